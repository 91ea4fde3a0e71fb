"""Benchmark of the 4-bit DiT linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: the MLP up-projection of a FLUX-class DiT block at 1024x1024
(4096 image + 512 text tokens): X bf16 [4608, 3072] with Student-t(3)
activations, W [3072, 12288] split into a rank-32 bf16 low-rank part (L1, L2) and
an MXFP4 residual R.  One step is one pass of the layer's hot path on inputs
already resident in HBM:

    quantize_act (MXFP4 codes + E8M0 scales of X, fused t = X L1)
    gemm_w4a4_lowrank (FP4 x FP4 block-scaled MFMA, t L2 + store in the epilogue)

The residual weight is packed once before timing (offline, as in deployment).
Eight independent input sets (about 460 MB, more than the 256 MB Infinity Cache)
are rotated so repeated steps cannot be served from the last-level cache.

Prints one JSON line: value = effective W4A4 TFLOP/s of the whole step
(2 M N K / step time; the low-rank flops are not counted), the GEMM kernel's
roofline (its own average duration from HIP events around every GEMM launch in
the timed region, against the MI355X dense MXFP4 peak), and the CPU oracle timed
on the host cores on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, K, N, RANK = 4608, 3072, 12288, 32
N_SETS = 8
MXFP4_PEAK_TFLOPS = 10100.0        # MI355X dense MXFP4 MFMA, published
HBM_PEAK_GBS = 8000.0
METRIC = "W4A4 FP4 GEMM effective TFLOPS + % MXFP4 MFMA peak at M=4608 K=3072 N=12288"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mx_traffic.json")
KERNEL_SOURCES = ["gemm_mx.hip", "q4_epilogue.h", "q4_device.h"]


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "bit_quantized_gemm_quantize_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter runs, if they
    were taken on the current GEMM kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(d, budget_s=12.0):
    """The CPU oracle as it stands, on a bounded sample of the step: quantize a
    block of rows of X, dequantize, fp64 GEMM against the (pre-dequantized)
    residual weight with the low-rank branch and the error bound.  Rows are added in
    chunks until the time budget is used; throughput is scaled to TFLOP/s of
    2 * rows * N * K."""
    import oracle
    from threadpoolctl import threadpool_info
    F, Q, L = oracle.formats, oracle.quant, oracle.layer
    B = Q.mx_dequantize(*Q.mx_quantize(d["rt"]))          # offline weight packing, untimed
    L1, L2 = F.bf16_to_f64(d["l1"]), F.bf16_to_f64(d["l2"])
    chunk = 256
    rows = 0
    t0 = time.perf_counter()
    while rows < M and time.perf_counter() - t0 < budget_s:
        xs = d["x"][rows:rows + chunk]
        A = Q.mx_dequantize(*Q.mx_quantize(xs))
        L.gemm_ref(A, B, x=F.bf16_to_f64(xs), l1=L1, l2=L2)
        rows += xs.shape[0]
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} of {M} rows of X through quantize + dequantize + fp64 GEMM "
                      f"(+ low-rank, + error bound) against all {N} columns; {dt:.1f} s"}


GEMM_KERNEL_PREFIX = "void q4::gemm_mx_kernel<32, false, 0>"
QUANT_KERNEL_PREFIX = "void q4::quant_act_kernel<0, 32, false>"
QUANT_SOURCES = ["quant.hip", "q4_device.h"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"
CAL_BYTES = 256 * 2 ** 20          # the calibration copy below: 64 Mi fp32 in, 64 Mi fp32 out


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def timed_region_avg_ns(trace_csv, steps):
    """Average duration of the GEMM over its last `steps` dispatches in a rocprofv3
    kernel trace: the launches of the timed region (the warmup launches come first)."""
    rows = [r for r in _csv_rows(trace_csv) if r["Kernel_Name"].startswith(GEMM_KERNEL_PREFIX)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows[-steps:]]
    return float(np.mean(d)) if d else None


def summarize_profiles(stats_csv, fetch_csv, write_csv, command, trace_csv=None, steps=None,
                       bench_log=None, util_csv=None):
    """Turns the rocprofv3 outputs of a bench run (one --kernel-trace --stats run,
    one --pmc FETCH_SIZE run, one --pmc WRITE_SIZE run, and optionally one --pmc run
    of the SQ/GRBM utilisation counters) into the committed text summary and the
    traffic record read by measured_traffic().  HBM bytes of a kernel are the
    counters' per-dispatch KiB, each scaled by the ratio of the bytes the
    calibration copy really moves to what the same counter reports for it."""
    lines = [f"# rocprofv3 summary: MXFP4 W4A4 GEMM + low-rank epilogue, M={M} K={K} N={N} r={RANK}",
             "", "commands (R = the repository root; each run after `cd /tmp && export TMPDIR=/tmp`):", ""]
    lines += ["    " + c for c in command]
    lines += ["", "## kernel stats (--kernel-trace --stats)", "",
              "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    gemm_avg_ns = None
    for r in _csv_rows(stats_csv):
        name = r["Name"]
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
        if name.startswith(GEMM_KERNEL_PREFIX):
            gemm_avg_ns = float(r["AverageNs"])

    def per_dispatch(path, counter, prefix=GEMM_KERNEL_PREFIX):
        vals = {}
        for r in _csv_rows(path):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        kern = [v for k, d in vals.items() if k.startswith(prefix) for v in d.values()]
        cal = [v for k, d in vals.items() if k.startswith(COPY_KERNEL) for v in d.values()]
        return float(np.mean(kern)), float(np.max(cal))

    fetch_kib, cal_fetch_kib = per_dispatch(fetch_csv, "FETCH_SIZE")
    write_kib, cal_write_kib = per_dispatch(write_csv, "WRITE_SIZE")
    q_fetch_kib, _ = per_dispatch(fetch_csv, "FETCH_SIZE", QUANT_KERNEL_PREFIX)
    q_write_kib, _ = per_dispatch(write_csv, "WRITE_SIZE", QUANT_KERNEL_PREFIX)
    f_scale = CAL_BYTES / (cal_fetch_kib * 1024.0)
    w_scale = CAL_BYTES / (cal_write_kib * 1024.0)
    fetch_b, write_b = fetch_kib * 1024.0 * f_scale, write_kib * 1024.0 * w_scale
    alg_in = M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + M * RANK * 4 + N * RANK * 2
    alg_out = M * N * 2
    lines += ["", "## HBM traffic of the GEMM (--pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              f"calibration copy `{COPY_KERNEL}` of {CAL_BYTES} bytes: FETCH_SIZE {cal_fetch_kib:.0f} KiB, "
              f"WRITE_SIZE {cal_write_kib:.0f} KiB -> scale {f_scale:.4f} (fetch), {w_scale:.4f} (write)", "",
              f"GEMM per dispatch: FETCH_SIZE {fetch_kib:.0f} KiB -> {fetch_b / 1e6:.2f} MB; "
              f"WRITE_SIZE {write_kib:.0f} KiB -> {write_b / 1e6:.2f} MB", "",
              f"algorithmic bytes per launch: read {alg_in / 1e6:.2f} MB (A, B codes + scales, t, L2^T), "
              f"write {alg_out / 1e6:.2f} MB (Y bf16); measured / algorithmic = "
              f"{(fetch_b + write_b) / (alg_in + alg_out):.3f}"]
    # the fused quantizer of the same step: reads X (bf16) and L1^T, writes codes,
    # scales and t (fp32)
    q_fetch_b, q_write_b = q_fetch_kib * 1024.0 * f_scale, q_write_kib * 1024.0 * w_scale
    q_alg_in = M * K * 2 + K * RANK * 2
    q_alg_out = M * K // 2 + M * K // 32 + M * RANK * 4
    lines += ["", "## HBM traffic of the fused quantizer (same two --pmc runs)", "",
              f"`{QUANT_KERNEL_PREFIX[5:]}` per dispatch: FETCH_SIZE {q_fetch_kib:.0f} KiB -> "
              f"{q_fetch_b / 1e6:.2f} MB; WRITE_SIZE {q_write_kib:.0f} KiB -> {q_write_b / 1e6:.2f} MB", "",
              f"algorithmic bytes per launch: read {q_alg_in / 1e6:.2f} MB (X bf16, L1^T), write "
              f"{q_alg_out / 1e6:.2f} MB (codes, scales, t fp32); measured / algorithmic = "
              f"{(q_fetch_b + q_write_b) / (q_alg_in + q_alg_out):.3f}"]
    util = None
    if util_csv:
        # per dispatch: counters summed over the chip's instances.  SQ_BUSY_CYCLES sums
        # over the 32 shader engines, SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs and
        # GRBM_GUI_ACTIVE over the 8 XCDs (its window also spans the dispatch set-up).
        acc = {}
        for r in _csv_rows(util_csv):
            if not r["Kernel_Name"].startswith(GEMM_KERNEL_PREFIX):
                continue
            d = acc.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        disp = [acc[k] for k in sorted(acc, key=int)][-max(1, len(acc) // 4):]
        mean = {c: float(np.mean([d[c] for d in disp])) for c in disp[0]}
        se_cycles = mean["SQ_BUSY_CYCLES"] / 32.0
        mfma_simd = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0
        grbm_xcd = mean["GRBM_GUI_ACTIVE"] / 8.0
        util = {"mfma_busy_per_simd": mfma_simd, "sq_busy_cycles_per_se": se_cycles,
                "grbm_gui_active_per_xcd": grbm_xcd,
                "mfma_util_vs_sq_busy": mfma_simd / se_cycles,
                "mfma_util_vs_grbm": mfma_simd / grbm_xcd,
                "wait_any_frac": mean["SQ_WAIT_ANY"] / mean["SQ_WAVE_CYCLES"],
                "lds_bank_conflict_per_active": mean["SQ_LDS_BANK_CONFLICT"] / max(mean["SQ_LDS_IDX_ACTIVE"], 1.0)}
        lines += ["", "## MFMA utilisation of the GEMM (--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
                      "GRBM_GUI_ACTIVE SQ_WAIT_ANY SQ_WAVE_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT)", "",
                  f"last {len(disp)} dispatches of {len(acc)}: MFMA busy {mfma_simd:.0f} cycles per SIMD "
                  f"(SQ_VALU_MFMA_BUSY_CYCLES / 1024); shader-engine busy {se_cycles:.0f} cycles "
                  f"(SQ_BUSY_CYCLES / 32); GPU busy {grbm_xcd:.0f} cycles (GRBM_GUI_ACTIVE / 8)", "",
                  f"MFMA busy / SQ busy = {100 * util['mfma_util_vs_sq_busy']:.1f}%; "
                  f"MFMA busy / GPU busy = {100 * util['mfma_util_vs_grbm']:.1f}%; "
                  f"SQ_WAIT_ANY / SQ_WAVE_CYCLES = {100 * util['wait_any_frac']:.1f}%; "
                  f"LDS bank-conflict cycles per LDS-active cycle = {util['lds_bank_conflict_per_active']:.3f}"]
    if trace_csv and steps:
        timed_ns = timed_region_avg_ns(trace_csv, steps)
        if timed_ns:
            lines += ["", f"GEMM average over the timed region (last {steps} dispatches of the kernel trace, "
                          f"the launches bench.py times with HIP events): {timed_ns / 1e3:.2f} us -> "
                          f"{2.0 * M * N * K / (timed_ns * 1e-9) / 1e12:.1f} TFLOP/s "
                          f"({100 * 2.0 * M * N * K / (timed_ns * 1e-9) / 1e12 / MXFP4_PEAK_TFLOPS:.1f}% "
                          f"of {MXFP4_PEAK_TFLOPS:.0f}); the stats average above also covers the warmup "
                          f"launches, run while the clocks ramp up"]
    if bench_log:
        with open(bench_log) as f:
            recs = [json.loads(l) for l in f if l.startswith("{")]
        if recs and "roofline" in recs[-1]:
            ev_ms = recs[-1]["roofline"]["avg_launch_ms"]
            lines += ["", f"bench.py's own line from the same profiled run: GEMM {ev_ms * 1e3:.2f} us by HIP "
                          f"events around each launch (the events add the gap between the event and "
                          f"the dispatch to the kernel's own duration)"]
    if gemm_avg_ns:
        lines += ["", f"GEMM average duration {gemm_avg_ns / 1e3:.2f} us -> "
                      f"{2.0 * M * N * K / (gemm_avg_ns * 1e-9) / 1e12:.1f} TFLOP/s "
                      f"({100 * 2.0 * M * N * K / (gemm_avg_ns * 1e-9) / 1e12 / MXFP4_PEAK_TFLOPS:.1f}% "
                      f"of {MXFP4_PEAK_TFLOPS:.0f})"]
    rec = {"kernel_source_hash": kernel_source_hash(), "hbm_bytes_per_launch": round(fetch_b + write_b),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "fetch_scale": f_scale, "write_scale": w_scale, "gemm_avg_us": gemm_avg_ns and gemm_avg_ns / 1e3,
           "quant_source_hash": kernel_source_hash(QUANT_SOURCES),
           "quant_hbm_bytes_per_launch": round(q_fetch_b + q_write_b), "gemm_util": util}
    return "\n".join(lines) + "\n", rec


def bench_rows(reps=50):
    """Times every other step of the path on its own workload and prints one JSON
    line per row: the quantizers and packers against the HBM peak (algorithmic
    bytes: X read once, codes and scales written once), the GEMMs against their MFMA
    peak, and W4A16 next to a plain bf16 GEMM (torch, hipBLASLt) of the same shape."""
    import torch
    from bit_quantized_gemm_quantize_amd import binding as B
    from bit_quantized_gemm_quantize_amd import synth, weight_prep

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def timed(fn, n_sets):
        # The clocks need about 40 ms of sustained load to settle after an idle gap
        # (the host work between rows is one): run about 80 ms of this launch back to
        # back, sized from one cold launch, before the timed launches.
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(1 % n_sets)
        e1.record(stream)
        torch.cuda.synchronize()
        n_warm = max(3, min(20000, int(80.0 / max(e0.elapsed_time(e1), 1e-3))))
        for i in range(n_warm):
            fn(i % n_sets)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            fn(i % n_sets)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def emit(row, ms, bytes_=None, flops=None, peak=None, note=""):
        rec = {"row": row, "us": round(ms * 1e3, 2)}
        if bytes_ is not None:
            gbs = bytes_ / (ms * 1e-3) / 1e9
            rec.update({"GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes": int(bytes_)})
        if flops is not None:
            tf = flops / (ms * 1e-3) / 1e12
            rec.update({"TFLOP/s": round(tf, 1), "peak": peak, "frac": round(tf / peak, 4)})
        if note:
            rec["note"] = note
        print(json.dumps(rec), flush=True)

    # ---- a1 + a3: MXFP4 activation quantizer (+ t = X L1), rotating 10 copies of X
    Mq, Kq = 4608, 3072
    x0 = bf16_dev(synth.activations(Mq, Kq, seed=0, dist="student_t3")[0])
    xs = [x0] + [x0.clone() for _ in range(9)]
    l1t = bf16_dev(synth.to_bf16_bits(np.random.default_rng(1).standard_normal((RANK, Kq)) * 0.05))
    ac, asc, _ = B.empty_quant("mxfp4", Mq, Kq, dev)
    tq = torch.empty((Mq, RANK), dtype=torch.float32, device=dev)
    for r in (0, RANK):
        ms = timed(lambda i: B.quantize_act("mxfp4", xs[i], ac, asc, None, l1t if r else None,
                                            tq if r else None, stream), len(xs))
        nbytes = 2 * Mq * Kq + Mq * Kq // 2 + Mq * Kq // 32 + (4 * Mq * r + 2 * Kq * r)
        emit(f"quantize_act mxfp4 r={r} {Mq}x{Kq}", ms, bytes_=nbytes,
             note="10 rotating copies of X (283 MB)")
    del xs

    # ---- a2: NVFP4 activation quantizer, QKV shape, 3 rotating copies of X (311 MB)
    Mn, Kn, Nn = 16896, 3072, 9216
    xn0 = bf16_dev(synth.qkv_nvfp4(step=0)["x"])
    xns = [xn0, xn0.clone(), xn0.clone()]
    nc, nsc, nts = B.empty_quant("nvfp4", Mn, Kn, dev)
    ms = timed(lambda i: B.quantize_act("nvfp4", xns[i], nc, nsc, nts, stream=stream), len(xns))
    emit(f"quantize_act nvfp4 {Mn}x{Kn}", ms, bytes_=2 * Mn * Kn + Mn * Kn // 2 + Mn * Kn // 16 + 4,
         note="algorithmic bytes count one read of X; the tensor amax pass reads it a second time")

    # ---- a7: NVFP4 GEMM, QKV shape
    wq = bf16_dev(synth.qkv_nvfp4_weight())
    bnc, bnsc, bnts = B.empty_quant("nvfp4", Nn, Kn, dev)
    B.pack_weights("nvfp4", wq, Kn, Nn, 1, Kn, bnc, bnsc, tensor_scale=bnts, stream=stream)
    yq = torch.empty((Mn, Nn), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda i: B.gemm_w4a4("nvfp4", nc, nsc, nts, bnc, bnsc, bnts, Mn, Nn, Kn, yq,
                                     stream=stream), 1)
    emit(f"gemm_w4a4 nvfp4 {Mn}x{Kn}x{Nn}", ms, flops=2.0 * Mn * Nn * Kn, peak=2500.0,
         note="exact fp16 dequant + fp16 MFMA; peak = dense bf16 and fp16 (2.5 PF)")
    del xns, xn0, yq, wq

    # ---- a4: packers, MLP up-projection residual weight [N, K]
    Np = 12288
    wt = bf16_dev(synth.weights(Np, Kq, seed=0))
    bc, bsc, _ = B.empty_quant("mxfp4", Np, Kq, dev)
    ms = timed(lambda i: B.pack_weights("mxfp4", wt, Kq, Np, 1, Kq, bc, bsc, stream=stream), 1)
    emit(f"pack_weights mxfp4 {Np}x{Kq}", ms, bytes_=2 * Np * Kq + Np * Kq // 2 + Np * Kq // 32,
         note="offline step")
    ic, isc, izc = B.empty_quant("int4_g64", Np, Kq, dev)
    ms = timed(lambda i: B.pack_weights("int4_g64", wt, Kq, Np, 1, Kq, ic, isc, izc, stream=stream), 1)
    emit(f"pack_weights int4_g64 {Np}x{Kq}", ms, bytes_=2 * Np * Kq + Np * Kq // 2 + Np * Kq // 16,
         note="offline step")

    # ---- a5: MXFP4 GEMM without the branch, MLP and attention-projection shapes
    B.quantize_act("mxfp4", x0, ac, asc, stream=stream)
    for n in (12288, 3072):
        y = torch.empty((Mq, n), dtype=torch.bfloat16, device=dev)
        ms = timed(lambda i: B.gemm_w4a4("mxfp4", ac, asc, None, bc[:n], bsc[:n], None, Mq, n, Kq, y,
                                         stream=stream), 1)
        emit(f"gemm_w4a4 mxfp4 {Mq}x{Kq}x{n} bf16 out", ms, flops=2.0 * Mq * n * Kq,
             peak=MXFP4_PEAK_TFLOPS, note="inputs warm in L2/MALL")

    # ---- the attention-projection step as one measured pass: quantize_act (MXFP4,
    # no branch) of X, then gemm_w4a4 into bf16, over 8 rotating sets of X (1% outlier
    # channels) and packed W (8 x 33 MB, more than the last-level cache holds)
    Na, n_sets_a = 3072, 8
    sets_a = []
    for j in range(n_sets_a):
        da = synth.attn_proj(seed=j, M=Mq, K=Kq, N=Na)
        wa = bf16_dev(da["wt"])
        wc_, ws_, _ = B.empty_quant("mxfp4", Na, Kq, dev)
        B.pack_weights("mxfp4", wa, Kq, Na, 1, Kq, wc_, ws_, stream=stream)
        xc_, xs_, _ = B.empty_quant("mxfp4", Mq, Kq, dev)
        sets_a.append((bf16_dev(da["x"]), wc_, ws_, xc_, xs_))
        del wa
    ya = torch.empty((Mq, Na), dtype=torch.bfloat16, device=dev)

    def attn_step(i):
        xa, wc_, ws_, xc_, xs_ = sets_a[i]
        B.quantize_act("mxfp4", xa, xc_, xs_, stream=stream)
        B.gemm_w4a4("mxfp4", xc_, xs_, None, wc_, ws_, None, Mq, Na, Kq, ya, stream=stream)
    ms = timed(attn_step, n_sets_a)
    emit(f"step quantize_act + gemm_w4a4 mxfp4 {Mq}x{Kq}x{Na}", ms, flops=2.0 * Mq * Na * Kq,
         peak=MXFP4_PEAK_TFLOPS, note="attention projection at 1024^2 as one pass: X quantized, then "
                                      "multiplied; 8 rotating sets of X and W, cold in HBM")
    del sets_a, ya

    # ---- f1: the MXFP4-emitting epilogue at the MLP up-projection with the rank-32
    # branch, against the unfused pair (bf16 store, then quantize_act reading it back)
    dm = weight_prep.mlp_up_svd(seed=0)
    tq2 = torch.empty((Mq, RANK), dtype=torch.float32, device=dev)
    l1m = bf16_dev(np.ascontiguousarray(dm["l1"].T))
    l2m = bf16_dev(np.ascontiguousarray(dm["l2"].T))
    bcm, bsm, _ = B.empty_quant("mxfp4", Np, Kq, dev)
    B.pack_weights("mxfp4", bf16_dev(dm["rt"]), Kq, Np, 1, Kq, bcm, bsm, stream=stream)
    acm, asm_, _ = B.empty_quant("mxfp4", Mq, Kq, dev)
    B.quantize_act("mxfp4", bf16_dev(dm["x"]), acm, asm_, l1t=l1m, t=tq2, stream=stream)
    yq_c, yq_s, _ = B.empty_quant("mxfp4", Mq, Np, dev)
    ym = torch.empty((Mq, Np), dtype=torch.bfloat16, device=dev)
    ms_f = timed(lambda i: B.gemm_w4a4_lowrank_mxout(acm, asm_, bcm, bsm, Mq, Np, Kq, yq_c, yq_s, t=tq2,
                                                     l2t=l2m, stream=stream), 1)
    emit(f"gemm_w4a4_lowrank_mxout mxfp4 {Mq}x{Kq}x{Np} r={RANK}", ms_f, flops=2.0 * Mq * Np * Kq,
         peak=MXFP4_PEAK_TFLOPS, note="output as MXFP4 codes + scales for the next layer (no bf16 store)")

    def unfused(i):
        B.gemm_w4a4_lowrank("mxfp4", acm, asm_, None, bcm, bsm, None, Mq, Np, Kq, tq2, l2m, ym, stream=stream)
        B.quantize_act("mxfp4", ym, yq_c, yq_s, stream=stream)
    ms_u = timed(unfused, 1)
    emit(f"gemm_w4a4_lowrank + quantize_act {Mq}x{Kq}x{Np} r={RANK}", ms_u, flops=2.0 * Mq * Np * Kq,
         peak=MXFP4_PEAK_TFLOPS, note=f"unfused: bf16 Y stored and read back; fused saves "
                                      f"{(ms_u - ms_f) * 1e3:.1f} us")

    # ---- f1: the SwiGLU epilogue on the same operands read as 6144 gate/up pairs
    # (weight rows grouped 32 gate + 32 up), against the GEMM's bf16 store followed by
    # torch's silu and product
    ysw = torch.empty((Mq, Np // 2), dtype=torch.bfloat16, device=dev)
    ms_s = timed(lambda i: B.gemm_w4a4_lowrank_swiglu(acm, asm_, bcm, bsm, Mq, Np, Kq, ysw, t=tq2, l2t=l2m,
                                                      stream=stream), 1)
    emit(f"gemm_w4a4_lowrank_swiglu mxfp4 {Mq}x{Kq}x{Np} r={RANK}", ms_s, flops=2.0 * Mq * Np * Kq,
         peak=MXFP4_PEAK_TFLOPS, note="SwiGLU epilogue: bf16 [M, N/2] out")

    def unfused_swiglu(i):
        B.gemm_w4a4_lowrank("mxfp4", acm, asm_, None, bcm, bsm, None, Mq, Np, Kq, tq2, l2m, ym, stream=stream)
        gu = ym.view(Mq, Np // 64, 2, 32)
        torch.mul(torch.nn.functional.silu(gu[:, :, 0, :]), gu[:, :, 1, :], out=ysw.view(Mq, Np // 64, 32))
    ms_su = timed(unfused_swiglu, 1)
    emit(f"gemm_w4a4_lowrank + torch silu*up {Mq}x{Kq}x{Np} r={RANK}", ms_su, flops=2.0 * Mq * Np * Kq,
         peak=MXFP4_PEAK_TFLOPS, note=f"unfused comparison; the fused epilogue saves {(ms_su - ms_s) * 1e3:.1f} us")
    del ysw

    # ---- f1: the QKV-split + RoPE epilogue on a fused QKV projection (3072 -> 3 x
    # 3072, head width 128), against the GEMM's bf16 store followed by torch's split
    # and rotation
    dq = weight_prep.mlp_up_svd(seed=1, N=9216)
    bcq, bsq, _ = B.empty_quant("mxfp4", 9216, Kq, dev)
    B.pack_weights("mxfp4", bf16_dev(dq["rt"]), Kq, 9216, 1, Kq, bcq, bsq, stream=stream)
    l2q = bf16_dev(np.ascontiguousarray(dq["l2"].T))
    hd = 128
    pos = torch.arange(Mq, device=dev, dtype=torch.float32)[:, None]
    ang = pos * (10000.0 ** (-torch.arange(hd // 2, device=dev, dtype=torch.float32) * 2.0 / hd))[None, :]
    csq = torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).contiguous()
    yqkv = [torch.empty((Mq, 3072), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    ms_q = timed(lambda i: B.gemm_w4a4_lowrank_qkv_rope(acm, asm_, bcq, bsq, Mq, 9216, Kq, *yqkv, t=tq2,
                                                        l2t=l2q, cs=csq, head_dim=hd, stream=stream), 1)
    emit(f"gemm_w4a4_lowrank_qkv_rope mxfp4 {Mq}x{Kq}x9216 r={RANK}", ms_q, flops=2.0 * Mq * 9216 * Kq,
         peak=MXFP4_PEAK_TFLOPS, note="Q, K, V outputs, RoPE on Q and K (head width 128)")
    yfull = torch.empty((Mq, 9216), dtype=torch.bfloat16, device=dev)
    cq, sq = csq[..., 0].repeat(1, 3072 // hd), csq[..., 1].repeat(1, 3072 // hd)

    def unfused_qkv(i):
        B.gemm_w4a4_lowrank("mxfp4", acm, asm_, None, bcq, bsq, None, Mq, 9216, Kq, tq2, l2q, yfull,
                            stream=stream)
        for sec in range(2):
            part = yfull[:, 3072 * sec:3072 * (sec + 1)].float()
            a, b = part[:, 0::2], part[:, 1::2]
            out = yqkv[sec].view(Mq, 3072 // 2, 2)
            out[:, :, 0] = (a * cq - b * sq).to(torch.bfloat16)
            out[:, :, 1] = (a * sq + b * cq).to(torch.bfloat16)
        yqkv[2].copy_(yfull[:, 6144:])
    ms_qu = timed(unfused_qkv, 1)
    emit(f"gemm_w4a4_lowrank + torch split/rope {Mq}x{Kq}x9216 r={RANK}", ms_qu, flops=2.0 * Mq * 9216 * Kq,
         peak=MXFP4_PEAK_TFLOPS, note=f"unfused comparison; the fused epilogue saves {(ms_qu - ms_q) * 1e3:.1f} us")
    del dq, yqkv, yfull
    del dm, ym

    # ---- f3: symmetric INT4 W4A4 on the INT8 MFMA (no 4-bit integer matrix
    # instruction on gfx950), same activations and weight as the MXFP4 row above
    xi, xis, _ = B.empty_quant("int4_sym", Mq, Kq, dev)
    B.quantize_act("int4_sym", x0, xi, xis, stream=stream)
    wi, wis, _ = B.empty_quant("int4_sym", Np, Kq, dev)
    B.pack_weights("int4_sym", wt, Kq, Np, 1, Kq, wi, wis, stream=stream)
    yi = torch.empty((Mq, Np), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda i: B.gemm_w4a4("int4_sym", xi, xis, None, wi, wis, None, Mq, Np, Kq, yi, stream=stream), 1)
    emit(f"gemm_w4a4 int4_sym {Mq}x{Kq}x{Np} bf16 out", ms, flops=2.0 * Mq * Np * Kq, peak=5000.0,
         note="int4 widened to int8 for the INT8 MFMA; peak = dense INT8 5.0 POP/s")
    ms = timed(lambda i: B.quantize_act("int4_sym", x0, xi, xis, stream=stream), 1)
    emit(f"quantize_act int4_sym {Mq}x{Kq}", ms, bytes_=2 * Mq * Kq + Mq * Kq // 2 + 4 * Mq,
         note="one wave per row, the row read once into registers (amax, then codes)")
    del yi, xi, wi

    # ---- f4: MXFP8 W8A8 on the same block-scaled MFMA with E4M3 operands
    x8, x8s, _ = B.empty_quant("mxfp8", Mq, Kq, dev)
    B.quantize_act("mxfp8", x0, x8, x8s, stream=stream)
    w8, w8s, _ = B.empty_quant("mxfp8", Np, Kq, dev)
    B.pack_weights("mxfp8", wt, Kq, Np, 1, Kq, w8, w8s, stream=stream)
    y8 = torch.empty((Mq, Np), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda i: B.gemm_w4a4("mxfp8", x8, x8s, None, w8, w8s, None, Mq, Np, Kq, y8, stream=stream), 1)
    emit(f"gemm_w4a4 mxfp8 {Mq}x{Kq}x{Np} bf16 out", ms, flops=2.0 * Mq * Np * Kq, peak=5000.0,
         note="E4M3 x E4M3 with E8M0 block scales; peak = dense FP8 5.0 PFLOP/s")
    ms = timed(lambda i: B.quantize_act("mxfp8", x0, x8, x8s, stream=stream), 1)
    emit(f"quantize_act mxfp8 {Mq}x{Kq}", ms, bytes_=2 * Mq * Kq + Mq * Kq + Mq * Kq // 32)
    try:
        a8v, b8v = x8.view(torch.float8_e4m3fn), w8.view(torch.float8_e4m3fn)
        sa8, sb8 = x8s.view(torch.float8_e8m0fnu), w8s.view(torch.float8_e8m0fnu)
        y_lib = torch._scaled_mm(a8v, b8v.t(), sa8, sb8, out_dtype=torch.bfloat16)
        diff = (y_lib.float() - y8.float()).abs().max().item() / max(y8.float().abs().max().item(), 1e-30)
        ms = timed(lambda i: torch._scaled_mm(a8v, b8v.t(), sa8, sb8, out_dtype=torch.bfloat16), 1)
        emit(f"torch._scaled_mm mxfp8 {Mq}x{Kq}x{Np} bf16 out", ms, flops=2.0 * Mq * Np * Kq, peak=5000.0,
             note=f"comparison: hipBLASLt MXFP8 on the same codes and scales; max |diff| / max |y| "
                  f"vs gemm_w4a4 = {diff:.2e}")
    except (RuntimeError, TypeError, AttributeError) as e:
        print(json.dumps({"row": "torch._scaled_mm mxfp8", "note": f"unavailable: {str(e)[:200]}"}),
              flush=True)
    del y8, x8, w8

    # ---- f4: FP8 attention at the FLUX-class joint attention of a 1024x1024 image
    # (4096 image + 512 text tokens, 24 heads of 128), Gaussian Q, K, V
    Sa, Ha = 4608, 24
    rng_a = np.random.default_rng(7)
    qa, ka, va = (bf16_dev(synth.to_bf16_bits(rng_a.standard_normal((Sa, Ha * 128)).astype(np.float32)))
                  for _ in range(3))
    ab = B.attn_buffers(1, Sa, Ha, dev)
    oa = torch.empty((Sa, Ha * 128), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda i: B.attention_fp8_quantize(qa, ka, va, 1, Sa, Ha, ab, stream=stream), 1)
    emit(f"attention_fp8_quantize {Sa} tokens x {Ha} heads x 128", ms,
         bytes_=3 * Sa * Ha * 128 * 2 + 3 * Sa * Ha * (128 + 4),
         note="Q, K MXFP8 along head_dim, V MXFP8 along the keys (transposed)")
    ms = timed(lambda i: B.attention_fp8(ab, 1, Sa, Ha, oa, stream=stream), 1)
    emit(f"attention_fp8 {Sa} tokens x {Ha} heads x 128", ms, flops=4.0 * Sa * Sa * 128 * Ha, peak=5000.0,
         note="Q K^T and P V on the E4M3 block-scaled MFMA, online softmax over 64-key blocks; "
              "peak = dense FP8 5.0 PFLOP/s")
    del qa, ka, va, ab, oa

    # ---- comparison: the vendor MXFP4 GEMM (hipBLASLt through torch._scaled_mm) on
    # the same codes and E8M0 scales, row-major scale layout
    y = torch.empty((Mq, Np), dtype=torch.bfloat16, device=dev)
    B.gemm_w4a4("mxfp4", ac, asc, None, bc, bsc, None, Mq, Np, Kq, y, stream=stream)
    try:
        a4, b4 = ac.view(torch.float4_e2m1fn_x2), bc.view(torch.float4_e2m1fn_x2)
        sa8, sb8 = asc.view(torch.float8_e8m0fnu), bsc.view(torch.float8_e8m0fnu)
        y_lib = torch._scaled_mm(a4, b4.t(), sa8, sb8, out_dtype=torch.bfloat16)
        diff = (y_lib.float() - y.float()).abs().max().item() / max(y.float().abs().max().item(), 1e-30)
        ms = timed(lambda i: torch._scaled_mm(a4, b4.t(), sa8, sb8, out_dtype=torch.bfloat16), 1)
        emit(f"torch._scaled_mm mxfp4 {Mq}x{Kq}x{Np} bf16 out", ms, flops=2.0 * Mq * Np * Kq,
             peak=MXFP4_PEAK_TFLOPS,
             note=f"comparison: hipBLASLt MXFP4 on the same codes and scales; max |diff| / max |y| "
                  f"vs gemm_w4a4 = {diff:.2e}")
    except (RuntimeError, TypeError, AttributeError) as e:
        print(json.dumps({"row": "torch._scaled_mm mxfp4", "note": f"unavailable: {str(e)[:200]}"}),
              flush=True)
    del y

    # ---- a8: W4A16 against a plain bf16 GEMM of the same shape
    wbf = wt
    for m in (512, 4608):
        xw = x0[:m].contiguous()
        y = torch.empty((m, Np), dtype=torch.bfloat16, device=dev)
        ms = timed(lambda i: B.gemm_w4a16(xw, ic, isc, izc, Np, y, stream=stream), 1)
        emit(f"gemm_w4a16 {m}x{Kq}x{Np}", ms, flops=2.0 * m * Np * Kq, peak=2500.0,
             note="int4 g64 dequant in LDS + bf16 MFMA")
        ms = timed(lambda i: torch.matmul(xw, wbf.t(), out=y), 1)
        emit(f"torch bf16 matmul {m}x{Kq}x{Np}", ms, flops=2.0 * m * Np * Kq, peak=2500.0,
             note="comparison: hipBLASLt via torch, unquantized bf16 weight")

    # ---- f2: SVDQuant pre-conditioning on the attention projection (X N(0,1) with 1% of
    # channels x U(30,100)): the smoothed quantizer's time, and the layer's error against
    # the unquantized bf16 product for plain W4A4, the unsmoothed SVD split and SVDQuant
    # (GPU outputs on 64 sampled rows, reference in fp64 on the host)
    del x0, xw, wt, wbf, y
    d = weight_prep.attn_proj_svdquant(seed=0)
    Ms, Ks, Ns, rs = d["M"], d["K"], d["N"], d["rank"]
    xsv = bf16_dev(d["x"])
    xsl = [xsv] + [xsv.clone() for _ in range(9)]
    inv = torch.from_numpy(d["inv_s"]).to(dev)
    l1t_s = bf16_dev(np.ascontiguousarray(d["l1"].T))
    l2t_s = bf16_dev(np.ascontiguousarray(d["l2"].T))
    sc_, ss_, _ = B.empty_quant("mxfp4", Ms, Ks, dev)
    ts_ = torch.empty((Ms, rs), dtype=torch.float32, device=dev)
    ms = timed(lambda i: B.quantize_act_smooth("mxfp4", xsl[i], inv, sc_, ss_, l1t_s, ts_, stream), len(xsl))
    emit(f"quantize_act_smooth mxfp4 r={rs} {Ms}x{Ks}", ms,
         bytes_=2 * Ms * Ks + Ms * Ks // 2 + Ms * Ks // 32 + 4 * Ks + 4 * Ms * rs + 2 * Ks * rs,
         note="SmoothQuant factors applied in the quantizer; 10 rotating copies of X")
    del xsl
    rows_q = np.sort(np.random.default_rng(1).choice(Ms, 64, replace=False))
    xf = synth.bf16_bits_to_f32(d["x"][rows_q]).astype(np.float64)
    exact = xf @ synth.bf16_bits_to_f32(d["wt"]).astype(np.float64).T

    def layer_err(wt_bits, l1_bits=None, l2_bits=None, smooth=False):
        bc_, bs_, _ = B.empty_quant("mxfp4", Ns, Ks, dev)
        B.pack_weights("mxfp4", bf16_dev(wt_bits), Ks, Ns, 1, Ks, bc_, bs_, stream=stream)
        yq = torch.empty((Ms, Ns), dtype=torch.float32, device=dev)
        if l1_bits is None:
            B.quantize_act("mxfp4", xsv, sc_, ss_, stream=stream)
            B.gemm_w4a4("mxfp4", sc_, ss_, None, bc_, bs_, None, Ms, Ns, Ks, yq, out=B.OUT_F32, stream=stream)
        else:
            l1d, l2d = bf16_dev(np.ascontiguousarray(l1_bits.T)), bf16_dev(np.ascontiguousarray(l2_bits.T))
            if smooth:
                B.quantize_act_smooth("mxfp4", xsv, inv, sc_, ss_, l1d, ts_, stream)
            else:
                B.quantize_act("mxfp4", xsv, sc_, ss_, l1t=l1d, t=ts_, stream=stream)
            B.gemm_w4a4_lowrank("mxfp4", sc_, ss_, None, bc_, bs_, None, Ms, Ns, Ks, ts_, l2d, yq,
                                out=B.OUT_F32, stream=stream)
        torch.cuda.synchronize()
        yh = yq.cpu().numpy()[rows_q].astype(np.float64)
        return float(np.linalg.norm(yh - exact) / np.linalg.norm(exact))

    l1p, l2p, rtp = weight_prep.lowrank_split(d["wt"], rs, 0)
    gd = weight_prep.guide_step1_split(d["x_cal"], d["wt"], rs)
    errs = {"w4a4": layer_err(d["wt"]), "svd_split": layer_err(rtp, l1p, l2p),
            "guide_step1_literal": layer_err(gd["rt"], gd["l1"], gd["l2"]),
            "svdquant": layer_err(d["rt"], d["l1"], d["l2"], smooth=True)}
    print(json.dumps({"row": f"svdquant quality attn_proj {Ms}x{Ks}x{Ns} r={rs}",
                      "rel_error_vs_bf16_product": {k: round(v, 5) for k, v in errs.items()},
                      "note": "64 sampled rows; plain W4A4, the unsmoothed rank-32 SVD split, the "
                              "Guide's Step-1 recipe as printed (SVD of dW C, residual W - L1 L2), "
                              "and smoothing + activation-weighted rank-32 split"}), flush=True)


def bench_bf16_gemms(reps=50):
    """The GEMMs on the 16-bit MFMA and the vendor bf16 GEMM they are compared with,
    timed like the rows (one JSON line each): the NVFP4 GEMM at the fused-QKV shape
    (16896x3072x9216), W4A16 at M = 512 and 4608 (K = 3072, N = 12288), and torch's
    bf16 matmul (hipBLASLt) at the W4A16 shapes.  A short pass for counter runs."""
    import torch
    from bit_quantized_gemm_quantize_amd import binding as B
    from bit_quantized_gemm_quantize_amd import synth

    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        for _ in range(max(3, min(2000, int(80.0 / max(e0.elapsed_time(e1), 1e-3))))):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def emit(row, ms, flops):
        tf = flops / (ms * 1e-3) / 1e12
        print(json.dumps({"row": row, "us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1), "peak": 2500.0,
                          "frac": round(tf / 2500.0, 4)}), flush=True)

    Mn, Kn, Nn = 16896, 3072, 9216
    xn = bf16_dev(synth.qkv_nvfp4(step=0)["x"])
    nc, nsc, nts = B.empty_quant("nvfp4", Mn, Kn, dev)
    B.quantize_act("nvfp4", xn, nc, nsc, nts, stream=stream)
    wq = bf16_dev(synth.qkv_nvfp4_weight())
    bnc, bnsc, bnts = B.empty_quant("nvfp4", Nn, Kn, dev)
    B.pack_weights("nvfp4", wq, Kn, Nn, 1, Kn, bnc, bnsc, tensor_scale=bnts, stream=stream)
    yq = torch.empty((Mn, Nn), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: B.gemm_w4a4("nvfp4", nc, nsc, nts, bnc, bnsc, bnts, Mn, Nn, Kn, yq, stream=stream))
    emit(f"gemm_w4a4 nvfp4 {Mn}x{Kn}x{Nn}", ms, 2.0 * Mn * Nn * Kn)
    del xn, wq, yq

    Kq, Np = 3072, 12288
    wt = bf16_dev(synth.weights(Np, Kq, seed=0))
    ic, isc, izc = B.empty_quant("int4_g64", Np, Kq, dev)
    B.pack_weights("int4_g64", wt, Kq, Np, 1, Kq, ic, isc, izc, stream=stream)
    for m in (512, 4608):
        xw = bf16_dev(synth.activations(m, Kq, seed=m)[0])
        y = torch.empty((m, Np), dtype=torch.bfloat16, device=dev)
        ms = timed(lambda: B.gemm_w4a16(xw, ic, isc, izc, Np, y, stream=stream))
        emit(f"gemm_w4a16 {m}x{Kq}x{Np}", ms, 2.0 * m * Np * Kq)
        ms = timed(lambda: torch.matmul(xw, wt.t(), out=y))
        emit(f"torch bf16 matmul {m}x{Kq}x{Np}", ms, 2.0 * m * Np * Kq)


def _per_kernel_means(csv_path):
    """Counter means per kernel over the last quarter of its dispatches (each counter
    summed over the chip per dispatch), and the kernel's dispatch count."""
    acc = {}
    for r in _csv_rows(csv_path):
        d = acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for name, per in acc.items():
        disp = [per[k] for k in sorted(per, key=int)]
        disp = disp[-max(1, len(disp) // 4):]
        out[name] = ({c: float(np.mean([d.get(c, 0.0) for d in disp])) for c in disp[0]}, len(per))
    return out


def summarize_kernel_util(util_csv, stats_csv, command, title, lds_csv=None):
    """Per kernel of a rocprofv3 --pmc run of the utilisation counters: the MFMA pipe's
    busy cycles against the shader engines' busy cycles and the GPU's, and the share
    of wave cycles spent waiting, averaged over the last quarter of each kernel's
    dispatches; with the kernel's average duration from a --stats run and, from a
    second --pmc run (lds_csv), its LDS-active cycles per shader-engine busy cycle and
    the bank-conflict share of them."""
    util = _per_kernel_means(util_csv)
    lds = _per_kernel_means(lds_csv) if lds_csv else {}
    dur = {r["Name"]: float(r["AverageNs"]) / 1e3 for r in _csv_rows(stats_csv)} if stats_csv else {}
    lines = [f"# rocprofv3 summary: {title}", "",
             "commands (R = the repository root; each run after `cd /tmp && export TMPDIR=/tmp`):", ""]
    lines += ["    " + c for c in command]
    lines += ["", "Counters per dispatch, summed over the chip: SQ_VALU_MFMA_BUSY_CYCLES over the 1024 "
                  "SIMDs, SQ_BUSY_CYCLES over the 32 shader engines, GRBM_GUI_ACTIVE over the 8 XCDs; "
                  "the last quarter of each kernel's dispatches (settled clocks).", "",
              "| kernel | dispatches | average us (stats run) | MFMA busy / SQ busy | MFMA busy / GPU busy | "
              "SQ_WAIT_ANY / SQ_WAVE_CYCLES | SQ_LDS_IDX_ACTIVE / SQ_BUSY_CYCLES | "
              "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE |", "|---|---|---|---|---|---|---|---|"]
    for name, (mean, n) in sorted(util.items(), key=lambda kv: -kv[1][1]):
        if mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) <= 0:
            continue
        mfma = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        us = dur.get(name)
        lm = lds.get(name, ({}, 0))[0]
        lds_cols = (f"{lm['SQ_LDS_IDX_ACTIVE'] / lm['SQ_BUSY_CYCLES']:.2f} | "
                    f"{lm['SQ_LDS_BANK_CONFLICT'] / max(lm['SQ_LDS_IDX_ACTIVE'], 1.0):.2f}"
                    if lm.get("SQ_BUSY_CYCLES") else " | ")
        lines.append(f"| `{short[:90]}` | {n} | {'' if us is None else f'{us:.2f}'} | "
                     f"{100 * mfma / (mean['SQ_BUSY_CYCLES'] / 32.0):.1f}% | "
                     f"{100 * mfma / (mean['GRBM_GUI_ACTIVE'] / 8.0):.1f}% | "
                     f"{100 * mean['SQ_WAIT_ANY'] / mean['SQ_WAVE_CYCLES']:.1f}% | {lds_cols} |")
    lines += ["", "The LDS ratios are on the counters' own scale (both summed over the chip), for "
                  "comparing kernels with one another.", "",
              "Kernels named `Cijk_*` are hipBLASLt's bf16 GEMMs behind torch.matmul."]
    return "\n".join(lines) + "\n"


def summarize_rows_profile(stats_csv, command):
    """rocprofv3 --kernel-trace --stats of `bench.py --rows` -> a text table of every
    kernel's average duration (the per-row numbers' own kernels)."""
    lines = ["# rocprofv3 summary: every kernel of `bench.py --rows` (one MI355X)", "",
             "commands (R = the repository root; each run after `cd /tmp && export TMPDIR=/tmp`):", ""]
    lines += ["    " + c for c in command]
    lines += ["", "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in _csv_rows(stats_csv):
        short = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        lines.append(f"| `{short[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "Kernels named `Cijk_*` are hipBLASLt's bf16 GEMMs behind the torch comparison rows;",
              "`__amd_rocclr_*` are runtime copies and fills of the input setup."]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks ramp up over the first ~40 ms of sustained load (after an idle
    # gap the GEMM runs ~25% slower for ~250 steps), so the default warmup is 400 steps
    # (~65 ms) and the timed region 200 steps (~32 ms), both well inside a second.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    # a floor on the warmup's GPU time: when W steps take less (a faster kernel, a
    # smaller --warmup), whole batches of 50 more untimed steps run until it is met
    ap.add_argument("--min-warmup-ms", type=float, default=80.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rows", action="store_true",
                    help="time every other step of the path, one JSON line per row")
    ap.add_argument("--bf16-gemms", action="store_true",
                    help="time the NVFP4 and W4A16 GEMMs and the vendor bf16 GEMM, one JSON line each")
    ap.add_argument("--summarize-util", nargs=2, metavar=("UTIL_CSV", "STATS_CSV"),
                    help="write the per-kernel counter summary of a `--bf16-gemms` run under profiles/")
    ap.add_argument("--lds", metavar="LDS_CSV",
                    help="with --summarize-util: the counter_collection CSV of the --pmc "
                         "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES run")
    ap.add_argument("--summarize", nargs=3, metavar=("STATS_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write the rocprofv3 summary under profiles/ (no GPU needed)")
    ap.add_argument("--summarize-rows", metavar="STATS_CSV",
                    help="write the rocprofv3 summary of `bench.py --rows` under profiles/")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize: a command line that produced the inputs")
    ap.add_argument("--bench-log", metavar="LOG",
                    help="with --summarize: the output of the profiled bench.py run")
    ap.add_argument("--util", metavar="UTIL_CSV",
                    help="with --summarize: the counter_collection CSV of the --pmc SQ/GRBM "
                         "utilisation run")
    ap.add_argument("--trace", metavar="TRACE_CSV",
                    help="with --summarize: the kernel trace of the stats run; the GEMM average "
                         "over its last --steps dispatches is added")
    a = ap.parse_args()
    if a.summarize:
        text, rec = summarize_profiles(*a.summarize, a.command, trace_csv=a.trace, steps=a.steps,
                                       bench_log=a.bench_log, util_csv=a.util)
        with open(os.path.join(ROOT, "profiles", "gemm_mx_mlp_up_4608x3072x12288.md"), "w") as f:
            f.write(text)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(text)
        return
    if a.summarize_rows:
        text = summarize_rows_profile(a.summarize_rows, a.command)
        with open(os.path.join(ROOT, "profiles", "rows_kernels.md"), "w") as f:
            f.write(text)
        print(text)
        return
    if a.summarize_util:
        text = summarize_kernel_util(*a.summarize_util, a.command,
                                     "MFMA utilisation of the 16-bit-MFMA GEMMs and the vendor bf16 GEMM "
                                     "(`bench.py --bf16-gemms`, one MI355X)", lds_csv=a.lds)
        with open(os.path.join(ROOT, "profiles", "bf16_gemms_counters.md"), "w") as f:
            f.write(text)
        print(text)
        return
    if a.rows:
        bench_rows()
        return
    if a.bf16_gemms:
        bench_bf16_gemms()
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_quantized_gemm_quantize_amd import binding as B
    from bit_quantized_gemm_quantize_amd import synth, weight_prep

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs: one weight split, eight activation sets, all resident in HBM
    d = weight_prep.mlp_up_svd(seed=0)
    sets = []
    for i in range(N_SETS):
        x_bits = d["x"] if i == 0 else synth.activations(M, K, seed=i, dist="student_t3")[0]
        rt = bf16_dev(d["rt"])
        bc, bsc, _ = B.empty_quant("mxfp4", N, K, dev)
        B.pack_weights("mxfp4", rt, K, N, 1, K, bc, bsc)            # offline packing
        del rt
        ac, asc, _ = B.empty_quant("mxfp4", M, K, dev)
        sets.append(dict(x=bf16_dev(x_bits), l1t=bf16_dev(np.ascontiguousarray(d["l1"].T)),
                         l2t=bf16_dev(np.ascontiguousarray(d["l2"].T)), bc=bc, bsc=bsc, ac=ac,
                         asc=asc, t=torch.empty((M, RANK), dtype=torch.float32, device=dev)))
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    # a plain copy of known size: the scale for rocprofv3's FETCH_SIZE / WRITE_SIZE
    cal_src = torch.empty(64 * 2 ** 20, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()

    lib = B.load()
    stream = torch.cuda.current_stream()
    sp = B._stream(stream)

    def step(i, ev=None):
        s = sets[i % N_SETS]
        y = ys[i % 2]
        st = lib.quantize_act(B.MXFP4, B._ptr(s["x"]), M, K, K, B._ptr(s["ac"]), B._ptr(s["asc"]),
                              None, B._ptr(s["l1t"]), RANK, B._ptr(s["t"]), sp)
        if st:
            raise B.Q4Error("quantize_act", st)
        if ev is not None:
            ev[0].record(stream)
        st = lib.gemm_w4a4_lowrank(B.MXFP4, B._ptr(s["ac"]), B._ptr(s["asc"]), None, B._ptr(s["bc"]),
                                   B._ptr(s["bsc"]), None, M, N, K, B._ptr(s["t"]), B._ptr(s["l2t"]),
                                   RANK, None, B._ptr(y), N, B.OUT_BF16, sp)
        if st:
            raise B.Q4Error("gemm_w4a4_lowrank", st)
        if ev is not None:
            ev[1].record(stream)

    t_w = time.perf_counter()
    n_warm = 0
    for _ in range(a.warmup):
        step(n_warm)
        n_warm += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t_w) * 1e3 < a.min_warmup_ms:
        for _ in range(50):
            step(n_warm)
            n_warm += 1
        torch.cuda.synchronize()
    warmup_ms = (time.perf_counter() - t_w) * 1e3
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = [e0.elapsed_time(e1) for e0, e1 in events]
    gemm_ms = float(np.mean(ev_ms))
    # the last quarter of the timed steps: the clocks have settled longest there
    gemm_ms_lq = float(np.mean(ev_ms[-max(1, a.steps // 4):]))
    ms_per_step = wall * 1e3 / a.steps

    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "warmup_steps_run": n_warm,
        "warmup_ms": round(warmup_ms, 1),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4_e2m1",
        "data": "synthetic",
        "config": {"workload": "mlp_up_svd_r32_mxfp4_4608x3072x12288", "M": M, "K": K, "N": N,
                   "rank": RANK, "format": "mxfp4", "output": "bf16",
                   "step": "quantize_act(+X L1) -> gemm_w4a4_lowrank", "input_sets": N_SETS},
        "pct_of_mxfp4_peak": round(100.0 * value / MXFP4_PEAK_TFLOPS, 2),
        "roofline": {"kernel": "gemm_mx_kernel<32,false,0>", "bound": "mfma",
                     "achieved": round(gemm_tflops, 2), "peak": MXFP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / MXFP4_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(), "avg_launch_ms": round(gemm_ms, 5),
                     "avg_launch_ms_last_quarter": round(gemm_ms_lq, 5),
                     "algorithmic_flop_per_launch": flops},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
