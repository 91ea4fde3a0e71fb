"""GPU parity of the GEMMs against the CPU oracle.

The whole hot path runs on the device through the C ABI (quantize_act ->
pack_weights -> gemm_*); the oracle quantizes the same bf16 inputs itself and
computes the fp64 product.  Outputs must lie within the per-element bound
1e-3 * sum|products| (+ half a bf16 ulp for bf16 output), checked element by
element at sizes spanning several 256 x 256 tiles with ragged tails, and on
sampled rows at the full layer sizes in the configuration bench.py times."""

import numpy as np
import pytest
import torch

from bit_quantized_gemm_quantize_amd import binding as B
from bit_quantized_gemm_quantize_amd import synth, weight_prep
from oracle import formats as F
from oracle import layer as L
from oracle import quant as Q

from _gpu import bf16_dev, device, out_buffer, pack, quantize, say, y_host

pytestmark = pytest.mark.gpu


def _check(y, y_ref, bound, out_bf16, what):
    ok, worst, idx = L.check_close(y, y_ref, bound, out_bf16)
    assert ok, f"{what}: worst |err|/tol = {worst:.4g} at {idx}: gpu {y[idx]!r} ref {y_ref[idx]!r}"
    return worst


def run_w4a4(fmt, x, wt, dev, bias=None, f32=True, l1=None, l2=None, rows=None):
    """GPU: quantize X (+ t), pack W, GEMM (+ low-rank).  Returns host Y."""
    M, K = x.shape
    N = wt.shape[0]
    g = quantize(fmt, x, dev, l1_bits=l1)
    w = pack(fmt, wt, dev)
    y = out_buffer(M, N, dev, f32)
    b = bf16_dev(bias[None, :], dev)[0] if bias is not None else None
    out = B.OUT_F32 if f32 else B.OUT_BF16
    ats = g["ts"] if fmt == "nvfp4" else None
    bts = w["extra"] if fmt == "nvfp4" else None
    if l1 is None:
        B.gemm_w4a4(fmt, g["codes"], g["scales"], ats, w["codes"], w["scales"], bts, M, N, K, y,
                    bias=b, out=out)
    else:
        l2t = bf16_dev(np.ascontiguousarray(l2.T), dev)
        B.gemm_w4a4_lowrank(fmt, g["codes"], g["scales"], ats, w["codes"], w["scales"], bts, M, N,
                            K, g["t"], l2t, y, bias=b, out=out)
    torch.cuda.synchronize()
    yh, canary_ok = y_host(y, N)
    assert canary_ok, "write outside the output"
    return yh


def ref_w4a4(fmt, x, wt, bias=None, l1=None, l2=None, rows=None):
    """Oracle: its own quantization of the same inputs, then the fp64 product."""
    if fmt == "mxfp4":
        xs = x if rows is None else x[rows]
        A = Q.mx_dequantize(*Q.mx_quantize(xs))
        Bm = Q.mx_dequantize(*Q.mx_quantize(wt))
    else:
        amax = np.abs(F.bf16_to_f32(x)).max()
        xs = x if rows is None else x[rows]
        A = Q.nv_dequantize(*Q.nv_quantize(xs, amax_t=amax))
        Bm = Q.nv_dequantize(*Q.nv_quantize(wt))
    kw = {}
    if l1 is not None:
        kw = dict(x=F.bf16_to_f64(xs), l1=F.bf16_to_f64(l1), l2=F.bf16_to_f64(l2))
    return L.gemm_ref(A, Bm, bias=None if bias is None else F.bf16_to_f64(bias), **kw)


# (M, N, K): one tile, several tiles with ragged M/N tails, a K tail of half a K-tile,
# a single row/column and a deep K
SHAPES = [(64, 256, 256), (300, 520, 384), (512, 512, 1024), (17, 8, 128), (1, 300, 640),
          (513, 257, 256)]


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_w4a4_parity(fmt, M, N, K):
    dev = device()
    x = synth.activations(M, K, seed=M + N, outliers=max(1, K // 100))[0]
    wt = synth.weights(N, K, seed=N)
    bias = synth.bias(N, seed=1)
    for f32, use_bias in [(True, False), (False, True)]:
        say(f"gemm_w4a4 {fmt} M={M} N={N} K={K} f32={f32} bias={use_bias}")
        y = run_w4a4(fmt, x, wt, dev, bias=bias if use_bias else None, f32=f32)
        y_ref, bound = ref_w4a4(fmt, x, wt, bias=bias if use_bias else None)
        _check(y, y_ref, bound, not f32, f"{fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("M,N,K,r", [(64, 256, 256, 32), (300, 520, 384, 16), (200, 384, 512, 32)])
def test_gemm_w4a4_lowrank_parity(fmt, M, N, K, r):
    dev = device()
    d = weight_prep.mlp_up_svd(seed=2, M=M, K=K, N=N, rank=r)
    bias = synth.bias(N, seed=3)
    for f32 in (True, False):
        say(f"gemm_w4a4_lowrank {fmt} M={M} N={N} K={K} r={r} f32={f32}")
        y = run_w4a4(fmt, d["x"], d["rt"], dev, bias=bias, f32=f32, l1=d["l1"], l2=d["l2"])
        y_ref, bound = ref_w4a4(fmt, d["x"], d["rt"], bias=bias, l1=d["l1"], l2=d["l2"])
        _check(y, y_ref, bound, not f32, f"{fmt} low-rank {M}x{N}x{K} r{r}")


def test_gemm_mx_exact_grid_values():
    # Inputs already on the E2M1 grid with a 6 (or 4) in every block: quantization
    # is exact with scale 2**0, every product is a multiple of 0.25 and every sum
    # is exact in fp32, so the fp32 output must equal the oracle exactly.
    dev = device()
    rng = np.random.default_rng(4)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    M, N, K = 260, 300, 768
    xv = grid[rng.integers(0, 8, (M, K))] * rng.choice([-1, 1], (M, K))
    wv = grid[rng.integers(0, 8, (N, K))] * rng.choice([-1, 1], (N, K))
    xv[:, ::32] = 6.0
    wv[:, ::32] = -4.0
    x, wt = synth.to_bf16_bits(xv), synth.to_bf16_bits(wv)
    say("gemm_w4a4 mxfp4 exact grid values")
    y = run_w4a4("mxfp4", x, wt, dev, f32=True)
    y_ref, _ = ref_w4a4("mxfp4", x, wt)
    assert np.array_equal(y, y_ref)
    assert np.array_equal(y_ref, xv @ wv.T)


def test_gemm_mx_all_ones_closed_form():
    # every element 4 * 2**a (activations) or 4 * 2**b (weights): each block gets
    # E = a (or b), every code is 4, and
    # Y = 16 K * 2**(a + b) exactly
    dev = device()
    M, N, K = 96, 160, 512
    for a, b in [(0, 0), (-5, 3), (20, -30)]:
        x = synth.to_bf16_bits(np.full((M, K), 2.0 ** a * 4))       # block max 4*2**a -> E = a
        wt = synth.to_bf16_bits(np.full((N, K), 2.0 ** b * 4))
        say(f"gemm_w4a4 mxfp4 all-ones a={a} b={b}")
        y = run_w4a4("mxfp4", x, wt, dev, f32=True)
        assert np.all(y == K * 16 * 2.0 ** (a + b))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8", "int4_sym"])
def test_gemm_k_zero_gives_bias(fmt):
    dev = device()
    M, N = 40, 72
    bias = synth.bias(N, seed=5)
    # no codes or block scales are read at K = 0; int4_sym reads its float row scales
    # [M] and [N] (zeros here)
    dummy = torch.zeros(4 * max(M, N), dtype=torch.uint8, device=dev)
    sdummy = torch.zeros(max(M, N), dtype=torch.float32, device=dev) if fmt == "int4_sym" else dummy
    y = out_buffer(M, N, dev, f32=True)
    b = bf16_dev(bias[None, :], dev)[0]
    say(f"gemm_w4a4 {fmt} K=0")
    B.gemm_w4a4(fmt, dummy, sdummy, None, dummy, sdummy, None, M, N, 0, y, bias=b, out=B.OUT_F32)
    torch.cuda.synchronize()
    yh, ok = y_host(y, N)
    assert ok and np.array_equal(yh, np.broadcast_to(F.bf16_to_f64(bias), (M, N)))


def test_gemm_deterministic():
    dev = device()
    d = weight_prep.mlp_up_svd(seed=6, M=512, K=1024, N=768, rank=32)
    say("gemm_w4a4_lowrank determinism")
    y1 = run_w4a4("mxfp4", d["x"], d["rt"], dev, f32=False, l1=d["l1"], l2=d["l2"])
    y2 = run_w4a4("mxfp4", d["x"], d["rt"], dev, f32=False, l1=d["l1"], l2=d["l2"])
    assert np.array_equal(y1, y2)


def test_gemm_mx_leftover_tiles_as_halves():
    """More 256 x 256 tiles than one round over the CUs (17 x 16 = 272 on 256 CUs):
    the leftover tiles run as two halves of 128 weight rows each.  Ragged M and N,
    rank-32 branch and bias, every element checked."""
    dev = device()
    M, N, K = 4335, 4024, 256
    d = weight_prep.mlp_up_svd(seed=10, M=M, K=K, N=N, rank=32)
    bias = synth.bias(N, seed=11)
    for f32 in (True, False):
        say(f"gemm_w4a4_lowrank mxfp4 leftover tiles M={M} N={N} K={K} f32={f32}")
        y = run_w4a4("mxfp4", d["x"], d["rt"], dev, bias=bias, f32=f32, l1=d["l1"], l2=d["l2"])
        y_ref, bound = ref_w4a4("mxfp4", d["x"], d["rt"], bias=bias, l1=d["l1"], l2=d["l2"])
        _check(y, y_ref, bound, not f32, f"leftover tiles {M}x{N}x{K}")


@pytest.mark.parametrize("K", [256, 1024])
def test_gemm_mx_several_tiles_per_workgroup(K):
    """About four work units per workgroup (864 tiles of 256 x 256, the leftover 96
    as halves): each tile queues the next one's first loads before its own stores,
    and with K a multiple of four K-tiles (K = 1024) a whole tile followed by a whole
    tile loads the next one's first K-tile and scale pairs in its own last K-tiles.
    Ragged M and N put masked edge tiles among the interior ones; rank-16 branch and
    bias, bf16 and fp32 output, every element checked."""
    dev = device()
    M, N = 4600, 12280
    d = weight_prep.mlp_up_svd(seed=12, M=M, K=K, N=N, rank=16)
    bias = synth.bias(N, seed=13)
    y_ref, bound = ref_w4a4("mxfp4", d["x"], d["rt"], bias=bias, l1=d["l1"], l2=d["l2"])
    for f32 in (False, True):
        say(f"gemm_w4a4_lowrank mxfp4 several tiles per workgroup M={M} N={N} K={K} f32={f32}")
        y = run_w4a4("mxfp4", d["x"], d["rt"], dev, bias=bias, f32=f32, l1=d["l1"], l2=d["l2"])
        _check(y, y_ref, bound, not f32, f"several tiles per workgroup {M}x{N}x{K}")


# ------------------------------------------------------------------ full layer sizes
def test_full_mlp_up_svd_layer_every_element():
    """The benchmarked configuration: M=4608, K=3072, N=12288, rank 32, bf16 output,
    quantize_act (+ t) -> gemm_w4a4_lowrank in the launch bench.py times, every one
    of the 56.6 M outputs checked against the oracle (in blocks of rows)."""
    dev = device()
    d = weight_prep.mlp_up_svd(seed=0)
    M, N = d["M"], d["N"]
    say("full layer mxfp4 4608x3072x12288 r=32 bf16, every element")
    y = run_w4a4("mxfp4", d["x"], d["rt"], dev, f32=False, l1=d["l1"], l2=d["l2"])
    Bm = Q.mx_dequantize(*Q.mx_quantize(d["rt"]))
    l1, l2 = F.bf16_to_f64(d["l1"]), F.bf16_to_f64(d["l2"])
    worst = 0.0
    for r0 in range(0, M, 512):
        xs = d["x"][r0:r0 + 512]
        A = Q.mx_dequantize(*Q.mx_quantize(xs))
        y_ref, bound = L.gemm_ref(A, Bm, x=F.bf16_to_f64(xs), l1=l1, l2=l2)
        worst = max(worst, _check(y[r0:r0 + 512], y_ref, bound, True, f"full MLP layer rows {r0}.."))
    print(f"full MLP layer: worst |err|/tol = {worst:.4g}")


def test_full_attention_projection_every_element():
    """The attention projection at 1024^2 (M=4608, K=N=3072), fp32 output: every one
    of the 14.2 M outputs against the oracle, in blocks of rows."""
    dev = device()
    d = synth.attn_proj(seed=0)
    M = d["M"]
    say("full layer mxfp4 4608x3072x3072 f32, every element")
    y = run_w4a4("mxfp4", d["x"], d["wt"], dev, f32=True)
    Bm = Q.mx_dequantize(*Q.mx_quantize(d["wt"]))
    worst = 0.0
    for r0 in range(0, M, 1152):
        A = Q.mx_dequantize(*Q.mx_quantize(d["x"][r0:r0 + 1152]))
        y_ref, bound = L.gemm_ref(A, Bm)
        worst = max(worst, _check(y[r0:r0 + 1152], y_ref, bound, False, f"attention projection rows {r0}.."))
    print(f"full attention projection: worst |err|/tol = {worst:.4g}")


@pytest.mark.parametrize("step", [0, 5])
def test_full_qkv_nvfp4(step):
    """Fused QKV at 2048^2, NVFP4, at two denoising steps with different outlier
    channel sets (and so different tensor scales): every one of the 155.7 M outputs
    at step 0, sampled rows at step 5."""
    dev = device()
    d = synth.qkv_nvfp4(step=step)
    wt = synth.qkv_nvfp4_weight()
    M = d["M"]
    say(f"full layer nvfp4 16896x3072x9216 bf16, denoising step {step}")
    y = run_w4a4("nvfp4", d["x"], wt, dev, f32=False)
    if step != 0:
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(9 + step).choice(M, 46)]))
        y_ref, bound = ref_w4a4("nvfp4", d["x"], wt, rows=rows)
        _check(y[rows], y_ref, bound, True, "full QKV NVFP4")
        return
    amax = np.abs(F.bf16_to_f32(d["x"])).max()
    Bm = Q.nv_dequantize(*Q.nv_quantize(wt))
    worst = 0.0
    for r0 in range(0, M, 2048):
        A = Q.nv_dequantize(*Q.nv_quantize(d["x"][r0:r0 + 2048], amax_t=amax))
        y_ref, bound = L.gemm_ref(A, Bm)
        worst = max(worst, _check(y[r0:r0 + 2048], y_ref, bound, True, f"QKV NVFP4 rows {r0}.."))
    print(f"full QKV NVFP4: worst |err|/tol = {worst:.4g}")


def _blockwise_range(rows, K, seed):
    """bf16 [rows, K]: N(0, 1) values, each 16-element block scaled by its own 2**u,
    u ~ U(-20, 0), so that the NVFP4 block scales (relative to the tensor maximum)
    run from E4M3 subnormals to the top of the range."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(-20, 0, size=(rows, K // 16))
    return synth.to_bf16_bits(rng.standard_normal((rows, K)) * np.repeat(2.0 ** u, 16, axis=1))


def test_gemm_nvfp4_block_scales_over_the_e4m3_range():
    """The NVFP4 GEMM dequantizes e2m1 * s_b exactly in fp16: check it where the block
    scales reach both ends of E4M3 (subnormal scales, products down to 2**-10, and
    scales near 448) in both operands, with ragged M and N."""
    dev = device()
    M, N, K = 200, 264, 512
    x = _blockwise_range(M, K, 21)
    wt = _blockwise_range(N, K, 22)
    for bits in (x, wt):
        sb = Q.nv_quantize(bits)[1]
        assert np.any(((sb & 0x78) == 0) & ((sb & 0x07) != 0))          # subnormal scales
        assert np.any((sb & 0x7F) >= 0x70)                               # scales of 256 and up
    say("gemm_w4a4 nvfp4 block scales over the E4M3 range, f32")
    y = run_w4a4("nvfp4", x, wt, dev, f32=True)
    y_ref, bound = ref_w4a4("nvfp4", x, wt)
    _check(y, y_ref, bound, False, "nvfp4 E4M3 range")


# ------------------------------------------------------------------ W4A16
def run_w4a16(x, wt, dev, bias=None, f32=True):
    M, K = x.shape
    N = wt.shape[0]
    w = pack("int4_g64", wt, dev)
    xd = bf16_dev(x, dev)
    y = out_buffer(M, N, dev, f32)
    b = bf16_dev(bias[None, :], dev)[0] if bias is not None else None
    B.gemm_w4a16(xd, w["codes"], w["scales"], w["extra"], N, y, bias=b,
                 out=B.OUT_F32 if f32 else B.OUT_BF16)
    torch.cuda.synchronize()
    yh, ok = y_host(y, N)
    assert ok, "write outside the output"
    return yh


def ref_w4a16(x, wt, bias=None, rows=None):
    W = Q.int4_g64_dequantize(*Q.int4_g64_quantize(wt))
    X = F.bf16_to_f64(x if rows is None else x[rows])
    return L.gemm_ref(X, W, bias=None if bias is None else F.bf16_to_f64(bias))


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (300, 520, 384), (17, 8, 128), (512, 512, 1024)])
def test_gemm_w4a16_parity(M, N, K):
    dev = device()
    x = synth.activations(M, K, seed=M)[0]
    wt = synth.weights(N, K, seed=N + 1)
    bias = synth.bias(N, seed=2)
    for f32, use_bias in [(True, False), (False, True)]:
        say(f"gemm_w4a16 M={M} N={N} K={K} f32={f32} bias={use_bias}")
        y = run_w4a16(x, wt, dev, bias=bias if use_bias else None, f32=f32)
        y_ref, bound = ref_w4a16(x, wt, bias=bias if use_bias else None)
        _check(y, y_ref, bound, not f32, f"w4a16 {M}x{N}x{K}")


# Both tilings of the W4A16 GEMM, with ragged M and N: few rows take 256 x 96 tiles
# (one round over the CUs), more rows 256 x 256 tiles and halves of the leftover
# ones.  Every element is checked.
@pytest.mark.parametrize("M,N,K", [(500, 11990, 192), (2100, 8000, 128), (257, 24576, 64)])
def test_gemm_w4a16_tilings(M, N, K):
    dev = device()
    x = synth.activations(M, K, seed=M + 7)[0]
    wt = synth.weights(N, K, seed=N + 3)
    bias = synth.bias(N, seed=4)
    say(f"gemm_w4a16 tilings M={M} N={N} K={K} bf16 bias")
    y = run_w4a16(x, wt, dev, bias=bias, f32=False)
    y_ref, bound = ref_w4a16(x, wt, bias=bias)
    _check(y, y_ref, bound, True, f"w4a16 {M}x{N}x{K}")


def test_full_w4a16_layer():
    """The comparison layer at M = 512 (every element) and M = 4608 (sampled rows)."""
    dev = device()
    for M in (512, 4608):
        d = synth.w4a16_layer(M)
        say(f"full layer w4a16 {M}x3072x12288")
        y = run_w4a16(d["x"], d["wt"], dev, f32=False)
        rows = (np.arange(M) if M <= 512 else
                np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).choice(M, 30)])))
        y_ref, bound = ref_w4a16(d["x"], d["wt"], rows=rows)
        _check(y[rows], y_ref, bound, True, f"full W4A16 M={M}")
