"""GPU parity of the SVDQuant-style smoothed activation quantizer
(quantize_act_smooth) against the CPU oracle -- codes and scales bit-exact -- and
of the whole smoothed layer (smoothed activations, activation-weighted low-rank
branch, 4-bit residual) within the GEMM bound.  Every call goes through the C ABI."""

import numpy as np
import pytest
import torch

from bit_quantized_gemm_quantize_amd import binding as B
from bit_quantized_gemm_quantize_amd import synth, weight_prep
from oracle import formats as F
from oracle import layer as L
from oracle import quant as Q

from _gpu import bf16_dev, device, out_buffer, pack, say, u8, y_host
from test_gpu_gemm import _check

pytestmark = pytest.mark.gpu


def quantize_smooth(x_bits, inv_s, dev, l1_bits=None, ldx_pad=0):
    M, K = x_bits.shape
    x = bf16_dev(x_bits, dev, ldx_pad)
    inv = torch.from_numpy(np.ascontiguousarray(inv_s, dtype=np.float32)).to(dev)
    codes, scales, _ = B.empty_quant("mxfp4", M, K, dev)
    l1t = t = None
    if l1_bits is not None:
        l1t = bf16_dev(np.ascontiguousarray(l1_bits.T), dev)
        t = torch.full((M, l1_bits.shape[1]), float("nan"), dtype=torch.float32, device=dev)
    B.quantize_act_smooth("mxfp4", x, inv, codes, scales, l1t=l1t, t=t)
    torch.cuda.synchronize()
    return dict(codes=codes, scales=scales, t=t)


@pytest.mark.parametrize("M,K", [(64, 256), (100, 352), (33, 32), (257, 1024), (31, 96)])
def test_quantize_smooth_bit_exact(M, K):
    dev = device()
    x = synth.activations(M, K, seed=M + 3 * K, outliers=max(1, K // 100))[0]
    rng = np.random.default_rng(M * K)
    inv = np.exp(rng.uniform(-4.0, 3.0, K)).astype(np.float32)     # factors over 2^-6 .. 2^4
    say(f"quantize_act_smooth mxfp4 M={M} K={K}")
    g = quantize_smooth(x, inv, dev)
    codes, scales = Q.mx_quantize_smoothed(x, inv)
    assert np.array_equal(u8(g["scales"]), scales)
    assert np.array_equal(u8(g["codes"]), codes)


def test_quantize_smooth_wide_range_and_padded_rows():
    # every finite bf16 pattern once (subnormals included) times factors spanning
    # 2^-20 .. 1 (none overflows), so products land subnormal, normal and, with the
    # unit factors, at the top of the range; rows padded past K
    dev = device()
    rng = np.random.default_rng(11)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF]
    rng.shuffle(pats)
    x = pats[:65280].reshape(-1, 256)
    inv = np.exp2(rng.uniform(-20.0, 0.0, 256)).astype(np.float32)
    inv[:32] = 1.0
    say(f"quantize_act_smooth mxfp4 all bf16 patterns rows={x.shape[0]} padded")
    g = quantize_smooth(x, inv, dev, ldx_pad=64)
    codes, scales = Q.mx_quantize_smoothed(x, inv)
    assert np.array_equal(u8(g["scales"]), scales)
    assert np.array_equal(u8(g["codes"]), codes)


@pytest.mark.parametrize("M,K,r", [(4700, 1056, 16), (600, 3104, 32)])
def test_quantize_smooth_fused_t_ring_shapes(M, K, r):
    """The smoothed pass with t over shapes that wrap the kernel's load ring and end
    in a partial chunk (K = 1056, 3104), with 19 rows per workgroup (M = 4700) and
    with fewer rows than CUs (M = 600): codes and scales bit-exact, t within the
    fp32 accumulation bound."""
    dev = device()
    x = synth.activations(M, K, seed=M + K, outliers=max(1, K // 100))[0]
    rng = np.random.default_rng(M + 2 * K)
    inv = np.exp(rng.uniform(-4.0, 3.0, K)).astype(np.float32)
    l1 = synth.to_bf16_bits(rng.standard_normal((K, r)) * 0.05)
    say(f"quantize_act_smooth mxfp4 + t=X L1 M={M} K={K} r={r}")
    g = quantize_smooth(x, inv, dev, l1_bits=l1)
    codes, scales = Q.mx_quantize_smoothed(x, inv)
    assert np.array_equal(u8(g["scales"]), scales)
    assert np.array_equal(u8(g["codes"]), codes)
    X, L1 = F.bf16_to_f64(x), F.bf16_to_f64(l1)
    t = g["t"].cpu().numpy().astype(np.float64)
    bound = np.abs(X) @ np.abs(L1)
    assert np.all(np.abs(t - L.lowrank_down(X, L1)) <= K * 2.0 ** -24 * bound * 1.01 + 1e-30)


def test_quantize_smooth_fused_t_uses_unsmoothed_x():
    dev = device()
    M, K, r = 96, 512, 32
    d = weight_prep.attn_proj_svdquant(seed=2, M=M, K=K, N=256, rank=r, calib=256)
    say(f"quantize_act_smooth mxfp4 + t=X L1 M={M} K={K} r={r}")
    g = quantize_smooth(d["x"], d["inv_s"], dev, l1_bits=d["l1"])
    X, L1 = F.bf16_to_f64(d["x"]), F.bf16_to_f64(d["l1"])
    t = g["t"].cpu().numpy().astype(np.float64)
    bound = np.abs(X) @ np.abs(L1)
    assert np.all(np.abs(t - L.lowrank_down(X, L1)) <= K * 2.0 ** -24 * bound * 1.01 + 1e-30)
    codes, scales = Q.mx_quantize_smoothed(d["x"], d["inv_s"])
    assert np.array_equal(u8(g["codes"]), codes) and np.array_equal(u8(g["scales"]), scales)


def run_svdquant_layer(d, dev, f32, rows=None):
    """quantize_act_smooth (+ t) -> pack R' -> gemm_w4a4_lowrank; host Y."""
    M, N, K = d["M"], d["N"], d["K"]
    g = quantize_smooth(d["x"], d["inv_s"], dev, l1_bits=d["l1"])
    w = pack("mxfp4", d["rt"], dev)
    y = out_buffer(M, N, dev, f32)
    l2t = bf16_dev(np.ascontiguousarray(d["l2"].T), dev)
    B.gemm_w4a4_lowrank("mxfp4", g["codes"], g["scales"], None, w["codes"], w["scales"], None, M, N, K,
                        g["t"], l2t, y, out=B.OUT_F32 if f32 else B.OUT_BF16)
    torch.cuda.synchronize()
    yh, ok = y_host(y, N)
    assert ok, "write outside the output"
    return yh


def ref_svdquant_layer(d, rows=None):
    xs = d["x"] if rows is None else d["x"][rows]
    A = Q.mx_dequantize(*Q.mx_quantize_smoothed(xs, d["inv_s"]))
    Bm = Q.mx_dequantize(*Q.mx_quantize(d["rt"]))
    return L.gemm_ref(A, Bm, x=F.bf16_to_f64(xs), l1=F.bf16_to_f64(d["l1"]), l2=F.bf16_to_f64(d["l2"]))


@pytest.mark.parametrize("f32", [True, False])
def test_svdquant_layer_parity(f32):
    dev = device()
    d = weight_prep.attn_proj_svdquant(seed=6, M=300, K=1024, N=520, rank=32, calib=512)
    say(f"svdquant layer 300x1024x520 r=32 f32={f32}")
    y = run_svdquant_layer(d, dev, f32)
    y_ref, bound = ref_svdquant_layer(d)
    _check(y, y_ref, bound, not f32, "svdquant layer")


def test_full_svdquant_attention_projection_sampled_rows():
    """The attention projection at 4608x3072x3072 prepared the SVDQuant way, checked
    on sampled rows against the oracle; and its error against the unquantized bf16
    product is far below plain W4A4's on the same activations (reported)."""
    dev = device()
    d = weight_prep.attn_proj_svdquant(seed=0)
    M = d["M"]
    say("full svdquant attention projection 4608x3072x3072 r=32 bf16")
    y = run_svdquant_layer(d, dev, f32=False)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(9).choice(M, 40)]))
    y_ref, bound = ref_svdquant_layer(d, rows=rows)
    _check(y[rows], y_ref, bound, True, "full svdquant attention projection")
    exact = F.bf16_to_f64(d["x"][rows]) @ F.bf16_to_f64(d["wt"]).T
    rel = np.linalg.norm(y[rows] - exact) / np.linalg.norm(exact)
    say(f"svdquant relative error vs the bf16 product: {rel:.4f}")
    assert rel < 0.05
