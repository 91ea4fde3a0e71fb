"""GPU parity of the symmetric INT4 path (per-row scales, the per-channel quantizer
of the SVDQuant Guide's "Step 1") run on the INT8 MFMA: quantizer and packer
bit-exact against the oracle, the GEMM within the bound and exactly equal where
the result is exact.  Every call goes through the C ABI."""

import numpy as np
import pytest
import torch

from bit_quantized_gemm_quantize_amd import binding as B
from bit_quantized_gemm_quantize_amd import synth
from oracle import formats as F
from oracle import layer as L
from oracle import quant as Q

from _gpu import bf16_dev, device, out_buffer, pack, quantize, say, u8, y_host
from test_gpu_gemm import _check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,pad", [(64, 256, 0), (100, 352, 0), (33, 32, 0), (257, 1024, 64), (5, 96, 8)])
def test_quantize_int4_sym_bit_exact(M, K, pad):
    dev = device()
    x = synth.activations(M, K, seed=M + 7 * K, outliers=max(1, K // 100))[0].copy()
    x[M // 2] = 0                                          # an all-zero row
    say(f"quantize_act int4_sym M={M} K={K} pad={pad}")
    g = quantize("int4_sym", x, dev, ldx_pad=pad)
    codes, scales = Q.int4_sym_quantize(x)
    assert np.array_equal(g["scales"].cpu().numpy(), scales)
    assert np.array_equal(u8(g["codes"]), codes)


@pytest.mark.parametrize("layout", ["nk", "kn", "nk_pad"])
def test_pack_int4_sym_bit_exact(layout):
    dev = device()
    wt = synth.weights(200, 384, seed=3)
    say(f"pack_weights int4_sym {layout}")
    w = pack("int4_sym", wt, dev, layout=layout)
    codes, scales = Q.int4_sym_quantize(wt)
    assert np.array_equal(w["scales"].cpu().numpy(), scales)
    assert np.array_equal(u8(w["codes"]), codes)


def run_i4(x, wt, dev, bias=None, f32=True):
    M, K = x.shape
    N = wt.shape[0]
    g = quantize("int4_sym", x, dev)
    w = pack("int4_sym", wt, dev)
    y = out_buffer(M, N, dev, f32)
    b = bf16_dev(bias[None, :], dev)[0] if bias is not None else None
    B.gemm_w4a4("int4_sym", g["codes"], g["scales"], None, w["codes"], w["scales"], None, M, N, K, y,
                bias=b, out=B.OUT_F32 if f32 else B.OUT_BF16)
    torch.cuda.synchronize()
    yh, ok = y_host(y, N)
    assert ok, "write outside the output"
    return yh


def ref_i4(x, wt, bias=None, rows=None):
    xs = x if rows is None else x[rows]
    A = Q.int4_sym_dequantize(*Q.int4_sym_quantize(xs))
    Bm = Q.int4_sym_dequantize(*Q.int4_sym_quantize(wt))
    return L.gemm_ref(A, Bm, bias=None if bias is None else F.bf16_to_f64(bias))


def test_gemm_int4_sym_exact_integers():
    # every row holds a 7 * 2^a: the scale is exactly 2^a, the codes are the integers
    # themselves, and the int32 sums times powers of two are exact in fp32
    dev = device()
    rng = np.random.default_rng(12)
    M, N, K = 260, 300, 768
    xq = rng.integers(-7, 8, (M, K))
    wq = rng.integers(-7, 8, (N, K))
    xq[:, 5] = 7
    wq[:, 9] = -7
    xa, wb = 2.0 ** rng.integers(-6, 6, (M, 1)), 2.0 ** rng.integers(-6, 6, (N, 1))
    x, wt = synth.to_bf16_bits(xq * xa), synth.to_bf16_bits(wq * wb)
    say("gemm_w4a4 int4_sym exact integers")
    y = run_i4(x, wt, dev, f32=True)
    assert np.array_equal(y, (xq * xa) @ (wq * wb).T)


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (300, 520, 384), (513, 257, 1024), (17, 8, 128)])
@pytest.mark.parametrize("f32", [True, False])
def test_gemm_int4_sym_parity(M, N, K, f32):
    dev = device()
    x = synth.activations(M, K, seed=M + N, outliers=max(1, K // 100))[0]
    wt = synth.weights(N, K, seed=K)
    bias = synth.bias(N, seed=N)
    say(f"gemm_w4a4 int4_sym {M}x{N}x{K} f32={f32}")
    y = run_i4(x, wt, dev, bias=bias, f32=f32)
    y_ref, bound = ref_i4(x, wt, bias=bias)
    _check(y, y_ref, bound, not f32, f"int4_sym {M}x{N}x{K}")


def test_gemm_int4_sym_half_tiles():
    # 2 x 130 tiles on 256 CUs: the 4 leftover tiles run as 8 halves (with ragged M
    # and N); every output checked
    dev = device()
    M, N, K = 300, 130 * 256 - 160, 512
    x = synth.activations(M, K, seed=13, outliers=3)[0]
    wt = synth.weights(N, K, seed=14)
    say(f"gemm_w4a4 int4_sym half tiles {M}x{N}x{K}")
    y = run_i4(x, wt, dev, f32=True)
    y_ref, bound = ref_i4(x, wt)
    _check(y, y_ref, bound, False, "int4_sym half tiles")


def test_full_int4_sym_mlp_up_sampled_rows():
    dev = device()
    d = synth.attn_proj(seed=1, N=12288)
    M = d["M"]
    say("gemm_w4a4 int4_sym full 4608x3072x12288 bf16")
    y = run_i4(d["x"], d["wt"], dev, f32=False)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(2).choice(M, 30)]))
    y_ref, bound = ref_i4(d["x"], d["wt"], rows=rows)
    _check(y[rows], y_ref, bound, True, "full int4_sym")
