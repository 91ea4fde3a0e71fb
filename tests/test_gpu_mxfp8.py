"""GPU parity of the MXFP8 path (E4M3 elements, E8M0 scales per 32 K elements) on
the block-scaled MFMA with the FP8 operand format: quantizer and packer bit-exact
against the oracle (every finite bf16 pattern under several block exponents), the
GEMM exactly equal where the result is exact and within the bound elsewhere.
Every call goes through the C ABI."""

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


def every_pattern_blocks(E, K=1024):
    """Blocks of 32 whose element 0 is the largest bf16 below 2**(E+9) (so the block
    exponent is E) and whose other 31 elements run through every finite bf16 pattern
    of magnitude at most that, both signs, zeros included; rows of K elements."""
    top = (E + 8 + 127) << 7 | 0x7F                         # 1.9921875 * 2**(E+8)
    mags = np.arange(0, top + 1, dtype=np.uint32)
    pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
    nb = -(-len(pats) // 31)
    body = np.zeros(nb * 31, dtype=np.uint16)
    body[:len(pats)] = pats
    blocks = np.concatenate([np.full((nb, 1), top, dtype=np.uint16), body.reshape(nb, 31)], axis=1)
    per_row = K // 32
    nrow = -(-nb // per_row)
    out = np.zeros((nrow * per_row, 32), dtype=np.uint16)
    out[:nb] = blocks
    return out.reshape(nrow, K)


@pytest.mark.parametrize("E", [0, -5, 40, -120, 119])
def test_quantize_mxfp8_every_pattern(E):
    dev = device()
    x = every_pattern_blocks(E)
    say(f"quantize_act mxfp8 every pattern E={E} rows={x.shape[0]}")
    g = quantize("mxfp8", x, dev)
    codes, scales = Q.mxfp8_quantize(x)
    assert np.all(scales[scales != 0] == E + 127)
    assert np.array_equal(u8(g["scales"]), scales)
    got = u8(g["codes"])
    bad = np.argwhere(got != codes)
    assert bad.size == 0, (f"{len(bad)} codes differ, first at {tuple(bad[0])}: x=0x{x[tuple(bad[0])]:04x} "
                           f"gpu 0x{got[tuple(bad[0])]:02x} oracle 0x{codes[tuple(bad[0])]:02x}")


@pytest.mark.parametrize("M,K,pad", [(64, 256, 0), (100, 352, 0), (33, 32, 0), (257, 1024, 64), (5, 96, 8)])
def test_quantize_mxfp8_bit_exact(M, K, pad):
    dev = device()
    x = synth.activations(M, K, seed=M + 3 * K, outliers=max(1, K // 100))[0].copy()
    x[M // 2] = 0                                          # an all-zero row
    x[0, :32] = 0x8000                                     # a block of negative zeros
    say(f"quantize_act mxfp8 M={M} K={K} pad={pad}")
    g = quantize("mxfp8", x, dev, ldx_pad=pad)
    codes, scales = Q.mxfp8_quantize(x)
    assert np.array_equal(u8(g["scales"]), scales)
    assert np.array_equal(u8(g["codes"]), codes)


@pytest.mark.parametrize("layout", ["nk", "kn", "nk_pad"])
def test_pack_mxfp8_bit_exact(layout):
    dev = device()
    wt = synth.weights(200, 384, seed=5)
    say(f"pack_weights mxfp8 {layout}")
    w = pack("mxfp8", wt, dev, layout=layout)
    codes, scales = Q.mxfp8_quantize(wt)
    assert np.array_equal(u8(w["scales"]), scales)
    assert np.array_equal(u8(w["codes"]), codes)


def run_x8(x, wt, dev, bias=None, f32=True):
    M, K = x.shape
    N = wt.shape[0]
    g = quantize("mxfp8", x, dev)
    w = pack("mxfp8", wt, dev)
    y = out_buffer(M, N, dev, f32)
    b = bf16_dev(bias[None, :], dev)[0] if bias is not None else None
    B.gemm_w4a4("mxfp8", g["codes"], g["scales"], None, w["codes"], w["scales"], None, M, N, K, y,
                bias=b, out=B.OUT_F32 if f32 else B.OUT_BF16)
    torch.cuda.synchronize()
    yh, ok = y_host(y, N)
    assert ok, "write outside the output"
    return yh


def ref_x8(x, wt, bias=None, rows=None):
    xs = x if rows is None else x[rows]
    A = Q.mxfp8_dequantize(*Q.mxfp8_quantize(xs))
    Bm = Q.mxfp8_dequantize(*Q.mxfp8_quantize(wt))
    return L.gemm_ref(A, Bm, bias=None if bias is None else F.bf16_to_f64(bias))


def test_gemm_mxfp8_exact_integers():
    # each block holds an 8 (block exponent -5, so the codes are the integers times
    # 32, exact in E4M3) and integers in [-7, 7]; rows and columns scaled by powers of
    # two: every product and partial sum is exact in fp32
    dev = device()
    rng = np.random.default_rng(21)
    M, N, K = 260, 300, 768
    xq = rng.integers(-7, 8, (M, K))
    wq = rng.integers(-7, 8, (N, K))
    xq[:, ::32] = 8
    wq[:, 5::32] = -8
    xa, wb = 2.0 ** rng.integers(-6, 6, (M, 1)), 2.0 ** rng.integers(-6, 6, (N, 1))
    x, wt = synth.to_bf16_bits(xq * xa), synth.to_bf16_bits(wq * wb)
    say("gemm_w4a4 mxfp8 exact integers")
    y = run_x8(x, wt, dev, f32=True)
    assert np.array_equal(y, (xq * xa) @ (wq * wb).T)


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (300, 520, 384), (513, 257, 1024), (17, 8, 128)])
@pytest.mark.parametrize("f32", [True, False])
def test_gemm_mxfp8_parity(M, N, K, f32):
    dev = device()
    x = synth.activations(M, K, seed=M + 2 * N, outliers=max(1, K // 100))[0]
    wt = synth.weights(N, K, seed=K + 1)
    bias = synth.bias(N, seed=N)
    say(f"gemm_w4a4 mxfp8 {M}x{N}x{K} f32={f32}")
    y = run_x8(x, wt, dev, bias=bias, f32=f32)
    y_ref, bound = ref_x8(x, wt, bias=bias)
    _check(y, y_ref, bound, not f32, f"mxfp8 {M}x{N}x{K}")


def test_gemm_mxfp8_half_tiles():
    # 2 x 130 tiles on 256 CUs: the 4 leftover tiles run as 8 halves (with ragged M
    # and N); every output checked
    dev = device()
    M, N, K = 300, 130 * 256 - 160, 256
    x = synth.activations(M, K, seed=11, outliers=3)[0]
    wt = synth.weights(N, K, seed=12)
    say(f"gemm_w4a4 mxfp8 half tiles {M}x{N}x{K}")
    y = run_x8(x, wt, dev, f32=True)
    y_ref, bound = ref_x8(x, wt)
    _check(y, y_ref, bound, False, "mxfp8 half tiles")


def test_full_mxfp8_mlp_up_sampled_rows():
    dev = device()
    d = synth.attn_proj(seed=1, N=12288)
    M = d["M"]
    say("gemm_w4a4 mxfp8 full 4608x3072x12288 bf16")
    y = run_x8(d["x"], d["wt"], dev, f32=False)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(3).choice(M, 30)]))
    y_ref, bound = ref_x8(d["x"], d["wt"], rows=rows)
    _check(y[rows], y_ref, bound, True, "full mxfp8")
