"""GPU tests of the MXFP4-emitting epilogue (gemm_w4a4_lowrank_mxout): the layer's
output handed to the next layer as MXFP4 codes and scales.  Bit-exact against the
oracle where the GEMM result is exact; elsewhere the bf16 output is checked against
the oracle within the GEMM bound and the emitted codes against the oracle's
quantization of that same stored output.  Every call goes through the C ABI."""

import numpy as np
import pytest
import torch

from bit_quantized_gemm_quantize_amd import binding as B
from bit_quantized_gemm_quantize_amd import synth, weight_prep
from oracle import formats as F
from oracle import layer as L
from oracle import quant as Q

from _gpu import bf16_dev, bits16, device, pack, quantize, say, u8
from test_gpu_gemm import _check, ref_w4a4

pytestmark = pytest.mark.gpu


def run_mxout(x, wt, dev, l1=None, l2=None, bias=None, with_y=True):
    """quantize_act (+ t) -> pack -> gemm_w4a4_lowrank_mxout.  Returns host
    (codes, scales, y bf16 bits or None); the code and scale rows are padded and the
    padding checked untouched."""
    M, K = x.shape
    N = wt.shape[0]
    g = quantize("mxfp4", x, dev, l1_bits=l1)
    w = pack("mxfp4", wt, dev)
    qc = torch.full((M, N // 2 + 16), 0xA5, dtype=torch.uint8, device=dev)
    qs = torch.full((M, N // 32 + 4), 0xA5, dtype=torch.uint8, device=dev)
    y = None
    if with_y:
        y = torch.full((M, N + 8), float("nan"), dtype=torch.bfloat16, device=dev)
    b = bf16_dev(bias[None, :], dev)[0] if bias is not None else None
    l2t = bf16_dev(np.ascontiguousarray(l2.T), dev) if l2 is not None else None
    B.gemm_w4a4_lowrank_mxout(g["codes"], g["scales"], w["codes"], w["scales"], M, N, K, qc, qs,
                              t=g["t"] if l1 is not None else None, l2t=l2t, y=y, bias=b)
    torch.cuda.synchronize()
    qch, qsh = u8(qc), u8(qs)
    assert np.all(qch[:, N // 2:] == 0xA5) and np.all(qsh[:, N // 32:] == 0xA5), "write past N"
    yb = None
    if y is not None:
        yb = bits16(y)
        assert np.all(yb[:, N:] == bits16(torch.full((1,), float("nan"), dtype=torch.bfloat16))[0])
        yb = yb[:, :N]
    return qch[:, :N // 2], qsh[:, :N // 32], yb


def grid_inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    xv = grid[rng.integers(0, 8, (M, K))] * rng.choice([-1, 1], (M, K))
    wv = grid[rng.integers(0, 8, (N, K))] * rng.choice([-1, 1], (N, K))
    xv[:, ::32] = 6.0
    wv[:, ::32] = -4.0
    return xv, wv


def test_mxout_exact_grid_values_bit_exact():
    # operands on the E2M1 grid: the GEMM result is exact in fp32 and equals the
    # oracle's, so its bf16 rounding and MXFP4 quantization must match bit for bit;
    # ragged M and N (N a multiple of 32), bias on a 0.25 grid
    dev = device()
    M, N, K = 260, 352, 768
    xv, wv = grid_inputs(M, N, K, 4)
    bias = synth.to_bf16_bits(np.random.default_rng(5).integers(-64, 64, N) * 0.25)
    say(f"gemm_w4a4_lowrank_mxout exact grid M={M} N={N} K={K}")
    qc, qs, yb = run_mxout(synth.to_bf16_bits(xv), synth.to_bf16_bits(wv), dev, bias=bias)
    y_exact = xv @ wv.T + F.bf16_to_f64(bias)[None, :]
    codes, scales = L.mx_output(y_exact)
    assert np.array_equal(qs, scales)
    assert np.array_equal(qc, codes)
    assert np.array_equal(yb, F.f32_to_bf16_rne(y_exact.astype(np.float32)))


def test_mxout_exact_grid_with_lowrank_bit_exact():
    # a low-rank branch on a small grid too: t = X L1 is exact in fp32 and in its
    # bf16 hi + lo split, t L2 is exact, so the output stays exact
    dev = device()
    M, N, K, r = 200, 256, 512, 16
    xv, wv = grid_inputs(M, N, K, 6)
    rng = np.random.default_rng(7)
    l1v = rng.integers(-2, 3, (K, r)) * 0.5
    l2v = rng.integers(-2, 3, (r, N)) * 0.25
    say(f"gemm_w4a4_lowrank_mxout exact grid + rank {r}")
    qc, qs, yb = run_mxout(synth.to_bf16_bits(xv), synth.to_bf16_bits(wv), dev,
                           l1=synth.to_bf16_bits(l1v), l2=synth.to_bf16_bits(l2v))
    y_exact = xv @ wv.T + (xv @ l1v) @ l2v
    codes, scales = L.mx_output(y_exact)
    assert np.array_equal(qs, scales) and np.array_equal(qc, codes)


@pytest.mark.parametrize("M,N,K,r", [(300, 512, 384, 16), (4600, 12256, 1024, 32)])
def test_mxout_matches_the_stored_output(M, N, K, r):
    """General data (several tiles per workgroup in the large case, ragged M and
    N): the bf16 output is within the GEMM bound of the oracle, the codes and
    scales are the oracle's quantization of exactly that stored output, and a launch
    without the bf16 output emits the same codes."""
    dev = device()
    d = weight_prep.mlp_up_svd(seed=M, M=M, K=K, N=N, rank=r)
    bias = synth.bias(N, seed=M + 1)
    say(f"gemm_w4a4_lowrank_mxout M={M} N={N} K={K} r={r}")
    qc, qs, yb = run_mxout(d["x"], d["rt"], dev, l1=d["l1"], l2=d["l2"], bias=bias)
    y_ref, bound = ref_w4a4("mxfp4", d["x"], d["rt"], bias=bias, l1=d["l1"], l2=d["l2"])
    _check(F.bf16_to_f64(yb), y_ref, bound, True, f"mxout bf16 {M}x{N}x{K}")
    codes, scales = Q.mx_quantize(yb)
    assert np.array_equal(qs, scales)
    assert np.array_equal(qc, codes)
    say(f"gemm_w4a4_lowrank_mxout M={M} N={N} K={K} r={r} without y")
    qc2, qs2, _ = run_mxout(d["x"], d["rt"], dev, l1=d["l1"], l2=d["l2"], bias=bias, with_y=False)
    assert np.array_equal(qc2, qc) and np.array_equal(qs2, qs)


def test_mxout_full_mlp_up_sampled_rows():
    """4608 x 3072 x 12288, rank 32: the codes equal quantize_act run on the bf16
    output of gemm_w4a4_lowrank over the same inputs (the unfused path), and their
    dequantized values on sampled rows lie within the MXFP4 step of the oracle's Y
    plus the GEMM bound."""
    dev = device()
    d = weight_prep.mlp_up_svd(seed=0)
    M, K, N = d["M"], d["K"], d["N"]
    say("gemm_w4a4_lowrank_mxout full 4608x3072x12288 r=32")
    qc, qs, _ = run_mxout(d["x"], d["rt"], dev, l1=d["l1"], l2=d["l2"], with_y=False)
    g = quantize("mxfp4", d["x"], dev, l1_bits=d["l1"])
    w = pack("mxfp4", d["rt"], dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    B.gemm_w4a4_lowrank("mxfp4", g["codes"], g["scales"], None, w["codes"], w["scales"], None, M, N, K,
                        g["t"], bf16_dev(np.ascontiguousarray(d["l2"].T), dev), y)
    c2, s2, _ = B.empty_quant("mxfp4", M, N, dev)
    B.quantize_act("mxfp4", y, c2, s2)
    torch.cuda.synchronize()
    assert np.array_equal(u8(c2), qc) and np.array_equal(u8(s2), qs)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(3).choice(M, 24)]))
    y_ref, bound = ref_w4a4("mxfp4", d["x"], d["rt"], l1=d["l1"], l2=d["l2"], rows=rows)
    deq = Q.mx_dequantize(qc[rows], qs[rows])
    step = np.ldexp(2.0, qs[rows].astype(np.int64) - 127).repeat(32, axis=1)  # <= 2 * 2**E
    assert np.all(np.abs(deq - y_ref) <= step + L.tolerance(y_ref, bound, True))
