"""GPU parity of the MXFP4 GEMM with the SwiGLU epilogue (gemm_w4a4_lowrank_swiglu):
the oracle's quantization of the same inputs, its fp64 product (+ low-rank term,
+ bias) and silu(gate) * up over the gate/up groups of 2 x 32 weight rows, within the
error bound propagated from the GEMM's.  Every call goes through the C ABI."""

import numpy as np
import pytest
import torch

from bit_quantized_gemm_quantize_amd import binding as B
from bit_quantized_gemm_quantize_amd import synth, weight_prep
from oracle import formats as F
from oracle import layer as L
from oracle import quant as Q

from _gpu import bf16_dev, device, out_buffer, pack, quantize, say, y_host
from test_gpu_gemm import _check

pytestmark = pytest.mark.gpu


def run_swiglu(x, wt, dev, bias=None, l1=None, l2=None):
    M, K = x.shape
    N = wt.shape[0]
    g = quantize("mxfp4", x, dev, l1_bits=l1)
    w = pack("mxfp4", wt, dev)
    y = out_buffer(M, N // 2, dev, f32=False)
    b = bf16_dev(bias[None, :], dev)[0] if bias is not None else None
    l2t = bf16_dev(np.ascontiguousarray(l2.T), dev) if l2 is not None else None
    B.gemm_w4a4_lowrank_swiglu(g["codes"], g["scales"], w["codes"], w["scales"], M, N, K, y,
                               t=g["t"] if l1 is not None else None, l2t=l2t, bias=b)
    torch.cuda.synchronize()
    yh, ok = y_host(y, N // 2)
    assert ok, "write outside the output"
    return yh


def ref_swiglu(x, wt, bias=None, l1=None, l2=None, rows=None):
    xs = x if rows is None else x[rows]
    A = Q.mx_dequantize(*Q.mx_quantize(xs))
    Bm = Q.mx_dequantize(*Q.mx_quantize(wt))
    kw = {}
    if l1 is not None:
        kw = dict(x=F.bf16_to_f64(xs), l1=F.bf16_to_f64(l1), l2=F.bf16_to_f64(l2))
    y, bound = L.gemm_ref(A, Bm, bias=None if bias is None else F.bf16_to_f64(bias), **kw)
    return L.swiglu_ref(y, bound)


def test_swiglu_exact_gemm_results():
    # operands on the E2M1 grid with unit block scales: the GEMM results are exact, so
    # only the epilogue's fp32 evaluation and the bf16 store remain
    dev = device()
    rng = np.random.default_rng(31)
    M, N, K = 64, 256, 256
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    xv = rng.choice(grid, (M, K)) * rng.choice([-1, 1], (M, K))
    wv = rng.choice(grid, (N, K)) * rng.choice([-1, 1], (N, K)) / 16
    xv[:, ::32] = 6                       # block maximum 6: block exponent 0
    wv[:, ::32] = 6 / 16                  # block maximum 0.375: exponent -4, codes exact
    x, wt = synth.to_bf16_bits(xv), synth.to_bf16_bits(wv)
    say("swiglu exact GEMM results")
    y = run_swiglu(x, wt, dev)
    exact = xv @ wv.T
    assert np.array_equal(exact, Q.mx_dequantize(*Q.mx_quantize(x)) @ Q.mx_dequantize(*Q.mx_quantize(wt)).T)
    y_ref, bound = L.swiglu_ref(exact, np.zeros_like(exact))
    _check(y, y_ref, bound, True, "swiglu exact")


@pytest.mark.parametrize("M,N,K,r", [(64, 256, 256, 0), (300, 384, 384, 32), (513, 640, 1024, 16),
                                     (1, 64, 128, 0), (257, 1344, 512, 32), (70, 320, 256, 16)])
def test_swiglu_parity(M, N, K, r):
    dev = device()
    x = synth.activations(M, K, seed=M + N, dist="student_t3")[0]
    wt = synth.weights(N, K, seed=K + r)
    bias = synth.bias(N, seed=N + 1)
    l1 = l2 = None
    if r:
        rng = np.random.default_rng(r)
        l1 = synth.to_bf16_bits(rng.standard_normal((K, r)) * 0.05)
        l2 = synth.to_bf16_bits(rng.standard_normal((r, N)) * 0.05)
    say(f"swiglu {M}x{N}x{K} r={r}")
    y = run_swiglu(x, wt, dev, bias=bias, l1=l1, l2=l2)
    y_ref, bound = ref_swiglu(x, wt, bias=bias, l1=l1, l2=l2)
    _check(y, y_ref, bound, True, f"swiglu {M}x{N}x{K} r={r}")


def test_swiglu_half_tiles():
    # 2 x 130 tiles on 256 CUs: the 4 leftover tiles run as 8 halves (64-row waves,
    # one gate/up group each); ragged M and N; every output checked
    dev = device()
    M, N, K = 300, 130 * 256 - 192, 256
    x = synth.activations(M, K, seed=15, dist="student_t3")[0]
    wt = synth.weights(N, K, seed=16)
    bias = synth.bias(N, seed=17)
    say(f"swiglu half tiles {M}x{N}x{K}")
    y = run_swiglu(x, wt, dev, bias=bias)
    y_ref, bound = ref_swiglu(x, wt, bias=bias)
    _check(y, y_ref, bound, True, "swiglu half tiles")


def test_swiglu_full_mlp_up_sampled_rows():
    # the MLP up-projection shape with its rank-32 branch: 4608 x 3072 against 12288
    # weight rows (6144 outputs); 40 sampled rows against the oracle
    dev = device()
    d = weight_prep.mlp_up_svd(seed=2)
    M = d["M"]
    say("swiglu full 4608x3072x12288 r=32")
    y = run_swiglu(d["x"], d["rt"], dev, l1=d["l1"], l2=d["l2"])
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(4).choice(M, 38)]))
    y_ref, bound = ref_swiglu(d["x"], d["rt"], l1=d["l1"], l2=d["l2"], rows=rows)
    _check(y[rows], y_ref, bound, True, "swiglu full")
