"""GPU parity of the MXFP4 GEMM with the QKV-split and RoPE epilogue
(gemm_w4a4_lowrank_qkv_rope): the oracle's quantization of the same inputs, its fp64
product (+ low-rank term, + bias), the split into Q, K, V and the rotation of Q's and
K's adjacent column pairs, within the error bound propagated from the GEMM's.  Every
call goes through the C ABI."""

import math

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


def rope_table(M, hd, seed, base=10000.0):
    """cos/sin [M, hd/2, 2] (fp32) of the angles pos(m) * base^(-2i/hd), with random
    token positions: the usual rotary frequencies."""
    pos = np.random.default_rng(seed).integers(0, 4096, M).astype(np.float64)
    inv = base ** (-np.arange(hd // 2) * 2.0 / hd)
    theta = pos[:, None] * inv[None, :]
    return np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)


def run_qkv(x, wt, dev, cs=None, hd=0, bias=None, l1=None, l2=None):
    M, K = x.shape
    N = wt.shape[0]
    D = N // 3
    g = quantize("mxfp4", x, dev, l1_bits=l1)
    w = pack("mxfp4", wt, dev)
    ys = [out_buffer(M, D, dev, f32=False) for _ in range(3)]
    b = bf16_dev(bias[None, :], dev)[0] if bias is not None else None
    l2t = bf16_dev(np.ascontiguousarray(l2.T), dev) if l2 is not None else None
    csd = torch.from_numpy(cs).to(dev) if cs is not None else None
    B.gemm_w4a4_lowrank_qkv_rope(g["codes"], g["scales"], w["codes"], w["scales"], M, N, K, *ys,
                                 t=g["t"] if l1 is not None else None, l2t=l2t, bias=b, cs=csd,
                                 head_dim=hd)
    torch.cuda.synchronize()
    out = []
    for y in ys:
        yh, ok = y_host(y, D)
        assert ok, "write outside the output"
        out.append(yh)
    return out


def ref_qkv(x, wt, cs, hd, bias=None, l1=None, l2=None, rows=None):
    xs = x if rows is None else x[rows]
    A = Q.mx_dequantize(*Q.mx_quantize(xs))
    Bm = Q.mx_dequantize(*Q.mx_quantize(wt))
    kw = {}
    if l1 is not None:
        kw = dict(x=F.bf16_to_f64(xs), l1=F.bf16_to_f64(l1), l2=F.bf16_to_f64(l2))
    y, bound = L.gemm_ref(A, Bm, bias=None if bias is None else F.bf16_to_f64(bias), **kw)
    if cs is None:                                 # the split alone: an identity rotation
        cs = np.zeros((len(y), 1, 2), np.float32)
        cs[:, :, 0] = 1.0
        hd = 2
    elif rows is not None:
        cs = cs[rows]
    return L.qkv_rope_ref(y, bound, cs, hd)


def check_all(got, ref, what):
    (q, k, v), (bq, bk, bv) = ref
    for g, r, b, name in zip(got, (q, k, v), (bq, bk, bv), "qkv"):
        _check(g, r, b, True, f"{what} {name}")


def test_quarter_turn_on_exact_gemm_results():
    # operands on the E2M1 grid: exact GEMM results; cos = 0, sin = 1 exactly, so Q and
    # K become (-b, a) pairs: the stored values equal the bf16 rounding of those
    dev = device()
    rng = np.random.default_rng(41)
    M, N, K, hd = 64, 384, 256, 32
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    xv = rng.choice(grid, (M, K)) * rng.choice([-1, 1], (M, K))
    wv = rng.choice(grid, (N, K)) * rng.choice([-1, 1], (N, K)) / 16
    xv[:, ::32] = 6
    wv[:, ::32] = 6 / 16
    x, wt = synth.to_bf16_bits(xv), synth.to_bf16_bits(wv)
    cs = np.zeros((M, hd // 2, 2), np.float32)
    cs[:, :, 1] = 1.0
    say("qkv rope quarter turn, exact")
    got = run_qkv(x, wt, dev, cs=cs, hd=hd)
    exact = xv @ wv.T
    (q, k, v), _ = L.qkv_rope_ref(exact, np.zeros_like(exact), cs, hd)
    for g, r in zip(got, (q, k, v)):
        want = F.bf16_to_f64(F.f32_to_bf16_rne(r.astype(np.float32)))
        assert np.array_equal(g, want)


@pytest.mark.parametrize("M,N,K,hd,r,rope", [(64, 384, 256, 64, 0, True), (300, 768, 384, 128, 32, True),
                                             (513, 1152, 512, 64, 16, True), (1, 384, 128, 2, 0, True),
                                             (200, 768, 256, 0, 32, False),
                                             # head widths that straddle the 32-column
                                             # passes, and one head over all of D
                                             (130, 1152, 256, 96, 0, True), (70, 1152, 128, 6, 16, True),
                                             (257, 1152, 256, 384, 32, True)])
def test_qkv_rope_parity(M, N, K, hd, r, rope):
    dev = device()
    x = synth.activations(M, K, seed=M + N + 7, dist="student_t3")[0]
    wt = synth.weights(N, K, seed=K + r + 3)
    bias = synth.bias(N, seed=N + 5)
    l1 = l2 = None
    if r:
        rng = np.random.default_rng(r + 1)
        l1 = synth.to_bf16_bits(rng.standard_normal((K, r)) * 0.05)
        l2 = synth.to_bf16_bits(rng.standard_normal((r, N)) * 0.05)
    cs = rope_table(M, hd, seed=M) if rope else None
    say(f"qkv rope {M}x{N}x{K} hd={hd} r={r} rope={rope}")
    got = run_qkv(x, wt, dev, cs=cs, hd=hd, bias=bias, l1=l1, l2=l2)
    check_all(got, ref_qkv(x, wt, cs, hd, bias=bias, l1=l1, l2=l2), f"qkv {M}x{N}x{K}")


def test_qkv_rope_half_tiles():
    # 2 x 132 tiles on 256 CUs (N = 3 x 11264): the 8 leftover tiles run as halves;
    # ragged M; every output checked
    dev = device()
    M, N, K, hd = 300, 3 * 11264, 256, 128
    x = synth.activations(M, K, seed=19, dist="student_t3")[0]
    wt = synth.weights(N, K, seed=20)
    cs = rope_table(M, hd, seed=21)
    say(f"qkv rope half tiles {M}x{N}x{K}")
    got = run_qkv(x, wt, dev, cs=cs, hd=hd)
    check_all(got, ref_qkv(x, wt, cs, hd), "qkv half tiles")


def test_qkv_rope_full_attention_qkv_sampled_rows():
    # a fused QKV projection of the attention blocks: 4608 tokens, 3072 -> 3 x 3072,
    # head width 128, rank-32 branch; 40 sampled rows against the oracle
    dev = device()
    d = weight_prep.mlp_up_svd(seed=3, N=9216)
    M, hd = d["M"], 128
    cs = rope_table(M, hd, seed=22)
    say("qkv rope full 4608x3072x9216 r=32")
    got = run_qkv(d["x"], d["rt"], dev, cs=cs, hd=hd, l1=d["l1"], l2=d["l2"])
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(5).choice(M, 38)]))
    ref = ref_qkv(d["x"], d["rt"], cs, hd, l1=d["l1"], l2=d["l2"], rows=rows)
    check_all([g[rows] for g in got], ref, "qkv full")
