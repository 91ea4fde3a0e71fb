"""Pins of the oracle's layer (GEMM, low-rank branch, bias, tolerance): closed
forms, brute-force rational arithmetic on tiny shapes, and the special cases in
which the layer reduces to something simpler."""

from fractions import Fraction

import numpy as np

from bit_quantized_gemm_quantize_amd import synth
from oracle import formats as F
from oracle import layer as L
from oracle import quant as Q


def test_all_ones_codes_closed_form():
    # every element code 0x2 (= 1.0), scales 2**a and 2**b: Y = K * 2**(a + b)
    M, N, K = 5, 7, 256
    for a, b in [(0, 0), (-3, 5), (20, -40), (-127, 100)]:
        ac = np.full((M, K // 2), 0x22, np.uint8)
        bc = np.full((N, K // 2), 0x22, np.uint8)
        asc = np.full((M, K // 32), a + 127, np.uint8)
        bsc = np.full((N, K // 32), b + 127, np.uint8)
        y, bound = L.gemm_ref(Q.mx_dequantize(ac, asc), Q.mx_dequantize(bc, bsc))
        assert np.all(y == K * 2.0 ** (a + b))
        assert np.all(bound == y)


def test_gemm_brute_force_rational_tiny():
    rng = np.random.default_rng(12)
    M, N, K, r = 3, 4, 64, 2
    ac = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    bc = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    asc = rng.integers(120, 135, (M, K // 32)).astype(np.uint8)
    bsc = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
    x = synth.activations(M, K, seed=1)[0]
    l1 = synth.to_bf16_bits(rng.standard_normal((K, r)) * 0.1)
    l2 = synth.to_bf16_bits(rng.standard_normal((r, N)) * 0.1)
    bias = synth.to_bf16_bits(rng.standard_normal(N))
    A, B = Q.mx_dequantize(ac, asc), Q.mx_dequantize(bc, bsc)
    X, L1, L2, b = (F.bf16_to_f64(v) for v in (x, l1, l2, bias))
    y, bound = L.gemm_ref(A, B, bias=b, x=X, l1=L1, l2=L2)
    # Python loops over exact fractions: sum_k A B + sum_j (sum_k X L1) L2 + bias
    fr = np.vectorize(Fraction)
    Af, Bf, Xf, L1f, L2f, bf = fr(A), fr(B), fr(X), fr(L1), fr(L2), fr(b)
    for m in range(M):
        t = [sum(Xf[m, k] * L1f[k, j] for k in range(K)) for j in range(r)]
        for n in range(N):
            exact = sum(Af[m, k] * Bf[n, k] for k in range(K))
            exact += sum(t[j] * L2f[j, n] for j in range(r)) + bf[n]
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 2 ** 40) * abs(Fraction(bound[m, n]))
            mag = sum(abs(Af[m, k] * Bf[n, k]) for k in range(K)) + abs(bf[n])
            mag += sum(sum(abs(Xf[m, k] * L1f[k, j]) for k in range(K)) * abs(L2f[j, n]) for j in range(r))
            assert abs(Fraction(bound[m, n]) - mag) <= Fraction(1, 2 ** 40) * mag


def test_zero_residual_reduces_to_lowrank_product():
    # R = 0 (all codes 0): the layer is (X L1) L2, evaluated right to left
    rng = np.random.default_rng(2)
    M, N, K, r = 4, 6, 64, 3
    x = F.bf16_to_f64(synth.activations(M, K, seed=3)[0])
    l1 = F.bf16_to_f64(synth.to_bf16_bits(rng.standard_normal((K, r))))
    l2 = F.bf16_to_f64(synth.to_bf16_bits(rng.standard_normal((r, N))))
    zeros_a = Q.mx_dequantize(np.zeros((M, K // 2), np.uint8), np.full((M, 2), 127, np.uint8))
    zeros_b = Q.mx_dequantize(np.zeros((N, K // 2), np.uint8), np.full((N, 2), 127, np.uint8))
    y, _ = L.gemm_ref(zeros_a, zeros_b, x=x, l1=l1, l2=l2)
    for m in range(M):
        for n in range(N):
            want = sum(sum(x[m, k] * l1[k, j] for k in range(K)) * l2[j, n] for j in range(r))
            assert abs(y[m, n] - want) <= 1e-12 * (1 + abs(want))


def test_zero_lowrank_reduces_to_plain_gemm():
    d = synth.tiny_layer()
    ac, asc = Q.mx_quantize(d["x"])
    bc, bsc = Q.mx_quantize(d["wt"])
    A, B = Q.mx_dequantize(ac, asc), Q.mx_dequantize(bc, bsc)
    y0, b0 = L.gemm_ref(A, B)
    X = F.bf16_to_f64(d["x"])
    y1, b1 = L.gemm_ref(A, B, x=X, l1=np.zeros((256, 16)), l2=np.zeros((16, 256)))
    assert np.array_equal(y0, y1) and np.array_equal(b0, b1)


def test_tolerance_values():
    y = np.array([1.0, 100.0, 0.0])
    bound = np.array([10.0, 100.0, 0.0])
    assert np.allclose(L.tolerance(y, bound, out_bf16=False), [1e-2, 0.1, 0.0])
    tb = L.tolerance(y, bound, out_bf16=True)
    # half a bf16 ulp at |y| + tol: 2**-8 at 1.01, 2**-2 at 100.1, 2**-134 at 0
    assert np.allclose(tb, [1e-2 + 2.0 ** -8, 0.1 + 2.0 ** -2, 2.0 ** -134])
    ok, worst, _ = L.check_close(np.array([1.0 + 9e-3, 100.0, 0.0]), y, bound, out_bf16=False)
    assert ok and 0.89 < worst < 0.91
    ok, _, _ = L.check_close(np.array([1.02, 100.0, 0.0]), y, bound, out_bf16=False)
    assert not ok
    ok, _, _ = L.check_close(np.array([1.0, 100.0, 1e-30]), y, bound, out_bf16=False)
    assert not ok


def test_quality_context_quantization_error_ordering():
    # Not a pass/fail claim of the pages (their quality figures need trained
    # models); a sanity check that the quantizers behave: W4A16 int4 error is
    # below W4A4 MXFP4 error against the unquantized bf16 layer.
    d = synth.attn_proj(seed=0, M=64, K=512, N=128)
    y_exact = L.unquantized_ref(d["x"], d["wt"])
    ac, asc = Q.mx_quantize(d["x"])
    bc, bsc = Q.mx_quantize(d["wt"])
    y44, _ = L.gemm_ref(Q.mx_dequantize(ac, asc), Q.mx_dequantize(bc, bsc))
    qc, qs, qz = Q.int4_g64_quantize(d["wt"])
    y416, _ = L.gemm_ref(F.bf16_to_f64(d["x"]), Q.int4_g64_dequantize(qc, qs, qz))
    e44 = L.relative_error(y44, y_exact)
    e416 = L.relative_error(y416, y_exact)
    assert e416 < e44 < 0.5
