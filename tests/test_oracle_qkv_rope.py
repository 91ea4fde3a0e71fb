"""Pins of the oracle's QKV-split and RoPE epilogue (oracle/layer.py qkv_rope_ref)
against what the mathematics fixes: a quarter turn, a turn and its inverse, the pair
norm, a per-element brute force of the head and pair indexing, and the error bound
checked against perturbations of the GEMM results."""

import math

import numpy as np
import pytest

from oracle import layer as L


def table(M, hd, theta):
    """cs [M, hd/2, 2] for the angles theta[m, i]."""
    return np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)


def test_quarter_turn_swaps_with_sign():
    M, hd, heads = 3, 8, 2
    D = hd * heads
    y = np.random.default_rng(0).standard_normal((M, 3 * D))
    cs = np.zeros((M, hd // 2, 2), np.float32)
    cs[:, :, 1] = 1.0                                   # c = 0, s = 1 exactly
    (q, k, v), _ = L.qkv_rope_ref(y, np.zeros_like(y), cs, hd)
    for part, src in ((q, y[:, :D]), (k, y[:, D:2 * D])):
        assert np.array_equal(part[:, 0::2], -src[:, 1::2])
        assert np.array_equal(part[:, 1::2], src[:, 0::2])
    assert np.array_equal(v, y[:, 2 * D:])


def test_turn_then_inverse_and_norm():
    rng = np.random.default_rng(1)
    M, hd, heads = 4, 16, 3
    D = hd * heads
    y = rng.standard_normal((M, 3 * D))
    theta = rng.uniform(-math.pi, math.pi, (M, hd // 2))
    cs = table(M, hd, theta)
    (q, k, v), _ = L.qkv_rope_ref(y, np.zeros_like(y), cs, hd)
    # the pair norms are kept (cos^2 + sin^2 = 1 up to the fp32 rounding of the table)
    for part, src in ((q, y[:, :D]), (k, y[:, D:2 * D])):
        n0 = part[:, 0::2] ** 2 + part[:, 1::2] ** 2
        n1 = src[:, 0::2] ** 2 + src[:, 1::2] ** 2
        assert np.allclose(n0, n1, rtol=1e-6)
    # rotating back by the transposed table restores the input
    back = cs.copy()
    back[:, :, 1] = -back[:, :, 1]
    y2 = np.concatenate([q, k, v], axis=1)
    (q2, k2, _), _ = L.qkv_rope_ref(y2, np.zeros_like(y2), back, hd)
    assert np.allclose(q2, y[:, :D], atol=1e-6) and np.allclose(k2, y[:, D:2 * D], atol=1e-6)


def test_indexing_against_brute_force():
    rng = np.random.default_rng(2)
    M, hd, heads = 2, 6, 4
    D = hd * heads
    y = rng.standard_normal((M, 3 * D))
    cs = table(M, hd, rng.uniform(-3, 3, (M, hd // 2)))
    (q, k, v), _ = L.qkv_rope_ref(y, np.zeros_like(y), cs, hd)
    out = np.concatenate([q, k, v], axis=1)
    for m in range(M):
        for n in range(3 * D):
            sec, col = divmod(n, D)
            if sec == 2:
                assert out[m, n] == y[m, n]
                continue
            i = (col % hd) // 2
            c, s = float(cs[m, i, 0]), float(cs[m, i, 1])
            a, b = y[m, n - (col % 2)], y[m, n - (col % 2) + 1]
            want = a * c - b * s if col % 2 == 0 else a * s + b * c
            assert math.isclose(out[m, n], want, rel_tol=1e-15, abs_tol=1e-15)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        L.qkv_rope_ref(np.zeros((2, 30)), np.zeros((2, 30)), np.zeros((2, 2, 2)), 4)   # D = 10
    with pytest.raises(ValueError):
        L.qkv_rope_ref(np.zeros((2, 24)), np.zeros((2, 24)), np.zeros((2, 3, 2)), 4)   # cs shape


def test_bound_covers_perturbed_gemm_results():
    rng = np.random.default_rng(3)
    M, hd, heads = 16, 8, 2
    D = hd * heads
    y = rng.standard_normal((M, 3 * D)) * 5
    bound = np.abs(y) * rng.uniform(0.5, 20, y.shape) + 0.1
    cs = table(M, hd, rng.uniform(-math.pi, math.pi, (M, hd // 2)))
    ref, bnd = L.qkv_rope_ref(y, bound, cs, hd)
    for trial in range(30):
        e = rng.choice([-1.0, 1.0], y.shape) if trial < 10 else rng.uniform(-1, 1, y.shape)
        yp = y + L.GEMM_REL_TOL * bound * e
        got, _ = L.qkv_rope_ref(yp, bound, cs, hd)
        # (V passes through: its change reaches the bound exactly at the corners, so
        # allow the fp64 rounding of the perturbation itself)
        for g, r, b in zip(got, ref, bnd):
            assert np.all(np.abs(g - r) <= L.GEMM_REL_TOL * b * (1 + 1e-12))
