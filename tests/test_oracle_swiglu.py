"""Pins of the oracle's SwiGLU epilogue (oracle/layer.py swiglu_ref, silu) against
what the mathematics fixes: SciPy's logistic function, the identity
silu(z) - silu(-z) = z, a column-by-column brute force of the gate/up layout, the
slope constant found by a library optimizer, and the error bound checked against
perturbations of the GEMM results."""

import numpy as np
import pytest
from scipy.optimize import minimize_scalar
from scipy.special import expit

from oracle import layer as L


def test_silu_is_z_times_logistic():
    z = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-30, -1e-30, 700.0, -700.0]])
    assert np.allclose(L.silu(z), z * expit(z), rtol=1e-15, atol=0.0)


def test_silu_odd_part_identity():
    # sigmoid(z) + sigmoid(-z) = 1, so silu(z) - silu(-z) = z
    z = np.random.default_rng(0).standard_normal(1000) * 8
    assert np.allclose(L.silu(z) - L.silu(-z), z, rtol=1e-14, atol=1e-14)


def test_silu_limits():
    assert L.silu(0.0) == 0.0
    assert L.silu(800.0) == 800.0                        # sigmoid rounds to 1
    assert L.silu(-800.0) == 0.0 and np.signbit(L.silu(-800.0))


def test_slope_constant_bounds_the_derivative():
    # d/dz silu(z) = s(z) (1 + z (1 - s(z))), s the logistic function; its maximum by
    # a bounded scalar optimizer, and its minimum (about -0.0998) is smaller in size
    def slope(z):
        s = expit(z)
        return s * (1 + z * (1 - s))

    top = minimize_scalar(lambda z: -slope(z), bounds=(0, 10), method="bounded")
    low = minimize_scalar(slope, bounds=(-10, 0), method="bounded")
    assert -top.fun <= L.SILU_SLOPE_MAX < -top.fun + 1e-4
    assert abs(low.fun) < L.SILU_SLOPE_MAX


def brute_force(y):
    M, N = y.shape
    out = np.zeros((M, N // 2))
    blk = L.SWIGLU_BLOCK
    for m in range(M):
        for j in range(N // (2 * blk)):
            for c in range(blk):
                g = y[m, 2 * blk * j + c]
                u = y[m, 2 * blk * j + blk + c]
                out[m, blk * j + c] = g * expit(g) * u
    return out


def test_layout_against_brute_force():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((3, 4 * L.SWIGLU_BLOCK)) * 4
    out, _ = L.swiglu_ref(y, np.ones_like(y))
    assert out.shape == (3, 2 * L.SWIGLU_BLOCK)
    assert np.allclose(out, brute_force(y), rtol=1e-14, atol=1e-14)
    # a plausible mistake: gate and up exchanged
    blk = L.SWIGLU_BLOCK
    swapped = y.reshape(3, 2, 2, blk)[:, :, ::-1, :].reshape(y.shape)
    assert not np.allclose(out, brute_force(swapped))


def test_rejects_n_not_a_multiple_of_two_blocks():
    with pytest.raises(ValueError):
        L.swiglu_ref(np.zeros((2, 3 * L.SWIGLU_BLOCK)), np.zeros((2, 3 * L.SWIGLU_BLOCK)))


def test_bound_covers_perturbed_gemm_results():
    # perturb gate and up by up to the GEMM tolerance (1e-3 bound), at the corners and
    # at random inside: the change of silu(gate) * up stays within 1e-3 out_bound
    rng = np.random.default_rng(2)
    blk = L.SWIGLU_BLOCK
    y = rng.standard_normal((64, 2 * blk)) * np.exp(rng.uniform(-3, 3, (64, 1)))
    bound = np.abs(y) * rng.uniform(0.5, 50, y.shape) + rng.uniform(0, 2, y.shape)
    out, out_bound = L.swiglu_ref(y, bound)
    tol = L.GEMM_REL_TOL * out_bound
    for trial in range(40):
        if trial < 4:
            sg, su = [(1, 1), (1, -1), (-1, 1), (-1, -1)][trial]
            e = np.concatenate([np.full((64, blk), sg), np.full((64, blk), su)], axis=1)
        else:
            e = rng.uniform(-1, 1, y.shape)
        yp = y + L.GEMM_REL_TOL * bound * e
        outp, _ = L.swiglu_ref(yp, bound)
        assert np.all(np.abs(outp - out) <= tol)
