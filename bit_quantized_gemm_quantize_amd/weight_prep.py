"""Offline weight preparation for the low-rank branch (host side, NumPy, fp64).

Nothing here runs on the layer's forward path: the library's calls take the
prepared L1, L2 and the packed residual as inputs.  These functions turn a bf16
weight (and, for the SVDQuant preparations, calibration activations) into those
inputs, once per model, as the SVDQuant Guide's offline decomposition does
("Step 1: Low-Rank Outlier Decomposition in PyTorch").  The tests and the bench
use them to build the layers they run; the CPU tests pin each of them (truncated
SVD and Eckart-Young optimality, closed forms, reconstruction of the weight).

Orientation: the weight arrives as W^T [N, K] bf16 bits (nn.Linear's [out, in]),
the layer computes Y = X W with L1 [K, r] and L2 [r, N], so X L1 L2 is the
branch.  The Guide writes the same factors the other way round ([out, r] and
[r, in]); its L1 is this module's L2^T and its L2 this module's L1^T.

Four preparations:

* ``lowrank_split``: rank-r truncated SVD of W itself, W = L1 L2 + R.
* ``guide_step1_split``: the Guide's Step-1 recipe as the page prints it: a
  per-output-channel symmetric INT4 estimate of W, its error dW = W - Q(W), the
  SVD of the covariance-weighted error dW C, and the residual W - L1 L2.
* ``svdquant_split``: smoothing factors, then the best rank-r approximation of
  the smoothed weight in the activation-weighted norm, then the residual.
* ``smoothing_factors`` / ``weighted_lowrank``: the two steps of the latter.
"""

import numpy as np

from . import synth


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def lowrank_split(wt_bits, rank, seed, oversample=10, power_iters=2):
    """Split the logical weight W [K, N] = (W^T)^T into a rank-r part L1 [K, r] @
    L2 [r, N] plus a residual R, with a seeded randomized truncated SVD.

    L1 = V_r sqrt(S_r), L2 = sqrt(S_r) U_r^T (the square-root split of the SVD that
    the Guide's Step 1 uses, written for this orientation), both rounded to bf16;
    the residual is R = bf16(W - L1 L2) with the product taken in fp64.
    Returns (l1_bits [K, r], l2_bits [r, N], rt_bits [N, K] = R^T).
    """
    wt = _f64(wt_bits)                                           # [N, K]
    N, K = wt.shape
    rng = synth.generator(seed + 3 * synth.W_SEED_OFFSET)
    omega = rng.standard_normal((K, rank + oversample))
    y = wt @ omega
    for _ in range(power_iters):
        y, _r = np.linalg.qr(y)
        y = wt @ (wt.T @ y)
    q, _r = np.linalg.qr(y)
    ub, s, vh = np.linalg.svd(q.T @ wt, full_matrices=False)
    u = q @ ub                                                   # [N, r+p]
    root = np.sqrt(s[:rank])
    l1 = synth.to_bf16_bits(vh[:rank].T * root[None, :])         # [K, r]
    l2 = synth.to_bf16_bits(root[:, None] * u[:, :rank].T)       # [r, N]
    approx_t = (_f64(l1) @ _f64(l2)).T
    rt = synth.to_bf16_bits(wt - approx_t)                       # [N, K]
    return l1, l2, rt


def int4_channel_estimate(w):
    """The Guide's base quantization estimate of a weight [out, in] in fp64: each
    output channel (row) on its own symmetric signed 4-bit grid.  The grid step is
    the row's largest magnitude over 7 (the largest positive 4-bit code), floored
    at 1e-8; each entry goes to the nearest grid point (ties to the even multiple),
    limited to the codes -8 .. 7.  Returns the dequantized estimate."""
    step = np.maximum(np.abs(w).max(axis=1, keepdims=True) / 7.0, 1e-8)
    return np.clip(np.rint(w / step), -8.0, 7.0) * step


def guide_step1_split(x_cal_bits, wt_bits, rank):
    """The Guide's Step-1 decomposition, taken literally (its "1. Mathematical
    Outlier Factorization" prose and its Step-1 code), in fp64:

      1. W_q = the per-channel INT4 estimate of W (``int4_channel_estimate``);
      2. dW = W - W_q;
      3. C = the covariance of the calibration activations (centred, n - 1
         normalisation, as a covariance of the columns);
      4. U S V^T = SVD(dW C); the Guide's factors U_r sqrt(S_r) [out, r] and
         sqrt(S_r) V_r^T [r, in];
      5. the residual W - (product of the two factors), which the layer quantizes.

    dW C carries the units of W times those of X squared, so the factors it yields
    are not an approximation of dW; on activations with large outlier channels the
    residual grows in those channels.  The layer built from it is reported next to
    the other preparations, as the page's own recipe.

    In this module's orientation L1 = (sqrt(S_r) V_r^T)^T [K, r] and L2 =
    (U_r sqrt(S_r))^T [r, N], rounded to bf16; the residual is formed from the
    unrounded factors, as the Guide does, and rounded to bf16.
    Returns dict(l1 bf16 [K, r], l2 bf16 [r, N], rt bf16 [N, K] = residual^T,
    singular_values)."""
    w = _f64(wt_bits)                                            # [out, in] = [N, K]
    left, right, s = guide_step1_factors(w, np.cov(_f64(x_cal_bits).T), rank)
    resid = w - left @ right
    return dict(l1=synth.to_bf16_bits(right.T), l2=synth.to_bf16_bits(left.T),
                rt=synth.to_bf16_bits(resid), singular_values=s)


def guide_step1_factors(w, c, rank):
    """Steps 1, 2 and 4 of ``guide_step1_split`` for a weight w [out, in] and a
    covariance c [in, in], in fp64: the factors U_r sqrt(S_r) [out, r] and
    sqrt(S_r) V_r^T [r, in] of the truncated SVD of (w - int4_channel_estimate(w)) c,
    and all singular values."""
    dw = w - int4_channel_estimate(w)
    u, s, vh = np.linalg.svd(dw @ c, full_matrices=False)
    root = np.sqrt(s[:rank])
    return u[:, :rank] * root[None, :], root[:, None] * vh[:rank], s


def smoothing_factors(x_cal_bits, wt_bits, alpha=0.5):
    """Per-input-channel smoothing factors s [K] for X' = X diag(s)^-1, W' = diag(s) W
    (the SVDQuant Guide, "2. SmoothQuant Pre-Conditioning for DiTs", gives the
    transform but not how s is chosen).  Taken from SmoothQuant: s_j =
    max|X_j|^alpha / max|W_j|^(1 - alpha) over the calibration rows and the weight's
    output columns, alpha = 0.5; 1 for a channel that is zero on either side.
    Returned as the fp32 reciprocals inv_s = fp32(1 / s) the quantizer multiplies
    by, and the fp64 factors s = 1 / inv_s that exactly undo them."""
    xa = np.abs(_f64(x_cal_bits)).max(axis=0)                    # [K]
    wa = np.abs(_f64(wt_bits)).max(axis=0)                       # [K] (W^T is [N, K])
    ok = (xa > 0) & (wa > 0)
    s = np.ones_like(xa)
    s[ok] = xa[ok] ** alpha / wa[ok] ** (1.0 - alpha)
    inv_s = (1.0 / s).astype(np.float32)
    return inv_s, 1.0 / inv_s.astype(np.float64)


def weighted_lowrank(w, c, rank, ridge=1e-6):
    """Best rank-r approximation L1 L2 of w [K, N] in the activation-weighted norm
    ||C^(1/2) (w - L1 L2)||_F, C [K, K] the calibration covariance (the norm of the
    output error X (w - L1 L2) for activations of that covariance).  Whitening with
    C^(1/2), a truncated SVD and un-whitening with C^(-1/2) is the exact minimizer
    of that weighted error.  A ridge of `ridge` times the mean diagonal keeps C
    invertible.  L1 = C^(-1/2) U_r sqrt(S_r), L2 = sqrt(S_r) V_r^T.
    Returns (l1 [K, r], l2 [r, N], s_all) in fp64, s_all the weighted singular values."""
    K = c.shape[0]
    c = 0.5 * (c + c.T) + ridge * np.trace(c) / K * np.eye(K)
    lam, q = np.linalg.eigh(c)
    root = (q * np.sqrt(lam)[None, :]) @ q.T
    inv_root = (q / np.sqrt(lam)[None, :]) @ q.T
    u, sv, vh = np.linalg.svd(root @ w, full_matrices=False)
    r = np.sqrt(sv[:rank])
    return inv_root @ (u[:, :rank] * r[None, :]), r[:, None] * vh[:rank], sv


def svdquant_split(x_cal_bits, wt_bits, rank, alpha=0.5):
    """SVDQuant preparation: smoothing factors from calibration activations, W' =
    diag(s) W, the activation-weighted rank-r split of W' (weighted by the
    covariance of the smoothed calibration activations), and the residual R' =
    W' - L1' L2 for 4-bit quantization.

    The Guide's Step 1 weights the quantization error by the covariance and then
    subtracts factors of that product from W; this preparation instead minimizes
    the error that weighting stands for, ||C^(1/2) (W' - L1' L2)||, over rank-r
    factors of the smoothed weight itself (``guide_step1_split`` is the literal
    recipe).

    The forward pass computes Q(X diag(s)^-1) Q(R')^T + (X L1) L2 with the folded
    down-projection L1 = diag(s)^-1 L1', so the low-rank branch takes the
    unsmoothed X.  L1 and L2 are rounded to bf16 first; R' = bf16(W' -
    diag(s) L1 L2) in fp64 absorbs that rounding.
    Returns dict(inv_s fp32 [K], l1 bf16 [K, r], l2 bf16 [r, N], rt bf16 [N, K] = R'^T,
    weighted singular values)."""
    inv_s, s = smoothing_factors(x_cal_bits, wt_bits, alpha)
    w = _f64(wt_bits).T * s[:, None]                             # W' [K, N]
    xc = _f64(x_cal_bits) * inv_s.astype(np.float64)[None, :]
    c = np.cov(xc.T)
    l1p, l2, sv = weighted_lowrank(w, c, rank)
    l1 = synth.to_bf16_bits(l1p * inv_s.astype(np.float64)[:, None])   # folded [K, r]
    l2 = synth.to_bf16_bits(l2)
    l1f = _f64(l1) * s[:, None]                                  # L1' as stored
    rt = synth.to_bf16_bits((w - l1f @ _f64(l2)).T)
    return dict(inv_s=inv_s, l1=l1, l2=l2, rt=rt, singular_values=sv)


# --------------------------------------------------------------------------- prepared layers

def mlp_up_svd(seed=0, M=4608, K=3072, N=12288, rank=32):
    """MLP up-projection with the low-rank branch: X Student-t(3); W N(0,0.02)
    split into bf16 L1 [K, r], L2 [r, N] and a residual R^T [N, K] to quantize."""
    x, _, _ = synth.activations(M, K, seed, dist="student_t3")
    wt = synth.weights(N, K, seed)
    l1, l2, rt = lowrank_split(wt, rank, seed)
    return dict(name=f"mlp_up_svd_r{rank}_{M}x{K}x{N}", x=x, wt=wt, l1=l1, l2=l2, rt=rt,
                M=M, K=K, N=N, rank=rank)


def attn_proj_calibrated(seed=0, M=4608, K=3072, N=3072, calib=512):
    """The attention projection's inputs (X N(0,1) with 1% of channels x U(30,100),
    W N(0,0.02)) plus `calib` calibration rows drawn with X (same outlier channels,
    disjoint rows)."""
    xa, ch, g = synth.activations(M + calib, K, seed, outliers=int(round(0.01 * K)))
    return dict(x=xa[:M], x_cal=xa[M:], wt=synth.weights(N, K, seed), outlier_channels=ch,
                outlier_gains=g, M=M, K=K, N=N)


def attn_proj_svdquant(seed=0, M=4608, K=3072, N=3072, rank=32, calib=512):
    """The attention projection prepared the SVDQuant way: smoothing, an
    activation-weighted rank-r split and a 4-bit residual, from the calibration
    rows of ``attn_proj_calibrated``."""
    d = attn_proj_calibrated(seed, M, K, N, calib)
    d.update(svdquant_split(d["x_cal"], d["wt"], rank))
    d.update(name=f"attn_proj_svdquant_r{rank}_{M}x{K}x{N}", rank=rank)
    return d
