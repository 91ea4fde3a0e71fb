"""Seeded synthetic inputs for the 4-bit DiT linear layer.

This module only *draws* inputs; it holds none of the layer's arithmetic (no
quantization, no GEMM).  Both the HIP path and the CPU oracle consume exactly the
bytes it returns, so they always see the same bf16 tensors.

Shapes stand in for the linear layers of a FLUX-class diffusion transformer: at
1024x1024 an image gives 4096 latent tokens, plus 512 text tokens (the text
embedding has 512 rows in "Four Bits", FLUX.2 [dev] architecture walk-through, and
in the SVDQuant Guide's text-encoder offloading advice), so M = 4608; at 2048x2048,
16384 + 512 = 16896 tokens.  Hidden size 3072 and a 4x MLP expansion (12288).
Activations carry the heavy outlier channels the SVDQuant Guide describes ("Why
Standard Low-Bit Quantization Fails on DiTs": a handful of channels far above the
median, moving with the timestep).

Random draws use NumPy's PCG64 generator; activations use seed s and weights seed
s + 1000.  fp32 draws are rounded to bf16 with round-to-nearest-even.
"""

import numpy as np

W_SEED_OFFSET = 1000


def generator(seed):
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x):
    """fp32/fp64 array -> bf16 bit patterns (uint16), round to nearest even.
    Rounds fp64 to fp32 first (numpy's cast), then fp32 to bf16 on the bit pattern."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    if not np.all(np.isfinite(np.asarray(x, dtype=np.float32))):
        raise ValueError("synthetic inputs must be finite")
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(rng, K, count):
    return np.sort(rng.choice(K, size=count, replace=False))


def activations(M, K, seed, dist="normal", outliers=0, outlier_gain=None):
    """X [M, K] bf16 bits.

    dist: "normal" (N(0,1)) or "student_t3" (Student-t, 3 degrees of freedom).
    outliers: number of channels (columns) scaled up; outlier_gain None draws each
    channel's gain from U(30, 100), a number uses that gain for every channel.
    Returns (x_bits, channel_indices, gains).
    """
    rng = generator(seed)
    if dist == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32)
    elif dist == "student_t3":
        x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    else:
        raise ValueError(dist)
    ch = outlier_channels(rng, K, outliers) if outliers else np.zeros(0, dtype=np.int64)
    if outliers:
        gains = (np.full(outliers, float(outlier_gain)) if outlier_gain is not None
                 else rng.uniform(30.0, 100.0, size=outliers))
        x[:, ch] *= gains.astype(np.float32)[None, :]
    else:
        gains = np.zeros(0)
    return to_bf16_bits(x), ch, gains


def weights(N, K, seed, std=0.02):
    """W^T [N, K] bf16 bits (out-features x in-features, in-features contiguous),
    i.i.d. N(0, std^2)."""
    rng = generator(seed + W_SEED_OFFSET)
    return to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(std))


def bias(N, seed, std=0.1):
    rng = generator(seed + 2 * W_SEED_OFFSET)
    return to_bf16_bits(rng.standard_normal(N, dtype=np.float32) * np.float32(std))


def lowrank_split(wt_bits, rank, seed, oversample=10, power_iters=2):
    """Offline weight preparation, not part of the layer's forward pass: split the
    logical weight W [K, N] = (W^T)^T into a rank-r part L1 [K, r] @ L2 [r, N]
    plus a residual R, using a seeded randomized truncated SVD.

    L1 = V_r sqrt(S_r), L2 = sqrt(S_r) U_r^T (the SVDQuant Guide's factorization
    U sqrt(S), sqrt(S) Vh of "Step 1", written for this orientation), both rounded
    to bf16; the residual is R = bf16(W - L1 L2) with the product taken in fp64.
    Returns (l1_bits [K, r], l2_bits [r, N], rt_bits [N, K] = R^T).
    """
    wt = bf16_bits_to_f32(wt_bits).astype(np.float64)          # [N, K]
    N, K = wt.shape
    rng = generator(seed + 3 * W_SEED_OFFSET)
    omega = rng.standard_normal((K, rank + oversample))
    y = wt @ omega
    for _ in range(power_iters):
        y, _r = np.linalg.qr(y)
        y = wt @ (wt.T @ y)
    q, _r = np.linalg.qr(y)
    ub, s, vh = np.linalg.svd(q.T @ wt, full_matrices=False)
    u = q @ ub                                                 # [N, r+p]
    root = np.sqrt(s[:rank])
    l1 = to_bf16_bits(vh[:rank].T * root[None, :])             # [K, r]
    l2 = to_bf16_bits(root[:, None] * u[:, :rank].T)           # [r, N]
    approx_t = (bf16_bits_to_f32(l1).astype(np.float64) @ bf16_bits_to_f32(l2).astype(np.float64)).T
    rt = to_bf16_bits(wt - approx_t)                           # [N, K]
    return l1, l2, rt


def smoothing_factors(x_cal_bits, wt_bits, alpha=0.5):
    """Per-input-channel smoothing factors s [K] for X' = X diag(s)^-1, W' = diag(s) W
    (the SVDQuant Guide, "2. SmoothQuant Pre-Conditioning for DiTs", gives the
    transform but not how s is chosen).  Taken from SmoothQuant: s_j =
    max|X_j|^alpha / max|W_j|^(1 - alpha) over the calibration rows and the weight's
    output columns, alpha = 0.5; 1 for a channel that is zero on either side.
    Returned as the fp32 reciprocals inv_s = fp32(1 / s) the quantizer multiplies
    by, and the fp64 factors s = 1 / inv_s that exactly undo them."""
    xa = np.abs(bf16_bits_to_f32(x_cal_bits).astype(np.float64)).max(axis=0)     # [K]
    wa = np.abs(bf16_bits_to_f32(wt_bits).astype(np.float64)).max(axis=0)        # [K] (W^T is [N, K])
    ok = (xa > 0) & (wa > 0)
    s = np.ones_like(xa)
    s[ok] = xa[ok] ** alpha / wa[ok] ** (1.0 - alpha)
    inv_s = (1.0 / s).astype(np.float32)
    return inv_s, 1.0 / inv_s.astype(np.float64)


def weighted_lowrank(w, c, rank, ridge=1e-6):
    """Best rank-r approximation L1 L2 of w [K, N] in the activation-weighted norm
    ||C^(1/2) (w - L1 L2)||_F, C [K, K] the calibration covariance (the norm of the
    output error X (w - L1 L2) for activations of that covariance).  The SVDQuant
    Guide's Step 1 weights the quantization error by the covariance before its SVD;
    whitening with C^(1/2), a truncated SVD and un-whitening with C^(-1/2) is the
    exact minimizer of that weighted error.  A ridge of `ridge` times the mean
    diagonal keeps C invertible.  L1 = C^(-1/2) U_r sqrt(S_r), L2 = sqrt(S_r) V_r^T.
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
    """Offline SVDQuant weight preparation, not part of the forward pass: smoothing
    factors from calibration activations, W' = diag(s) W, the activation-weighted
    rank-r split of W' (weighted by the covariance of the smoothed calibration
    activations, torch.cov's centring as in the SVDQuant Guide's Step 1), and the
    residual R' = W' - L1' L2 for 4-bit quantization.

    The forward pass computes Q(X diag(s)^-1) Q(R')^T + (X L1) L2 with the folded
    down-projection L1 = diag(s)^-1 L1', so the low-rank branch takes the
    unsmoothed X.  L1 and L2 are rounded to bf16 first; R' = bf16(W' -
    diag(s) L1 L2) in fp64 absorbs that rounding.
    Returns dict(inv_s fp32 [K], l1 bf16 [K, r], l2 bf16 [r, N], rt bf16 [N, K] = R'^T,
    weighted singular values)."""
    inv_s, s = smoothing_factors(x_cal_bits, wt_bits, alpha)
    w = bf16_bits_to_f32(wt_bits).astype(np.float64).T * s[:, None]           # W' [K, N]
    xc = bf16_bits_to_f32(x_cal_bits).astype(np.float64) * inv_s.astype(np.float64)[None, :]
    c = np.cov(xc.T)
    l1p, l2, sv = weighted_lowrank(w, c, rank)
    l1 = to_bf16_bits(l1p * inv_s.astype(np.float64)[:, None])                # folded [K, r]
    l2 = to_bf16_bits(l2)
    l1f = bf16_bits_to_f32(l1).astype(np.float64) * s[:, None]                 # L1' as stored
    rt = to_bf16_bits((w - l1f @ bf16_bits_to_f32(l2).astype(np.float64)).T)
    return dict(inv_s=inv_s, l1=l1, l2=l2, rt=rt, singular_values=sv)


# --------------------------------------------------------------------------- workloads
# Named by what they are; the full-size ones are the shapes of the layers above.

def tiny_layer(seed=0):
    """64 x 256 x 256 MXFP4 layer: X N(0,1) with 2 outlier channels x50, W N(0,0.02)."""
    x, ch, g = activations(64, 256, seed, outliers=2, outlier_gain=50.0)
    return dict(name="tiny_mxfp4_64x256x256", x=x, wt=weights(256, 256, seed),
                outlier_channels=ch, outlier_gains=g, M=64, K=256, N=256)


def attn_proj(seed=0, M=4608, K=3072, N=3072):
    """Attention projection at 1024^2: X N(0,1) with 1% of channels x U(30,100)."""
    x, ch, g = activations(M, K, seed, outliers=int(round(0.01 * K)))
    return dict(name=f"attn_proj_mxfp4_{M}x{K}x{N}", x=x, wt=weights(N, K, seed),
                outlier_channels=ch, outlier_gains=g, M=M, K=K, N=N)


def mlp_up_svd(seed=0, M=4608, K=3072, N=12288, rank=32):
    """MLP up-projection with the low-rank branch: X Student-t(3); W N(0,0.02)
    split into bf16 L1 [K, r], L2 [r, N] and a residual R^T [N, K] to quantize."""
    x, _, _ = activations(M, K, seed, dist="student_t3")
    wt = weights(N, K, seed)
    l1, l2, rt = lowrank_split(wt, rank, seed)
    return dict(name=f"mlp_up_svd_r{rank}_{M}x{K}x{N}", x=x, wt=wt, l1=l1, l2=l2, rt=rt,
                M=M, K=K, N=N, rank=rank)


def attn_proj_svdquant(seed=0, M=4608, K=3072, N=3072, rank=32, calib=512):
    """The attention projection's inputs (X N(0,1) with 1% of channels x U(30,100),
    W N(0,0.02)) prepared the SVDQuant way: smoothing, an activation-weighted rank-r
    split and a 4-bit residual, from `calib` calibration rows drawn with X (same
    outlier channels, disjoint rows)."""
    xa, ch, g = activations(M + calib, K, seed, outliers=int(round(0.01 * K)))
    x, x_cal = xa[:M], xa[M:]
    wt = weights(N, K, seed)
    d = svdquant_split(x_cal, wt, rank)
    return dict(name=f"attn_proj_svdquant_r{rank}_{M}x{K}x{N}", x=x, x_cal=x_cal, wt=wt,
                outlier_channels=ch, outlier_gains=g, M=M, K=K, N=N, rank=rank, **d)


def qkv_nvfp4(step, seed=0, M=16896, K=3072, N=9216):
    """Fused QKV at 2048^2, NVFP4-style: X N(0,1) whose 1% outlier channel set
    (gains U(30,100)) is redrawn for each denoising step (seed + step)."""
    x, ch, g = activations(M, K, seed + step, outliers=int(round(0.01 * K)))
    return dict(name=f"qkv_nvfp4_{M}x{K}x{N}_step{step}", x=x, outlier_channels=ch,
                outlier_gains=g, M=M, K=K, N=N)


def qkv_nvfp4_weight(seed=0, K=3072, N=9216):
    return weights(N, K, seed)


def w4a16_layer(M, seed=0, K=3072, N=12288):
    """Weight-only comparison: X N(0,1), W N(0,0.02) to be packed as int4 g64."""
    x, _, _ = activations(M, K, seed)
    return dict(name=f"w4a16_int4g64_{M}x{K}x{N}", x=x, wt=weights(N, K, seed), M=M, K=K, N=N)
