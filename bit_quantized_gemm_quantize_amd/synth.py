"""Seeded synthetic inputs for the 4-bit DiT linear layer.

This module only *draws* inputs and rounds them to bf16: no quantization, no GEMM
and no weight preparation (the low-rank splits live in ``weight_prep``).  Both the
HIP path and the CPU oracle consume exactly the bytes it returns, so they always
see the same bf16 tensors.

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
