"""FP8 attention of the DiT block in fp64 (test infrastructure only).

Source: the NVIDIA Technical Blog summary (disconfirmai, "NVIDIA Technical Blog
Details FLUX 3 Image Klein Blackwell Inference Optimization Methods"), its second
optimization layer: attention quantized to FP8 ("VC-Attention FP8", with a repair
budget rho = 0.005).  The page names the method and its budget, nothing more, and
says attention is about 60% of the DiT's kernel time at 2048x2048 (same page,
third paragraph).  The steps below are the plainest FP8 reading of "quantized
attention" on block-scaled matrix units, with the MX element and scale rules the
rest of the oracle uses (OCP MX v1.0, E4M3 with emax 8):

1. Q and K: MXFP8 along head_dim, per token and head (``quant.mxfp8_quantize`` on
   the [tokens, heads * head_dim] rows; head_dim is a multiple of 32, so no block
   straddles two heads).
2. V: MXFP8 along the key axis, per (batch, head, channel): blocks of 32
   consecutive keys; a last block of fewer than 32 keys is padded with zeros.
3. Scores s = q^ . k^ (exact products, fp64 sums), logits c * s with c the softmax
   scale (1 / sqrt(head_dim) by default).  The maximum of each block is taken over
   the logits, so that the probability of a row's largest logit is exp(0) = 1
   exactly.
4. Softmax online over blocks of KEY_BLOCK keys, in key order (the flash-attention
   recurrence): m' = max(m, max of the block's s), alpha = exp(c (m - m')),
   p = exp(c (s - m')), l' = alpha l + sum p.  Keys past the sequence end are
   masked (p = 0).
5. P is quantized to MXFP8 along the keys, per query and 32-key chunk of the block,
   before the product with V: O' = alpha O + P^ V^.  Since P is quantized against
   the running maximum of its block, the block size is part of the result.
6. Output O / l rounded to bf16.

Readings of the pages' open points are listed in the design notes (attention
section): the quantization granularities, the key block, the order of the steps,
and the repair budget, which this function leaves at rho = 0.

Every step that decides a code (an E4M3 rounding, an E8M0 exponent) is taken in
fp64 here; the kernel takes it in fp32 after its own exp2, so a value within a
few fp32 ulps of a rounding boundary may round the other way there.  ``attention_fp8``
therefore also returns, per output element, the largest change such flips could
make (``ambiguity``), for the parity test to allow.
"""

import numpy as np

from .formats import E4M3_MAX, bf16_to_f64, check_finite, e4m3_decode, e4m3_encode, f32_to_bf16_rne, floor_log2
from .quant import MX_BLOCK, mxfp8_dequantize, mxfp8_quantize

KEY_BLOCK = 64
E4M3_EMAX = 8
# a code whose fp64 input lies this close (relative) to a rounding boundary, or a
# block whose amax lies this close to a power of two, counts as undecided
AMBIGUOUS_REL = 1e-5
FP32_TINY = 2.0 ** -126


def mx8_real(x):
    """MXFP8 of real (fp64) values along the last axis, whose length is a multiple
    of 32, by the same rule as ``quant.mxfp8_quantize`` (E = floor(log2 amax) - 8,
    E4M3 round to nearest even of x * 2**-E, saturating at 448).

    Returns (dequantized fp64 values, step, undecided):
    * step: the spacing of the E4M3 grid at each element times 2**E (the most a
      one-code change of that element moves its value),
    * undecided: elements whose code an fp32 evaluation of the same rule might
      decide differently (the value within AMBIGUOUS_REL of a rounding boundary,
      or the block's amax within AMBIGUOUS_REL of a power of two).
    """
    x = np.asarray(x, dtype=np.float64)
    check_finite(x, "attention operand")
    shape = x.shape
    blocks = x.reshape(shape[:-1] + (shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    pos = amax > 0
    lg = floor_log2(np.where(pos, amax, 1.0))
    E = np.clip(np.where(pos, lg - E4M3_EMAX, -127), -127, 127)
    scale = np.ldexp(1.0, E)[..., None]
    u = np.minimum(np.abs(blocks) / scale, E4M3_MAX)           # exact: a power of two
    codes = e4m3_encode(u)
    mag = e4m3_decode(codes)
    vals = np.where(np.signbit(blocks), -mag, mag) * scale
    # grid spacing at u: 2**(max(floor(log2 u), -6) - 3)
    eu = np.maximum(floor_log2(np.where(u > 0, u, 1.0)), -6)
    eu = np.where(u > 0, eu, -6)
    spacing = np.ldexp(1.0, eu - 3)
    # distance to the nearest rounding boundary (midpoints between grid values)
    # (a power of two is a grid value, not a boundary; u >= 448 saturates)
    frac = u / spacing - np.floor(u / spacing)
    near_mid = np.abs(frac - 0.5) * spacing <= AMBIGUOUS_REL * np.maximum(u, spacing)
    undecided = near_mid & (u < E4M3_MAX)
    # amax within AMBIGUOUS_REL of a power of two, from either side.  amax = 1 exactly
    # is decided: it is the chunk holding the row's running maximum, whose
    # probability exp(0) both sides compute as exactly 1
    lo = np.ldexp(1.0, lg)
    dist = np.minimum(amax - lo, 2.0 * lo - amax)
    amb_scale = pos & (amax != 1.0) & (dist <= AMBIGUOUS_REL * np.where(pos, amax, 1.0))
    undecided = undecided | amb_scale[..., None]
    # a changed block exponent halves or doubles the grid: allow twice the spacing
    step = spacing * scale * np.where(amb_scale[..., None], 2.0, 1.0)
    return vals.reshape(shape), step.reshape(shape), undecided.reshape(shape)


def quantize_qk(bits):
    """Q or K bf16 bits [tokens, heads * head_dim] -> MXFP8 (codes, scales) along
    head_dim (step 1)."""
    return mxfp8_quantize(bits)


def quantize_v(v_bits, batch, seq, heads, head_dim):
    """V bf16 bits [batch * seq, heads * head_dim] -> MXFP8 along the keys (step 2).

    Returns (codes uint8 [batch, heads * head_dim, seq32], scales uint8
    [batch, heads * head_dim, seq32 / 32]) with seq32 = seq rounded up to 32: row
    h * head_dim + d of batch b holds channel d of head h over the keys, padded with
    zero codes (and a zero block's scale 0) past seq.
    """
    v_bits = np.asarray(v_bits, dtype=np.uint16).reshape(batch, seq, heads * head_dim)
    seq32 = -(-seq // MX_BLOCK) * MX_BLOCK
    codes = np.zeros((batch, heads * head_dim, seq32), dtype=np.uint8)
    scales = np.zeros((batch, heads * head_dim, seq32 // MX_BLOCK), dtype=np.uint8)
    for b in range(batch):
        vt = np.zeros((heads * head_dim, seq32), dtype=np.uint16)
        vt[:, :seq] = v_bits[b].T
        c, s = mxfp8_quantize(vt)
        codes[b], scales[b] = c, s
    return codes, scales


def attention_fp8(q_bits, k_bits, v_bits, batch, seq, heads, head_dim=128, scale=None,
                  key_block=KEY_BLOCK, quantize=True):
    """FP8 attention (steps 1-6 above) of Q, K, V given as bf16 bits
    [batch * seq, heads * head_dim] (token-major, head h in columns
    h * head_dim .. +head_dim, as the QKV projection writes them).

    Returns dict(out_bits uint16 [batch * seq, heads * head_dim] (bf16 RNE of o),
    o fp64 (before rounding), ambiguity fp64 (per element: the most that codes of P
    left undecided in fp64 can move o), l fp64 [batch, heads, seq]).

    quantize=False skips every quantization (steps 1, 2 and 5 become identities):
    the recurrence then computes exact softmax attention, which the tests use to pin
    steps 3, 4 and 6.
    """
    n = batch * seq
    width = heads * head_dim
    c = 1.0 / np.sqrt(head_dim) if scale is None else float(scale)
    if quantize:
        qc, qs = quantize_qk(q_bits)
        kc, ks = quantize_qk(k_bits)
        q = mxfp8_dequantize(qc, qs)
        k = mxfp8_dequantize(kc, ks)
        vc, vs = quantize_v(v_bits, batch, seq, heads, head_dim)
        vt = np.stack([mxfp8_dequantize(vc[b], vs[b]) for b in range(batch)])   # [B, HD, seq32]
    else:
        q = bf16_to_f64(np.asarray(q_bits, dtype=np.uint16))
        k = bf16_to_f64(np.asarray(k_bits, dtype=np.uint16))
        v = bf16_to_f64(np.asarray(v_bits, dtype=np.uint16)).reshape(batch, seq, width)
        vt = np.transpose(v, (0, 2, 1))
    q = q.reshape(batch, seq, heads, head_dim)
    k = k.reshape(batch, seq, heads, head_dim)
    o = np.zeros((batch, seq, heads, head_dim))
    amb = np.zeros_like(o)
    lsum = np.zeros((batch, heads, seq))
    nblocks = -(-seq // key_block)
    for b in range(batch):
        for h in range(heads):
            s_all = q[b, :, h, :] @ k[b, :, h, :].T                    # [seq, seq]
            v_h = vt[b, h * head_dim:(h + 1) * head_dim, :seq].T       # [seq keys, head_dim]
            m = np.full(seq, -np.inf)
            l = np.zeros(seq)
            acc = np.zeros((seq, head_dim))
            bnd = np.zeros((seq, head_dim))
            for blk in range(nblocks):
                j0 = blk * key_block
                j1 = min(j0 + key_block, seq)
                s = s_all[:, j0:j1]
                m_new = np.maximum(m, s.max(axis=1))
                alpha = np.where(np.isfinite(m), np.exp(c * (m - m_new)), 0.0)
                p = np.exp(c * (s - m_new[:, None]))
                if quantize:
                    # below fp32's normal range a probability counts as zero: it moves
                    # o by less than 2**-126 |v|
                    p = np.where(p < FP32_TINY, 0.0, p)
                l = alpha * l + p.sum(axis=1)
                if quantize:
                    width_pad = -(-(j1 - j0) // MX_BLOCK) * MX_BLOCK
                    pp = np.zeros((seq, width_pad))
                    pp[:, :j1 - j0] = p
                    ph, step, und = mx8_real(pp)
                    ph, step, und = ph[:, :j1 - j0], step[:, :j1 - j0], und[:, :j1 - j0]
                    flips = np.where(und, step, 0.0) @ np.abs(v_h[j0:j1])
                else:
                    ph = p
                    flips = 0.0
                acc = alpha[:, None] * acc + ph @ v_h[j0:j1]
                bnd = alpha[:, None] * bnd + flips
                m = m_new
            o[b, :, h, :] = acc / l[:, None]
            amb[b, :, h, :] = bnd / l[:, None]
            lsum[b, h] = l
    o = o.reshape(n, width)
    return dict(out_bits=f32_to_bf16_rne(o), o=o, ambiguity=amb.reshape(n, width), l=lsum)
