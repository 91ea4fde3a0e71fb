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
# default margin of mx8_real: a code whose input lies this close (relative) to a
# rounding boundary, or a block whose amax lies this close to a power of two,
# counts as undecided
AMBIGUOUS_REL = 1e-5
FP32_TINY = 2.0 ** -126


def mx8_real(x, rel=AMBIGUOUS_REL, force_chunk=None):
    """MXFP8 of real (fp64) values along the last axis, whose length is a multiple
    of 32, by the same rule as ``quant.mxfp8_quantize`` (E = floor(log2 amax) - 8,
    E4M3 round to nearest even of x * 2**-E, saturating at 448).

    rel: the relative error (scalar, or per element) with which another evaluation
    of the same values may see them.  force_chunk (optional, bool per block of 32):
    blocks whose exponent is to be counted as undecided whatever their amax.

    Returns (dequantized fp64 values, step, undecided):
    * step: the spacing of the E4M3 grid at each element times 2**E (the most a
      one-code change of that element moves its value), doubled where the block
      exponent is undecided (the grid then halves or doubles),
    * undecided: elements whose code such an evaluation might decide differently
      (the value within rel of a rounding boundary, or the block's amax within rel
      of a power of two, or a forced block).
    """
    x = np.asarray(x, dtype=np.float64)
    check_finite(x, "attention operand")
    shape = x.shape
    bshape = shape[:-1] + (shape[-1] // MX_BLOCK, MX_BLOCK)
    blocks = x.reshape(bshape)
    relb = np.broadcast_to(np.asarray(rel, dtype=np.float64), shape).reshape(bshape)
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
    near_mid = np.abs(frac - 0.5) * spacing <= relb * np.maximum(u, spacing)
    undecided = near_mid & (u < E4M3_MAX)
    # amax within rel of a power of two, from either side.  amax = 1 exactly is
    # decided here: it is the chunk holding the row's running maximum, whose
    # probability exp(0) is exactly 1 in any evaluation (a near tie for that
    # maximum is the caller's to force)
    relc = relb.max(axis=-1)
    lo = np.ldexp(1.0, lg)
    dist = np.minimum(amax - lo, 2.0 * lo - amax)
    amb_scale = pos & (amax != 1.0) & (dist <= relc * np.where(pos, amax, 1.0))
    if force_chunk is not None:
        amb_scale = amb_scale | np.asarray(force_chunk, dtype=bool)
    undecided = undecided | amb_scale[..., None]
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
                  key_block=KEY_BLOCK, quantize=True, query_rows=None, score_err=0.0, sum_err=0.0):
    """FP8 attention (steps 1-6 above) of Q, K, V given as bf16 bits
    [batch * seq, heads * head_dim] (token-major, head h in columns
    h * head_dim .. +head_dim, as the QKV projection writes them).

    Returns dict(out_bits uint16 [batch * seq, heads * head_dim] (bf16 RNE of o),
    o fp64 (before rounding), l fp64 [batch, heads, seq], and two per-element
    bounds for comparing another evaluation of the same steps in finite precision:
    * ambiguity: the most that codes or exponents of P it may decide the other way
      can move o (values within its error of a decision boundary),
    * error_bound: the most its rounding can move o otherwise: the errors of the
      probabilities (through l and the rescaling factors) and of the P V sums.
    score_err is that evaluation's error bound on a score, relative to
    sum_d |q^_d k^_d| (its matrix unit's accumulation error), and sum_err the same
    for the sums of P^ V^ (relative to sum |p^ v^|); its fp32 exp2 and logit
    arithmetic add a relative 2**-20 (1 + |c s| + |c m|) to each probability.
    Neither bound changes o.

    quantize=False skips every quantization (steps 1, 2 and 5 become identities):
    the recurrence then computes exact softmax attention, which the tests use to pin
    steps 3, 4 and 6.

    query_rows (optional, indices into the seq queries of every batch item): only
    those queries are computed (every query is independent of the others); the
    returned arrays then hold batch * len(query_rows) rows, batch-major.
    """
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
    rows = np.arange(seq) if query_rows is None else np.asarray(query_rows, dtype=np.int64)
    q = q[:, rows]
    nq = len(rows)
    o = np.zeros((batch, nq, heads, head_dim))
    amb = np.zeros_like(o)
    lsum = np.zeros((batch, heads, nq))
    err = np.zeros_like(o)
    nblocks = -(-seq // key_block)
    for b in range(batch):
        for h in range(heads):
            qh, kh = q[b, :, h, :], k[b, :, h, :]
            s_all = qh @ kh.T                                          # [queries, seq]
            ds = score_err * (np.abs(qh) @ np.abs(kh).T)               # score error bounds
            dsmax = ds.max(axis=1)
            v_h = vt[b, h * head_dim:(h + 1) * head_dim, :seq].T       # [seq keys, head_dim]
            m = np.full(nq, -np.inf)
            l = np.zeros(nq)
            acc = np.zeros((nq, head_dim))
            acc_abs = np.zeros((nq, head_dim))                         # sum of |p^ v^|, rescaled
            bnd = np.zeros((nq, head_dim))
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
                    pp = np.zeros((nq, width_pad))
                    pp[:, :j1 - j0] = p
                    # relative error of each probability as the other evaluation sees
                    # it: its score's and the maximum's errors, and fp32's exp2
                    rel = np.full((nq, width_pad), 1.0)
                    rel[:, :j1 - j0] = (c * (ds[:, j0:j1] + dsmax[:, None])
                                        + 2.0 ** -20 * (1 + np.abs(c * s) + np.abs(c * m_new)[:, None]))
                    # the chunk holding the row maximum (amax exactly 1) loses it when
                    # a rival score (in another chunk, or an earlier block's maximum)
                    # lies within the two scores' errors: its exponent is undecided
                    # then.  Rounding the logits to fp32 keeps their order, so exact
                    # scores (score_err = 0) never trade places.
                    cmax = pp.reshape(nq, -1, MX_BLOCK).max(axis=2)
                    top = cmax == 1.0
                    rival = np.maximum(np.where(top, 0.0, cmax).max(axis=1), alpha)
                    tie = (score_err > 0) & (rival >= np.exp(-2.0 * c * dsmax))
                    ph, step, und = mx8_real(pp, rel, force_chunk=top & tie[:, None])
                    ph, step, und = ph[:, :j1 - j0], step[:, :j1 - j0], und[:, :j1 - j0]
                    flips = np.where(und, step, 0.0) @ np.abs(v_h[j0:j1])
                else:
                    ph = p
                    flips = 0.0
                acc = alpha[:, None] * acc + ph @ v_h[j0:j1]
                acc_abs = alpha[:, None] * acc_abs + np.abs(ph) @ np.abs(v_h[j0:j1])
                bnd = alpha[:, None] * bnd + flips
                m = m_new
            o[b, :, h, :] = acc / l[:, None]
            amb[b, :, h, :] = bnd / l[:, None]
            # e bounds the relative error of every probability, of every rescaling
            # factor and of l: O' = sum A' p^ v / sum A' p' moves by at most
            # (2 e + sum_err) sum |p^ v^| / l + 4 e |O|
            e = c * 2.0 * dsmax + 2.0 ** -20 * (1 + 2.0 * np.abs(c * s_all).max(axis=1))
            err[b, :, h, :] = ((2.0 * e + sum_err)[:, None] * acc_abs / l[:, None]
                               + 4.0 * e[:, None] * np.abs(o[b, :, h, :]))
            lsum[b, h] = l
    o = o.reshape(batch * nq, width)
    return dict(out_bits=f32_to_bf16_rne(o), o=o, ambiguity=amb.reshape(batch * nq, width),
                error_bound=err.reshape(batch * nq, width), l=lsum)
