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
3. Scores s = q^ . k^ (exact products, fp64 sums); logits in base 2,
   t = log2(e) c s, with c the softmax scale (1 / sqrt(head_dim) by default).
4. Softmax numerators shifted by a power of two: per query, M = ceil(max t) and
   p = 2**(t - M), in (0, 1], over the seq keys of the query's batch item.
5. P quantized to MXFP8 along the keys, per query and 32-key chunk (keys 32 j ..
   32 j + 31, the last chunk padded with zeros): P^.
6. O = P^ V^ / l with l = sum P^ (the weights actually used, so O is a weighted
   mean of the V^ rows: one-hot scores return one row exactly), rounded to bf16.

MX quantization commutes with scaling by a power of two (the block exponent moves,
the codes stay), so in steps 4-5 any integer M at or above the maximum gives the
same P^ 2**M: P^ is the MXFP8 form of exp(c s) itself, up to the range limits of
E8M0 and fp32, and does not depend on how an implementation walks the keys (its
key blocks, their order, or the running maximum it keeps).  The integer shift is
this reading's choice: quantizing against the exact maximum (p = exp(c (s - m)))
would make the result depend on where a blocked evaluation sees the maximum.

Readings of the pages' open points are listed in the design notes (attention
section): the quantization granularities, the shift, the order of the steps, and
the repair budget, which this function leaves at rho = 0.

Every step that decides a code (an E4M3 rounding, an E8M0 exponent) is taken in
fp64 here; a device takes it in fp32, from scores its matrix unit accumulates, so
a value near a rounding boundary may round the other way there.
``attention_fp8`` therefore also returns per output element the largest change
such flips could make (``ambiguity``) and a bound on the rest of the device's
rounding (``error_bound``), for the parity test to allow.
"""

import numpy as np

from .formats import E4M3_MAX, bf16_to_f64, check_finite, e4m3_decode, e4m3_encode, f32_to_bf16_rne, floor_log2
from .quant import MX_BLOCK, mxfp8_dequantize, mxfp8_quantize

E4M3_EMAX = 8
LOG2E = 1.4426950408889634
# default margin of mx8_real: a code whose input lies this close (relative) to a
# rounding boundary, or a block whose amax lies this close to a power of two,
# counts as undecided
AMBIGUOUS_REL = 1e-5
FP32_TINY = 2.0 ** -126


def mx8_real(x, rel=AMBIGUOUS_REL):
    """MXFP8 of real (fp64) values along the last axis, whose length is a multiple
    of 32, by the same rule as ``quant.mxfp8_quantize`` (E = floor(log2 amax) - 8,
    E4M3 round to nearest even of x * 2**-E, saturating at 448).

    rel: the relative error (scalar, or per element) with which another evaluation
    of the same values may see them (0: it sees them exactly).

    Returns (dequantized fp64 values, step, undecided):
    * step: the spacing of the E4M3 grid at each element times 2**E (the most a
      one-code change of that element moves its value), doubled where the block
      exponent is undecided (the grid then halves or doubles),
    * undecided: elements whose code such an evaluation might decide differently
      (the value within rel of a rounding boundary, or the block's amax within rel
      of a power of two).
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
    # amax within rel of a power of two, from either side (an amax exactly on one
    # is undecided too unless it carries no error)
    relc = relb.max(axis=-1)
    lo = np.ldexp(1.0, lg)
    dist = np.minimum(amax - lo, 2.0 * lo - amax)
    amb_scale = pos & (dist <= relc * np.where(pos, amax, 1.0)) & (relc > 0)
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
                  quantize=True, query_rows=None, score_err=0.0, sum_err=0.0, shift=0):
    """FP8 attention (steps 1-6 above) of Q, K, V given as bf16 bits
    [batch * seq, heads * head_dim] (token-major, head h in columns
    h * head_dim .. +head_dim, as the QKV projection writes them).

    Returns dict(out_bits uint16 [batch * seq, heads * head_dim] (bf16 RNE of o),
    o fp64 (before rounding), l fp64 [batch, heads, seq] (sum P^, relative to
    2**M), and two per-element bounds for comparing another evaluation of the same
    steps in finite precision:
    * ambiguity: the most that codes or exponents of P it may decide the other way
      can move o (values within its error of a decision boundary),
    * error_bound: the most the rounding of its sums of P^ V^ and of P^ can move o.
    score_err is that evaluation's error bound on a score, relative to
    sum_d |q^_d k^_d| (its matrix unit's accumulation error), and sum_err the same
    for the sums of P^ V^ and of P^ (relative to the sums of magnitudes); its fp32
    exp2 of an fp32 exponent adds a relative 2**-20 (|t - M| + 1) to each
    probability (nothing for an integer exponent).  Neither bound changes o.

    quantize=False skips every quantization (steps 1, 2 and 5 become identities):
    the result is then exact softmax attention, which the tests use to pin steps 3,
    4 and 6.  query_rows (optional, indices into the seq queries of every batch
    item): only those queries are computed (every query is independent of the
    others); the returned arrays then hold batch * len(query_rows) rows,
    batch-major.  shift: an integer added to every M (the result does not change).
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
    seq32 = -(-seq // MX_BLOCK) * MX_BLOCK
    o = np.zeros((batch, nq, heads, head_dim))
    amb = np.zeros_like(o)
    err = np.zeros_like(o)
    lsum = np.zeros((batch, heads, nq))
    for b in range(batch):
        for h in range(heads):
            qh, kh = q[b, :, h, :], k[b, :, h, :]
            v_h = vt[b, h * head_dim:(h + 1) * head_dim, :seq].T       # [seq keys, head_dim]
            t = LOG2E * c * (qh @ kh.T)                                # [queries, seq]
            M = np.ceil(t.max(axis=1)) + shift
            p = np.exp2(t - M[:, None])
            if quantize:
                # below fp32's normal range a probability counts as zero: it moves
                # o by less than 2**-126 |v|
                p = np.where(p < FP32_TINY, 0.0, p)
            if quantize:
                # relative error of each probability as another evaluation sees it:
                # its score's error, and fp32's rounding of the exponent t - M (an
                # integer exponent, as for scores of 0, is exact)
                tm = t - M[:, None]
                rel = (c * score_err * (np.abs(qh) @ np.abs(kh).T)
                       + 2.0 ** -20 * (np.abs(tm) + (tm != np.round(tm))))
                pp = np.zeros((nq, seq32))
                pp[:, :seq] = p
                relp = np.zeros((nq, seq32))
                relp[:, :seq] = rel
                ph, step, und = mx8_real(pp, relp)
                ph, step, und = ph[:, :seq], step[:, :seq], und[:, :seq]
            else:
                ph, step, und = p, np.zeros_like(p), np.zeros(p.shape, dtype=bool)
            l = ph.sum(axis=1)
            acc = ph @ v_h
            o_h = acc / l[:, None]
            o[b, :, h, :] = o_h
            lsum[b, h] = l
            # a code decided the other way moves p^_j by at most step_j, so O = sum p^ v
            # / sum p^ by at most step_j (|v_j| + |O|) / l; the sums of p^ v^ and of p^
            # (the matrix unit's) move O by sum_err (sum |p^ v^| / l + |O|)
            amb[b, :, h, :] = (np.where(und, step, 0.0) @ np.abs(v_h)
                               + np.where(und, step, 0.0).sum(axis=1)[:, None] * np.abs(o_h)) / l[:, None]
            err[b, :, h, :] = sum_err * ((np.abs(ph) @ np.abs(v_h)) / l[:, None] + np.abs(o_h))
    o = o.reshape(batch * nq, width)
    return dict(out_bits=f32_to_bf16_rne(o), o=o, ambiguity=amb.reshape(batch * nq, width),
                error_bound=err.reshape(batch * nq, width), l=lsum)
