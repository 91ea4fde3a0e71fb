"""Pins of the FP8 attention oracle (oracle/attention.py) to things other than
itself: a library softmax, closed forms (uniform and one-hot attention), an
invariance of the blocked recurrence, and the already pinned MXFP8 quantizer."""

import numpy as np
import pytest
from scipy.special import softmax

from bit_quantized_gemm_quantize_amd import synth
from oracle import attention as A
from oracle.formats import bf16_to_f64
from oracle.quant import mxfp8_dequantize, mxfp8_quantize


def _bits(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float32))


def _qkv(seed, batch, seq, heads, d=128, sd=1.0):
    rng = np.random.default_rng(seed)
    shape = (batch * seq, heads * d)
    return tuple(_bits(sd * rng.standard_normal(shape)) for _ in range(3))


@pytest.mark.parametrize("seq", [150, 64, 37, 1])
def test_unquantized_is_softmax_attention(seq):
    """quantize=False: steps 3, 4 and 6 (base-2 logits, the power-of-two shift, the
    normalization) must equal softmax(c Q K^T) V computed with scipy's softmax, per
    batch item and head."""
    batch, heads, d = 2, 2, 128
    q, k, v = _qkv(1, batch, seq, heads, sd=2.0)
    r = A.attention_fp8(q, k, v, batch, seq, heads, d, quantize=False)
    c = 1.0 / np.sqrt(d)
    qf = bf16_to_f64(q).reshape(batch, seq, heads, d)
    kf = bf16_to_f64(k).reshape(batch, seq, heads, d)
    vf = bf16_to_f64(v).reshape(batch, seq, heads, d)
    for b in range(batch):
        for h in range(heads):
            p = softmax(c * qf[b, :, h] @ kf[b, :, h].T, axis=1)
            ref = p @ vf[b, :, h]
            got = r["o"].reshape(batch, seq, heads, d)[b, :, h]
            np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_uniform_scores_average_the_quantized_values():
    """K = 0: every logit is 0, every probability exp(0) = 1 (an exact MXFP8 value),
    so O is the plain mean of the MXFP8-dequantized V over the seq keys (a ragged
    seq: the masked keys of the last block must not count)."""
    batch, seq, heads, d = 1, 100, 2, 128
    q, _, v = _qkv(2, batch, seq, heads)
    k = np.zeros_like(q)
    r = A.attention_fp8(q, k, v, batch, seq, heads, d)
    vt = np.zeros((heads * d, 128), dtype=np.uint16)                           # keys padded to 128
    vt[:, :seq] = v.reshape(seq, heads * d).T
    vhat = mxfp8_dequantize(*mxfp8_quantize(vt))[:, :seq]                      # [heads*d, seq]
    expect = np.broadcast_to(vhat.mean(axis=1), (seq, heads * d))
    np.testing.assert_allclose(r["o"], expect, rtol=1e-12, atol=1e-15)
    assert np.all(r["ambiguity"] == 0)
    assert np.all(r["l"] == seq)            # M = 0, every p^ = 1


def test_one_hot_scores_select_one_value_row():
    """Query i scores a * e_{pi(i)} against keys e_j (one-hot, exact in MXFP8): one
    logit per row is a c = 64 larger than the rest, so every other probability is
    below e^-64 and, l being the sum of the quantized weights, O row i is row pi(i)
    of the dequantized V, whatever the quantization error of that weight."""
    batch, seq, heads, d = 1, 128, 1, 128
    rng = np.random.default_rng(3)
    pi = rng.permutation(seq)
    a = 64.0 * np.sqrt(d)                      # c * a = 64
    qf = np.zeros((seq, d))
    qf[np.arange(seq), pi] = a
    kf = np.eye(seq, d)
    _, _, v = _qkv(4, batch, seq, heads)
    r = A.attention_fp8(_bits(qf), _bits(kf), v, batch, seq, heads, d)
    vc, vs = mxfp8_quantize(np.ascontiguousarray(v.T))
    vhat = mxfp8_dequantize(vc, vs).T                                          # [seq, d]
    np.testing.assert_allclose(r["o"], vhat[pi], rtol=1e-20, atol=1e-24)


@pytest.mark.parametrize("shift", [1, 7, -3])
def test_power_of_two_shift_changes_nothing(shift):
    """MX quantization commutes with powers of two, so shifting M by an integer
    leaves P^ 2**M, l 2**M and O unchanged, bit for bit (the property that makes
    the result independent of how an implementation walks the keys)."""
    batch, seq, heads, d = 2, 100, 2, 128
    q, k, v = _qkv(5, batch, seq, heads, sd=2.0)
    r0 = A.attention_fp8(q, k, v, batch, seq, heads, d)
    r1 = A.attention_fp8(q, k, v, batch, seq, heads, d, shift=shift)
    np.testing.assert_array_equal(r0["o"], r1["o"])
    np.testing.assert_array_equal(r0["l"], r1["l"] * 2.0 ** shift)


def test_real_valued_mx8_matches_the_pinned_mxfp8_quantizer():
    """mx8_real (used for P) and quant.mxfp8_quantize (pinned against the golden
    blocks) give the same values on bf16 inputs, including zero blocks, values
    that saturate, and signed values."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    x[5] = 0.0
    x[6, :32] = 0.0
    bits = _bits(x)
    codes, scales = mxfp8_quantize(bits)
    vals, step, und = A.mx8_real(bf16_to_f64(bits))
    np.testing.assert_array_equal(vals, mxfp8_dequantize(codes, scales))
    assert np.all(step > 0)


def test_fp8_error_against_exact_attention_is_a_few_percent():
    """Gaussian Q, K, V: the FP8 result stays within the error FP8 allows (E4M3
    keeps 3 mantissa bits: a few percent relative RMS), and is not exact."""
    batch, seq, heads, d = 1, 160, 2, 128
    q, k, v = _qkv(8, batch, seq, heads)
    r = A.attention_fp8(q, k, v, batch, seq, heads, d)
    e = A.attention_fp8(q, k, v, batch, seq, heads, d, quantize=False)
    rel = np.sqrt(np.mean((r["o"] - e["o"]) ** 2) / np.mean(e["o"] ** 2))
    assert 1e-3 < rel < 0.1
    # the allowance for codes an fp32 evaluation may decide the other way stays a
    # small fraction of the result
    assert np.all(r["ambiguity"] >= 0)
    assert r["ambiguity"].mean() < 0.01 * np.sqrt(np.mean(r["o"] ** 2))


def test_quantize_v_layout():
    """V is quantized along the keys per (batch, head, channel), padded to 32 keys."""
    batch, seq, heads, d = 2, 40, 2, 128
    _, _, v = _qkv(9, batch, seq, heads)
    codes, scales = A.quantize_v(v, batch, seq, heads, d)
    assert codes.shape == (batch, heads * d, 64) and scales.shape == (batch, heads * d, 2)
    vb = v.reshape(batch, seq, heads * d)
    for b in range(batch):
        c, s = mxfp8_quantize(np.ascontiguousarray(vb[b, :32].T))
        np.testing.assert_array_equal(codes[b, :, :32], c)
        np.testing.assert_array_equal(scales[b, :, :1], s)
    assert np.all(codes[:, :, seq:] == 0)


@pytest.mark.parametrize("seq,second", [(64, 40), (128, 100)])
def test_two_live_keys_worked_by_hand(seq, second):
    """A worked example whose codes are derived by hand.  Query 0 is 14 e_0 (14 =
    1.75 * 2**3 is exact in E4M3, so its MXFP8 form is exact); key 0 is e_0, key
    `second` is 0 and every other key is -64 e_0.  With c = 1/sqrt(128):
      base-2 logits t = log2(e) c s: 14 c log2(e) = 1.78525..., 0, and -114.3;
      M = ceil(1.785) = 2, so p = 2**-0.21475 = 0.861763 for key 0, 2**-2 = 0.25
      for key `second`, below 2**-116 for the rest (zero codes);
      chunk of key 0: amax 0.8618, E = floor(log2 0.8618) - 8 = -9, 0.8618 * 2**9 =
      441.2 lies in [256, 512) where E4M3 steps by 32, so it rounds to 448 (the
      midpoint is 432): p^ = 448 / 512 = 0.875;
      chunk of key `second`: 0.25 = 2**-2, E = -10, code 256 exact: p^ = 0.25;
      l = 0.875 + 0.25 = 1.125.
    V rows 0 and `second` are exact in MXFP8 along the keys (values 1 and 2 in
    channel d, all other keys 0), so O[0, d] = (0.875 * 1 + 0.25 * 2) / 1.125 = 11/9."""
    batch, heads, d = 1, 1, 128
    qf = np.zeros((seq, d))
    qf[0, 0] = 14.0
    kf = np.zeros((seq, d))
    kf[:, 0] = -64.0
    kf[0, 0] = 1.0
    kf[second, 0] = 0.0
    vf = np.zeros((seq, d))
    vf[0, :] = 1.0
    vf[second, :] = 2.0
    r = A.attention_fp8(_bits(qf), _bits(kf), _bits(vf), batch, seq, heads, d)
    np.testing.assert_allclose(r["o"][0], 11.0 / 9.0, rtol=1e-14)
    np.testing.assert_allclose(r["l"][0, 0, 0], 1.125, rtol=1e-14)
