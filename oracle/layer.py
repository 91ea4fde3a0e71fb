"""The quantized linear layer in fp64 (test infrastructure only).

Structure from the SVDQuant Guide (aifetchly):
* "The Three Pillars of SVDQuant", 1. Mathematical Outlier Factorization: the
  forward projection is the 4-bit GEMM of the quantized weight and the quantized
  activation, plus the low-rank branch L1 (L2 X) applied to the *unquantized*
  activation.
* "Step 2: The SVDQuant Dual-Branch Linear Layer": the low-rank branch is evaluated
  right to left (down-projection to rank r first), the two branches are summed,
  the bias is added last.

Orientation used here: X [M, K] (tokens x in-features), the weight as W^T [N, K]
(out-features x in-features), Y [M, N].  The low-rank factors are taken as
L1 [K, r] (the down-projection, applied first) and L2 [r, N]; in the page's
notation (W of shape d_out x d_in acting on column activations) these are the
transposes of its L2 and L1.
"""

import numpy as np

from .formats import bf16_to_f64, bf16_ulp, f32_to_bf16_rne
from .quant import mx_quantize

GEMM_REL_TOL = 1e-3


def gemm_ref(a_deq, b_deq, bias=None, x=None, l1=None, l2=None):
    """Y = A_deq B_deq^T (+ (X L1) L2) (+ bias) in fp64, and the per-element bound.

    a_deq [M, K], b_deq [N, K]: dequantized operands (fp64, exact).
    x [M, K], l1 [K, r], l2 [r, N]: the low-rank branch on the unquantized X.
    bias [N].

    Returns (y, bound) where bound[m, n] is the sum of the magnitudes of every
    product that enters y[m, n]:
        sum_k |a_mk b_nk| + sum_j (sum_k |x_mk l1_kj|) |l2_jn| + |bias_n|.
    """
    a_deq = np.asarray(a_deq, dtype=np.float64)
    b_deq = np.asarray(b_deq, dtype=np.float64)
    y = a_deq @ b_deq.T
    bound = np.abs(a_deq) @ np.abs(b_deq).T
    if l1 is not None:
        x = np.asarray(x, dtype=np.float64)
        l1 = np.asarray(l1, dtype=np.float64)
        l2 = np.asarray(l2, dtype=np.float64)
        t = x @ l1                       # rank-r down-projection first
        y = y + t @ l2
        bound = bound + (np.abs(x) @ np.abs(l1)) @ np.abs(l2)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64)
        y = y + bias[None, :]
        bound = bound + np.abs(bias)[None, :]
    return y, bound


def lowrank_down(x, l1):
    """t = X L1 in fp64: the low-rank branch's rank-r intermediate."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(l1, dtype=np.float64)


def tolerance(y_ref, bound, out_bf16):
    """Allowed |Y_gpu - Y_ref| per element.

    fp32 output: 1e-3 * bound (the bound of ``gemm_ref``).
    bf16 output: the stored value is the bf16 rounding of a result that is itself
    within 1e-3 * bound, so half a bf16 ulp at that result is added; the ulp is
    taken at |y_ref| + 1e-3 * bound, which is at least the result's magnitude.
    """
    tol = GEMM_REL_TOL * np.asarray(bound, dtype=np.float64)
    if out_bf16:
        tol = tol + 0.5 * bf16_ulp(np.abs(y_ref) + tol)
    return tol


def check_close(y_gpu, y_ref, bound, out_bf16):
    """Returns (ok, worst_ratio, index): worst |err| / tol over all elements."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    tol = tolerance(y_ref, bound, out_bf16)
    err = np.abs(y_gpu - y_ref)
    # an exact zero tolerance only admits an exact match
    ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), np.where(err > 0, np.inf, 0.0))
    if not np.all(np.isfinite(y_gpu)):
        return False, np.inf, None
    i = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else None
    worst = float(ratio[i]) if ratio.size else 0.0
    return worst <= 1.0, worst, i


def relative_error(y, y_exact):
    """Quality context (not pass/fail): ||Y - Y_exact||_F / ||Y_exact||_F."""
    y = np.asarray(y, dtype=np.float64)
    y_exact = np.asarray(y_exact, dtype=np.float64)
    return float(np.linalg.norm(y - y_exact) / max(np.linalg.norm(y_exact), 1e-300))


def unquantized_ref(x_bits, wt_bits, bias_bits=None):
    """The unquantized bf16 layer X W^T (+ bias) in fp64: the quality context."""
    y = bf16_to_f64(x_bits) @ bf16_to_f64(wt_bits).T
    if bias_bits is not None:
        y = y + bf16_to_f64(bias_bits)[None, :]
    return y


def mx_output(y):
    """The layer output handed to the next layer in MXFP4: Y rounded to bf16 (nearest
    even), then quantized along N in 32-column blocks as mx_quantize quantizes any
    bf16 activation.  Defined here for results that are exact fp32 values (the exact
    special cases of the tests), so the bf16 rounding is a single rounding, as in a
    kernel that rounds its fp32 result once.  Returns (codes [M, N/2], scales
    [M, N/32])."""
    y = np.asarray(y, dtype=np.float64)
    if not np.array_equal(y, y.astype(np.float32).astype(np.float64)):
        raise ValueError("mx_output takes results that are exact fp32 values")
    return mx_quantize(f32_to_bf16_rne(y.astype(np.float32)))


# ----------------------------------------------------------------------------- SwiGLU epilogue
SWIGLU_BLOCK = 32          # output columns per gate/up group of weight rows
SILU_SLOPE_MAX = 1.0999    # max over z of |d/dz (z sigmoid(z))| (1.09984 near z = 2.40)


def silu(z):
    """z * sigmoid(z) = z / (1 + e^-z) in fp64 (SiLU, the Swish of SwiGLU's gate)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ref(y, bound, block=SWIGLU_BLOCK):
    """The SwiGLU epilogue fused into the GEMM (a fusion the NVIDIA Technical Blog
    summary names for its FLUX kernels, first optimization layer), on the GEMM's
    fp64 result y [M, N] and its bound (both from ``gemm_ref``, bias included).

    Weight rows come in groups of 2 * block: the first `block` are the gate and the
    next `block` the up projection of output columns block * j .. + block - 1 of
    group j.  out = silu(gate) * up, [M, N / 2].

    Returns (out, out_bound): out_bound is in the units of ``gemm_ref``'s bound, so
    that ``check_close`` applies: with |gate error| <= 1e-3 bound_g and |up error|
    <= 1e-3 bound_u,
        |d out| <= 1e-3 (SILU_SLOPE_MAX bound_g (|up| + 1e-3 bound_u) + |silu(gate)| bound_u)
    plus the fp32 evaluation of silu(gate) * up (an exp whose argument carries a
    relative error of 2^-23, a division or a reciprocal within an ulp, and a
    product): |out| (|gate| 2^-23 + 2^-20).
    """
    y = np.asarray(y, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    M, N = y.shape
    if N % (2 * block):
        raise ValueError("N must be a multiple of 2 * block")
    groups = N // (2 * block)

    def split(a):
        a = a.reshape(M, groups, 2, block)
        return a[:, :, 0, :].reshape(M, N // 2), a[:, :, 1, :].reshape(M, N // 2)

    gate, up = split(y)
    bg, bu = split(bound)
    sg = silu(gate)
    out = sg * up
    eval_err = np.abs(out) * (np.abs(gate) * 2.0 ** -23 + 2.0 ** -20)
    out_bound = (SILU_SLOPE_MAX * bg * (np.abs(up) + GEMM_REL_TOL * bu) + np.abs(sg) * bu
                 + eval_err / GEMM_REL_TOL)
    return out, out_bound


# ----------------------------------------------------------------------------- QKV split + RoPE
def qkv_rope_ref(y, bound, cs, head_dim):
    """The QKV-split and RoPE epilogue fused into the GEMM (the NVIDIA Technical Blog
    summary names QKV-projection and RoPE epilogues for its FLUX kernels, first
    optimization layer), on the GEMM's fp64 result y [M, 3 D] and its bound (both from
    ``gemm_ref``, bias included).

    Columns [0, D) are Q, [D, 2 D) K and [2 D, 3 D) V.  In Q and K, each head's
    adjacent column pair (2 i, 2 i + 1) (i < head_dim / 2, counted inside the head) is
    rotated by the angle whose cosine and sine are cs[m, i] = (c, s) for row m:
        (a, b) -> (a c - b s, a s + b c);
    V is passed through.  cs: fp32 [M, head_dim / 2, 2], used exactly.

    Returns ((q, k, v), (bq, bk, bv)): the outputs [M, D] each and their bounds in the
    units of ``gemm_ref``'s bound: a rotated element's error is at most
    |c| e_a + |s| e_b (or |s| e_a + |c| e_b) for input errors e_a, e_b, plus the fp32
    evaluation (two products and a sum: 2^-22 (|a c| + |b s|)).
    """
    y = np.asarray(y, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    M, N = y.shape
    if N % 3 or (N // 3) % head_dim or head_dim % 2:
        raise ValueError("N = 3 D with D a multiple of an even head_dim")
    D = N // 3
    cs = np.asarray(cs, dtype=np.float64)
    if cs.shape != (M, head_dim // 2, 2):
        raise ValueError("cs must be [M, head_dim / 2, 2]")
    heads = D // head_dim
    c = np.tile(cs[:, :, 0], (1, heads))          # [M, D / 2]: pair p of the section
    s = np.tile(cs[:, :, 1], (1, heads))

    def rotate(part, bpart):
        a, b = part[:, 0::2], part[:, 1::2]
        ea, eb = bpart[:, 0::2], bpart[:, 1::2]
        out = np.empty_like(part)
        ob = np.empty_like(part)
        out[:, 0::2] = a * c - b * s
        out[:, 1::2] = a * s + b * c
        ev = (np.abs(a * c) + np.abs(b * s)) * 2.0 ** -22 / GEMM_REL_TOL
        ev2 = (np.abs(a * s) + np.abs(b * c)) * 2.0 ** -22 / GEMM_REL_TOL
        ob[:, 0::2] = np.abs(c) * ea + np.abs(s) * eb + ev
        ob[:, 1::2] = np.abs(s) * ea + np.abs(c) * eb + ev2
        return out, ob

    q, bq = rotate(y[:, :D], bound[:, :D])
    k, bk = rotate(y[:, D:2 * D], bound[:, D:2 * D])
    return (q, k, y[:, 2 * D:].copy()), (bq, bk, bound[:, 2 * D:].copy())
