"""ctypes binding of libq4lin (the C ABI in include/q4lin.h).

Argument marshalling only: every function passes device pointers, sizes and the
current HIP stream of torch to the C entry point of the same name and raises
``Q4Error`` on a non-OK status.  All arithmetic runs in the library's kernels.
torch is used for device memory and streams.  There is no fallback: if the
library is not built, the first call raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; Q4LIN_LIBRARY names another build of the same library
LIB_PATH = os.environ.get("Q4LIN_LIBRARY") or os.path.join(_PKG, "libq4lin.so")

Q4_OK, Q4_ERR_NULL, Q4_ERR_SHAPE, Q4_ERR_ALIGN, Q4_ERR_FORMAT, Q4_ERR_LAUNCH = range(6)
MXFP4, NVFP4, INT4_G64, INT4_SYM, MXFP8 = 0, 1, 2, 3, 4
OUT_BF16, OUT_F32 = 0, 1
FORMATS = {"mxfp4": MXFP4, "nvfp4": NVFP4, "int4_g64": INT4_G64, "int4_sym": INT4_SYM, "mxfp8": MXFP8}

# name -> (restype, argtypes), in the order of include/q4lin.h
_c = ctypes
_P = _c.c_void_p
_I64 = _c.c_int64
_I32 = _c.c_int32
SIGNATURES = {
    "quantize_act": (_c.c_int, [_c.c_int, _P, _I64, _I64, _I64, _P, _P, _P, _P, _I32, _P, _P]),
    "quantize_act_noalloc": (_c.c_int, [_c.c_int, _P, _I64, _I64, _I64, _P, _P, _P, _P, _I32, _P, _P]),
    "quantize_act_smooth": (_c.c_int, [_c.c_int, _P, _I64, _I64, _I64, _P, _P, _P, _P, _I32, _P, _P]),
    "pack_weights": (_c.c_int, [_c.c_int, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "gemm_w4a4": (_c.c_int, [_c.c_int, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64,
                             _c.c_int, _P]),
    "gemm_w4a4_lowrank": (_c.c_int, [_c.c_int, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P,
                                     _I32, _P, _P, _I64, _c.c_int, _P]),
    "gemm_w4a4_lowrank_mxout": (_c.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I32, _P, _P,
                                           _I64, _P, _I64, _P, _I64, _P]),
    "gemm_w4a4_lowrank_swiglu": (_c.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I32, _P, _P,
                                            _I64, _P]),
    "gemm_w4a4_lowrank_qkv_rope": (_c.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I32, _P, _P,
                                              _I32, _P, _P, _P, _I64, _P]),
    "gemm_w4a16": (_c.c_int, [_P, _I64, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _I64, _c.c_int,
                              _P]),
    "attention_fp8_quantize": (_c.c_int, [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P,
                                          _P, _P, _P, _P]),
    "attention_fp8": (_c.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _c.c_float, _P, _I64, _P]),
    "q4_status_string": (_c.c_char_p, [_c.c_int]),
}

_lib = None


class Q4Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {status_string(status)} ({status})")


def load(path=LIB_PATH):
    """Load libq4lin.so (after torch, so the library binds to the HIP runtime
    torch already loaded).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m bit_quantized_gemm_quantize_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status):
    return load().q4_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != Q4_OK:
        raise Q4Error(fn, status)


def _rowmajor(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


# ----------------------------------------------------------------------------- host checks
# The C ABI takes bare pointers and cannot see a buffer's size, type or device, so
# every wrapper checks its tensors here first: a short or mistyped buffer would
# otherwise be read or written past its end by the kernels.

def _device(t, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.device


def _span_ok(t, nbytes):
    avail = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    return nbytes <= avail


def _packed(t, name, dtype, rows, cols, dev):
    """A buffer the library reads or writes as a dense [rows, cols] array."""
    if _device(t, name) != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < rows * cols:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {rows} x {cols}")


def _strided(t, name, dtypes, rows, cols, dev):
    """A [rows, cols] matrix with contiguous rows and the row stride t.stride(0)."""
    if _device(t, name) != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1 or t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} must be a 2-D tensor of at least {rows} x {cols} with contiguous rows")
    if rows and cols and not _span_ok(t, ((rows - 1) * t.stride(0) + cols) * t.element_size()):
        raise ValueError(f"{name} is too small for {rows} x {cols}")


def _scales_spec(fmt, K):
    """(dtype, columns) of a format's scale buffer per row, and the code bytes per row."""
    if fmt == MXFP4:
        return torch.uint8, K // 32, K // 2
    if fmt == NVFP4:
        return torch.uint8, K // 16, K // 2
    if fmt == INT4_SYM:
        return torch.float32, 1, K // 2
    if fmt == MXFP8:
        return torch.uint8, K // 32, K
    if fmt == INT4_G64:
        return torch.bfloat16, K // 64, K // 2
    raise ValueError(f"unknown format {fmt}")


def _operand(fmt, codes, scales, tscale, rows, K, dev, name):
    sdt, scols, cbytes = _scales_spec(fmt, K)
    _packed(codes, f"{name}_codes", torch.uint8, rows, cbytes, dev)
    _packed(scales, f"{name}_scales", sdt, rows, scols, dev)
    if fmt == NVFP4:
        _packed(tscale, f"{name}_tscale", torch.float32, 1, 1, dev)


def _out_dtype(out):
    return torch.float32 if int(out) == OUT_F32 else torch.bfloat16


# ----------------------------------------------------------------------------- entry points
def quantize_act(fmt, x, codes, scales, tensor_scale=None, l1t=None, t=None, stream=None):
    """x bf16 [M, K] -> codes uint8 [M, K/2], scales uint8 [M, K/32|K/16],
    tensor_scale float32 [1] (NVFP4), t float32 [M, r] = X L1 (l1t bf16 [r, K])."""
    _rowmajor(x, "x")
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    f = _fmt(fmt)
    dev = _device(x, "x")
    _strided(x, "x", (torch.bfloat16,), M, K, dev)
    _operand(f, codes, scales, tensor_scale, M, K, dev, "x")
    if r:
        _packed(l1t, "l1t", torch.bfloat16, r, K, dev)
        _packed(t, "t", torch.float32, M, r, dev)
    st = load().quantize_act(_fmt(fmt), _ptr(x), M, K, x.stride(0), _ptr(codes), _ptr(scales),
                             _ptr(tensor_scale), _ptr(l1t), r, _ptr(t), _stream(stream))
    _check("quantize_act", st)


def quantize_act_noalloc(fmt, x, codes, scales, tensor_scale=None, l1t=None, t=None, stream=None):
    """quantize_act through the entry point that allocates nothing (its NVFP4 scratch
    is a static device array shared by every call on the GPU)."""
    _rowmajor(x, "x")
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    f = _fmt(fmt)
    dev = _device(x, "x")
    _strided(x, "x", (torch.bfloat16,), M, K, dev)
    _operand(f, codes, scales, tensor_scale, M, K, dev, "x")
    if r:
        _packed(l1t, "l1t", torch.bfloat16, r, K, dev)
        _packed(t, "t", torch.float32, M, r, dev)
    st = load().quantize_act_noalloc(f, _ptr(x), M, K, x.stride(0), _ptr(codes), _ptr(scales),
                                     _ptr(tensor_scale), _ptr(l1t), r, _ptr(t), _stream(stream))
    _check("quantize_act_noalloc", st)


def quantize_act_smooth(fmt, x, inv_s, codes, scales, l1t=None, t=None, stream=None):
    """quantize_act of x * inv_s (per channel, fp32 [K]); t = X L1 of the unsmoothed x."""
    _rowmajor(x, "x")
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    dev = _device(x, "x")
    _strided(x, "x", (torch.bfloat16,), M, K, dev)
    _operand(_fmt(fmt), codes, scales, None, M, K, dev, "x")
    _packed(inv_s, "inv_s", torch.float32, 1, K, dev)
    if r:
        _packed(l1t, "l1t", torch.bfloat16, r, K, dev)
        _packed(t, "t", torch.float32, M, r, dev)
    st = load().quantize_act_smooth(_fmt(fmt), _ptr(x), M, K, x.stride(0), _ptr(inv_s), _ptr(codes),
                                    _ptr(scales), _ptr(l1t), r, _ptr(t), _stream(stream))
    _check("quantize_act_smooth", st)


def pack_weights(fmt, w, K, N, stride_k, stride_n, codes, scales, zeros=None, tensor_scale=None,
                 stream=None):
    """w bf16, logical [K, N] with element strides (stride_k, stride_n)."""
    f = _fmt(fmt)
    dev = _device(w, "w")
    if w.dtype != torch.bfloat16:
        raise ValueError("w must be bfloat16")
    if K > 0 and N > 0 and not _span_ok(w, ((K - 1) * stride_k + (N - 1) * stride_n + 1) * 2):
        raise ValueError(f"w is too small for [{K}, {N}] with strides ({stride_k}, {stride_n})")
    _operand(f, codes, scales, tensor_scale, N, K, dev, "w")
    if f == INT4_G64:
        _packed(zeros, "zeros", torch.bfloat16, N, K // 64, dev)
    st = load().pack_weights(_fmt(fmt), _ptr(w), K, N, stride_k, stride_n, _ptr(codes),
                             _ptr(scales), _ptr(zeros), _ptr(tensor_scale), _stream(stream))
    _check("pack_weights", st)


def _gemm_checks(f, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, y, bias, ydt,
                 ycols=None):
    dev = _device(y, "y")
    _operand(f, a_codes, a_scales, a_tscale, M, K, dev, "a")
    _operand(f, b_codes, b_scales, b_tscale, N, K, dev, "b")
    _strided(y, "y", ydt, M, N if ycols is None else ycols, dev)
    if bias is not None:
        _packed(bias, "bias", torch.bfloat16, 1, N, dev)
    return dev


def gemm_w4a4(fmt, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, y,
              bias=None, out=OUT_BF16, stream=None):
    _gemm_checks(_fmt(fmt), a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, y, bias,
                 (_out_dtype(out),))
    st = load().gemm_w4a4(_fmt(fmt), _ptr(a_codes), _ptr(a_scales), _ptr(a_tscale), _ptr(b_codes),
                          _ptr(b_scales), _ptr(b_tscale), M, N, K, _ptr(bias), _ptr(y), y.stride(0),
                          int(out), _stream(stream))
    _check("gemm_w4a4", st)


def gemm_w4a4_lowrank(fmt, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, t,
                      l2t, y, bias=None, out=OUT_BF16, stream=None):
    r = 0 if l2t is None else l2t.shape[1]
    dev = _gemm_checks(_fmt(fmt), a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, y,
                       bias, (_out_dtype(out),))
    if r:
        _packed(t, "t", torch.float32, M, r, dev)
        _packed(l2t, "l2t", torch.bfloat16, N, r, dev)
    st = load().gemm_w4a4_lowrank(_fmt(fmt), _ptr(a_codes), _ptr(a_scales), _ptr(a_tscale),
                                  _ptr(b_codes), _ptr(b_scales), _ptr(b_tscale), M, N, K, _ptr(t),
                                  _ptr(l2t), r, _ptr(bias), _ptr(y), y.stride(0), int(out),
                                  _stream(stream))
    _check("gemm_w4a4_lowrank", st)


def gemm_w4a4_lowrank_mxout(a_codes, a_scales, b_codes, b_scales, M, N, K, y_codes, y_scales, t=None,
                            l2t=None, y=None, bias=None, stream=None):
    """MXFP4 GEMM (+ t L2) whose output is written as MXFP4 codes [M, N/2] and scales
    [M, N/32] (and as bf16 into y when given)."""
    r = 0 if l2t is None else l2t.shape[1]
    dev = _device(y_codes, "y_codes")
    _operand(MXFP4, a_codes, a_scales, None, M, K, dev, "a")
    _operand(MXFP4, b_codes, b_scales, None, N, K, dev, "b")
    _strided(y_codes, "y_codes", (torch.uint8,), M, N // 2, dev)
    _strided(y_scales, "y_scales", (torch.uint8,), M, N // 32, dev)
    if y is not None:
        _strided(y, "y", (torch.bfloat16,), M, N, dev)
    if bias is not None:
        _packed(bias, "bias", torch.bfloat16, 1, N, dev)
    if r:
        _packed(t, "t", torch.float32, M, r, dev)
        _packed(l2t, "l2t", torch.bfloat16, N, r, dev)
    st = load().gemm_w4a4_lowrank_mxout(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M,
                                        N, K, _ptr(t), _ptr(l2t), r, _ptr(bias), _ptr(y),
                                        0 if y is None else y.stride(0), _ptr(y_codes),
                                        y_codes.stride(0), _ptr(y_scales), y_scales.stride(0),
                                        _stream(stream))
    _check("gemm_w4a4_lowrank_mxout", st)


def gemm_w4a4_lowrank_swiglu(a_codes, a_scales, b_codes, b_scales, M, N, K, y, t=None, l2t=None,
                             bias=None, stream=None):
    """MXFP4 GEMM (+ t L2) over N weight rows grouped as 32 gate + 32 up rows per 32
    output columns; y bf16 [M, N/2] receives silu(gate) * up."""
    r = 0 if l2t is None else l2t.shape[1]
    dev = _gemm_checks(MXFP4, a_codes, a_scales, None, b_codes, b_scales, None, M, N, K, y, bias,
                       (torch.bfloat16,), ycols=N // 2)
    if r:
        _packed(t, "t", torch.float32, M, r, dev)
        _packed(l2t, "l2t", torch.bfloat16, N, r, dev)
    st = load().gemm_w4a4_lowrank_swiglu(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M,
                                         N, K, _ptr(t), _ptr(l2t), r, _ptr(bias), _ptr(y), y.stride(0),
                                         _stream(stream))
    _check("gemm_w4a4_lowrank_swiglu", st)


def gemm_w4a4_lowrank_qkv_rope(a_codes, a_scales, b_codes, b_scales, M, N, K, yq, yk, yv, t=None,
                               l2t=None, bias=None, cs=None, head_dim=0, stream=None):
    """MXFP4 GEMM (+ t L2) of a fused QKV projection (N = 3 D weight rows): Q, K, V
    stored to yq, yk, yv (bf16 [M, D], one row stride), Q and K rotated by cs
    (float [M, head_dim/2, 2] of cos, sin) when given."""
    r = 0 if l2t is None else l2t.shape[1]
    dev = _gemm_checks(MXFP4, a_codes, a_scales, None, b_codes, b_scales, None, M, N, K, yq, bias,
                       (torch.bfloat16,), ycols=N // 3)
    for name, yo in (("yk", yk), ("yv", yv)):
        _strided(yo, name, (torch.bfloat16,), M, N // 3, dev)
    if yk.stride(0) != yq.stride(0) or yv.stride(0) != yq.stride(0):
        raise ValueError("yq, yk, yv share one row stride")
    if cs is not None:
        _packed(cs, "cs", torch.float32, M, max(head_dim, 0), dev)
    if r:
        _packed(t, "t", torch.float32, M, r, dev)
        _packed(l2t, "l2t", torch.bfloat16, N, r, dev)
    st = load().gemm_w4a4_lowrank_qkv_rope(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M,
                                           N, K, _ptr(t), _ptr(l2t), r, _ptr(bias), _ptr(cs), head_dim,
                                           _ptr(yq), _ptr(yk), _ptr(yv), yq.stride(0), _stream(stream))
    _check("gemm_w4a4_lowrank_qkv_rope", st)


def gemm_w4a16(x, w_codes, w_scales, w_zeros, N, y, bias=None, group=64, out=OUT_BF16, stream=None):
    _rowmajor(x, "x")
    M, K = x.shape
    dev = _device(x, "x")
    _strided(x, "x", (torch.bfloat16,), M, K, dev)
    _operand(INT4_G64, w_codes, w_scales, None, N, K, dev, "w")
    _packed(w_zeros, "w_zeros", torch.bfloat16, N, K // 64, dev)
    _strided(y, "y", (_out_dtype(out),), M, N, dev)
    if bias is not None:
        _packed(bias, "bias", torch.bfloat16, 1, N, dev)
    st = load().gemm_w4a16(_ptr(x), x.stride(0), _ptr(w_codes), _ptr(w_scales), _ptr(w_zeros), M, N,
                           K, group, _ptr(bias), _ptr(y), y.stride(0), int(out), _stream(stream))
    _check("gemm_w4a16", st)


HEAD_DIM = 128


def _attn_bufs_check(bufs, batch, seq, heads, dev):
    tokens, width = batch * seq, heads * HEAD_DIM
    seq64 = -(-seq // 64) * 64
    _packed(bufs["qc"], "qc", torch.uint8, tokens, width, dev)
    _packed(bufs["kc"], "kc", torch.uint8, tokens, width, dev)
    _packed(bufs["qs"], "qs", torch.uint8, tokens, heads * 4, dev)
    _packed(bufs["ks"], "ks", torch.uint8, tokens, heads * 4, dev)
    _packed(bufs["vc"], "vc", torch.uint8, batch * width, seq64, dev)
    _packed(bufs["vs"], "vs", torch.uint8, batch * heads * (seq64 // 64), 256, dev)


def attention_fp8_quantize(q, k, v, batch, seq, heads, bufs, stream=None):
    """q, k, v bf16 [batch*seq, heads*128] (contiguous rows, any row stride) -> the
    MXFP8 operands of attention_fp8 in bufs (from attn_buffers)."""
    dev = _device(q, "q")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _strided(t, name, (torch.bfloat16,), batch * seq, heads * HEAD_DIM, dev)
    _attn_bufs_check(bufs, batch, seq, heads, dev)
    st = load().attention_fp8_quantize(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), batch,
                                       seq, heads, HEAD_DIM, _ptr(bufs["qc"]), _ptr(bufs["qs"]), _ptr(bufs["kc"]),
                                       _ptr(bufs["ks"]), _ptr(bufs["vc"]), _ptr(bufs["vs"]), _stream(stream))
    _check("attention_fp8_quantize", st)


def attention_fp8(bufs, batch, seq, heads, out, softmax_scale=None, stream=None):
    """FP8 attention of the operands in bufs -> out bf16 [batch*seq, heads*128]."""
    dev = _device(out, "out")
    _strided(out, "out", (torch.bfloat16,), batch * seq, heads * HEAD_DIM, dev)
    _attn_bufs_check(bufs, batch, seq, heads, dev)
    c = HEAD_DIM ** -0.5 if softmax_scale is None else float(softmax_scale)
    st = load().attention_fp8(_ptr(bufs["qc"]), _ptr(bufs["qs"]), _ptr(bufs["kc"]), _ptr(bufs["ks"]),
                              _ptr(bufs["vc"]), _ptr(bufs["vs"]), batch, seq, heads, HEAD_DIM, c, _ptr(out),
                              out.stride(0), _stream(stream))
    _check("attention_fp8", st)


# ----------------------------------------------------------------------------- buffers
def attn_buffers(batch, seq, heads, device="cuda"):
    """Output buffers of attention_fp8_quantize (the MXFP8 Q, K, V), as a dict."""
    tokens, width = batch * seq, heads * HEAD_DIM
    seq64 = -(-seq // 64) * 64
    u8 = dict(dtype=torch.uint8, device=device)
    return dict(qc=torch.empty((tokens, width), **u8), qs=torch.empty((tokens, heads * 4), **u8),
                kc=torch.empty((tokens, width), **u8), ks=torch.empty((tokens, heads * 4), **u8),
                vc=torch.empty((batch * width, seq64), **u8),
                vs=torch.empty((batch * heads * (seq64 // 64), 256), **u8))


def empty_quant(fmt, rows, K, device="cuda"):
    """Output buffers for quantize_act / pack_weights: (codes, scales, tensor_scale|zeros)."""
    fmt = _fmt(fmt)
    if fmt == MXFP8:
        return (torch.empty((rows, K), dtype=torch.uint8, device=device),
                torch.empty((rows, K // 32), dtype=torch.uint8, device=device), None)
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=device)
    if fmt == MXFP4:
        return codes, torch.empty((rows, K // 32), dtype=torch.uint8, device=device), None
    if fmt == NVFP4:
        return (codes, torch.empty((rows, K // 16), dtype=torch.uint8, device=device),
                torch.empty(1, dtype=torch.float32, device=device))
    if fmt == INT4_SYM:
        return codes, torch.empty(rows, dtype=torch.float32, device=device), None
    return (codes, torch.empty((rows, K // 64), dtype=torch.bfloat16, device=device),
            torch.empty((rows, K // 64), dtype=torch.bfloat16, device=device))
