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
LIB_PATH = os.path.join(_PKG, "libq4lin.so")

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


# ----------------------------------------------------------------------------- entry points
def quantize_act(fmt, x, codes, scales, tensor_scale=None, l1t=None, t=None, stream=None):
    """x bf16 [M, K] -> codes uint8 [M, K/2], scales uint8 [M, K/32|K/16],
    tensor_scale float32 [1] (NVFP4), t float32 [M, r] = X L1 (l1t bf16 [r, K])."""
    _rowmajor(x, "x")
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    st = load().quantize_act(_fmt(fmt), _ptr(x), M, K, x.stride(0), _ptr(codes), _ptr(scales),
                             _ptr(tensor_scale), _ptr(l1t), r, _ptr(t), _stream(stream))
    _check("quantize_act", st)


def quantize_act_smooth(fmt, x, inv_s, codes, scales, l1t=None, t=None, stream=None):
    """quantize_act of x * inv_s (per channel, fp32 [K]); t = X L1 of the unsmoothed x."""
    _rowmajor(x, "x")
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    st = load().quantize_act_smooth(_fmt(fmt), _ptr(x), M, K, x.stride(0), _ptr(inv_s), _ptr(codes),
                                    _ptr(scales), _ptr(l1t), r, _ptr(t), _stream(stream))
    _check("quantize_act_smooth", st)


def pack_weights(fmt, w, K, N, stride_k, stride_n, codes, scales, zeros=None, tensor_scale=None,
                 stream=None):
    """w bf16, logical [K, N] with element strides (stride_k, stride_n)."""
    st = load().pack_weights(_fmt(fmt), _ptr(w), K, N, stride_k, stride_n, _ptr(codes),
                             _ptr(scales), _ptr(zeros), _ptr(tensor_scale), _stream(stream))
    _check("pack_weights", st)


def gemm_w4a4(fmt, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, y,
              bias=None, out=OUT_BF16, stream=None):
    st = load().gemm_w4a4(_fmt(fmt), _ptr(a_codes), _ptr(a_scales), _ptr(a_tscale), _ptr(b_codes),
                          _ptr(b_scales), _ptr(b_tscale), M, N, K, _ptr(bias), _ptr(y), y.stride(0),
                          int(out), _stream(stream))
    _check("gemm_w4a4", st)


def gemm_w4a4_lowrank(fmt, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, t,
                      l2t, y, bias=None, out=OUT_BF16, stream=None):
    r = 0 if l2t is None else l2t.shape[1]
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
    assert yk.stride(0) == yq.stride(0) == yv.stride(0), "yq, yk, yv share one row stride"
    st = load().gemm_w4a4_lowrank_qkv_rope(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M,
                                           N, K, _ptr(t), _ptr(l2t), r, _ptr(bias), _ptr(cs), head_dim,
                                           _ptr(yq), _ptr(yk), _ptr(yv), yq.stride(0), _stream(stream))
    _check("gemm_w4a4_lowrank_qkv_rope", st)


def gemm_w4a16(x, w_codes, w_scales, w_zeros, N, y, bias=None, group=64, out=OUT_BF16, stream=None):
    _rowmajor(x, "x")
    M, K = x.shape
    st = load().gemm_w4a16(_ptr(x), x.stride(0), _ptr(w_codes), _ptr(w_scales), _ptr(w_zeros), M, N,
                           K, group, _ptr(bias), _ptr(y), y.stride(0), int(out), _stream(stream))
    _check("gemm_w4a16", st)


# ----------------------------------------------------------------------------- buffers
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
