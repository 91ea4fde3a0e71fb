"""Helpers for the GPU parity tests: host <-> device copies of the seeded inputs
and one call per hot-path step through the C ABI binding."""

import sys

import numpy as np
import torch

from bit_quantized_gemm_quantize_amd import binding as B


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU (run them with -m gpu on the MI355X box)")
    B.load()
    return torch.device("cuda:0")


def say(msg):
    """Name the case before its GPU work, so a fault can be traced to it."""
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(bits, dev, pad_cols=0):
    """uint16 bf16 patterns [rows, cols] -> torch bfloat16 on the device, rows padded
    to cols + pad_cols elements (the padding is filled with a canary)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if pad_cols:
        padded = np.full((bits.shape[0], bits.shape[1] + pad_cols), 0x7F7F, np.uint16)
        padded[:, :bits.shape[1]] = bits
        t = torch.from_numpy(padded.view(np.int16)).view(torch.bfloat16).to(dev)
        return t[:, :bits.shape[1]]
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)


def u8(t):
    return t.cpu().numpy().view(np.uint8) if t.dtype == torch.uint8 else t.cpu().numpy()


def bits16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def quantize(fmt, x_bits, dev, l1_bits=None, ldx_pad=0):
    """quantize_act on the device; returns dict of host arrays (and device tensors)."""
    M, K = x_bits.shape
    x = bf16_dev(x_bits, dev, ldx_pad)
    codes, scales, ts = B.empty_quant(fmt, M, K, dev)
    l1t = t = None
    if l1_bits is not None:
        r = l1_bits.shape[1]
        l1t = bf16_dev(np.ascontiguousarray(l1_bits.T), dev)
        t = torch.full((M, r), float("nan"), dtype=torch.float32, device=dev)
    B.quantize_act(fmt, x, codes, scales, tensor_scale=ts, l1t=l1t, t=t)
    return dict(x=x, codes=codes, scales=scales, ts=ts, t=t)


def pack(fmt, wt_bits, dev, layout="nk"):
    """pack_weights of W^T [N, K] given either as [N, K] ("nk": stride_k 1) or as the
    row-major [K, N] transpose ("kn": stride_n 1), or with a padded row ("nk_pad")."""
    N, K = wt_bits.shape
    if layout == "nk":
        w = bf16_dev(wt_bits, dev)
        sk, sn = 1, K
    elif layout == "nk_pad":
        w = bf16_dev(wt_bits, dev, pad_cols=24)
        sk, sn = 1, w.stride(0)
    elif layout == "kn":
        w = bf16_dev(np.ascontiguousarray(wt_bits.T), dev)
        sk, sn = N, 1
    else:
        raise ValueError(layout)
    codes, scales, extra = B.empty_quant(fmt, N, K, dev)
    if fmt == "int4_g64":
        B.pack_weights(fmt, w, K, N, sk, sn, codes, scales, zeros=extra)
    else:
        B.pack_weights(fmt, w, K, N, sk, sn, codes, scales, tensor_scale=extra)
    return dict(codes=codes, scales=scales, extra=extra)


CANARY = -31744.0     # exact in bf16 and fp32, far from any output here


def out_buffer(M, N, dev, f32, pad=8):
    """Output with ldy = N rounded up to 8 plus `pad`, the whole buffer filled with a
    canary so writes outside [M, N] can be seen."""
    ldy = ((N + 7) // 8) * 8 + pad
    return torch.full((M, ldy), CANARY, dtype=torch.float32 if f32 else torch.bfloat16, device=dev)


def y_host(y, N):
    """(values fp64 [M, N], padding columns untouched?)"""
    a = y.float().cpu().numpy().astype(np.float64)
    return a[:, :N], bool(np.all(a[:, N:] == CANARY))
