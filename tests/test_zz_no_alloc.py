"""quantize_act_noalloc (the entry point that allocates nothing, its NVFP4 scratch
in a static device array) against quantize_act, through the C ABI: codes, scales
and the tensor scale must be identical, on two calls in a row, the second with a
smaller input (the array keeps the first call's partial maxima)."""

import numpy as np
import pytest
import torch

from bit_quantized_gemm_quantize_amd import binding as B
from bit_quantized_gemm_quantize_amd import synth

from _gpu import bf16_dev, device, say, u8

pytestmark = pytest.mark.gpu


def _both(fmt, x_bits, dev, l1_bits=None):
    M, K = x_bits.shape
    x = bf16_dev(x_bits, dev)
    outs = []
    for fn in (B.quantize_act, B.quantize_act_noalloc):
        codes, scales, ts = B.empty_quant(fmt, M, K, dev)
        codes.fill_(0xAB)
        scales.fill_(0xCD)
        l1t = t = None
        if l1_bits is not None:
            l1t = bf16_dev(np.ascontiguousarray(l1_bits.T), dev)
            t = torch.full((M, l1_bits.shape[1]), float("nan"), dtype=torch.float32, device=dev)
        fn(fmt, x, codes, scales, tensor_scale=ts, l1t=l1t, t=t)
        torch.cuda.synchronize()
        outs.append((u8(codes), u8(scales), None if ts is None else float(ts.item()),
                     None if t is None else t.cpu().numpy()))
    return outs


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_noalloc_matches_quantize_act_twice(fmt):
    dev = device()
    rng = np.random.default_rng(4)
    # a large input, then a smaller one whose tensor amax is much smaller, so stale
    # partial maxima left in the array by the first call would change the result
    # NVFP4: odd numbers of 16-element blocks; MXFP4: K a multiple of 32
    kb, ks = (1040, 272) if fmt == "nvfp4" else (1056, 288)
    big = synth.activations(3000, kb, seed=1, outliers=12)[0]
    small = synth.to_bf16_bits(rng.standard_normal((130, ks)) * 0.01)
    l1 = synth.to_bf16_bits(rng.standard_normal((kb, 32)) * 0.05) if fmt == "mxfp4" else None
    for i, (x, l1b) in enumerate([(big, l1), (small, None)]):
        say(f"quantize_act_noalloc {fmt} call {i + 1}: {x.shape}")
        a, b = _both(fmt, x, dev, l1b)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert a[2] == b[2]
        if a[3] is not None:
            assert np.array_equal(a[3], b[3])
