"""The §8(b) K contract on the GPU: MXFP4 at any K that is a multiple of 32 and
NVFP4 at any K that is a multiple of 16, through the same calls (quantize_act,
pack_weights, gemm_w4a4, gemm_w4a4_lowrank).  K not a multiple of 128 runs the
any-K GEMM; the quantizer and packer take NVFP4 rows of an odd number of
16-element blocks.  Codes and scales bit-exact against the oracle, GEMM outputs
within the per-element bound, element by element."""

import numpy as np
import pytest

from bit_quantized_gemm_quantize_amd import synth
from oracle import formats as F
from oracle import quant as Q

from _gpu import device, pack, quantize, say, u8
from test_gpu_gemm import _check, ref_w4a4, run_w4a4

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,K", [("mxfp4", 32), ("mxfp4", 96), ("mxfp4", 160), ("mxfp4", 3104),
                                   ("nvfp4", 16), ("nvfp4", 48), ("nvfp4", 3088)])
def test_gemm_any_k_parity(fmt, K):
    dev = device()
    M, N = 300, 200
    x = synth.activations(M, K, seed=K + 1, outliers=max(1, K // 100))[0]
    wt = synth.weights(N, K, seed=K + 2)
    bias = synth.bias(N, seed=3)
    for f32, use_bias in [(True, False), (False, True)]:
        say(f"gemm_w4a4 {fmt} any K: M={M} N={N} K={K} f32={f32} bias={use_bias}")
        b = bias if use_bias else None
        y = run_w4a4(fmt, x, wt, dev, bias=b, f32=f32)
        y_ref, bound = ref_w4a4(fmt, x, wt, bias=b)
        _check(y, y_ref, bound, not f32, f"{fmt} any-K {M}x{N}x{K}")


@pytest.mark.parametrize("fmt,K,r", [("mxfp4", 96, 32), ("mxfp4", 3104, 16), ("nvfp4", 160, 32)])
def test_gemm_any_k_lowrank(fmt, K, r):
    dev = device()
    M, N = 260, 136
    x = synth.activations(M, K, seed=K + 5, dist="student_t3")[0]
    wt = synth.weights(N, K, seed=K + 6)
    rng = np.random.default_rng(K)
    l1 = synth.to_bf16_bits(rng.standard_normal((K, r)) * 0.05)
    l2 = synth.to_bf16_bits(rng.standard_normal((r, N)) * 0.05)
    bias = synth.bias(N, seed=7)
    for f32 in (True, False):
        say(f"gemm_w4a4_lowrank {fmt} any K: M={M} N={N} K={K} r={r} f32={f32}")
        y = run_w4a4(fmt, x, wt, dev, bias=bias, f32=f32, l1=l1, l2=l2)
        y_ref, bound = ref_w4a4(fmt, x, wt, bias=bias, l1=l1, l2=l2)
        _check(y, y_ref, bound, not f32, f"{fmt} any-K low-rank {M}x{N}x{K}")


@pytest.mark.parametrize("M,K", [(37, 16), (64, 48), (129, 3088), (5, 1040)])
def test_quantize_nv_odd_block_count(M, K):
    dev = device()
    x = synth.activations(M, K, seed=M + K, outliers=max(1, K // 100))[0]
    say(f"quantize_act nvfp4 M={M} K={K}")
    g = quantize("nvfp4", x, dev)
    codes, sb, st = Q.nv_quantize(x)
    assert float(g["ts"].item()) == float(st)
    assert np.array_equal(u8(g["scales"]), sb)
    assert np.array_equal(u8(g["codes"]), codes)


@pytest.mark.parametrize("layout", ["nk", "kn", "nk_pad"])
def test_pack_nv_odd_block_count(layout):
    dev = device()
    N, K = 72, 80
    wt = synth.weights(N, K, seed=13)
    say(f"pack_weights nvfp4 layout={layout} N={N} K={K}")
    g = pack("nvfp4", wt, dev, layout)
    codes, sb, st = Q.nv_quantize(wt)
    assert float(g["extra"].item()) == float(st)
    assert np.array_equal(u8(g["scales"]), sb)
    assert np.array_equal(u8(g["codes"]), codes)
