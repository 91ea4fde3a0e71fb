"""GPU parity of the quantizers and packers against the CPU oracle: codes and scales
bit-exact, the fused low-rank intermediate t = X L1 within the fp32 accumulation
bound.  Every call goes through the C ABI."""

import numpy as np
import pytest

from bit_quantized_gemm_quantize_amd import synth
from oracle import formats as F
from oracle import quant as Q
from oracle import layer as L

from _gpu import bf16_dev, bits16, device, pack, quantize, say, u8

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ MXFP4 activations
MX_SHAPES = [(64, 256), (100, 352), (33, 32), (1, 64), (257, 1024), (31, 96)]


@pytest.mark.parametrize("M,K", MX_SHAPES)
def test_quantize_mx_bit_exact(M, K):
    dev = device()
    x = synth.activations(M, K, seed=M + K, outliers=max(1, K // 100))[0]
    say(f"quantize_act mxfp4 M={M} K={K}")
    g = quantize("mxfp4", x, dev)
    codes, scales = Q.mx_quantize(x)
    assert np.array_equal(u8(g["codes"]), codes)
    assert np.array_equal(u8(g["scales"]), scales)


def test_quantize_mx_every_bf16_pattern():
    # every finite bf16 pattern once, shuffled into 32-element blocks, plus blocks of
    # only subnormals and blocks of only tiny normals (exponent clamp at -127)
    dev = device()
    rng = np.random.default_rng(0)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF]
    rng.shuffle(pats)
    sub = np.concatenate([np.arange(1, 128), np.arange(0x8001, 0x8080)]).astype(np.uint16)
    tiny = np.concatenate([np.arange(0x0080, 0x0200), np.arange(0x8080, 0x8200)]).astype(np.uint16)
    rows = [pats[:65280].reshape(-1, 32), rng.choice(sub, (64, 32)), rng.choice(tiny, (64, 32))]
    x = np.concatenate(rows).reshape(-1, 256)      # 8 blocks per row
    say(f"quantize_act mxfp4 all bf16 patterns rows={x.shape[0]}")
    g = quantize("mxfp4", x, dev)
    codes, scales = Q.mx_quantize(x)
    assert np.array_equal(u8(g["scales"]), scales)
    assert np.array_equal(u8(g["codes"]), codes)


def test_quantize_mx_golden_blocks_and_padded_rows():
    dev = device()
    x = synth.activations(40, 512, seed=3, outliers=4)[0]
    say("quantize_act mxfp4 ldx > K")
    g = quantize("mxfp4", x, dev, ldx_pad=64)
    codes, scales = Q.mx_quantize(x)
    assert np.array_equal(u8(g["codes"]), codes) and np.array_equal(u8(g["scales"]), scales)


def test_quantize_mx_full_attention_projection():
    dev = device()
    d = synth.attn_proj(seed=0)
    say("quantize_act mxfp4 4608x3072 (attention projection activations)")
    g = quantize("mxfp4", d["x"], dev)
    codes, scales = Q.mx_quantize(d["x"])
    assert np.array_equal(u8(g["scales"]), scales)
    assert np.array_equal(u8(g["codes"]), codes)


# ------------------------------------------------------------------ low-rank t = X L1
@pytest.mark.parametrize("M,K,r,fmt", [(64, 256, 32, "mxfp4"), (100, 352, 16, "mxfp4"),
                                       (70, 512, 32, "nvfp4"), (4608, 3072, 32, "mxfp4"),
                                       (8192, 3104, 32, "mxfp4"), (4700, 1056, 16, "nvfp4")])
def test_quantize_fused_lowrank_t(M, K, r, fmt):
    dev = device()
    x = synth.activations(M, K, seed=5, dist="student_t3")[0]
    rng = np.random.default_rng(M)
    l1 = synth.to_bf16_bits(rng.standard_normal((K, r)) * 0.05)
    say(f"quantize_act {fmt} + t=X L1 M={M} K={K} r={r}")
    g = quantize(fmt, x, dev, l1_bits=l1)
    t = g["t"].cpu().numpy().astype(np.float64)
    X, L1 = F.bf16_to_f64(x), F.bf16_to_f64(l1)
    t_ref = L.lowrank_down(X, L1)
    # fp32 accumulation of K products: |error| <= K * 2**-24 * sum_k |x l1| (to first order)
    bound = np.abs(X) @ np.abs(L1)
    assert np.all(np.abs(t - t_ref) <= K * 2.0 ** -24 * bound * 1.01 + 1e-30)
    # the codes, scales and tensor scale are unaffected by the fused branch
    ref = Q.mx_quantize(x) if fmt == "mxfp4" else Q.nv_quantize(x)
    assert np.array_equal(u8(g["codes"]), ref[0])
    assert np.array_equal(u8(g["scales"]), ref[1])
    if fmt == "nvfp4":
        assert float(g["ts"].item()) == float(ref[2])


# ------------------------------------------------------------------ NVFP4 activations
@pytest.mark.parametrize("M,K", [(64, 256), (100, 352), (33, 32), (257, 1024)])
def test_quantize_nv_bit_exact(M, K):
    dev = device()
    x = synth.activations(M, K, seed=M * 7 + K, outliers=max(1, K // 100))[0]
    say(f"quantize_act nvfp4 M={M} K={K}")
    g = quantize("nvfp4", x, dev)
    codes, sb, st = Q.nv_quantize(x)
    assert float(g["ts"].item()) == float(st)
    assert np.array_equal(u8(g["scales"]), sb)
    assert np.array_equal(u8(g["codes"]), codes)


def test_quantize_nv_wide_dynamic_range():
    # blocks spanning many binades relative to the tensor maximum: E4M3 subnormal
    # block scales, block scales that round to 0, ties in the fp32 quotient
    dev = device()
    rng = np.random.default_rng(1)
    mags = 2.0 ** rng.uniform(-30, 8, size=(96, 512))
    x = synth.to_bf16_bits(mags * rng.choice([-1, 1], size=mags.shape))
    x[5, :16] = 0                                       # an all-zero block
    say("quantize_act nvfp4 wide dynamic range")
    g = quantize("nvfp4", x, dev)
    codes, sb, st = Q.nv_quantize(x)
    assert float(g["ts"].item()) == float(st)
    assert np.array_equal(u8(g["scales"]), sb)
    assert np.array_equal(u8(g["codes"]), codes)


@pytest.mark.parametrize("step", range(8))
def test_quantize_nv_full_qkv_sampled_rows(step):
    """The fused-QKV activations at 2048^2 for each of the 8 denoising steps, each
    with its own outlier channel set: the tensor scale and the sampled rows' codes
    and block scales bit-exact."""
    dev = device()
    d = synth.qkv_nvfp4(step=step)
    x = d["x"]
    say(f"quantize_act nvfp4 16896x3072 (QKV activations, denoising step {step})")
    g = quantize("nvfp4", x, dev)
    amax_t = np.abs(F.bf16_to_f32(x)).max()
    rows = np.unique(np.concatenate([[0, x.shape[0] - 1],
                                     np.random.default_rng(2 + step).choice(x.shape[0], 126)]))
    codes, sb, st = Q.nv_quantize(x[rows], amax_t=amax_t)
    assert float(g["ts"].item()) == float(st)
    assert np.array_equal(u8(g["scales"])[rows], sb)
    assert np.array_equal(u8(g["codes"])[rows], codes)


def test_quantize_empty_is_a_no_op():
    import torch
    from bit_quantized_gemm_quantize_amd import binding as B
    dev = device()
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    codes = torch.zeros((1, 32), dtype=torch.uint8, device=dev)
    scales = torch.zeros((1, 4), dtype=torch.uint8, device=dev)
    say("quantize_act M=0")
    st = B.load().quantize_act(0, B._ptr(codes), 0, 64, 64, B._ptr(codes), B._ptr(scales), None,
                               None, 0, None, B._stream(None))
    assert st == B.Q4_OK
    torch.cuda.synchronize()
    assert int(codes.sum()) == 0


# ------------------------------------------------------------------ weight packing
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4_g64"])
@pytest.mark.parametrize("layout", ["nk", "kn", "nk_pad"])
def test_pack_weights_bit_exact(fmt, layout):
    dev = device()
    N, K = 136, 512
    wt = synth.weights(N, K, seed=11)
    say(f"pack_weights {fmt} layout={layout} N={N} K={K}")
    g = pack(fmt, wt, dev, layout)
    if fmt == "mxfp4":
        codes, scales = Q.mx_quantize(wt)
        assert np.array_equal(u8(g["codes"]), codes) and np.array_equal(u8(g["scales"]), scales)
    elif fmt == "nvfp4":
        codes, sb, st = Q.nv_quantize(wt)
        assert float(g["extra"].item()) == float(st)
        assert np.array_equal(u8(g["codes"]), codes) and np.array_equal(u8(g["scales"]), sb)
    else:
        codes, sc, zc = Q.int4_g64_quantize(wt)
        assert np.array_equal(u8(g["codes"]), codes)
        assert np.array_equal(bits16(g["scales"]), sc)
        assert np.array_equal(bits16(g["extra"]), zc)


def test_pack_int4_edge_groups():
    # all-zero group (s = 1), all-positive group (z = 0), all-negative group (z = 15),
    # a group holding a single value
    dev = device()
    wt = synth.weights(8, 256, seed=12)
    wt[0, :64] = 0
    wt[1, :64] = synth.to_bf16_bits(np.abs(F.bf16_to_f32(wt[1, :64])))
    wt[2, :64] = synth.to_bf16_bits(-np.abs(F.bf16_to_f32(wt[2, :64])))
    wt[3, 64:128] = synth.to_bf16_bits(np.full(64, 0.3))
    say("pack_weights int4_g64 edge groups")
    g = pack("int4_g64", wt, dev)
    codes, sc, zc = Q.int4_g64_quantize(wt)
    assert np.array_equal(u8(g["codes"]), codes)
    assert np.array_equal(bits16(g["scales"]), sc) and np.array_equal(bits16(g["extra"]), zc)


def test_pack_full_size_residual_weight():
    dev = device()
    wt = synth.weights(12288, 3072, seed=0)
    say("pack_weights mxfp4 12288x3072 (MLP up-projection weight)")
    g = pack("mxfp4", wt, dev)
    codes, scales = Q.mx_quantize(wt)
    assert np.array_equal(u8(g["scales"]), scales)
    assert np.array_equal(u8(g["codes"]), codes)
