"""The NVFP4 GEMM dequantizes each operand value e2m1 * s_b to fp16 (and multiplies
on the fp16 MFMA).  That is exact only if every such product is an fp16 value: this
checks it for every E2M1 code and every finite E4M3 scale code, against the oracle's
decoders (NVFP4 in the Blackwell summary: E2M1 elements with an E4M3 scale per
16-element block).  No GPU needed."""
import numpy as np

from oracle import formats as F


def test_every_e2m1_times_e4m3_product_is_an_fp16_value():
    e2m1 = F.e2m1_decode(np.arange(16, dtype=np.uint8))               # 16 codes, signed
    e4m3 = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))             # 0x00 .. 0x7E: finite, >= 0
    prod = np.multiply.outer(e2m1, e4m3)                               # exact in fp64
    as16 = prod.astype(np.float16)
    assert np.all(np.isfinite(as16))
    assert np.array_equal(as16.astype(np.float64), prod)               # no rounding
    nz = np.abs(prod[prod != 0])
    # every nonzero product is an fp16 normal (no subnormal or flush path involved)
    assert nz.min() >= 2.0 ** -14 and nz.min() == 2.0 ** -10 and nz.max() == 6 * 448


def test_every_e4m3_scale_is_an_fp16_value():
    e4m3 = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.array_equal(e4m3.astype(np.float16).astype(np.float64), e4m3)
