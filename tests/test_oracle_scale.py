"""Pins of the oracle's group scale against exact rational arithmetic.

For every non-negative finite bf16 value a used as a group's absmax, and for
both format maxima (448 for e4m3, 127 for int8):
  * fp32 scale == fl(max(a, eps) / qmax), the IEEE quotient numpy computes;
  * UE8M0 byte == the smallest k with 2^(k-127) >= that quotient, decided with
    Python's exact Fractions (the power-of-two ceiling of the quotient, which is
    what the exponent-plus-carry bit trick of the sglang #30924 reference
    computes, and what the vllm #41326 page states is bit-identical to
    exp2(ceil(log2(.)))).
The group is [a, 0, ..., 0] so its absmax is a; the first code must then be the
e4m3/int8 code of a times the multiplier (2^(127-k) for UE8M0).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

EPS = np.float32(1e-10)


def all_bf16_magnitudes():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)         # +0 .. largest finite
    return bits


def groups_with_amax(bits, G=128):
    x = np.zeros((bits.size, G), dtype=np.uint16)
    x[:, 0] = bits
    return x


def pow2_ceil_byte(r: np.float32) -> int:
    fr = Fraction(float(r))
    if fr == 0:
        return 0
    k = fr.numerator.bit_length() - fr.denominator.bit_length()   # 2^k near fr
    while Fraction(2) ** k < fr:
        k += 1
    while Fraction(2) ** (k - 1) >= fr:
        k -= 1
    return k + 127


@pytest.mark.parametrize("out_dtype,qmax", [("e4m3", 448.0), ("int8", 127.0)])
def test_scales_over_all_bf16_amax(out_dtype, qmax):
    bits = all_bf16_magnitudes()
    a = (bits.astype(np.uint32) << 16).view(np.float32)
    x = groups_with_amax(bits)
    M = bits.size
    r_expect = np.maximum(a, EPS) / np.float32(qmax)        # IEEE fp32 division
    assert r_expect.dtype == np.float32

    _, s32 = oracle.ptgq(x, "bf16", M, 128, 128, False, out_dtype, "f32", "row", eps=1e-10)
    assert np.array_equal(s32.view(np.float32), r_expect)

    q, s8 = oracle.ptgq(x, "bf16", M, 128, 128, False, out_dtype, "ue8m0", "row", eps=1e-10)
    expect_bytes = np.array([pow2_ceil_byte(r) for r in r_expect], dtype=np.uint8)
    assert np.array_equal(s8, expect_bytes)

    # first code = narrowing of a * 2^(127 - byte), which is exact in fp32
    mult = np.ldexp(np.float64(1.0), 127 - expect_bytes.astype(np.int64))
    v = (a.astype(np.float64) * mult).astype(np.float32)
    assert np.array_equal(v.astype(np.float64), a.astype(np.float64) * mult)
    narrowed = oracle.e4m3(v) if out_dtype == "e4m3" else oracle.int8(v).view(np.uint8)
    assert np.array_equal(q[:, 0], narrowed)
    assert np.all(q[:, 1:] == 0)


def test_ue8m0_scale_covers_amax():
    """2^(byte-127) * qmax >= max(a, eps) > 2^(byte-128) * qmax up to fp32 rounding."""
    bits = all_bf16_magnitudes()[::7]
    a = (bits.astype(np.uint32) << 16).view(np.float32)
    _, s8 = oracle.ptgq(groups_with_amax(bits), "bf16", bits.size, 128, 128, False,
                        "e4m3", "ue8m0", "row")
    scale = np.ldexp(1.0, s8.astype(np.int64) - 127)
    aa = np.maximum(a, EPS).astype(np.float64)
    assert np.all(scale * 448.0 >= aa * (1 - 2.0 ** -23))
    assert np.all(scale * 448.0 / 2 < aa * (1 + 2.0 ** -23))


def test_fp32_codes_use_reciprocal_multiply_and_stay_in_range():
    """fp32-scale codes never exceed the format maximum (the scale keeps
    |v| <= qmax*(1 + 2^-22)), and the group maximum maps to +-qmax."""
    rng = np.random.default_rng(11)
    vals = rng.standard_normal((512, 128)).astype(np.float32) * rng.uniform(
        1e-3, 1e3, (512, 1)).astype(np.float32)
    bits = (vals.view(np.uint32) + 0x8000) >> 16            # RN-ish to bf16, fine for a test
    x = bits.astype(np.uint16)
    q, s = oracle.ptgq(x, "bf16", 512, 128, 128, False, "e4m3", "f32", "row")
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    amax_col = np.argmax(np.abs(xf), axis=1)
    top = q[np.arange(512), amax_col]
    assert np.all((top & 0x7F) == 0x7E)
    qi, _ = oracle.ptgq(x, "bf16", 512, 128, 128, False, "int8", "f32", "row")
    topi = qi.view(np.int8)[np.arange(512), amax_col]
    assert np.all(np.abs(topi.astype(np.int32)) == 127)


@pytest.mark.parametrize("eps", [0.0, 1e-10])
@pytest.mark.parametrize("out_dtype,qmax", [("e4m3", 448.0), ("int8", 127.0)])
def test_vector_scale_export_equals_the_pins(out_dtype, qmax, eps):
    """oracle.scale (the vector form the device probes are compared with):
    every bf16 absmax plus fp32 values around the subnormal quotients, against
    numpy's IEEE quotients and the exact power-of-two ceiling."""
    bits = all_bf16_magnitudes()
    a16 = (bits.astype(np.uint32) << 16).view(np.float32)
    tiny = np.arange(0, 1 << 24, 4099, dtype=np.uint32).view(np.float32)   # up to 2^-126 * 2
    a = np.concatenate([a16, tiny])
    e32 = np.float32(eps)
    r, e, inv = oracle.scale(a, eps, out_dtype, "f32")
    r_expect = (np.maximum(a, e32) / np.float32(qmax)).astype(np.float32)
    assert np.array_equal(r.view(np.uint32), r_expect.view(np.uint32))
    with np.errstate(divide="ignore", over="ignore"):
        inv_expect = np.where(r_expect == 0, np.float32(0), np.float32(1) / r_expect)
    assert np.array_equal(inv.view(np.uint32), inv_expect.astype(np.float32).view(np.uint32))
    assert np.all(e == 0)
    r8, e8, inv8 = oracle.scale(a, eps, out_dtype, "ue8m0")
    assert np.array_equal(r8.view(np.uint32), r_expect.view(np.uint32))
    # a subnormal quotient has exponent field 0 and a non-zero fraction: the
    # exponent-plus-carry rule gives byte 1 (2^-126), the power-of-two ceiling
    # clamped to the normal range
    want = np.array([max(pow2_ceil_byte(x), 1) if x > 0 else 0 for x in r_expect],
                    dtype=np.uint8)
    assert np.array_equal(e8, want)
    assert np.array_equal(inv8.astype(np.float64), np.ldexp(1.0, 127 - want.astype(np.int64)))
