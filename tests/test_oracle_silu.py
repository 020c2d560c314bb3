"""Pin of the oracle's fused SiLU step against a 60-digit decimal evaluation.

The reading: silu(g) * u = (g / (1 + e^-g)) * u with e^-g correctly rounded to
binary32 and every other operation one IEEE fp32 rounding.  exp_cr is checked
for every finite bf16 and fp16 gate against Python's Decimal exp at 60 digits,
rounded to the nearest binary32 exactly (Fractions); the composition is
checked against numpy's IEEE float32 add / divide / multiply.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle

getcontext().prec = 60
F32_MAX = Fraction(float(np.finfo(np.float32).max))
OVERFLOW = F32_MAX + Fraction(2) ** 103      # half an ulp above the largest float


def nearest_f32(exact: Fraction) -> np.float32:
    """Round a positive rational to the nearest binary32 (ties impossible here)."""
    if exact >= OVERFLOW:
        return np.float32(np.inf)
    c = np.float32(float(exact))
    best, bestd = None, None
    cands = {np.float32(v) for v in (np.nextafter(c, np.float32(0)), c,
                                     np.nextafter(c, np.float32(np.inf)))}
    for cand in sorted(cands):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - exact)
        if bestd is None or d < bestd:
            best, bestd = cand, d
        elif d == bestd:
            raise AssertionError("exact tie: cannot decide the correctly rounded value")
    return np.float32(best)


def cr_exp(x: np.float32) -> np.float32:
    return nearest_f32(Fraction(Decimal(float(x)).exp()))


def finite_gates(dtype):
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    g = oracle.decode(bits, dtype)
    return g[np.isfinite(g)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_exp_is_correctly_rounded_for_every_16bit_gate(dtype):
    g = finite_gates(dtype)
    x = np.unique(-g)
    got = oracle.exp_f32(x)
    # beyond these bounds the result is +inf / 0 whatever the method
    big = x > 89.0
    small = x < -104.0
    assert np.all(np.isposinf(got[big]))
    assert np.all(got[small] == 0)
    mid = x[~big & ~small]
    exp = np.array([cr_exp(v) for v in mid], dtype=np.float32)
    assert np.array_equal(got[~big & ~small].view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_silu_mul_composition_is_ieee_fp32(dtype):
    g = finite_gates(dtype)
    e = oracle.exp_f32(-g)                       # pinned above
    with np.errstate(over="ignore", invalid="ignore"):
        d = np.float32(1.0) + e
        s = g / d
        for u in (np.float32(1.0), np.float32(-3.0), np.float32(0.7109375), np.float32(1e-30)):
            y = s * u
            got = oracle.silu_mul(g, np.full_like(g, u))
            assert np.array_equal(got.view(np.uint32), y.view(np.uint32))


def test_silu_known_values():
    g = np.array([0.0, 1.0, -1.0, 100.0, -100.0, 20.0], np.float32)
    y = oracle.silu_mul(g, np.ones_like(g))
    assert y[0] == 0.0 and y[3] == 100.0 and y[5] == 20.0
    assert y[4] == 0.0 and np.signbit(y[4])            # e^100 overflows: -100/inf = -0
    assert abs(y[1] - 0.7310586) < 1e-6 and abs(y[2] + 0.26894143) < 1e-6


def test_decode_fp16_matches_numpy():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
