"""The argument behind the fused kernels' direct SiLU evaluation, checked on
the host over every finite 16-bit gate (no GPU).  The kernels compute e^-g
with fp64 FMAs (Cody and Waite's reduction by ln 2, the degree-9 Taylor
polynomial of e^r by Horner's rule, a scale by 2^k) and round it once to
fp32, and form g / d from an fp64 reciprocal; the device probe test compares
the kernels' own code with the oracle for every gate.  Here:

- the same fp64 steps, simulated with exactly rounded FMAs (rational
  arithmetic), give the oracle's correctly rounded e^-g for every bf16 and
  fp16 gate (degree 8 does not);
- no quotient g / d of the oracle's steps that is not itself an fp32 value
  lies within 2^-48 of an fp32 rounding midpoint, so an fp64 approximation of
  it within 2^-48.5 rounds as the IEEE fp32 division does.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

INV_LN2 = float.fromhex("0x1.71547652b82fep+0")
LN2_HI = float.fromhex("0x1.62e42fee00000p-1")      # 32 significant bits: k * LN2_HI is exact
LN2_LO = float.fromhex("0x1.a39ef35793c76p-33")


def fma(a, b, c):
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def exp_neg_steps(g, degree):
    """The kernels' fp64 steps for e^-g, rounded to fp32."""
    x = -min(max(g, -100.0), 120.0)
    k = float(round(x * INV_LN2))                   # round half to even, as rint
    r = fma(-k, LN2_HI, x)
    r = fma(-k, LN2_LO, r)
    p = 1.0 / math.factorial(degree)
    for i in range(degree - 1, -1, -1):
        p = fma(p, r, 1.0 / math.factorial(i))
    with np.errstate(over="ignore"):
        return np.float32(math.ldexp(p, int(k)))


def finite_gates(dtype):
    g = oracle.decode(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16), dtype)
    return g[np.isfinite(g)].astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fp64_exp_steps_round_correctly_for_every_gate(dtype):
    g = finite_gates(dtype)
    want = oracle.exp_f32(-g).view(np.uint32)
    got = np.array([exp_neg_steps(float(v), 9) for v in g], dtype=np.float32).view(np.uint32)
    assert int((got != want).sum()) == 0


def test_degree_eight_is_not_enough():
    bad = 0
    for dtype in ("bf16", "fp16"):
        g = finite_gates(dtype)
        near = g[np.abs(g) > 0.2]                    # where a short polynomial errs most
        want = oracle.exp_f32(-near).view(np.uint32)
        got = np.array([exp_neg_steps(float(v), 8) for v in near],
                       dtype=np.float32).view(np.uint32)
        bad += int((got != want).sum())
    assert bad > 0


def test_quotients_stay_clear_of_fp32_midpoints():
    limit = Fraction(1, 1 << 48)
    closest = Fraction(1)
    for dtype in ("bf16", "fp16"):
        g = finite_gates(dtype)
        e = oracle.exp_f32(-g)
        with np.errstate(over="ignore"):
            d = (np.float32(1.0) + e).astype(np.float32)
        for gv, dv in zip(g.tolist(), d.tolist()):
            if gv == 0.0 or math.isinf(dv):
                continue
            q = abs(Fraction(gv) / Fraction(dv))
            if q < Fraction(1, 1 << 126):
                continue                              # subnormal results: the device probe
            lo = np.float32(float(q))
            if Fraction(float(lo)) > q:
                lo = np.nextafter(lo, np.float32(0))
            if Fraction(float(lo)) == q:
                continue                              # exact quotient
            hi = np.nextafter(lo, np.float32(np.inf))
            mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
            closest = min(closest, abs(q - mid) / q)
    assert closest >= limit, float(closest)
