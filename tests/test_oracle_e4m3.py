"""Pins of the oracle's 8-bit narrowing against things other than itself.

e4m3: PyTorch's float8_e4m3fn decoding/encoding (a library routine) over every
fp32 value where a plain cast and a saturating cast agree (|v| < 464), an exact
nearest-code brute force over a random sample, the exact midpoints between
neighbouring codes, saturation, and the sign of zero.
int8: numpy's rint (round half to even) plus clamping over a dense sweep.
"""
import numpy as np
import pytest
import torch

import oracle

F8 = torch.float8_e4m3fn


def e4m3_values():
    """The 127 non-negative finite e4m3 values, decoded by PyTorch."""
    codes = torch.arange(0, 127, dtype=torch.uint8)
    return codes.view(F8).to(torch.float64).numpy()


def test_every_finite_code_roundtrips():
    vals = e4m3_values()
    assert vals[126] == 448.0 and vals[8] == 2.0 ** -6 and vals[1] == 2.0 ** -9
    pos = oracle.e4m3(vals.astype(np.float32))
    neg = oracle.e4m3(-vals.astype(np.float32))
    assert np.array_equal(pos, np.arange(127, dtype=np.uint8))
    assert np.array_equal(neg, np.arange(127, dtype=np.uint8) | 0x80)


def test_midpoints_go_to_even_and_neighbours_to_nearest():
    vals = e4m3_values()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    lo = np.arange(126)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(oracle.e4m3(mids), even)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    assert np.array_equal(oracle.e4m3(up), (lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.e4m3(dn), lo.astype(np.uint8))
    assert np.array_equal(oracle.e4m3(-mids), even | 0x80)


def test_saturation_and_signed_zero():
    big = np.array([448.0, 449.0, 463.99, 464.0, 470.0, 480.0, 1e6, 3.4e38, np.inf], np.float32)
    assert np.all(oracle.e4m3(big) == 0x7E)
    assert np.all(oracle.e4m3(-big) == 0xFE)
    tiny = np.array([0.0, 1e-45, 1e-20, 2.0 ** -11, 2.0 ** -10], np.float32)
    assert np.all(oracle.e4m3(tiny) == 0x00)
    assert np.all(oracle.e4m3(-tiny) == 0x80)
    assert oracle.e4m3(np.array([np.nextafter(np.float32(2.0 ** -10), np.float32(1))]))[0] == 1


def test_brute_force_nearest_on_random_sample():
    """Exhaustive nearest-code search (exact, in float64) on 200k values."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0x30000000, 0x43F00000, size=200_000, dtype=np.uint32)
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    vals = e4m3_values()
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # ties: choose the even code
    idx = np.where(cand.sum(axis=1) == 1, cand.argmax(axis=1),
                   np.where(cand[:, ::2].any(axis=1),
                            np.argmax(cand & (np.arange(127) % 2 == 0)[None, :], axis=1), 0))
    idx = np.where(a >= 448.0, 126, idx).astype(np.uint8)
    expect = idx | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    assert np.array_equal(oracle.e4m3(v), expect)


@pytest.mark.slow
def test_exhaustive_against_torch_cast():
    """Every fp32 pattern with 2^-12 <= |v| < 464, both signs (~350M values)."""
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(464.0).view(np.uint32))
    step = 1 << 24
    for b0 in range(lo, hi, step):
        b1 = min(hi, b0 + step)
        v = np.arange(b0, b1, dtype=np.uint32).view(np.float32)
        t = torch.from_numpy(v).to(F8).view(torch.uint8).numpy()
        assert np.array_equal(oracle.e4m3(v), t), hex(b0)
        t = torch.from_numpy(-v).to(F8).view(torch.uint8).numpy()
        assert np.array_equal(oracle.e4m3(-v), t), hex(b0)
    # everything below 2^-12 is a signed zero
    v = np.arange(0, lo, 4099, dtype=np.uint32).view(np.float32)
    assert np.all(oracle.e4m3(v) == 0) and np.all(oracle.e4m3(-v) == 0x80)


def test_int8_round_half_even_and_clamp():
    k = np.arange(-140 * 8, 140 * 8 + 1, dtype=np.float64) / 8.0   # quarter/half/eighth points
    rng = np.random.default_rng(3)
    r = rng.uniform(-140, 140, 100_000)
    v = np.concatenate([k, r]).astype(np.float32)
    v = np.concatenate([v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(-np.inf))])
    expect = np.clip(np.rint(v.astype(np.float64)), -128, 127).astype(np.int8)
    assert np.array_equal(oracle.int8(v), expect)
