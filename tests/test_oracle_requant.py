"""Pins of the oracle's per-token-group fp8 -> per-tensor fp8 requantization
(the sglang #35593 page): the page's exact-arithmetic test design (integers in
[-8, 8], power-of-two group scales, output scale 2, sentinel rows past
masked_m, k in {7168, 3584, 1152}), PyTorch's e4m3 decoding, and the IEEE
composition against numpy float32 products."""
import numpy as np
import pytest
import torch

import oracle
from workloads import splitmix64, substream

F8 = torch.float8_e4m3fn
SENTINEL = 0x2C           # e4m3 code of 0.375 (1.5 * 2^-2)


def to_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(F8).view(torch.uint8).numpy()


def test_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(F8).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(ours[~fin]))
    assert to_e4m3([0.375])[0] == SENTINEL


def build_exact(E, T, K, seed):
    """Integers in [-8, 8] as e4m3 codes; group scales 2^{-1, 0, 1} stored
    column-major per expert ([E][K/128][T])."""
    z = splitmix64(seed, 0, E * T * K)
    xi = (z % np.uint64(17)).astype(np.int64) - 8
    x = to_e4m3(xi.astype(np.float32)).reshape(E, T, K)
    ze = splitmix64(substream(seed, 1), 0, E * (K // 128) * T)
    ex = (ze % np.uint64(3)).astype(np.int64) - 1
    s = np.ldexp(np.float32(1.0), ex).astype(np.float32).reshape(E, K // 128, T)
    return x, xi.reshape(E, T, K), s


@pytest.mark.parametrize("k", [7168, 3584, 1152])
def test_page_design_exact_values_and_sentinels(k):
    E, T = 4, 48
    masked = np.array([0, 1, 17, T], np.int32)
    x, xi, s = build_exact(E, T, k, seed=k)
    out0 = np.full((E, T, k), SENTINEL, np.uint8)
    out = oracle.requant_fp8(x, E, T, k, 128, s, (k // 128 * T, 1, T), masked, 2.0, out_init=out0)
    for e, live in enumerate(masked):
        sc = np.repeat(s[e].T, 128, axis=1)[:live]              # [live, k]
        want = to_e4m3(xi[e, :live] * sc * 0.5)                 # every value exact in e4m3
        assert np.array_equal(out[e, :live], want)
        assert np.all(out[e, live:] == SENTINEL)


def test_saturation_rounding_and_composition():
    """Random codes and scales: the oracle equals e4m3(fl(fl(dec(x) * s) * fl(1/os)))
    computed with numpy float32 products; large products saturate."""
    E, T, K = 3, 9, 384
    rng = np.random.default_rng(5)
    x = rng.integers(0, 256, (E, T, K)).astype(np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x11                                # no NaN codes
    s = rng.uniform(0.001, 40.0, (E, T, K // 128)).astype(np.float32)   # row-major scales
    os_ = np.float32(0.7)
    out = oracle.requant_fp8(x, E, T, K, 128, s, (T * (K // 128), K // 128, 1), None, os_)
    dec = torch.from_numpy(x).view(F8).to(torch.float32).numpy()
    inv = np.float32(1.0) / os_
    v = (dec * np.repeat(s, 128, axis=2)).astype(np.float32) * inv
    assert np.array_equal(out, oracle.e4m3(v.astype(np.float32)))
    assert np.any(out == 0x7E) and np.any(out == 0xFE)          # saturated both ways


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.requant_fp8(np.zeros((1, 1, 100), np.uint8), 1, 1, 100, 128,
                           np.ones(1, np.float32), (1, 1, 1), None, 1.0)
