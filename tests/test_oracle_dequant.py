"""Pins of the oracle's dequantization (codes x group scales -> bf16 / fp16 /
fp32): its round-to-nearest-even narrowings against numpy's float16 cast and
PyTorch's bfloat16 cast, and quantize-then-dequantize identities."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def fp32_sweep(step):
    lo = int(np.float32(2.0 ** -27).view(np.uint32))
    hi = int(np.float32(2.0 ** 17).view(np.uint32))
    b = np.arange(lo, hi, step, dtype=np.uint32)
    v = b.view(np.float32)
    extra = np.array([0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e30, 2.0 ** -24, 2.0 ** -25,
                      3 * 2.0 ** -26, 2.0 ** -14, 6.1e-5], np.float32)
    v = np.concatenate([v, extra])
    return np.concatenate([v, -v])


def test_fp16_rounding_matches_numpy():
    v = fp32_sweep(7)
    assert np.array_equal(oracle.fp16_rne(v), v.astype(np.float16).view(np.uint16))


def test_bf16_rounding_matches_torch():
    v = fp32_sweep(5)
    v = np.concatenate([v, np.array([3.3895e38, 3.4e38, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne(v), ref)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("code", ["e4m3", "int8"])
def test_exactness_family_round_trips(layout, code):
    """Integers in [-8, 8]: with UE8M0 (power-of-two) scales the dequantized
    codes are the inputs exactly, in every output dtype."""
    fmt = "ue8m0"
    d = W.cfg5c(M=12, K=1024)
    x = d["x"]
    q, s = oracle.ptgq(x, "fp16", 12, 1024, 128, False, code, fmt, layout)
    xf = x.view(np.float16).astype(np.float32)
    for out in ("fp32", "fp16", "bf16"):
        y = oracle.dequant(q, code, 12, 1024, 128, s, fmt, layout, out)
        if out == "fp32":
            assert np.array_equal(y, xf)
        elif out == "fp16":
            assert np.array_equal(y.view(np.float16).astype(np.float32), xf)
        else:
            assert np.array_equal(W.bf16_bits_to_f32(y), xf)


def test_dequant_is_decode_times_scale():
    """Random codes and fp32 scales: fp32 output = numpy float32 product of
    PyTorch's decoded codes and the scales; bf16/fp16 outputs are its casts."""
    rng = np.random.default_rng(3)
    M, K, G = 7, 512, 64
    q = rng.integers(0, 256, (M, K)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x40
    s = rng.uniform(1e-4, 10, (M, K // G)).astype(np.float32)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    want = (dec * np.repeat(s, G, axis=1)).astype(np.float32)
    y = oracle.dequant(q, "e4m3", M, K, G, s, "f32", "row", "fp32")
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    y16 = oracle.dequant(q, "e4m3", M, K, G, s, "f32", "row", "fp16")
    assert np.array_equal(y16, want.astype(np.float16).view(np.uint16))
    qi = q.view(np.int8)
    yi = oracle.dequant(q, "int8", M, K, G, s, "f32", "row", "fp32")
    assert np.array_equal(yi, (qi.astype(np.float32) * np.repeat(s, G, axis=1)).astype(np.float32))


def test_col_major_and_ue8m0_scale_addressing():
    """Scales written by hand in each layout (fp32 column-major with M padded
    to 4; UE8M0 packed four groups to a 32-bit word) address the same group
    as the row-major fp32 form.  Exponent byte 0 stands for 2^-127."""
    rng = np.random.default_rng(5)
    M, K, G = 6, 1024, 128
    ng = K // G
    q = rng.integers(0, 0x7E, (M, K)).astype(np.uint8)
    e = rng.integers(100, 140, (M, ng)).astype(np.uint8)
    e[0, 0] = 0
    e[5, 7] = 0
    sf = np.where(e == 0, np.float32(2.0 ** -127), np.ldexp(1.0, e.astype(np.int32) - 127)
                  ).astype(np.float32)
    want = oracle.dequant(q, "e4m3", M, K, G, sf, "f32", "row", "fp32")
    mp = 8
    col = np.zeros((ng, mp), np.float32)
    col[:, :M] = sf.T
    assert np.array_equal(oracle.dequant(q, "e4m3", M, K, G, col, "f32", "col", "fp32"), want)
    assert np.array_equal(oracle.dequant(q, "e4m3", M, K, G, e, "ue8m0", "row", "fp32"), want)
    packed = np.zeros((ng // 4, mp, 4), np.uint8)
    for g in range(ng):
        packed[g // 4, :M, g % 4] = e[:, g]
    assert np.array_equal(oracle.dequant(q, "e4m3", M, K, G, packed, "ue8m0", "col", "fp32"),
                          want)
    dec = oracle.e4m3_decode(q)
    exact = dec.astype(np.float64) * np.repeat(sf, G, axis=1).astype(np.float64)
    assert np.array_equal(want.astype(np.float64)[exact >= 2.0 ** -126],
                          exact[exact >= 2.0 ** -126])
