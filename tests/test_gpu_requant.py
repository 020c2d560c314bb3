"""Bit-exact parity of the fp8 requantization path (ptgq_requant_fp8) with
the oracle, including the sglang #35593 page's own test design."""
import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
from gpu_util import DEV, Guarded, compare
from workloads import splitmix64, substream

pytestmark = pytest.mark.gpu
F8 = torch.float8_e4m3fn
SENTINEL = 0x2C          # e4m3 code of 0.375


def to_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(F8).view(torch.uint8).numpy()


def run(x, E, T, K, G, s, strides, mm, exp_m, os_, fill=SENTINEL):
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    sd = torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).to(DEV)
    md = None if mm is None else torch.from_numpy(np.ascontiguousarray(mm, dtype=np.int32)).to(DEV)
    od = torch.tensor([os_], dtype=torch.float32, device=DEV)
    out = Guarded((E, T, K), torch.uint8, fill)
    aq.ptgq_requant_fp8(xd, E, T, K, G, sd, strides, md, exp_m, od, out.t)
    torch.cuda.synchronize()
    out.check("ptgq_requant_fp8 out")
    return out.host()


@pytest.mark.parametrize("k", [7168, 3584, 1152])
def test_page_design(k):
    """Integers in [-8, 8], power-of-two group scales (column-major per
    expert), output scale 2, sentinel past masked_m in {0, 1, 17, 48}."""
    E, T = 4, 48
    masked = np.array([0, 1, 17, T], np.int32)
    z = splitmix64(k, 0, E * T * k)
    xi = (z % np.uint64(17)).astype(np.int64) - 8
    x = to_e4m3(xi.astype(np.float32)).reshape(E, T, k)
    ze = splitmix64(substream(k, 1), 0, E * (k // 128) * T)
    s = np.ldexp(np.float32(1.0), (ze % np.uint64(3)).astype(np.int64) - 1).astype(np.float32)
    strides = ((k // 128) * T, 1, T)
    got = run(x, E, T, k, 128, s, strides, masked, 0, 2.0)
    want = oracle.requant_fp8(x, E, T, k, 128, s, strides, masked, 2.0,
                              out_init=np.full((E, T, k), SENTINEL, np.uint8))
    compare(f"requant page design k={k}", got, np.zeros(0, np.uint8), want, np.zeros(0, np.uint8))
    s3 = s.reshape(E, k // 128, T)
    for e, live in enumerate(masked):
        exact = to_e4m3(xi.reshape(E, T, k)[e, :live] * np.repeat(s3[e].T, 128, axis=1)[:live] * 0.5)
        assert np.array_equal(got[e, :live], exact)


def test_every_code_round_trips_with_unit_scales():
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                     # finite codes only
    E, T, K = 2, 3, 2048
    x = np.resize(codes, E * T * K).reshape(E, T, K).astype(np.uint8)
    s = np.ones(E * T * (K // 128), np.float32)
    got = run(x, E, T, K, 128, s, (T * (K // 128), K // 128, 1), None, 0, 1.0)
    assert np.array_equal(got, x)


@pytest.mark.parametrize("G", [16, 32, 64, 128])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_random_codes_and_scales(G, layout):
    rng = np.random.default_rng(G + (layout == "col"))
    E, T, K = 5, 37, 1152 + 2 * G
    K -= K % G
    x = rng.integers(0, 256, (E, T, K)).astype(np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x3A
    ng = K // G
    s = rng.uniform(1e-3, 30.0, E * T * ng).astype(np.float32)
    strides = (T * ng, ng, 1) if layout == "row" else (T * ng, 1, T)
    mm = rng.integers(-3, T + 5, E).astype(np.int32)
    for os_, exp_m in ((0.37, 0), (3.0, 7), (1e-3, T)):
        got = run(x, E, T, K, G, s, strides, mm, exp_m, os_)
        want = oracle.requant_fp8(x, E, T, K, G, s, strides, mm, os_,
                                  out_init=np.full((E, T, K), SENTINEL, np.uint8))
        compare(f"requant G={G} {layout} os={os_}", got, np.zeros(0, np.uint8), want,
                np.zeros(0, np.uint8))


def test_many_experts_and_all_rows():
    rng = np.random.default_rng(9)
    E, T, K = 130, 6, 640
    x = rng.integers(0, 127, (E, T, K)).astype(np.uint8)
    s = rng.uniform(0.5, 2.0, E * T * (K // 128)).astype(np.float32)
    strides = (T * (K // 128), 1, T)
    mm = rng.integers(0, T + 1, E).astype(np.int32)
    for masked in (mm, None):
        got = run(x, E, T, K, 128, s, strides, masked, 0, 0.75)
        want = oracle.requant_fp8(x, E, T, K, 128, s, strides, masked, 0.75,
                                  out_init=np.full((E, T, K), SENTINEL, np.uint8))
        compare(f"requant E=130 masked={masked is not None}", got, np.zeros(0, np.uint8), want,
                np.zeros(0, np.uint8))


@pytest.mark.parametrize("grid", [0, 1])
@pytest.mark.parametrize("E", [64, 65])
def test_grid_modes_at_the_expert_window(E, grid):
    """Both grids (capped persistent, uncapped XCD-chunked) at 64 experts,
    whose prefix sum each wave holds in registers, and 65, which the kernel
    sums in LDS; the last expert is full, the first empty."""
    rng = np.random.default_rng(6400 + E + 7 * grid)
    T, K = 40, 1152
    x = rng.integers(0, 256, (E, T, K)).astype(np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x30
    s = rng.uniform(0.25, 4.0, E * T * (K // 128)).astype(np.float32)
    strides = (T * (K // 128), 1, T)
    mm = rng.integers(-2, T + 3, E).astype(np.int32)
    mm[0], mm[E - 1] = 0, T
    try:
        aq.ptgq_set_tuning(6, grid)
        aq.ptgq_set_tuning(5, 1)        # chunks of one block: a ragged last span
        got = run(x, E, T, K, 128, s, strides, mm, 8, 1.5)
    finally:
        aq.ptgq_set_tuning(6, -1)
        aq.ptgq_set_tuning(5, -1)
    want = oracle.requant_fp8(x, E, T, K, 128, s, strides, mm, 1.5,
                              out_init=np.full((E, T, K), SENTINEL, np.uint8))
    compare(f"requant E={E} grid={grid}", got, np.zeros(0, np.uint8), want,
            np.zeros(0, np.uint8))
