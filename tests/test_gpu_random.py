"""Seeded random parity sweep: shapes, traits and masks drawn at random (fixed
seeds, so every run checks the same cases) across every entry point, each
compared byte for byte with the oracle.  PTGQ_RANDOM_<FAMILY>=n widens a
family to its first n seeds (the defaults keep the suite short)."""
import os

import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
import workloads as W
from gpu_util import DEV, Guarded, compare, run_flat, run_masked, run_per_token

pytestmark = pytest.mark.gpu
GS = (16, 32, 64, 128)


def cases(family, default):
    return range(int(os.environ.get(f"PTGQ_RANDOM_{family}", default)))


def draw_x(rng, shape, in_dtype, seed):
    if in_dtype == "fp32":
        x = W.normal_f32(seed, shape) * np.float32(rng.choice([1e-3, 1.0, 50.0]))
        return x.astype(np.float32)
    if in_dtype == "fp16":
        return W.normal_fp16(seed, shape)
    return W.normal_bf16(seed, shape, factor_cols=[int(rng.integers(0, shape[-1]))],
                         factor=float(rng.choice([1.0, 30.0, 300.0])))


def random_flat(case, seed, m_lo, m_hi):
    rng = np.random.default_rng(seed)
    G = int(rng.choice(GS))
    fuse = bool(rng.integers(0, 2))
    in_dtype = str(rng.choice(["bf16", "fp16"] if fuse else ["bf16", "fp16", "fp32"]))
    M = int(rng.integers(m_lo, m_hi))
    K = G * int(rng.integers(1, 9000 // G))
    out = str(rng.choice(["e4m3", "int8"]))
    fmt = str(rng.choice(["f32", "ue8m0"]))
    lay = str(rng.choice(["row", "col"]))
    eps = float(rng.choice([1e-10, 0.0, 1e-3]))
    x = draw_x(rng, (M, 2 * K if fuse else K), in_dtype, 5000 + case)
    args = (x, in_dtype, M, K, G, fuse, out, fmt, lay)
    compare(f"random flat #{case} {args[1:]} eps={eps}", *run_flat(*args, eps=eps),
            *oracle.ptgq(*args, eps=eps))


@pytest.mark.parametrize("case", cases("FLAT", 24))
def test_random_flat(case):
    random_flat(case, 1000 + case, 1, 700)


@pytest.mark.parametrize("case", cases("FLAT_LARGE", 6))
def test_random_flat_large(case):
    """Sizes where two-slab tasks, flat-slab tasks, the uncapped grid, its XCD
    chunks and the SiLU table take over."""
    random_flat(case, 1500 + case, 700, 5000)


@pytest.mark.parametrize("case", cases("MASKED", 12))
def test_random_masked(case):
    rng = np.random.default_rng(2000 + case)
    G = int(rng.choice(GS))
    fuse = bool(rng.integers(0, 2))
    in_dtype = str(rng.choice(["bf16", "fp16"] if fuse else ["bf16", "fp16", "fp32"]))
    E = int(rng.integers(1, 80))
    T = int(rng.integers(1, 120))
    K = G * int(rng.integers(1, 3000 // G))
    out = str(rng.choice(["e4m3", "int8"]))
    fmt = str(rng.choice(["f32", "ue8m0"]))
    lay = str(rng.choice(["row", "col"]))
    mm = rng.integers(-5, T + 10, E).astype(np.int32)
    x = draw_x(rng, (E, T, 2 * K if fuse else K), in_dtype, 6000 + case)
    gq, gs = run_masked(x, in_dtype, E, T, K, G, fuse, mm, int(rng.integers(0, T + 1)), out, fmt,
                        lay)
    sb = aq.ptgq_scale_bytes(T, K, G, fmt, lay)
    rq, rs = oracle.ptgq_masked(x, in_dtype, E, T, K, G, fuse, mm, out, fmt, lay,
                                q_init=np.full((E, T, K), 0x7F, np.uint8),
                                s_init=np.full(E * sb, 0xFF, np.uint8))
    compare(f"random masked #{case} E={E} T={T} K={K} G={G} {in_dtype} fuse={fuse} {out} "
            f"{fmt} {lay}", gq, gs, rq, rs)


@pytest.mark.parametrize("case", cases("PER_TOKEN", 10))
def test_random_per_token(case):
    rng = np.random.default_rng(3000 + case)
    in_dtype = str(rng.choice(["bf16", "fp16", "fp32"]))
    M = int(rng.integers(1, 3000))
    K = 4 * int(rng.integers(1, 6000))
    x = draw_x(rng, (M, K), in_dtype, 7000 + case)
    compare(f"random per-token #{case} M={M} K={K} {in_dtype}",
            *run_per_token(x, in_dtype, M, K), *oracle.ptq_fp8(x, in_dtype, M, K))


@pytest.mark.parametrize("case", cases("REQUANT", 10))
def test_random_requant(case):
    rng = np.random.default_rng(4000 + case)
    G = int(rng.choice(GS))
    E = int(rng.integers(1, 20))
    T = int(rng.integers(1, 200))
    K = G * int(rng.integers(1, 5000 // G))
    ng = K // G
    x = rng.integers(0, 256, (E, T, K)).astype(np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x31
    s = rng.uniform(1e-3, 20.0, E * T * ng).astype(np.float32)
    strides = [(T * ng, ng, 1), (T * ng, 1, T)][int(rng.integers(0, 2))]
    mm = None if rng.integers(0, 4) == 0 else rng.integers(-3, T + 5, E).astype(np.int32)
    os_ = float(rng.uniform(0.05, 8.0))
    xd = torch.from_numpy(x).to(DEV)
    sd = torch.from_numpy(s).to(DEV)
    md = None if mm is None else torch.from_numpy(mm).to(DEV)
    od = torch.tensor([os_], dtype=torch.float32, device=DEV)
    outd = Guarded((E, T, K), torch.uint8, 0x2C)
    aq.ptgq_requant_fp8(xd, E, T, K, G, sd, strides, md, int(rng.integers(0, T + 1)), od, outd.t)
    torch.cuda.synchronize()
    outd.check("random requant out")
    want = oracle.requant_fp8(x, E, T, K, G, s, strides, mm, os_,
                              out_init=np.full((E, T, K), 0x2C, np.uint8))
    compare(f"random requant #{case} E={E} T={T} K={K} G={G} strides={strides}",
            outd.host(), np.zeros(0, np.uint8), want, np.zeros(0, np.uint8))


@pytest.mark.parametrize("case", cases("DEQUANT", 10))
def test_random_dequant(case):
    rng = np.random.default_rng(5000 + case)
    G = int(rng.choice(GS))
    M = int(rng.integers(1, 900))
    K = G * int(rng.integers(1, 8000 // G))
    code = str(rng.choice(["e4m3", "int8"]))
    fmt = str(rng.choice(["f32", "ue8m0"]))
    lay = str(rng.choice(["row", "col"]))
    outd = str(rng.choice(["bf16", "fp16", "fp32"]))
    q = rng.integers(0, 256, (M, K)).astype(np.uint8)
    nb = oracle.scale_bytes(M, K, G, fmt, lay)
    if fmt == "f32":
        s = np.ldexp(rng.uniform(1, 2, nb // 4), rng.integers(-40, 20, nb // 4)).astype(np.float32)
        s = s.view(np.uint8)
    else:
        s = rng.integers(90, 160, nb).astype(np.uint8)
    qd = torch.from_numpy(q).to(DEV)
    sd = torch.from_numpy(s).to(DEV)
    osz = 4 if outd == "fp32" else 2
    y = Guarded((M * K * osz,), torch.uint8, 0x5A)
    aq.ptgq_dequant(qd, code, M, K, G, sd, fmt, lay, outd, y.t)
    torch.cuda.synchronize()
    y.check("random dequant y")
    got = y.host().view(np.float32 if outd == "fp32" else np.uint16).reshape(M, K)
    want = oracle.dequant(q, code, M, K, G, s, fmt, lay, outd)
    gf = got.astype(np.float32) if outd == "fp32" else None
    nan_g = np.isnan(gf) if outd == "fp32" else np.zeros(got.shape, bool)
    nan_w = np.isnan(want) if outd == "fp32" else np.zeros(got.shape, bool)
    if outd == "bf16":
        nan_g = (got & 0x7FFF) > 0x7F80
        nan_w = (want & 0x7FFF) > 0x7F80
    elif outd == "fp16":
        nan_g = (got & 0x7FFF) > 0x7C00
        nan_w = (want & 0x7FFF) > 0x7C00
    bad = (got.view(np.uint32 if outd == "fp32" else np.uint16) !=
           want.view(np.uint32 if outd == "fp32" else np.uint16)) & ~(nan_g & nan_w)
    print(f"[parity] random dequant #{case} M={M} K={K} G={G} {code} {fmt} {lay} {outd}: "
          f"{int(bad.sum())} mismatches", flush=True)
    assert not bad.any()
