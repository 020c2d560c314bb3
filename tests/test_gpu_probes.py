"""Device probes, each against the oracle: the gfx950 e4m3 narrowing over
every relevant fp32 value, the fused SiLU step over every 16-bit gate, the
UE8M0 scale byte over every non-negative finite fp32 absmax, fp32 scales and
multipliers over every bf16 absmax and a dense fp32 sample, and the int8
narrowing over every non-NaN fp32."""
import os

import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def probe_e4m3(v_dev):
    out = torch.empty(v_dev.numel(), dtype=torch.uint8, device=DEV)
    aq.ptgq_probe_e4m3(v_dev, out, v_dev.numel())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_e4m3_narrowing_every_fp32_in_range():
    """All fp32 patterns with 2^-12 <= |v| <= 480, both signs; a sample below;
    specials above (saturation)."""
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(480.0).view(np.uint32)) + 1
    step = 1 << 26
    total = 0
    for b0 in range(lo, hi, step):
        b1 = min(hi, b0 + step)
        bits = torch.arange(b0, b1, dtype=torch.int64, device=DEV).to(torch.int32)
        for sign in (0, 1):
            b = bits | (-(1 << 31)) if sign else bits
            v = b.view(torch.float32)
            got = probe_e4m3(v)
            ref = oracle.e4m3(v.cpu().numpy())
            bad = int((got != ref).sum())
            total += got.size
            if bad:
                i = int(np.flatnonzero(got != ref)[0])
                print(f"e4m3 probe: {bad} mismatches in [{b0:#x},{b1:#x}) sign {sign}; first "
                      f"v={v.cpu().numpy()[i]!r} got {got[i]:#04x} want {ref[i]:#04x}", flush=True)
            assert bad == 0
    print(f"e4m3 probe: {total} values, 0 mismatches", flush=True)
    small = np.arange(0, lo, 997, dtype=np.uint32).view(np.float32)
    special = np.array([480.0, 500.0, 1e6, 3.4e38, np.inf, 448.0, 464.0, 463.9, 0.0],
                       dtype=np.float32)
    v = np.concatenate([small, -small, special, -special]).astype(np.float32)
    got = probe_e4m3(torch.from_numpy(v).to(DEV))
    assert np.array_equal(got, oracle.e4m3(v))


@pytest.mark.parametrize("in_dtype,path", [("bf16", 0), ("bf16", 1), ("fp16", 0), ("fp16", 1)])
def test_silu_mul_every_16bit_gate(in_dtype, path):
    g_bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    gf = oracle.decode(g_bits, in_dtype)
    keep = np.isfinite(gf)
    from workloads import to_bf16_bits, to_fp16_bits
    conv = to_bf16_bits if in_dtype == "bf16" else to_fp16_bits
    for u in (1.0, -3.0, 0.7109375, 1e-3, 40.0):
        u_bits = np.full_like(g_bits, conv(np.array([u]))[0])
        gd = torch.from_numpy(g_bits.view(np.int16)).to(DEV)
        ud = torch.from_numpy(u_bits.view(np.int16)).to(DEV)
        out = torch.empty(g_bits.size, dtype=torch.float32, device=DEV)
        aq.ptgq_probe_silu_mul(gd, ud, in_dtype, path, out, g_bits.size)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = oracle.silu_mul(gf, oracle.decode(u_bits, in_dtype))
        bad = (got.view(np.uint32) != ref.view(np.uint32)) & keep
        print(f"silu probe {in_dtype} path {path} u={u}: {int(bad.sum())} mismatches over {int(keep.sum())} "
              f"finite gates", flush=True)
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            print(f"  first: g={gf[i]!r} got {got[i]!r} want {ref[i]!r}", flush=True)
        assert not bad.any()


# ------------------------------------------------ scale step and int8 narrowing

from concurrent.futures import ThreadPoolExecutor

CHUNK = 1 << 26
SUB = 1 << 22
WORKERS = min(16, os.cpu_count() or 1)


def host_bits(b0, b1):
    return np.arange(b0, b1, dtype=np.uint64).astype(np.uint32)


def oracle_over(fn, b0, b1):
    """fn(float32 values) over the bit patterns [b0, b1), in sub-chunks on a
    thread pool (the oracle's C loops release the interpreter lock)."""
    starts = list(range(b0, b1, SUB))
    with ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(lambda s: fn(host_bits(s, min(b1, s + SUB)).view(np.float32)), starts))
    return np.concatenate(parts)


@pytest.mark.parametrize("eps", [0.0, 1e-10])
@pytest.mark.parametrize("out_dtype", ["e4m3", "int8"])
def test_ue8m0_scale_every_finite_amax(out_dtype, eps):
    """The division-free UE8M0 byte of the kernels (exponent arithmetic above
    a threshold, the quotient's bits below it) over every non-negative finite
    fp32 absmax, against the oracle's byte from the IEEE quotient; the
    multiplier 2^(127 - e) is checked on every 4099th value."""
    end = 0x7F800000
    dev_e = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    dev_inv = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    total = bad = 0
    for b0 in range(0, end, CHUNK):
        b1 = min(end, b0 + CHUNK)
        n = b1 - b0
        aq.ptgq_probe_scale(b0, n, eps, out_dtype, "ue8m0", dev_e[:n], dev_inv[:n])
        torch.cuda.synchronize()
        got = dev_e[:n].cpu().numpy()
        want = oracle_over(lambda a: oracle.scale(a, eps, out_dtype, "ue8m0")[1], b0, b1)
        nb = int((got != want).sum())
        if nb:
            i = int(np.flatnonzero(got != want)[0])
            print(f"scale probe {out_dtype} eps={eps}: {nb} byte mismatches in [{b0:#x},{b1:#x});"
                  f" first amax bits {b0 + i:#x} got {got[i]} want {want[i]}", flush=True)
        bad += nb
        total += n
        inv = dev_inv[:n:4099].cpu().numpy().astype(np.float64)
        assert np.array_equal(inv, np.ldexp(1.0, 127 - got[::4099].astype(np.int64)))
    print(f"UE8M0 scale probe {out_dtype} eps={eps}: {total} amax values, {bad} mismatches",
          flush=True)
    assert bad == 0


@pytest.mark.parametrize("eps", [0.0, 1e-10])
@pytest.mark.parametrize("out_dtype", ["e4m3", "int8"])
def test_fp32_scale_and_multiplier(out_dtype, eps):
    """fp32 scales r = fl(max(a, eps) / qmax) and multipliers fl(1/r) (0 for
    r = 0, +inf once r is below ~2^-128): every bf16 absmax, every fp32 bit
    pattern below 2^-100 (subnormal and overflowing quotients) with a stride
    of 3, and every 61st pattern above, against the oracle."""
    lo_end = int(np.float32(2.0 ** -100).view(np.uint32))
    pats = np.concatenate([
        (np.arange(0, 0x7F80, dtype=np.uint32) << 16),
        np.arange(0, lo_end, 3, dtype=np.uint32),
        np.arange(lo_end, 0x7F800000, 61, dtype=np.uint32)]).astype(np.uint32)
    r_got = np.empty(pats.size, np.float32)
    inv_got = np.empty(pats.size, np.float32)
    # the probe runs over whole ranges of patterns; the sampled ones are
    # gathered on the device and copied back
    dev_r = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    dev_inv = torch.empty(CHUNK, dtype=torch.float32, device=DEV)
    order = np.argsort(pats, kind="stable")
    sp = pats[order]
    for b0 in range(0, 0x7F800000, CHUNK):
        b1 = min(0x7F800000, b0 + CHUNK)
        i0, i1 = np.searchsorted(sp, [b0, b1])
        if i0 == i1:
            continue
        aq.ptgq_probe_scale(b0, b1 - b0, eps, out_dtype, "f32", dev_r[:b1 - b0], dev_inv[:b1 - b0])
        idx = torch.from_numpy((sp[i0:i1] - b0).astype(np.int64)).to(DEV)
        r_got[order[i0:i1]] = dev_r[idx].cpu().numpy()
        inv_got[order[i0:i1]] = dev_inv[idx].cpu().numpy()
    r_want, _, inv_want = oracle.scale(pats.view(np.float32), eps, out_dtype, "f32")
    nr = int((r_got.view(np.uint32) != r_want.view(np.uint32)).sum())
    ni = int((inv_got.view(np.uint32) != inv_want.view(np.uint32)).sum())
    print(f"fp32 scale probe {out_dtype} eps={eps}: {pats.size} amax values, r mismatches {nr},"
          f" multiplier mismatches {ni}, overflowed multipliers {int(np.isinf(inv_want).sum())}",
          flush=True)
    assert nr == 0 and ni == 0


def test_int8_narrowing_every_fp32():
    """The kernels' int8 narrowing (clamp, add 1.5 * 2^23, byte) over every
    fp32 bit pattern except NaNs, against the oracle's round-half-even and
    clamp."""
    dev = torch.empty(CHUNK, dtype=torch.int8, device=DEV)
    total = bad = 0
    for b0 in range(0, 1 << 32, CHUNK):
        b1 = b0 + CHUNK
        aq.ptgq_probe_int8(b0, CHUNK, dev)
        torch.cuda.synchronize()
        got = dev.cpu().numpy()
        want = oracle_over(oracle.int8, b0, b1)
        bits = host_bits(b0, b1)
        finite_or_inf = (bits & 0x7FFFFFFF) <= 0x7F800000
        mism = (got != want) & finite_or_inf
        nb = int(mism.sum())
        if nb:
            i = int(np.flatnonzero(mism)[0])
            print(f"int8 probe: {nb} mismatches in [{b0:#x},{b1:#x}); first bits {b0 + i:#x} "
                  f"got {got[i]} want {want[i]}", flush=True)
        bad += nb
        total += int(finite_or_inf.sum())
    print(f"int8 probe: {total} non-NaN fp32 values, {bad} mismatches", flush=True)
    assert bad == 0
