"""Device probes: the gfx950 e4m3 narrowing over every relevant fp32 value and
the fused SiLU step over every 16-bit gate, each against the oracle."""
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


@pytest.mark.parametrize("in_dtype,path", [("bf16", 0), ("bf16", 1), ("fp16", 0)])
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
