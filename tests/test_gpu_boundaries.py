"""Bit-exact parity on both sides of every size threshold of the launch
chooser: one-slab against two-slab tasks (flat row tasks and flat-slab tasks),
the direct SiLU evaluation against the lookup table (flat and masked), and the
dequantization's one- against four-sub-slab tasks.  The shapes are derived
from the device's compute-unit count, and the host plan report confirms that
each pair straddles its threshold."""
import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
import workloads as W
from gpu_util import DEV, Guarded, compare, run_flat, run_masked

pytestmark = pytest.mark.gpu


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def plan(in_dtype, rows, K, fuse=False, E=0, expected_m=0):
    return aq.ptgq_plan_group(in_dtype, E, rows, K, 128, fuse, expected_m, rows, cus())


@pytest.mark.parametrize("in_dtype,K,out,fmt,layout", [
    ("bf16", 7168, "e4m3", "ue8m0", "col"),      # 14 slabs per row: row tasks
    ("fp16", 3584, "int8", "f32", "row"),        # 7 slabs per row: flat-slab tasks
])
def test_two_slab_threshold_of_unfused_calls(in_dtype, K, out, fmt, layout):
    spr = K // 512
    lo = (cus() * 16 - 1) // spr
    p_lo, p_hi = plan(in_dtype, lo, K), plan(in_dtype, lo + 1, K)
    assert p_lo["slabs_per_task"] == 1 and p_hi["slabs_per_task"] == 2 and p_hi["uncapped"] == 1
    for M in (lo, lo + 1):
        if in_dtype == "bf16":
            x = W.normal_bf16(700 + M, (M, K), factor_cols=[3, K - 1], factor=40.0)
        else:
            x = W.normal_fp16(700 + M, (M, K))
        x[M // 2, :128] = 0
        args = (x, in_dtype, M, K, 128, False, out, fmt, layout)
        compare(f"two-slab threshold {in_dtype} M={M} K={K}", *run_flat(*args),
                *oracle.ptgq(*args, eps=1e-10))


def test_silu_table_threshold_of_flat_calls():
    K = 4096
    lo = (cus() * 16 - 1) // (K // 512)
    assert plan("bf16", lo, K, fuse=True)["silu_table"] == 0
    assert plan("bf16", lo + 1, K, fuse=True)["silu_table"] == 1
    for M in (lo, lo + 1):
        x = W.normal_bf16(800 + M, (M, 2 * K))
        args = (x, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col")
        compare(f"table threshold fused M={M}", *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


def test_silu_table_threshold_of_masked_calls():
    E, T, K = 4, 384, 2048
    e_hi = (cus() * 16 + E * 4 - 1) // (E * 4)          # expected rows from which the table is read
    assert plan("bf16", T, K, fuse=True, E=E, expected_m=e_hi - 1)["silu_table"] == 0
    assert plan("bf16", T, K, fuse=True, E=E, expected_m=e_hi)["silu_table"] == 1
    rng = np.random.default_rng(31)
    for exp_m in (e_hi - 1, e_hi):
        mm = rng.integers(0, T + 1, E).astype(np.int32)
        mm[0] = T
        x = W.normal_bf16(900 + exp_m, (E, T, 2 * K))
        gq, gs = run_masked(x, "bf16", E, T, K, 128, True, mm, exp_m, "e4m3", "ue8m0", "col")
        sb = oracle.scale_bytes(T, K, 128, "ue8m0", "col")
        rq, rs = oracle.ptgq_masked(x, "bf16", E, T, K, 128, True, mm, "e4m3", "ue8m0", "col",
                                    q_init=np.full((E, T, K), 0x7F, np.uint8),
                                    s_init=np.full(E * sb, 0xFF, np.uint8))
        compare(f"table threshold masked expected_m={exp_m} masked_m={list(mm)}", gq, gs, rq, rs)


@pytest.mark.parametrize("out,sub", [("bf16", 512), ("fp32", 256)])
def test_dequant_task_size_threshold(out, sub):
    K, G = 7168, 128
    lo = (cus() * 16 * sub - 1) // K                   # last M with one-sub-slab tasks
    rng = np.random.default_rng(41)
    for M in (lo, lo + 1):
        q = rng.integers(0, 256, (M, K), dtype=np.uint8)
        s = rng.integers(100, 150, oracle.scale_bytes(M, K, G, "ue8m0", "col")).astype(np.uint8)
        osz = 4 if out == "fp32" else 2
        y = Guarded((M * K * osz,), torch.uint8, 0x5A)
        aq.ptgq_dequant(torch.from_numpy(q).to(DEV), "e4m3", M, K, G,
                        torch.from_numpy(s).to(DEV), "ue8m0", "col", out, y.t)
        torch.cuda.synchronize()
        y.check(f"dequant M={M}")
        got = y.host().view(np.float32 if out == "fp32" else np.uint16).reshape(M, K)
        want = oracle.dequant(q, "e4m3", M, K, G, s, "ue8m0", "col", out)
        if out == "fp32":
            gb, wb = got.view(np.uint32), want.view(np.uint32)
            nan = np.isnan(got) & np.isnan(want)
        else:
            gb, wb = got, want
            f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
            nan = np.isnan(f(got)) & np.isnan(f(want))
        bad = int(((gb != wb) & ~nan).sum())
        print(f"dequant threshold {out} M={M}: {bad} mismatches", flush=True)
        assert bad == 0
