"""Host logic of the benchmark's correctness counts: with the oracle's own
outputs standing in for the GPU's, the sampled checks report no mismatch and
a dequantization error within its bound; a planted code or scale error is
counted.  (CPU only: the stand-in buffers are CPU tensors.)"""
import numpy as np
import torch

import bench
import oracle
import workloads as W


def test_flat_checks_count_nothing_on_oracle_outputs_and_count_planted_errors():
    M, K, G = 40, 2048, 128
    x = W.normal_bf16(5, (M, K), factor_cols=[3], factor=30.0)
    for out, fmt, lay in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row"), ("e4m3", "f32", "col")):
        q, s = oracle.ptgq(x, "bf16", M, K, G, False, out, fmt, lay)
        rows = [0, 7, 39]
        res = bench.capture_flat(x, "bf16", M, K, G, False, out, fmt, lay, torch.from_numpy(q),
                                 torch.from_numpy(s), rows)(oracle)
        assert res["code_mismatches"] == 0 and res["scale_mismatches"] == 0
        assert 0.0 < res["max_error_over_bound"] <= 1.0
        q2 = q.copy()
        q2[7, 100] ^= 1
        res = bench.capture_flat(x, "bf16", M, K, G, False, out, fmt, lay, torch.from_numpy(q2),
                                 torch.from_numpy(s), rows)(oracle)
        assert res["code_mismatches"] == 1


def test_fused_and_fp32_checks():
    M, K, G = 16, 1024, 128
    x = W.normal_bf16(6, (M, 2 * K))
    q, s = oracle.ptgq(x, "bf16", M, K, G, True, "e4m3", "ue8m0", "col")
    res = bench.capture_flat(x, "bf16", M, K, G, True, "e4m3", "ue8m0", "col",
                             torch.from_numpy(q), torch.from_numpy(s), [0, 15])(oracle)
    assert res["code_mismatches"] == 0 and res["scale_mismatches"] == 0
    assert res["max_error_over_bound"] <= 1.0
    x32 = W.normal_f32(7, (M, K))
    q, s = oracle.ptgq(x32, "fp32", M, K, G, False, "int8", "ue8m0", "row")
    s2 = s.copy()
    s2[3] ^= 1
    res = bench.capture_flat(x32, "fp32", M, K, G, False, "int8", "ue8m0", "row",
                             torch.from_numpy(q), torch.from_numpy(s2), [0, 5])(oracle)
    assert res["scale_mismatches"] == 1


def test_error_bound_is_tight_for_a_half_ulp_miss():
    """A code one step away from the nearest exceeds the bound."""
    y = np.array([[1.0625, 3.0]], dtype=np.float32)          # e4m3 1.0625 is a tie: 0x38
    sc = np.ones((1, 2))
    good = oracle.e4m3(y)
    assert bench.error_over_bound(oracle, y, good, "e4m3", sc, False) <= 1.0
    bad = good.copy()
    bad[0, 1] += 1                                          # 3.0 -> 3.25
    assert bench.error_over_bound(oracle, y, bad, "e4m3", sc, False) > 1.0


def test_bench_refuses_more_than_one_gpu():
    """The path needs no exchange between GPUs; bench.py measures one and says
    so for any other count, before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "--gpus 1" in res.stderr
