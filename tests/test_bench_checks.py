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
    """A code one step away from the nearest exceeds both bounds and is
    counted past the strict one."""
    y = np.array([[1.0625, 3.0]], dtype=np.float32)          # e4m3 1.0625 is a tie: 0x38
    sc = np.ones((1, 2))
    good = oracle.e4m3(y)
    assert bench.error_stats(oracle, y, good, "e4m3", sc, False) == (1.0, 0)
    bad = good.copy()
    bad[0, 1] += 1                                          # 3.0 -> 3.25
    worst, strict = bench.error_stats(oracle, y, bad, "e4m3", sc, False)
    assert worst > 1.0 and strict == 1


def test_strict_bound_counts_the_fp32_multiplier_drift():
    """With an fp32 scale the reciprocal-multiply drift can move a value across
    an e4m3 midpoint: y / s a hair below the midpoint 1.0625 while
    fl(y * fl(1/s)) lands on it (ties to the even code 1.0): within the
    drift-aware bound, past the strict one.  Independent of the oracle's
    quantizer: the code is the nearest-even e4m3 of the fp32 product."""
    s = np.float32(3.0)
    inv = np.float32(1.0) / s
    # search y near 1.0625 * 3 whose product rounds onto the midpoint
    base = np.float32(1.0625) * s
    found = None
    for k in range(-64, 64):
        y = np.nextafter(base, np.float32(np.inf if k > 0 else -np.inf))
        for _ in range(abs(k)):
            y = np.nextafter(y, np.float32(np.inf if k > 0 else -np.inf))
        v = np.float32(y * inv)
        if v == np.float32(1.0625) and float(y) / float(s) != 1.0625:
            found = y
            break
    if found is None:
        import pytest
        pytest.skip("no drift case near this midpoint")
    y = np.array([[found]], dtype=np.float32)
    code = torch.from_numpy(np.array([[1.0625]], np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    worst, strict = bench.error_stats(oracle, y, code, "e4m3", np.full((1, 1), float(s)), True)
    exact = float(y[0, 0]) / float(s)
    nearest = 1.125 if exact > 1.0625 else 1.0
    if torch.from_numpy(np.array([[nearest]], np.float32)).to(torch.float8_e4m3fn) \
            .view(torch.uint8).numpy()[0, 0] != code[0, 0]:
        assert worst <= 1.0 and strict == 1
    else:
        assert worst <= 1.0 and strict == 0


def test_bf16_strict_bound_count():
    """Half a bf16 ulp around exact values: the nearest bf16 passes, one ulp
    off fails, ties pass either way, subnormals and zero included."""
    exact = np.array([1.0, 1.0 + 2.0 ** -8, 3.0 * 2.0 ** -130, 0.0, -448.0, 1.0 + 2.0 ** -9])
    near = torch.tensor(exact, dtype=torch.float64).to(torch.bfloat16).view(torch.int16)
    bits = near.numpy().view(np.uint16)
    assert bench.bf16_past_half_ulp(exact, bits) == 0
    off = bits.copy()
    off[0] += 1                      # 1 + 2^-7: one ulp above 1.0
    off[2] += 1                      # subnormal, one ulp (2^-133) off
    assert bench.bf16_past_half_ulp(exact, off) == 2
    tie = bits.copy()
    tie[1] = np.uint16(0x3F81)       # 1 + 2^-8 is a tie: 1 + 2^-7 is half an ulp away too
    assert bench.bf16_past_half_ulp(exact, tie) == 0


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
