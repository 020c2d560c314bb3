"""Hand-worked groups (tests/golden/hand_worked.json) and the vllm #41326 page's
all-zero worked example (packed column-major UE8M0 layout)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import to_bf16_bits

with open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")) as fh:
    GOLDEN = json.load(fh)


def bf16_exact(values):
    f = np.array([float.fromhex(v) if "p" in v else float(v) for v in values], dtype=np.float64)
    b = to_bf16_bits(f)
    back = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, f) and np.array_equal(np.signbit(back), np.signbit(f))
    return b


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["id"] for c in GOLDEN["cases"]])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_hand_worked_group(case, layout):
    n = len(case["values"])
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, :n] = bf16_exact(case["values"])
    q, s = oracle.ptgq(x, "bf16", 1, 128, 128, False, case["out_dtype"], case["scale_fmt"],
                       layout, eps=case["eps"])
    assert list(q[0, :n]) == case["codes"]
    assert np.all(q[0, n:] == 0)
    if case["scale_fmt"] == "ue8m0":
        assert s[0] == case["scale_byte"]
        if layout == "col":        # one packed word, rows padded to 4: bytes 1..3 and rows 1..3 are 0
            assert s.size == 16 and np.all(s[1:] == 0)
    else:
        assert int(s[:4].view(np.uint32)[0]) == int(case["scale_bits"], 16)
        if layout == "col":
            assert s.size == 16 and np.all(s[4:] == 0)


@pytest.mark.parametrize("case", GOLDEN["per_token"], ids=[c["id"] for c in GOLDEN["per_token"]])
def test_hand_worked_per_token(case):
    x = bf16_exact(case["values"]).reshape(1, -1)
    n = x.shape[1]
    x = np.concatenate([x, np.zeros((1, 4 - n), np.uint16)], axis=1) if n < 4 else x
    q, s = oracle.ptq_fp8(x, "bf16", 1, x.shape[1])
    assert list(q[0, :n]) == case["codes"]
    assert int(s.view(np.uint32)[0]) == int(case["scale_bits"], 16)


def test_vllm_all_zero_example_packed_layout():
    """The vllm #41326 page's all-zero test: 4 x 7168 bf16 zeros, G=128.
    Its expected tensor is built as idx = pack_col * tma_aligned_mn + row, byte
    g % 4, over num_scale_elems = mn + (k_num_packed - 1) * tma_aligned_mn words;
    its byte is 0x5E under its own composition of eps.  Under the reading used
    here (eps floors amax once, before the division) the byte is 0x55.
    """
    mn, hidden, gs = 4, 7168, 128
    # the page's number, recomputed from the page's composition:
    page_scale = max(1e-10 / 448.0, 1e-10)
    assert math.ceil(math.log2(page_scale)) == -33 and 127 - 33 == 0x5E
    # our reading: fl(1e-10f / 448f) has exponent field 84 and a non-zero fraction
    r = np.float32(1e-10) / np.float32(448.0)
    assert (int(r.view(np.uint32)) >> 23) == 84 and (int(r.view(np.uint32)) & 0x7FFFFF) != 0
    byte = 85
    assert Fraction(2) ** (byte - 127) >= Fraction(float(r)) > Fraction(2) ** (byte - 128)

    x = np.zeros((mn, hidden), dtype=np.uint16)
    q, s = oracle.ptgq(x, "bf16", mn, hidden, gs, False, "e4m3", "ue8m0", "col")
    assert np.all(q == 0)
    groups_per_row = hidden // gs
    k_num_packed = (groups_per_row + 3) // 4
    tma_aligned_mn = ((mn + 3) // 4) * 4
    num_scale_elems = mn + (k_num_packed - 1) * tma_aligned_mn
    expected = np.zeros(num_scale_elems, dtype=np.int64)
    for row in range(mn):
        for g in range(groups_per_row):
            expected[(g // 4) * tma_aligned_mn + row] |= byte << ((g % 4) * 8)
    words = s.view(np.uint32).astype(np.int64)
    assert words.size == k_num_packed * tma_aligned_mn
    assert np.array_equal(words[:num_scale_elems], expected)
