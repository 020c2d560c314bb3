"""The launch-geometry chooser on the host (no GPU): the plans it makes for the
seeded workloads on a 256-CU MI355X, and the rules every plan keeps."""
import numpy as np
import pytest

import activation_quantization_amd as aq

CUS = 256            # MI355X
SLAB = 512           # elements of a row per slab


@pytest.fixture(autouse=True)
def _reset_knobs():
    for k in range(8):
        aq.ptgq_set_tuning(k, -1)
    yield
    for k in range(8):
        aq.ptgq_set_tuning(k, -1)


def plan(in_dtype, rows, K, G=128, fuse=False, E=0, expected_m=0, q_rows=None, cus=CUS):
    return aq.ptgq_plan_group(in_dtype, E, rows, K, G, fuse, expected_m,
                              rows if q_rows is None else q_rows, cus)


def test_headline_uncapped_xcd_chunked():
    p = plan("bf16", 16384, 7168)
    assert p["slabs_per_task"] == 2 and p["tasks_per_row"] == 7
    assert p["tasks"] == 16384 * 7
    assert p["uncapped"] == 1 and p["block"] == 256
    assert p["grid"] == 16384 * 7 // 4             # one wave per task
    assert p["xcd_chunk"] == 64 and p["silu_table"] == 0


@pytest.mark.parametrize("M", [1, 16])
def test_decode_sizes_spread_one_slab_tasks_over_one_wave_blocks(M):
    p = plan("bf16", M, 7168)
    assert p["slabs_per_task"] == 1 and p["block"] == 64
    assert p["tasks"] == M * 14 and p["grid"] == M * 14
    assert p["uncapped"] == 0 and p["xcd_chunk"] == 0


def test_m256_one_slab_tasks_capped_grid_covers_every_task_once():
    p = plan("bf16", 256, 7168)
    assert p["slabs_per_task"] == 1 and p["tasks"] == 256 * 14
    assert p["uncapped"] == 0 and p["xcd_chunk"] == 0
    assert p["grid"] * p["block"] // 64 >= p["tasks"]


@pytest.mark.parametrize("M", [512, 1024])
def test_mid_sizes_take_two_slab_tasks_on_the_uncapped_grid(M):
    p = plan("bf16", M, 7168)                     # from 4096 slabs on (half a wave per slot)
    assert p["slabs_per_task"] == 2 and p["uncapped"] == 1 and p["grid"] == M * 7 // 4
    # fused calls of the same size keep one-slab tasks on a capped grid
    p = plan("bf16", M, 3584, fuse=True)
    assert p["slabs_per_task"] == 1 and p["uncapped"] == 0


def test_fused_large_call_takes_the_silu_table_one_block_per_cu():
    p = plan("bf16", 8192, 4096, fuse=True)
    assert p["silu_table"] == 1 and p["block"] == 1024 and p["grid"] == CUS
    assert p["slabs_per_task"] == 1 and p["uncapped"] == 0
    # small fused calls evaluate directly
    assert plan("bf16", 64, 4096, fuse=True)["silu_table"] == 0
    # from 16 slabs per CU (one per wave of the table grid) on
    assert plan("bf16", 256, 4096, fuse=True)["silu_table"] == 0
    assert plan("bf16", 512, 4096, fuse=True)["silu_table"] == 1
    # fp16 gates: the 144 KiB table from 32 slabs per CU on
    assert plan("fp16", 8192, 4096, fuse=True)["silu_table"] == 1
    assert plan("fp16", 1023, 4096, fuse=True)["silu_table"] == 0
    assert plan("fp16", 1024, 4096, fuse=True)["silu_table"] == 1
    # masked: not beside the 2 E ints of a prefix sum of more than 1024 experts
    assert plan("fp16", 384, 2048, fuse=True, E=1024)["silu_table"] == 1
    assert plan("fp16", 384, 2048, fuse=True, E=1025)["silu_table"] == 0


def test_masked_workload_sized_by_expected_rows():
    p = plan("bf16", 384, 2048, fuse=True, E=32, expected_m=189)
    assert p["silu_table"] == 1 and p["grid"] == CUS and p["block"] == 1024
    assert p["tasks"] == 32 * 189 * 4
    # unknown expected_m: every row of every expert
    assert plan("bf16", 384, 2048, fuse=True, E=32)["tasks"] == 32 * 384 * 4
    # masked grids are never uncapped (the task count is only known on the device)
    assert plan("bf16", 384, 7168, E=32)["uncapped"] == 0


def test_small_masked_fused_calls_take_chunk_tasks():
    # decode-sized masked calls: chunk tasks over the expected live rows
    p = plan("bf16", 384, 2048, fuse=True, E=32, expected_m=4)
    assert p["flat_slabs"] == 4 and p["tasks"] == 32 * 4 * 16 and p["tasks_per_row"] == 16
    assert plan("bf16", 384, 2048, fuse=True, E=32, expected_m=5)["flat_slabs"] == 0
    assert plan("bf16", 384, 2048, E=32, expected_m=1)["flat_slabs"] == 0     # unfused
    assert plan("bf16", 384, 2048, fuse=True, E=32)["flat_slabs"] == 0        # all rows expected


def test_small_fused_calls_take_chunk_tasks():
    # up to 8 chunk tasks of 128 output elements per CU, on the direct SiLU path
    p = plan("bf16", 64, 4096, fuse=True)
    assert p["flat_slabs"] == 4 and p["tasks"] == 64 * 32 and p["tasks_per_row"] == 32
    assert p["uncapped"] == 1 and p["grid"] * p["block"] // 64 >= p["tasks"]
    assert plan("bf16", 65, 4096, fuse=True)["flat_slabs"] == 0
    assert plan("fp16", 1, 4160, G=64, fuse=True)["tasks_per_row"] == 33  # a short last chunk
    assert plan("bf16", 64, 4096)["flat_slabs"] == 0                       # unfused: never
    aq.ptgq_set_tuning(0, 1)                      # slab tasks forced
    assert plan("bf16", 64, 4096, fuse=True)["flat_slabs"] == 0
    aq.ptgq_set_tuning(0, -1)
    aq.ptgq_set_tuning(7, 0)
    assert plan("bf16", 64, 4096, fuse=True)["flat_slabs"] == 0
    aq.ptgq_set_tuning(7, 2)                      # forced; the table still wins unless off
    assert plan("bf16", 1000, 4096, fuse=True)["silu_table"] == 1
    aq.ptgq_set_tuning(4, 0)
    assert plan("bf16", 1000, 4096, fuse=True)["flat_slabs"] == 4


@pytest.mark.parametrize("K", [640, 1408, 1152, 384, 128, 2944])
def test_masked_rows_not_whole_slabs_take_flattened_slabs(K):
    # each expert's live rows are one sequence of slabs: the expected task
    # count is per expert, rounded up to whole tasks
    for fuse in (False, True):
        for E, exp_m in ((32, 300), (3, 5), (80, 0)):
            p = plan("bf16", 384, K, fuse=fuse, E=E, expected_m=exp_m)
            hint = exp_m if exp_m > 0 else 384
            if fuse and hint * E * -(-K // 128) <= CUS * 8:
                # small fused calls: chunk tasks of the live rows
                assert p["flat_slabs"] == 4 and p["tasks"] == hint * E * -(-K // 128)
                continue
            per = p["slabs_per_task"] * SLAB
            assert p["flat_slabs"] == 3 and p["tasks_per_row"] == 1 and p["uncapped"] == 0
            assert p["tasks"] == E * (-(-hint * K // per))
    # two-slab tasks once the expected slabs pass half a wave per slot (unfused)
    assert plan("bf16", 384, 1408, E=32, expected_m=300)["slabs_per_task"] == 2
    assert plan("bf16", 384, 1408, E=3, expected_m=5)["slabs_per_task"] == 1
    # unfused rows of an odd number of whole slabs too; fused ones, and rows
    # of an even number, keep row tasks unless the slab-sequence knob forces
    # flattened slabs
    assert plan("bf16", 384, 1536, E=32)["flat_slabs"] == 3
    assert plan("fp16", 384, 512, E=32)["flat_slabs"] == 3
    assert plan("bf16", 384, 1536, fuse=True, E=32)["flat_slabs"] == 0
    assert plan("bf16", 384, 2048, E=32)["flat_slabs"] == 0
    aq.ptgq_set_tuning(7, 1)
    assert plan("bf16", 384, 1536, fuse=True, E=32)["flat_slabs"] == 3
    assert plan("bf16", 384, 2048, E=32)["flat_slabs"] == 3
    aq.ptgq_set_tuning(7, 0)
    assert plan("bf16", 384, K, E=32)["flat_slabs"] == 0


@pytest.mark.parametrize("K", [7168, 4096, 14336, 2048, 1024])
def test_fp32_input_uncapped_and_xcd_chunked_for_every_row_length(K):
    p = plan("fp32", 8192 * 7168 // K, K)
    assert p["slabs_per_task"] == 2 and p["uncapped"] == 1
    assert p["block"] == 128 and p["xcd_chunk"] == 256     # two-wave blocks


@pytest.mark.parametrize("K,chunk", [(1536, 512), (2560, 512), (1024, 64), (2048, 64), (3072, 64)])
def test_short_16bit_rows_are_xcd_chunked_too(K, chunk):
    # odd slab counts: flat-slab tasks in one-wave blocks; even: row tasks
    p = plan("fp16", 16384, K)
    assert p["uncapped"] == 1 and p["tasks_per_row"] < 4 and p["xcd_chunk"] == chunk


def test_small_uncapped_grids_keep_contiguous_xcd_ranges():
    # 12288 one-wave blocks: under 4 spans of 8 x 512
    p = plan("fp16", 8192, 1536)
    assert p["uncapped"] == 1 and p["flat_slabs"] == 1 and p["block"] == 64
    assert p["grid"] == 12288 and p["xcd_chunk"] == 0


def test_odd_slab_rows_take_flat_slab_tasks_across_row_ends():
    p = plan("fp16", 8192, 3584)                   # 7 slabs per row
    assert p["slabs_per_task"] == 2 and p["uncapped"] == 1 and p["flat_slabs"] == 1
    assert p["tasks"] == 8192 * 7 // 2             # no half task per row
    # one-wave blocks, dealt to the XCDs in chunks of 512
    assert p["block"] == 64 and p["grid"] == p["tasks"] and p["xcd_chunk"] == 512
    # fp32 rows of an odd slab count too
    p = plan("fp32", 4096, 3584)
    assert p["slabs_per_task"] == 2 and p["flat_slabs"] == 1 and p["tasks"] == 4096 * 7 // 2
    # rows that are not whole slabs: slabs of the flattened tensor, crossing
    # row ends anywhere
    p = plan("fp16", 8192, 3584 + 128)
    assert p["flat_slabs"] == 3 and p["slabs_per_task"] == 2
    assert p["tasks"] == -(-(-(-(8192 * 3712) // 512)) // 2)
    # fp32 input too
    assert plan("fp32", 8192, 3584 + 128)["flat_slabs"] == 3
    # rows of an even slab count keep row tasks (the same tasks)
    p = plan("bf16", 4096, 7168)
    assert p["flat_slabs"] == 0 and p["tasks"] == 4096 * 7
    # the override: 0 restores row tasks, whose last task per row holds one
    # slab; 1 takes flat-slab tasks for even slab counts too
    aq.ptgq_set_tuning(7, 0)
    p = plan("fp16", 8192, 3584)
    assert p["flat_slabs"] == 0 and p["tasks_per_row"] == 4 and p["tasks"] == 8192 * 4
    aq.ptgq_set_tuning(7, 1)
    assert plan("bf16", 4096, 7168)["flat_slabs"] == 1


@pytest.mark.parametrize("K", [16, 64, 128, 256])
def test_short_rows_take_multi_row_slabs(K):
    rows = 8192 * SLAB // K + 3                    # 8193 slabs of 512 // K rows, the last partial
    p = plan("bf16", rows, K, G=16)
    assert p["flat_slabs"] == 2 and p["slabs_per_task"] == 2 and p["uncapped"] == 1
    assert p["tasks"] == (8193 + 1) // 2 and p["block"] == 64
    # fp32 input and fused calls take slabs of the flattened tensor
    assert plan("fp32", rows, K, G=16)["flat_slabs"] == 3
    assert plan("bf16", rows, K, G=16, fuse=True)["flat_slabs"] == 3
    # K not dividing the slab: slabs of the flattened tensor
    assert plan("bf16", 65536, 384)["flat_slabs"] == 3
    # the override's 0 restores one row per slab
    aq.ptgq_set_tuning(7, 0)
    assert plan("bf16", rows, K, G=16)["flat_slabs"] == 0


def test_padded_rows_get_waves_for_the_zero_fill():
    # nothing to quantize, 28 MiB of code rows to zero: a full capped grid
    # whose waves loop over the fill (1 KiB per wave store)
    p = plan("bf16", 0, 7168, q_rows=4096)
    assert p["tasks"] == 0 and p["uncapped"] == 0
    assert p["grid"] % CUS == 0 and p["grid"] * p["block"] // 64 >= CUS * 16
    # a few rows and no padding: one-wave blocks, as many as the tasks
    # rounded up to a multiple of the 8 XCDs
    p = plan("bf16", 5, 7168)
    assert p["block"] == 64 and p["grid"] == 72 and p["tasks"] == 70


@pytest.mark.parametrize("cus", [80, 256, 304])
def test_rules_hold_for_random_shapes(cus):
    rng = np.random.default_rng(cus)
    for _ in range(300):
        G = int(rng.choice([16, 32, 64, 128]))
        K = G * int(rng.integers(1, 30000 // G))
        if rng.integers(0, 4) == 0:                       # rows shorter than a slab
            K = int(rng.choice([k for k in (16, 32, 64, 128, 256) if k >= G] or [G]))
        rows = int(rng.integers(1, 200000 if K < SLAB else 20000))
        dt = str(rng.choice(["bf16", "fp16", "fp32"]))
        fuse = dt != "fp32" and bool(rng.integers(0, 2))
        p = plan(dt, rows, K, G, fuse, cus=cus)
        spr = -(-K // SLAB)
        U = p["slabs_per_task"]
        assert U in (1, 2)
        if p["flat_slabs"] == 4:
            assert p["tasks_per_row"] == -(-K // 128)
        elif p["flat_slabs"] >= 2:
            assert p["tasks_per_row"] == 1
        else:
            assert p["tasks_per_row"] == -(-spr // U)
        if p["flat_slabs"] == 4:
            # chunk tasks: fused calls of fewer slabs than SIMDs, direct SiLU
            assert fuse and U == 1 and not p["silu_table"] and rows * -(-K // 128) <= cus * 8
            assert p["tasks"] == rows * -(-K // 128) and p["uncapped"]
        elif p["flat_slabs"] == 3:
            assert K % SLAB != 0 and (fuse or U == 2)
            assert fuse or dt == "fp32" or not (K < SLAB and SLAB % K == 0)
            assert p["tasks"] == -(-(-(-(rows * K) // SLAB)) // U)
        elif p["flat_slabs"] == 2:
            assert U == 2 and not fuse and dt != "fp32" and K < SLAB and SLAB % K == 0
            assert p["tasks"] == -(-(-(-(rows * K) // SLAB)) // 2)
        elif p["flat_slabs"]:
            assert U == 2 and not fuse and K % SLAB == 0 and spr % 2 == 1
            assert p["tasks"] == -(-(rows * spr) // 2)
        else:
            assert p["tasks"] == rows * p["tasks_per_row"]
            assert U == 1 or fuse or spr % 2 == 0
        assert p["block"] in (64, 128, 256, 1024) and p["grid"] >= 1
        if p["block"] == 128:
            assert dt == "fp32" and p["uncapped"]
        waves = p["grid"] * p["block"] // 64
        if p["uncapped"]:
            assert waves >= p["tasks"]                  # one wave per task
            assert (not fuse and U == 2) or p["flat_slabs"] == 4
        elif waves < p["tasks"]:
            assert p["grid"] % cus == 0                 # looping grids: equal blocks per CU
        if p["xcd_chunk"]:
            assert p["uncapped"] and p["grid"] >= 4 * 8 * p["xcd_chunk"]
        if p["silu_table"]:
            assert fuse and dt in ("bf16", "fp16") and p["block"] == 1024
            assert rows * spr >= cus * (16 if dt == "bf16" else 32)


def test_tuning_knobs_are_honoured():
    aq.ptgq_set_tuning(6, 0)                      # capped grid
    p = plan("bf16", 16384, 7168)
    assert p["uncapped"] == 0 and p["grid"] % CUS == 0
    aq.ptgq_set_tuning(6, -1)
    aq.ptgq_set_tuning(5, 16)                     # XCD chunk
    assert plan("bf16", 16384, 7168)["xcd_chunk"] == 16
    aq.ptgq_set_tuning(5, -1)
    aq.ptgq_set_tuning(0, 1)                      # one-slab tasks
    assert plan("bf16", 16384, 7168)["tasks_per_row"] == 14


def test_plan_validation():
    lib = aq.load_library()
    with pytest.raises(aq.PtgqError):
        plan("bf16", 16, 7168, cus=0)
    with pytest.raises(aq.PtgqError):
        plan("bf16", 16, 7100)                    # K % G != 0
    with pytest.raises(aq.PtgqError):
        plan("fp32", 16, 7168, fuse=True)         # fused fp32 is unsupported
    with pytest.raises(aq.PtgqError):
        plan("bf16", 16, 7168, q_rows=8)          # q buffer shorter than the rows
    assert lib.ptgq_plan_group(0, 0, 16, 7168, 128, 0, 0, 16, 256, None) == aq.PTGQ_EINVAL
    assert all(v == 0 for v in plan("bf16", 0, 7168).values())     # nothing launched
    assert all(v == 0 for v in plan("bf16", 0, 2048, E=4).values())
