"""Bit-exact parity of the HIP path (through the C ABI) with the CPU oracle,
on the five seeded workloads at their full sizes and on a sweep of every trait
combination at small ragged shapes."""
import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
import workloads as W
from gpu_util import compare, run_flat, run_masked, run_per_token, to_dev, DEV

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ the workloads

def test_cfg1_plain_fp32_rowmajor():
    d = W.cfg1()
    args = (d["x"], "bf16", d["M"], d["K"], d["G"], False, "e4m3", "f32", "row")
    compare("cfg1", *run_flat(*args), *oracle.ptgq(*args, eps=d["eps"]))


@pytest.mark.parametrize("M", W.CFG2_M)
def test_cfg2_deepseek_shape_ue8m0_colmajor(M):
    d = W.cfg2(M)
    args = (d["x"], "bf16", M, d["K"], 128, False, "e4m3", "ue8m0", "col")
    compare(f"cfg2 M={M}", *run_flat(*args), *oracle.ptgq(*args, eps=d["eps"]))


@pytest.mark.parametrize("M", W.CFG3_M)
def test_cfg3_fused_silu_mul(M):
    d = W.cfg3(M)
    args = (d["x"], "bf16", M, d["K"], 128, True, "e4m3", "ue8m0", "col")
    compare(f"cfg3 M={M}", *run_flat(*args), *oracle.ptgq(*args, eps=d["eps"]))


@pytest.mark.parametrize("expected_m", [0, 1, 64, 384])
def test_cfg4_masked_moe(expected_m):
    d = W.cfg4()
    E, T, K, mm = d["E"], d["T"], d["K"], d["masked_m"]
    gq, gs = run_masked(d["x"], "bf16", E, T, K, 128, True, mm, expected_m, "e4m3", "ue8m0", "col")
    sb = aq.ptgq_scale_bytes(T, K, 128, "ue8m0", "col")
    rq, rs = oracle.ptgq_masked(d["x"], "bf16", E, T, K, 128, True, mm, "e4m3", "ue8m0", "col",
                                q_init=np.full((E, T, K), 0x7F, np.uint8),
                                s_init=np.full(E * sb, 0xFF, np.uint8))
    compare(f"cfg4 expected_m={expected_m} live={int(mm.sum())}", gq, gs, rq, rs)


@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_cfg5a_fp16_int8_group_sweep(G):
    d = W.cfg5()
    args = (d["x"], "fp16", d["M"], d["K"], G, False, "int8", "f32", "row")
    compare(f"cfg5a G={G}", *run_flat(*args), *oracle.ptgq(*args, eps=d["eps"]))


def test_cfg5b_per_token_fp8():
    d = W.cfg5()
    gq, gs = run_per_token(d["x"], "fp16", d["M"], d["K"], extra_rows=4)
    rq, rs = oracle.ptq_fp8(d["x"], "fp16", d["M"], d["K"])
    compare("cfg5b", gq, gs, rq, rs)


@pytest.mark.parametrize("out_dtype", ["int8", "e4m3"])
@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_cfg5c_exactness_family(G, out_dtype):
    d = W.cfg5c()
    M, K = d["M"], d["K"]
    args = (d["x"], "fp16", M, K, G, False, out_dtype, "ue8m0", "row")
    gq, gs = run_flat(*args)
    compare(f"cfg5c G={G} {out_dtype}", gq, gs, *oracle.ptgq(*args, eps=d["eps"]))
    # implementation-independent: dequantized codes equal the integers exactly
    scale = np.ldexp(1.0, gs.reshape(M, K // G).astype(np.int64) - 127)
    if out_dtype == "int8":
        deq = gq.view(np.int8).astype(np.float64)
    else:
        deq = torch.from_numpy(gq).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    deq = deq.reshape(M, K // G, G) * scale[:, :, None]
    assert np.array_equal(deq.reshape(M, K), d["x"].view(np.float16).astype(np.float64))


# ------------------------------------------------ every trait combination

SHAPES = [(1, 128), (3, 640), (5, 2048 + 128), (37, 512), (6, 7168)]


@pytest.mark.parametrize("fuse", [False, True])
@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
@pytest.mark.parametrize("out_dtype", ["e4m3", "int8"])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_trait_sweep(G, in_dtype, out_dtype, fmt, layout, fuse):
    for i, (M, K) in enumerate(SHAPES):
        if K % G:
            continue
        shape = (M, 2 * K if fuse else K)
        seed = 100 * G + 10 * i + fuse
        x = W.normal_bf16(seed, shape, factor_cols=[1, K - 1], factor=37.0) \
            if in_dtype == "bf16" else W.normal_fp16(seed, shape)
        args = (x, in_dtype, M, K, G, fuse, out_dtype, fmt, layout)
        compare(f"sweep G={G} {in_dtype} {out_dtype} {fmt} {layout} fuse={fuse} M={M} K={K}",
                *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
@pytest.mark.parametrize("fuse", [False, True])
def test_masked_sweep(fuse, fmt, layout):
    d = W.cfg4(seed=4200 + fuse, E=5, T=45, K=640)
    E, T, K = d["E"], d["T"], d["K"]
    mm = d["masked_m"].copy()
    mm[2], mm[3] = -7, T + 100
    x = d["x"] if fuse else np.ascontiguousarray(d["x"][:, :, :K])
    gq, gs = run_masked(x, "bf16", E, T, K, 64, fuse, mm, 16, "int8", fmt, layout)
    sb = aq.ptgq_scale_bytes(T, K, 64, fmt, layout)
    rq, rs = oracle.ptgq_masked(x, "bf16", E, T, K, 64, fuse, mm, "int8", fmt, layout,
                                q_init=np.full((E, T, K), 0x7F, np.uint8),
                                s_init=np.full(E * sb, 0xFF, np.uint8))
    compare(f"masked fuse={fuse} {fmt} {layout} mm={list(mm)}", gq, gs, rq, rs)


@pytest.mark.parametrize("dist", ["one_expert", "alternating", "many_experts", "single",
                                  "all_empty", "all_full", "e64", "e65"])
def test_masked_balanced_schedule(dist):
    """The balanced masked schedule under skewed live-row distributions, more
    than 64 experts (several search windows), the 64 / 65 expert boundary
    between the prefix sum held in registers and the one in LDS, and
    degenerate cases."""
    rng = np.random.default_rng(sum(map(ord, dist)))
    if dist in ("e64", "e65"):
        E, T, K = int(dist[1:]), 21, 1024
        mm = rng.integers(-3, T + 4, E).astype(np.int32)
        mm[E - 1] = T
    elif dist == "one_expert":
        E, T, K, mm = 16, 200, 1024, np.zeros(16, np.int32)
        mm[11] = 200
    elif dist == "alternating":
        E, T, K = 12, 96, 2048
        mm = np.array([0, 96] * 6, np.int32)
    elif dist == "many_experts":
        E, T, K = 150, 9, 512
        mm = rng.integers(-2, 12, E).astype(np.int32)
    elif dist == "single":
        E, T, K, mm = 1, 77, 1536, np.array([77], np.int32)
    elif dist == "all_empty":
        E, T, K, mm = 8, 40, 512, np.zeros(8, np.int32)
    else:
        E, T, K = 8, 33, 640
        mm = np.full(8, 33, np.int32)
    x = W.normal_bf16(E * 1000 + T, (E, T, 2 * K))
    for fuse in (False, True):
        xi = x if fuse else np.ascontiguousarray(x[:, :, :K])
        for exp_m in (0, 3):
            gq, gs = run_masked(xi, "bf16", E, T, K, 128, fuse, mm, exp_m, "e4m3", "ue8m0", "col")
            sb = aq.ptgq_scale_bytes(T, K, 128, "ue8m0", "col")
            rq, rs = oracle.ptgq_masked(xi, "bf16", E, T, K, 128, fuse, mm, "e4m3", "ue8m0", "col",
                                        q_init=np.full((E, T, K), 0x7F, np.uint8),
                                        s_init=np.full(E * sb, 0xFF, np.uint8))
            compare(f"masked {dist} fuse={fuse} expected_m={exp_m}", gq, gs, rq, rs)


# --------------------------------------------------------------- per-token

@pytest.mark.parametrize("mode", [-1, 0, 1, 2, 3])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp16", "fp32"])
def test_per_token_modes(in_dtype, mode):
    try:
        aq.ptgq_set_tuning(3, mode)
        for M, K in [(39, 1076), (39, 1368), (300, 4096), (7, 4), (2, 8192 * 3), (64, 3584)]:
            seed = M * 7 + K
            if in_dtype == "bf16":
                x = W.normal_bf16(seed, (M, K))
            elif in_dtype == "fp16":
                x = W.normal_fp16(seed, (M, K))
            else:
                x = W.normal_f32(seed, (M, K))
            x[M // 2] = 0          # a zero row: scale 0, codes 0
            gq, gs = run_per_token(x, in_dtype, M, K)
            rq, rs = oracle.ptq_fp8(x, in_dtype, M, K)
            compare(f"per-token {in_dtype} mode={mode} M={M} K={K}", gq, gs, rq, rs)
    finally:
        aq.ptgq_set_tuning(3, -1)


@pytest.mark.parametrize("waves", [1, 2, 3, 5, 7, 8])
def test_per_token_block_waves_per_row(waves):
    """One block per row with every block size the override allows (rows
    whose vector count does not divide the block, idle lanes and waves, the
    XCD-chunked row order at M >= 1024)."""
    try:
        aq.ptgq_set_tuning(3, 1)
        aq.ptgq_set_tuning(1, waves)
        for in_dtype, M, K in [("fp16", 1100, 3584), ("bf16", 37, 7168), ("fp32", 64, 1076),
                               ("bf16", 1030, 2048), ("fp32", 9, 7168)]:
            gen = {"bf16": W.normal_bf16, "fp16": W.normal_fp16, "fp32": W.normal_f32}[in_dtype]
            x = gen(M * 13 + K + waves, (M, K))
            x[M // 3] = 0
            gq, gs = run_per_token(x, in_dtype, M, K)
            compare(f"per-token block waves={waves} {in_dtype} M={M} K={K}", gq, gs,
                    *oracle.ptq_fp8(x, in_dtype, M, K))
    finally:
        aq.ptgq_set_tuning(1, -1)
        aq.ptgq_set_tuning(3, -1)


@pytest.mark.parametrize("K", [1368, 3584, 1076, 4096])
def test_per_token_many_rows_wave_dispatch(K):
    """Enough rows for the persistent wave loop (several rows per wave, an odd
    count for some waves), each row length class."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M = cus * 16 + 37
    x = W.normal_bf16(31 + K, (M, K))
    x[5] = 0
    gq, gs = run_per_token(x, "bf16", M, K)
    compare(f"per-token wave-dispatch M={M} K={K}", gq, gs, *oracle.ptq_fp8(x, "bf16", M, K))


# ---------------------------------------------------------------- edges

def test_zero_rows_touch_nothing():
    q = torch.full((4, 256), 0x5A, dtype=torch.uint8, device=DEV)
    s = torch.full((64,), 0x5A, dtype=torch.uint8, device=DEV)
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device=DEV)
    aq.ptgq_quant(x, "bf16", 0, 256, 128, False, "e4m3", "ue8m0", "col", 1e-10, q, s)
    aq.ptgq_quant_masked(x, "bf16", 0, 4, 256, 128, False, s, 0, "e4m3", "ue8m0", "col", 1e-10, q, s)
    aq.ptq_quant_fp8(x, "bf16", 0, 256, q, s)
    torch.cuda.synchronize()
    assert bool((q == 0x5A).all()) and bool((s == 0x5A).all())


@pytest.mark.parametrize("eps", [0.0, 1e-10, 1e-3])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_special_values(eps, fmt):
    """All-zero groups (eps floor; eps = 0 gives scale 0 / byte 0 and +-0
    codes), signed zeros, bf16 subnormals, values near the bf16 maximum."""
    M, K = 8, 1024
    x = W.normal_bf16(55, (M, K))
    x[0] = 0
    x[1, :128] = 0x8000                      # -0
    # bf16 subnormals (with eps = 0 and fp32 scales the multiplier overflows:
    # zeros keep their sign, the rest saturate)
    x[2] = (np.arange(K) % 128).astype(np.uint16)
    x[3, :256] = 0x7F7F                      # largest finite bf16
    x[3, 256:512] = 0xFF7F
    x[4] = W.to_bf16_bits(np.full(K, 448.0))
    x[5] = W.to_bf16_bits(np.linspace(-450.0, 450.0, K))
    for out_dtype in ("e4m3", "int8"):
        for layout in ("row", "col"):
            args = (x, "bf16", M, K, 128, False, out_dtype, fmt, layout)
            compare(f"special eps={eps} {fmt} {out_dtype} {layout}", *run_flat(*args, eps=eps),
                    *oracle.ptgq(*args, eps=eps))


def reset_knobs():
    for k in range(8):
        aq.ptgq_set_tuning(k, -1)


@pytest.mark.parametrize("fuse", [False, True])
def test_tuning_knobs_never_change_results(fuse):
    M, K = 300, 7168 if not fuse else 3584
    x = W.normal_bf16(808 + fuse, (M, 2 * K if fuse else K), factor_cols=[7, 99], factor=30.0)
    args = (x, "bf16", M, K, 128, fuse, "e4m3", "ue8m0", "col")
    ref = oracle.ptgq(*args)
    try:
        # knob 5 (XCD chunk): 1, 3 and 64 leave a ragged last span of blocks
        for knob, values in ((0, [1, 2, 4]), (1, [1, 2, 4]), (2, [1, 2, 64]), (4, [0, 1]),
                             (5, [0, 1, 3, 64]), (6, [0, 1]), (7, [0, 1])):
            for v in values:
                aq.ptgq_set_tuning(knob, v)
                compare(f"fuse={fuse} knob {knob}={v}", *run_flat(*args), *ref)
                aq.ptgq_set_tuning(knob, -1)
    finally:
        reset_knobs()


@pytest.mark.parametrize("table", [0, 1])
@pytest.mark.parametrize("U", [1, 2])
def test_fused_paths_ragged(U, table):
    """Both SiLU paths and both fused task sizes, rows whose last task runs past
    the row (K = 640: 2 slabs, second one ragged), masked and flat."""
    try:
        aq.ptgq_set_tuning(0, U)
        aq.ptgq_set_tuning(4, table)
        for M, K in ((7, 640), (33, 1664), (2, 4096)):
            x = W.normal_bf16(M * 10 + K, (M, 2 * K), factor_cols=[0, K + 3], factor=9.0)
            for fmt, lay in (("ue8m0", "col"), ("f32", "row")):
                args = (x, "bf16", M, K, 128, True, "e4m3", fmt, lay)
                compare(f"fused U={U} table={table} M={M} K={K} {fmt} {lay}", *run_flat(*args),
                        *oracle.ptgq(*args))
        d = W.cfg4(seed=4300, E=6, T=50, K=640)
        gq, gs = run_masked(d["x"], "bf16", 6, 50, 640, 128, True, d["masked_m"], 0, "e4m3",
                            "ue8m0", "col")
        sb = aq.ptgq_scale_bytes(50, 640, 128, "ue8m0", "col")
        rq, rs = oracle.ptgq_masked(d["x"], "bf16", 6, 50, 640, 128, True, d["masked_m"], "e4m3",
                                    "ue8m0", "col", q_init=np.full((6, 50, 640), 0x7F, np.uint8),
                                    s_init=np.full(6 * sb, 0xFF, np.uint8))
        compare(f"masked fused U={U} table={table}", gq, gs, rq, rs)
    finally:
        reset_knobs()


@pytest.mark.parametrize("U", [1, 2, 4])
def test_plain_task_sizes_ragged(U):
    try:
        aq.ptgq_set_tuning(0, U)
        for M, K, G in ((5, 7168, 128), (9, 3584, 64), (3, 640, 32), (4, 128, 16), (17, 2560, 128)):
            x = W.normal_fp16(M + K + G, (M, K))
            for out_dtype, fmt, lay in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row"),
                                        ("e4m3", "f32", "col"), ("int8", "ue8m0", "row")):
                args = (x, "fp16", M, K, G, False, out_dtype, fmt, lay)
                compare(f"U={U} M={M} K={K} G={G} {out_dtype} {fmt} {lay}", *run_flat(*args),
                        *oracle.ptgq(*args))
    finally:
        reset_knobs()


def test_runs_on_a_side_stream():
    d = W.cfg2(16)
    args = (d["x"], "bf16", 16, d["K"], 128, False, "e4m3", "ue8m0", "col")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        got = run_flat(*args, stream=st)
    compare("side stream", *got, *oracle.ptgq(*args))
