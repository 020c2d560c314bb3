"""GPU parity for the contract points beside the workloads: the overflowed
multiplier corner (zeros keep their sign, other values saturate), the
per-token host contract on padded output rows, flat-slab tasks across row
ends, multi-row slabs for rows shorter than a slab, slabs of the flattened
tensor for other row lengths, the first call of a process made inside a graph capture, and the
no-arithmetic stream reference.  Every output sits between guard bands."""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
import workloads as W
from gpu_util import DEV, Guarded, compare, run_flat, run_masked, run_per_token, to_dev

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def tiny_rows(seed, M, K, in_dtype):
    """Rows whose largest magnitude lies in [1e-38, 4e-36] (so 1 / (max / qmax)
    overflows for most of them), about a third zeros of both signs, one zero
    row and one ordinary row."""
    rng = np.random.default_rng(seed)
    amax = np.exp(rng.uniform(np.log(1e-38), np.log(4e-36), M))
    y = rng.uniform(-1.0, 1.0, (M, K)) * amax[:, None]
    y[rng.random((M, K)) < 0.25] = 0.0
    y[rng.random((M, K)) < 0.1] = -0.0
    y[1] = 0.0
    y[2] = rng.normal(size=K)
    return y.astype(np.float32) if in_dtype == "fp32" else W.to_bf16_bits(y)


@pytest.mark.parametrize("mode", [-1, 0, 1, 2, 3])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp32"])
def test_overflowed_multiplier_per_token(in_dtype, mode):
    try:
        aq.ptgq_set_tuning(3, mode)
        for M, K in ((40, 1076), (9, 3584), (5, 8192 * 3)):
            x = tiny_rows(M + K, M, K, in_dtype)
            compare(f"tiny per-token {in_dtype} mode={mode} M={M} K={K}",
                    *run_per_token(x, in_dtype, M, K), *oracle.ptq_fp8(x, in_dtype, M, K))
    finally:
        aq.ptgq_set_tuning(3, -1)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("out_dtype", ["e4m3", "int8"])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp32"])
def test_overflowed_multiplier_group_fp32_scales(in_dtype, out_dtype, layout):
    for M, K, G in ((12, 512, 64), (33, 7168, 128), (7, 640, 16)):
        x = tiny_rows(M * K + G, M, K, in_dtype)
        args = (x, in_dtype, M, K, G, False, out_dtype, "f32", layout)
        compare(f"tiny group {in_dtype} {out_dtype} {layout} M={M} K={K} G={G}",
                *run_flat(*args, eps=0.0), *oracle.ptgq(*args, eps=0.0))


def test_overflowed_multiplier_fused_and_masked():
    """Fused silu(g)*u products that are zero or tiny, eps = 0, fp32 scales:
    gates of 0 give silu 0; tiny ups give tiny products."""
    M, K = 6, 1024
    rng = np.random.default_rng(88)
    g = rng.normal(size=(M, K))
    u = rng.normal(size=(M, K)) * 1e-37
    g[:, ::3] = 0.0
    x = W.to_bf16_bits(np.concatenate([g, u], axis=1))
    for fmt in ("f32", "ue8m0"):
        args = (x, "bf16", M, K, 128, True, "e4m3", fmt, "row")
        compare(f"tiny fused {fmt}", *run_flat(*args, eps=0.0), *oracle.ptgq(*args, eps=0.0))


def test_overflowed_multiplier_requant():
    E, T, K = 3, 20, 1152
    rng = np.random.default_rng(89)
    x = rng.integers(0, 256, (E, T, K)).astype(np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x00
    x[:, :, :40] = 0x80
    s = rng.uniform(0.5, 2.0, E * T * (K // 128)).astype(np.float32)
    strides = (T * (K // 128), 1, T)
    mm = np.array([20, 0, 7], np.int32)
    out = Guarded((E, T, K), torch.uint8, 0x2C)
    aq.ptgq_requant_fp8(to_dev(x), E, T, K, 128, to_dev(s), strides, to_dev(mm), 0,
                        torch.tensor([1e-39], dtype=torch.float32, device=DEV), out.t)
    torch.cuda.synchronize()
    out.check("requant out")
    want = oracle.requant_fp8(x, E, T, K, 128, s, strides, mm, np.float32(1e-39),
                              out_init=np.full((E, T, K), 0x2C, np.uint8))
    compare("requant, overflowed 1/output_scale", out.host(), np.zeros(0, np.uint8), want,
            np.zeros(0, np.uint8))


@pytest.mark.parametrize("mode", [-1, 0, 1, 2, 3])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp16", "fp32"])
def test_per_token_writes_only_the_first_M_rows(in_dtype, mode):
    """The host contract of the sglang #34257 page: output buffers may hold
    more rows than M; rows past M keep their contents."""
    try:
        aq.ptgq_set_tuning(3, mode)
        for M, K, extra in ((39, 1076, 5), (64, 3584, 1), (3, 8192 * 3, 4)):
            seed = 3 * M + K
            x = {"bf16": W.normal_bf16, "fp16": W.normal_fp16, "fp32": W.normal_f32}[in_dtype](
                seed, (M, K))
            compare(f"per-token padded outputs {in_dtype} mode={mode} M={M}+{extra} K={K}",
                    *run_per_token(x, in_dtype, M, K, extra_rows=extra),
                    *oracle.ptq_fp8(x, in_dtype, M, K))
    finally:
        aq.ptgq_set_tuning(3, -1)


# ------------------------------------------------------------ flat-slab tasks

@pytest.mark.parametrize("flat", [1, 0])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp16", "fp32"])
def test_flat_slab_tasks_across_row_ends(in_dtype, flat):
    """Rows of 1, 3, 7 and 14 slabs with row counts that leave a last task of
    one slab, every scale format and layout, with flat-slab tasks forced on
    (whatever the slab count) and off (row tasks); large enough that two-slab
    tasks are chosen."""
    try:
        aq.ptgq_set_tuning(7, flat)
        for M, K in ((16385, 512), (5463, 1536), (2341, 3584), (1171, 7168)):
            seed = M + K
            x = {"bf16": W.normal_bf16, "fp16": W.normal_fp16, "fp32": W.normal_f32}[in_dtype](
                seed, (M, K))
            p = aq.ptgq_plan_group(in_dtype, 0, M, K, 128, False, 0, M,
                                   torch.cuda.get_device_properties(0).multi_processor_count)
            assert p["flat_slabs"] == flat
            assert p["slabs_per_task"] == 2 or flat == 0   # row tasks may take one slab
            for out_dtype, fmt, layout in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row"),
                                           ("e4m3", "f32", "col"), ("int8", "ue8m0", "row")):
                G = 128 if fmt == "ue8m0" else 32
                args = (x, in_dtype, M, K, G, False, out_dtype, fmt, layout)
                compare(f"flat-slab={flat} {in_dtype} M={M} K={K} G={G} {out_dtype} {fmt} {layout}",
                        *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))
    finally:
        aq.ptgq_set_tuning(7, -1)


@pytest.mark.parametrize("K", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp16"])
def test_multi_row_slabs(in_dtype, K):
    """Rows shorter than a slab (K divides 512): each slab holds 512 / K rows,
    the last slab of the tensor is partial; every group size up to K, scale
    format and layout (column-major packed words of fewer than four groups
    included); large enough that two-slab tasks are chosen."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M = cus * 16 * 512 // K + 3                         # >= 16 slabs per CU, ragged
    x = (W.normal_bf16(M + K, (M, K), factor_cols=[K - 1], factor=40.0) if in_dtype == "bf16"
         else W.normal_fp16(M + K, (M, K)))
    x[M // 2] = 0                                       # a zero row: scale from eps
    for G in [g for g in (16, 32, 64, 128) if g <= K]:
        p = aq.ptgq_plan_group(in_dtype, 0, M, K, G, False, 0, M, cus)
        assert p["flat_slabs"] == 2 and p["slabs_per_task"] == 2
        for out_dtype, fmt, layout in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row"),
                                       ("e4m3", "f32", "col"), ("int8", "ue8m0", "row")):
            args = (x, in_dtype, M, K, G, False, out_dtype, fmt, layout)
            compare(f"multi-row slabs {in_dtype} M={M} K={K} G={G} {out_dtype} {fmt} {layout}",
                    *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


@pytest.mark.parametrize("K,Gs", [(48, (16,)), (96, (16, 32)), (384, (32, 128)),
                                  (640, (64, 128)), (1152, (16, 128)), (2880, (32, 64)),
                                  (3712, (128,)), (11008, (128,))])
def test_flattened_slabs(K, Gs):
    """16-bit rows that are not whole slabs and do not divide one: slabs of
    the flattened tensor cross row ends at any column; packed column-major
    words whose groups come from two slabs, partial last words (ng % 4 != 0),
    a last slab ending inside the tensor; every scale format and layout."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M = -(-(cus * 16 * 512) // K) + 5
    for in_dtype in ("bf16", "fp16", "fp32"):
        x = {"bf16": lambda: W.normal_bf16(M + K, (M, K), factor_cols=[K - 1], factor=40.0),
             "fp16": lambda: W.normal_fp16(M + K, (M, K)),
             "fp32": lambda: W.normal_f32(M + K, (M, K))}[in_dtype]()
        x[M // 3] = 0
        for G in Gs:
            p = aq.ptgq_plan_group(in_dtype, 0, M, K, G, False, 0, M, cus)
            assert p["flat_slabs"] == 3 and p["slabs_per_task"] == 2
            for out_dtype, fmt, layout in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row"),
                                           ("e4m3", "f32", "col"), ("int8", "ue8m0", "row")):
                args = (x, in_dtype, M, K, G, False, out_dtype, fmt, layout)
                compare(f"flattened slabs {in_dtype} M={M} K={K} G={G} {out_dtype} {fmt} "
                        f"{layout}", *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


@pytest.mark.parametrize("K,G", [(48, 16), (96, 32), (256, 128), (640, 64), (1152, 128),
                                 (1408, 128), (2880, 64)])
def test_flattened_slabs_fused(K, G):
    """Fused silu(gate)*up over rows that are not whole slabs: each lane reads
    the gate and up halves of its own row; bf16 with the SiLU table (large)
    and the direct evaluation (small), fp16 (direct); a last slab ending
    inside the tensor."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        for in_dtype, M in (("bf16", -(-(cus * 16 * 512) // K) + 3), ("bf16", 37),
                            ("fp16", -(-(cus * 4 * 512) // K) + 1)):
            # a small call takes chunk tasks unless slab tasks are forced
            aq.ptgq_set_tuning(0, 1 if M == 37 else -1)
            p = aq.ptgq_plan_group(in_dtype, 0, M, K, G, True, 0, M, cus)
            assert p["flat_slabs"] == 3
            x = (W.normal_bf16(M * 3 + K, (M, 2 * K)) if in_dtype == "bf16"
                 else W.normal_fp16(M * 3 + K, (M, 2 * K)))
            for out_dtype, fmt, layout in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row")):
                args = (x, in_dtype, M, K, G, True, out_dtype, fmt, layout)
                compare(f"flattened slabs fused {in_dtype} M={M} K={K} G={G} "
                        f"table={p['silu_table']} {out_dtype} {fmt} {layout}", *run_flat(*args),
                        *oracle.ptgq(*args, eps=1e-10))
    finally:
        aq.ptgq_set_tuning(0, -1)


@pytest.mark.parametrize("K,Gs", [(4096, (128, 64)), (640, (128, 32)), (1408, (64, 16)),
                                  (4160, (64, 32)), (48, (16,)), (192, (64, 32))])
def test_chunk_tasks_of_small_fused_calls(K, Gs):
    """Fused calls of fewer slabs than SIMDs run one wave per 128 output
    elements of a row, two per lane: groups of 8 to 64 lanes (the whole wave
    at G = 128), a short last chunk when 128 does not divide K, packed
    column-major words from several waves, every format and layout."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for in_dtype in ("bf16", "fp16"):
        for M in (1, 2, 7, 37):
            x = (W.normal_bf16(M * 7 + K, (M, 2 * K), factor_cols=[1, K + 2], factor=30.0)
                 if in_dtype == "bf16" else W.normal_fp16(M * 7 + K, (M, 2 * K)))
            x[M // 2, : min(K, 64)] = 0
            for G in Gs:
                p = aq.ptgq_plan_group(in_dtype, 0, M, K, G, True, 0, M, cus)
                assert p["flat_slabs"] == 4 and p["tasks"] == M * -(-K // 128)
                for out_dtype, fmt, layout in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row"),
                                               ("e4m3", "f32", "col"), ("int8", "ue8m0", "row")):
                    args = (x, in_dtype, M, K, G, True, out_dtype, fmt, layout)
                    compare(f"chunk tasks {in_dtype} M={M} K={K} G={G} {out_dtype} {fmt} "
                            f"{layout}", *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


@pytest.mark.parametrize("E,T,K,G", [(32, 384, 2048, 128), (5, 40, 640, 32), (70, 12, 1408, 64),
                                     (3, 9, 48, 16)])
def test_masked_chunk_tasks(E, T, K, G):
    """Decode-sized masked fused calls run chunk tasks over the live rows,
    with the prefix sum in registers (E <= 64) or in LDS (E = 70); live rows
    beyond the expected count make the waves loop; rows past masked_m keep
    their sentinels."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(E * 100 + K)
    exp_m = 1
    assert aq.ptgq_plan_group("bf16", E, T, K, G, True, exp_m, T, cus)["flat_slabs"] == 4
    for mm in (np.ones(E, np.int32), rng.integers(-2, 5, E).astype(np.int32),
               rng.integers(0, T + 3, E).astype(np.int32)):
        for in_dtype in ("bf16", "fp16"):
            for out_dtype, fmt, layout in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row")):
                masked_case(E, T, K, G, True, in_dtype, mm, exp_m, int(mm.sum()) + K,
                            out_dtype, fmt, layout)


def fp16_gates_with_large_values(seed, shape, K):
    """N(0,1) fp16 [gate | up] rows whose gate columns 5 and K - 3 are scaled
    x 40 (gates of magnitude 8 and more, outside the fp16 lookup table)."""
    x = W.normal_fp16(seed, shape).view(np.float16).copy()
    x[..., 5] *= np.float16(40)
    x[..., K - 3] *= np.float16(40)
    return x.view(np.uint16)


@pytest.mark.parametrize("K", [4096, 1408])
def test_fp16_silu_table_flat(K):
    """Large fused fp16 calls read the 144 KiB fp16 SiLU table (row tasks at
    K = 4096, flattened slabs at K = 1408); gates of magnitude 8 and more fall
    back to the direct evaluation."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M = -(-(cus * 32 * 512) // K) + 3
    p = aq.ptgq_plan_group("fp16", 0, M, K, 128, True, 0, M, cus)
    assert p["silu_table"] == 1 and p["block"] == 1024
    x = fp16_gates_with_large_values(M + K, (M, 2 * K), K)
    for out_dtype, fmt, layout in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row")):
        args = (x, "fp16", M, K, 128, True, out_dtype, fmt, layout)
        compare(f"fp16 table M={M} K={K} {out_dtype} {fmt} {layout}", *run_flat(*args),
                *oracle.ptgq(*args, eps=1e-10))


@pytest.mark.parametrize("E,K", [(32, 2048), (32, 1408), (100, 2048), (100, 1408)])
def test_fp16_silu_table_masked(E, K):
    """Masked fused fp16 calls with the fp16 table: row tasks and flattened
    slabs, the prefix sum in registers (32 experts) or beside the table in
    LDS (100 experts)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    T = 384 if E == 32 else 64
    exp_m = 128 if E == 32 else 48                # at least 32 slabs per CU
    assert aq.ptgq_plan_group("fp16", E, T, K, 128, True, exp_m, T, cus)["silu_table"] == 1
    rng = np.random.default_rng(K)
    mm = rng.integers(0, T + 1, E).astype(np.int32)
    mm[0], mm[1] = 0, T
    x = fp16_gates_with_large_values(K + 1, (E, T, 2 * K), K)
    gq, gs = run_masked(x, "fp16", E, T, K, 128, True, mm, exp_m, "e4m3", "ue8m0", "col")
    sb = aq.ptgq_scale_bytes(T, K, 128, "ue8m0", "col")
    rq, rs = oracle.ptgq_masked(x, "fp16", E, T, K, 128, True, mm, "e4m3", "ue8m0", "col",
                                q_init=np.full((E, T, K), 0x7F, np.uint8),
                                s_init=np.full(E * sb, 0xFF, np.uint8))
    compare(f"fp16 table masked E={E} K={K}", gq, gs, rq, rs)


def test_chunk_tasks_forced_and_padded():
    """Chunk tasks forced at a size that would take the SiLU table, and with
    a padded code buffer: rows past M and the column-major pad slots are zero."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        aq.ptgq_set_tuning(7, 2)
        aq.ptgq_set_tuning(4, 0)
        M, K, G = 1203, 4096, 128
        assert aq.ptgq_plan_group("bf16", 0, M, K, G, True, 0, M, cus)["flat_slabs"] == 4
        x = W.normal_bf16(1203, (M, 2 * K))
        args = (x, "bf16", M, K, G, True, "e4m3", "ue8m0", "col")
        compare("chunk tasks forced", *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))
    finally:
        aq.ptgq_set_tuning(7, -1)
        aq.ptgq_set_tuning(4, -1)
    M, K, G = 5, 640, 128                          # 5 groups: a partial packed word
    q_rows = M + 6
    x = W.normal_bf16(55, (M, 2 * K))
    assert aq.ptgq_plan_group("bf16", 0, M, K, G, True, 0, q_rows, cus)["flat_slabs"] == 4
    q = Guarded((q_rows, K), torch.uint8, 0xCD)
    sb = aq.ptgq_scale_bytes(M, K, G, "ue8m0", "col")
    s = Guarded((sb,), torch.uint8, 0xCD)
    aq.ptgq_quant_padded(to_dev(x), "bf16", M, K, G, True, "e4m3", "ue8m0", "col", 1e-10, q.t,
                         q_rows, s.t)
    torch.cuda.synchronize()
    q.check("padded q")
    s.check("padded s")
    qh = q.host()
    rq, rs = oracle.ptgq(x, "bf16", M, K, G, True, "e4m3", "ue8m0", "col", eps=1e-10)
    compare("chunk tasks padded", qh[:M], s.host(), rq, rs)
    assert np.all(qh[M:] == 0)


@pytest.mark.parametrize("K", [16, 64, 256])
def test_flattened_slabs_fp32_short_rows(K):
    """fp32 rows shorter than a slab take slabs of the flattened tensor."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M = cus * 16 * 512 // K + 3
    x = W.normal_f32(M + 3 * K, (M, K))
    x[M // 2] = 0
    for G in [g for g in (16, 32, 64, 128) if g <= K]:
        assert aq.ptgq_plan_group("fp32", 0, M, K, G, False, 0, M, cus)["flat_slabs"] == 3
        for out_dtype, fmt, layout in (("e4m3", "ue8m0", "col"), ("int8", "f32", "row"),
                                       ("e4m3", "f32", "col"), ("int8", "ue8m0", "row")):
            args = (x, "fp32", M, K, G, False, out_dtype, fmt, layout)
            compare(f"flattened slabs fp32 M={M} K={K} G={G} {out_dtype} {fmt} {layout}",
                    *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


def test_flattened_slabs_padded_codes():
    """ptgq_quant_padded with slabs of the flattened tensor: rows past M are
    zero, the column-major pad slots and partial-word bytes too."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K, G = 640, 128                                     # 5 groups: partial words
    M = -(-(cus * 16 * 512) // K) + 2
    q_rows = M + 9
    x = W.normal_bf16(78, (M, K))
    assert aq.ptgq_plan_group("bf16", 0, M, K, G, False, 0, q_rows, cus)["flat_slabs"] == 3
    q = Guarded((q_rows, K), torch.uint8, 0xCD)
    sb = aq.ptgq_scale_bytes(M, K, G, "ue8m0", "col")
    s = Guarded((sb,), torch.uint8, 0xCD)
    aq.ptgq_quant_padded(to_dev(x), "bf16", M, K, G, False, "e4m3", "ue8m0", "col", 1e-10, q.t,
                         q_rows, s.t)
    torch.cuda.synchronize()
    q.check("padded q")
    s.check("padded s")
    qh = q.host()
    rq, rs = oracle.ptgq(x, "bf16", M, K, G, False, "e4m3", "ue8m0", "col", eps=1e-10)
    compare("flattened slabs padded", qh[:M], s.host(), rq, rs)
    assert np.all(qh[M:] == 0)


def masked_case(E, T, K, G, fuse, in_dtype, mm, exp_m, seed, out_dtype, fmt, layout):
    gen = {"bf16": W.normal_bf16, "fp16": W.normal_fp16, "fp32": W.normal_f32}[in_dtype]
    x = gen(seed, (E, T, 2 * K if fuse else K))
    gq, gs = run_masked(x, in_dtype, E, T, K, G, fuse, mm, exp_m, out_dtype, fmt, layout)
    sb = aq.ptgq_scale_bytes(T, K, G, fmt, layout)
    rq, rs = oracle.ptgq_masked(x, in_dtype, E, T, K, G, fuse, mm, out_dtype, fmt, layout,
                                q_init=np.full((E, T, K), 0x7F, np.uint8),
                                s_init=np.full(E * sb, 0xFF, np.uint8))
    compare(f"masked flattened slabs E={E} T={T} K={K} G={G} {in_dtype} fuse={fuse} "
            f"expected_m={exp_m} {out_dtype} {fmt} {layout} masked_m={list(mm)}", gq, gs, rq, rs)


@pytest.mark.parametrize("E,T,K,G,in_dtype", [
    (5, 45, 640, 64, "bf16"),       # one-slab tasks, partial packed words
    (65, 30, 1408, 128, "bf16"),    # prefix sums in LDS
    (7, 33, 384, 128, "fp16"),      # rows shorter than a slab, not dividing it
    (6, 50, 128, 32, "bf16"),       # rows dividing the slab
    (4, 21, 1152, 128, "fp32"),
])
def test_masked_flattened_slabs(E, T, K, G, in_dtype):
    """Masked layout, rows that are not whole slabs: each expert's live rows
    are one flattened sequence of slabs whose tasks stop at the expert's end;
    fused lanes read their own rows' gate and up halves.  One- and two-slab
    tasks, the SiLU table and the direct evaluation, masked_m below 0, 0,
    tokens_pad and past it; rows past masked_m keep their sentinels."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(E * 1000 + K)
    mm = rng.integers(-3, T + 4, E).astype(np.int32)
    mm[0], mm[-1] = T, 0
    fuses = (False,) if in_dtype == "fp32" else (False, True)
    try:
        for fuse in fuses:
            for U, table in ((1, -1), (2, 0), (1, 1)):
                if table == 1 and not (fuse and in_dtype == "bf16"):
                    continue
                aq.ptgq_set_tuning(0, U)
                aq.ptgq_set_tuning(4, table)
                p = aq.ptgq_plan_group(in_dtype, E, T, K, G, fuse, 0, T, cus)
                assert p["flat_slabs"] == 3 and p["slabs_per_task"] == U
                masked_case(E, T, K, G, fuse, in_dtype, mm, 0, 50 + U + table + fuse,
                            "e4m3", "ue8m0", "col")
                masked_case(E, T, K, G, fuse, in_dtype, mm, 7, 60 + U + table + fuse,
                            "int8", "f32", "row")
    finally:
        aq.ptgq_set_tuning(0, -1)
        aq.ptgq_set_tuning(4, -1)


@pytest.mark.parametrize("fuse", [False, True])
def test_masked_flattened_slabs_large(fuse):
    """Masked flattened slabs at a size where the chooser itself takes
    two-slab tasks (unfused) or the SiLU table (fused): 32 experts of up to
    384 rows of 1408."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    E, T, K = 32, 384, 1408
    rng = np.random.default_rng(1408)
    mm = rng.integers(0, T + 1, E).astype(np.int32)
    mm[3], mm[9] = T, 0
    p = aq.ptgq_plan_group("bf16", E, T, K, 128, fuse, int(mm.mean()), T, cus)
    assert p["flat_slabs"] == 3
    assert (p["silu_table"], p["slabs_per_task"]) == ((1, 1) if fuse else (0, 2))
    masked_case(E, T, K, 128, fuse, "bf16", mm, int(mm.mean()), 1408 + fuse, "e4m3", "ue8m0",
                "col")


@pytest.mark.parametrize("K", [1536, 2048])
def test_masked_flattened_slabs_whole_slab_rows(K):
    """Masked rows of whole slabs: unfused rows of an odd number of slabs take
    flattened slabs by themselves, the others when the slab-sequence knob
    forces them."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    E, T = 9, 40
    mm = np.array([40, 0, 13, 41, -1, 7, 40, 1, 39], np.int32)
    try:
        for knob in (-1, 1):
            aq.ptgq_set_tuning(7, knob)
            for fuse in (False, True):
                natural = not fuse and (K // 512) % 2 == 1
                want = 3 if natural or knob == 1 else 0
                assert aq.ptgq_plan_group("bf16", E, T, K, 128, fuse, 0, T, cus)[
                    "flat_slabs"] == want
                if want == 3:
                    masked_case(E, T, K, 128, fuse, "bf16", mm, 0, K + fuse, "e4m3", "ue8m0",
                                "col")
    finally:
        aq.ptgq_set_tuning(7, -1)


def test_multi_row_slabs_padded_codes():
    """ptgq_quant_padded with multi-row slabs: rows past M are zero, the
    column-major pad slots too."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K, G = 128, 32
    M = cus * 16 * 4 + 1
    q_rows = M + 7
    x = W.normal_bf16(77, (M, K))
    assert aq.ptgq_plan_group("bf16", 0, M, K, G, False, 0, q_rows, cus)["flat_slabs"] == 2
    q = Guarded((q_rows, K), torch.uint8, 0xCD)
    sb = aq.ptgq_scale_bytes(M, K, G, "ue8m0", "col")
    s = Guarded((sb,), torch.uint8, 0xCD)
    aq.ptgq_quant_padded(to_dev(x), "bf16", M, K, G, False, "e4m3", "ue8m0", "col", 1e-10, q.t,
                         q_rows, s.t)
    torch.cuda.synchronize()
    q.check("padded q")
    s.check("padded s")
    qh = q.host()
    rq, rs = oracle.ptgq(x, "bf16", M, K, G, False, "e4m3", "ue8m0", "col", eps=1e-10)
    compare("multi-row slabs padded", qh[:M], s.host(), rq, rs)
    assert np.all(qh[M:] == 0)


def test_flat_slab_padded_codes():
    """ptgq_quant_padded with flat-slab tasks: rows past M are zero."""
    M, K, q_rows = 3001, 3584, 3008
    x = W.normal_fp16(3001, (M, K))
    q = Guarded((q_rows, K), torch.uint8, 0xA7)
    sb = aq.ptgq_scale_bytes(M, K, 64, "f32", "row")
    s = Guarded((sb,), torch.uint8, 0xA7)
    aq.ptgq_quant_padded(to_dev(x), "fp16", M, K, 64, False, "int8", "f32", "row", 1e-10, q.t,
                         q_rows, s.t)
    torch.cuda.synchronize()
    q.check("padded q")
    s.check("padded s")
    qh = q.host()
    rq, rs = oracle.ptgq(x, "fp16", M, K, 64, False, "int8", "f32", "row", eps=1e-10)
    compare("flat-slab padded", qh[:M], s.host(), rq, rs)
    assert np.all(qh[M:] == 0)


# ------------------------------------------- first call inside a graph capture

CAPTURE_CHILD = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    import numpy as np
    import torch
    import activation_quantization_amd as aq
    import oracle
    import workloads as W

    dev = "cuda"
    M, K = 2048, 4096                    # fused bf16, large enough for the SiLU table
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert aq.ptgq_plan_group("bf16", 0, M, K, 128, True, 0, M, cus)["silu_table"] == 1
    xh = W.normal_bf16(2048, (M, 2 * K))
    x = torch.from_numpy(xh.view(np.int16)).to(dev)
    ph = W.normal_bf16(2049, (64, 7168))
    p = torch.from_numpy(ph.view(np.int16)).to(dev)
    sb = aq.ptgq_scale_bytes(M, K, 128, "ue8m0", "col")
    spb = aq.ptgq_scale_bytes(64, 7168, 128, "ue8m0", "col")
    q = torch.full((M, K), 0xCD, dtype=torch.uint8, device=dev)
    s = torch.full((sb,), 0xCD, dtype=torch.uint8, device=dev)
    qp = torch.full((64, 7168), 0xCD, dtype=torch.uint8, device=dev)
    sp = torch.full((spb,), 0xCD, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc1 = aq.ptgq_quant(x, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col", 1e-10, q, s,
                            check=False)
        rc2 = aq.ptgq_quant(p, "bf16", 64, 7168, 128, False, "e4m3", "ue8m0", "col", 1e-10, qp,
                            sp, check=False)
    print("captured first calls: status", rc1, rc2, flush=True)
    rq, rs = oracle.ptgq(xh, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col", eps=1e-10)
    rpq, rps = oracle.ptgq(ph, "bf16", 64, 7168, 128, False, "e4m3", "ue8m0", "col", eps=1e-10)
    for replay in range(3):
        q.fill_(0xCD); s.fill_(0xCD); qp.fill_(0xCD); sp.fill_(0xCD)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if rc1 == 0:
            assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy(), rs)
        if rc2 == 0:
            assert np.array_equal(qp.cpu().numpy(), rpq) and np.array_equal(sp.cpu().numpy(), rps)
        print("replay", replay, "bit-exact", flush=True)
    assert rc1 in (0, aq.PTGQ_EDEVICE) and rc2 in (0, aq.PTGQ_EDEVICE)
    # eager calls afterwards, on the default stream and on a side stream
    for st in (None, torch.cuda.Stream()):
        q.fill_(0xCD); s.fill_(0xCD)
        torch.cuda.synchronize()
        if st is None:
            aq.ptgq_quant(x, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col", 1e-10, q, s)
        else:
            with torch.cuda.stream(st):
                aq.ptgq_quant(x, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col", 1e-10, q, s)
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy(), rs)
        print("eager call after the capture bit-exact", flush=True)
    print("CHILD OK", flush=True)
""")


def test_first_call_inside_a_graph_capture():
    """A fresh process whose first library call is made while torch captures a
    graph: the call builds nothing and never synchronizes; replays are
    bit-exact (or the call reports a clean error status), and eager calls
    afterwards are bit-exact on the default and on a side stream."""
    res = subprocess.run([sys.executable, "-c", CAPTURE_CHILD.format(root=ROOT)],
                         capture_output=True, text=True, timeout=150)
    print(res.stdout[-3000:], flush=True)
    if res.returncode != 0:
        print(res.stderr[-3000:], flush=True)
    assert res.returncode == 0 and "CHILD OK" in res.stdout


STREAMS_CHILD = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    import numpy as np
    import torch
    import activation_quantization_amd as aq
    import oracle
    import workloads as W

    dev = "cuda"
    M, K = 2048, 4096                    # fused bf16, large enough for the SiLU table
    xh = W.normal_bf16(2050, (M, 2 * K))
    x = torch.from_numpy(xh.view(np.int16)).to(dev)
    sb = aq.ptgq_scale_bytes(M, K, 128, "ue8m0", "col")
    outs = [(torch.full((M, K), 0xCD, dtype=torch.uint8, device=dev),
             torch.full((sb,), 0xCD, dtype=torch.uint8, device=dev)) for _ in range(3)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    # the first call builds the table on s1; the next two, on s2 and on the
    # default stream, are enqueued at once, with no host synchronization
    with torch.cuda.stream(s1):
        aq.ptgq_quant(x, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col", 1e-10, *outs[0])
    with torch.cuda.stream(s2):
        aq.ptgq_quant(x, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col", 1e-10, *outs[1])
    aq.ptgq_quant(x, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col", 1e-10, *outs[2])
    torch.cuda.synchronize()
    rq, rs = oracle.ptgq(xh, "bf16", M, K, 128, True, "e4m3", "ue8m0", "col", eps=1e-10)
    for i, (q, s) in enumerate(outs):
        assert np.array_equal(q.cpu().numpy(), rq) and np.array_equal(s.cpu().numpy(), rs), i
        print("stream call", i, "bit-exact", flush=True)
    print("CHILD OK", flush=True)
""")


def test_first_calls_on_several_streams():
    """A fresh process whose first fused call runs on a side stream (building
    the SiLU table there) and whose next calls are enqueued at once on another
    side stream and on the default stream: each orders itself after the build
    on the device and is bit-exact."""
    res = subprocess.run([sys.executable, "-c", STREAMS_CHILD.format(root=ROOT)],
                         capture_output=True, text=True, timeout=150)
    print(res.stdout[-3000:], flush=True)
    if res.returncode != 0:
        print(res.stderr[-3000:], flush=True)
    assert res.returncode == 0 and "CHILD OK" in res.stdout


# ----------------------------------------------------- the stream reference

def test_stream_probe_moves_the_low_bytes():
    n = 1024 * 3001
    xh = np.random.default_rng(9).integers(0, 1 << 16, n).astype(np.uint16)
    q = Guarded((n,), torch.uint8, 0x11)
    aq.ptgq_probe_stream(to_dev(xh), n, q.t)
    torch.cuda.synchronize()
    q.check("stream probe")
    assert np.array_equal(q.host(), (xh & 0xFF).astype(np.uint8))
