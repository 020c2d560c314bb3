"""Bit-exact parity of the trait extensions with the oracle: fp32 input for the
group quantizer (flat and masked), and the padded code buffer whose rows past M
are zero-filled (ptgq_quant_padded)."""
import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
import workloads as W
from gpu_util import DEV, Guarded, compare, run_flat, run_masked, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(1, 128), (3, 640), (5, 2048 + 128), (37, 512), (6, 7168)]


def f32_input(seed, shape):
    """N(0,1) fp32 with two outlier columns x37, a few exact zeros, values near
    the fp32 extremes of the normal range and tiny normals."""
    x = W.normal_f32(seed, shape)
    x[..., 1] *= 37.0
    x[..., -1] *= 37.0
    flat = x.reshape(-1)
    z = W.splitmix64(W.substream(seed, 7), 0, 8)
    idx = (z % np.uint64(flat.size)).astype(np.int64)
    flat[idx[:2]] = 0.0
    flat[idx[2]] = 3.0e38
    flat[idx[3]] = -1.0e-30
    flat[idx[4]] = 1.17549435e-38
    return x


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
@pytest.mark.parametrize("out_dtype", ["e4m3", "int8"])
@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_fp32_input_sweep(G, out_dtype, fmt, layout):
    for i, (M, K) in enumerate(SHAPES):
        if K % G:
            continue
        x = f32_input(500 * G + i, (M, K))
        args = (x, "fp32", M, K, G, False, out_dtype, fmt, layout)
        compare(f"fp32 input G={G} {out_dtype} {fmt} {layout} M={M} K={K}",
                *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


def test_fp32_input_large_flat():
    """[4096, 7168] fp32 -> e4m3, packed column-major UE8M0: two-slab tasks and
    the capped grid, every element."""
    M, K = 4096, 7168
    x = f32_input(4096, (M, K))
    args = (x, "fp32", M, K, 128, False, "e4m3", "ue8m0", "col")
    compare("fp32 input [4096, 7168]", *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_fp32_input_masked(fmt, layout):
    E, T, K = 6, 45, 1152
    x = f32_input(777, (E, T, K))
    mm = np.array([0, 45, 3, -2, 60, 17], np.int32)
    gq, gs = run_masked(x, "fp32", E, T, K, 128, False, mm, 16, "e4m3", fmt, layout)
    sb = aq.ptgq_scale_bytes(T, K, 128, fmt, layout)
    rq, rs = oracle.ptgq_masked(x, "fp32", E, T, K, 128, False, mm, "e4m3", fmt, layout,
                                q_init=np.full((E, T, K), 0x7F, np.uint8),
                                s_init=np.full(E * sb, 0xFF, np.uint8))
    compare(f"fp32 masked {fmt} {layout}", gq, gs, rq, rs)


def test_fused_fp32_is_refused():
    x = torch.zeros((2, 256), dtype=torch.float32, device=DEV)
    q = torch.zeros((2, 128), dtype=torch.uint8, device=DEV)
    s = torch.zeros(64, dtype=torch.uint8, device=DEV)
    rc = aq.ptgq_quant(x, "fp32", 2, 128, 128, True, "e4m3", "f32", "row", 1e-10, q, s,
                       check=False)
    assert rc == aq.PTGQ_EUNSUPPORTED


# ------------------------------------------------------ padded code buffer

SENT = 0xA7


def run_padded(x, in_dtype, M, K, G, fuse, out_dtype, fmt, layout, q_rows):
    xd = to_dev(x) if M > 0 else None
    q = Guarded((q_rows, K), torch.uint8, SENT)
    sb = aq.ptgq_scale_bytes(M, K, G, fmt, layout)
    s = Guarded((sb,), torch.uint8, SENT)
    aq.ptgq_quant_padded(xd, in_dtype, M, K, G, fuse, out_dtype, fmt, layout, 1e-10, q.t, q_rows,
                         s.t if M > 0 else None)
    torch.cuda.synchronize()
    q.check("ptgq_quant_padded q")
    s.check("ptgq_quant_padded s")
    return q.host(), s.host()


@pytest.mark.parametrize("M,K,q_rows,fuse", [(1, 7168, 4, False), (5, 7168, 8, False),
                                             (6, 1152, 8, True), (16, 2048, 16, False),
                                             (3, 640, 5000, False), (777, 512, 780, True)])
@pytest.mark.parametrize("fmt,layout", [("ue8m0", "col"), ("f32", "row")])
def test_padded_rows_are_zero(M, K, q_rows, fuse, fmt, layout):
    """Rows < M equal the oracle's codes, rows M .. q_rows-1 are zero, nothing
    past the buffer is written; the scales are the unpadded ones."""
    x = W.normal_bf16(M * 7 + K, (M, 2 * K if fuse else K))
    q, s = run_padded(x, "bf16", M, K, 128, fuse, "e4m3", fmt, layout, q_rows)
    rq, rs = oracle.ptgq(x, "bf16", M, K, 128, fuse, "e4m3", fmt, layout, eps=1e-10)
    compare(f"padded M={M} q_rows={q_rows} fuse={fuse} {fmt} {layout}", q[:M], s, rq, rs)
    assert np.all(q[M:] == 0)


def test_padded_with_no_rows_only_zero_fills():
    q, _ = run_padded(None, "bf16", 0, 4096, 128, False, "e4m3", "ue8m0", "col", 12)
    assert np.all(q == 0)


def test_padded_equals_plain_call():
    """Same bytes as ptgq_quant when q_rows == M (no fill)."""
    M, K = 300, 7168
    x = W.normal_bf16(300, (M, K))
    q, s = run_padded(x, "bf16", M, K, 128, False, "int8", "ue8m0", "row", M)
    pq, ps = run_flat(x, "bf16", M, K, 128, False, "int8", "ue8m0", "row")
    assert np.array_equal(q, pq) and np.array_equal(s, ps)
