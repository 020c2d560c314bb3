"""Bit-exact parity of group dequantization (ptgq_dequant) with the oracle:
every code, scale format, layout and output dtype, ragged rows, the group
sizes, the full headline shape, and writes confined to the output."""
import zlib

import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
import workloads as W
from gpu_util import DEV, Guarded

pytestmark = pytest.mark.gpu
OUTS = ("bf16", "fp16", "fp32")
CODES = ("e4m3", "int8")
LAYOUTS = (("f32", "row"), ("f32", "col"), ("ue8m0", "row"), ("ue8m0", "col"))
OSZ = {"bf16": 2, "fp16": 2, "fp32": 4}


def random_scales(rng, M, K, G, fmt, layout):
    """Scale tensor in the given format/layout, pad slots included.  fp32
    scales span 2^-130..2^12 (products reach fp32 subnormals and, after
    narrowing, bf16/fp16 overflow); exponent bytes cover 0..254."""
    nb = oracle.scale_bytes(M, K, G, fmt, layout)
    if fmt == "f32":
        e = rng.integers(-130, 13, nb // 4)
        m = rng.uniform(1.0, 2.0, nb // 4)
        return np.ldexp(m, e).astype(np.float32).view(np.uint8)
    b = rng.integers(0, 255, nb).astype(np.uint8)
    b[::7] = rng.integers(110, 135, b[::7].size).astype(np.uint8)
    return b


def run(q, code, M, K, G, s, fmt, layout, out, fill=0x5A):
    qd = torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
    sd = torch.from_numpy(np.ascontiguousarray(s).view(np.uint8)).to(DEV)
    n = M * K * OSZ[out]
    y = Guarded((n,), torch.uint8, fill)
    aq.ptgq_dequant(qd, code, M, K, G, sd, fmt, layout, out, y.t)
    torch.cuda.synchronize()
    y.check("ptgq_dequant y")
    return y.host().view(np.float32 if out == "fp32" else np.uint16).reshape(M, K)


def as_f32(y, out):
    if out == "fp32":
        return y
    if out == "fp16":
        return y.view(np.float16).astype(np.float32)
    return W.bf16_bits_to_f32(y)


def compare(tag, got, want, out):
    """Bit-exact, except that any NaN matches any NaN."""
    gn, wn = np.isnan(as_f32(got, out)), np.isnan(as_f32(want, out))
    bad = (got != want) & ~(gn & wn)
    print(f"[parity] {tag}: {int(bad.sum())}/{want.size} mismatches, {int(wn.sum())} NaN",
          flush=True)
    if bad.any():
        i = np.argwhere(bad)[0]
        print(f"  first at {tuple(i)}: got {got[tuple(i)]!r} want {want[tuple(i)]!r}", flush=True)
    assert not bad.any()


@pytest.mark.parametrize("fmt,layout", LAYOUTS)
@pytest.mark.parametrize("code", CODES)
@pytest.mark.parametrize("out", OUTS)
def test_every_code_format_layout_and_output(out, code, fmt, layout):
    """M = 37 (column-major pad rows), K = 3200 (three full 1024-code slabs
    and a ragged 128-code tail); all 256 code bytes, NaN codes included."""
    rng = np.random.default_rng(zlib.crc32(f"{out}/{code}/{fmt}/{layout}".encode()))
    M, K, G = 37, 3200, 128
    q = rng.integers(0, 256, (M, K)).astype(np.uint8)
    q[0, :256] = np.arange(256)
    s = random_scales(rng, M, K, G, fmt, layout)
    got = run(q, code, M, K, G, s, fmt, layout, out)
    want = oracle.dequant(q, code, M, K, G, s, fmt, layout, out)
    compare(f"dequant {code}->{out} {fmt}/{layout}", got, want, out)


@pytest.mark.parametrize("G", [16, 32, 64, 128])
@pytest.mark.parametrize("out", OUTS)
def test_group_sizes(G, out):
    rng = np.random.default_rng(G)
    M, K = 19, 2048 + G
    q = rng.integers(0, 256, (M, K)).astype(np.uint8)
    for fmt, layout in LAYOUTS:
        s = random_scales(rng, M, K, G, fmt, layout)
        got = run(q, "e4m3", M, K, G, s, fmt, layout, out)
        want = oracle.dequant(q, "e4m3", M, K, G, s, fmt, layout, out)
        compare(f"dequant G={G} ->{out} {fmt}/{layout}", got, want, out)


@pytest.mark.parametrize("M,K,G", [(1, 16, 16), (1, 128, 128), (3, 48, 16), (2, 65536, 128),
                                   (5, 1024, 64), (4, 1040, 16), (777, 256, 128)])
def test_edge_shapes(M, K, G):
    """One row, one group, K below one slab, very wide rows (few tasks: one-wave
    blocks), many short rows."""
    rng = np.random.default_rng(M * 100003 + K)
    q = rng.integers(0, 256, (M, K)).astype(np.uint8)
    for fmt, layout in LAYOUTS:
        s = random_scales(rng, M, K, G, fmt, layout)
        for out in OUTS:
            got = run(q, "e4m3", M, K, G, s, fmt, layout, out)
            want = oracle.dequant(q, "e4m3", M, K, G, s, fmt, layout, out)
            compare(f"dequant edge M={M} K={K} G={G} ->{out} {fmt}/{layout}", got, want, out)


def test_empty_calls_write_nothing():
    y = torch.full((64,), 0x5A, dtype=torch.uint8, device=DEV)
    q = torch.zeros(64, dtype=torch.uint8, device=DEV)
    s = torch.zeros(64, dtype=torch.uint8, device=DEV)
    aq.ptgq_dequant(q, "e4m3", 0, 1024, 128, s, "ue8m0", "col", "bf16", y)
    aq.ptgq_dequant(q, "e4m3", 4, 0, 128, s, "ue8m0", "col", "bf16", y)
    torch.cuda.synchronize()
    assert torch.all(y == 0x5A)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("code", CODES)
def test_quantized_exactness_family_round_trips(code, layout):
    """Codes and UE8M0 scales that the oracle's quantizer writes for integers
    in [-8, 8] dequantize to those integers exactly, in every output dtype."""
    d = W.cfg5c(M=12, K=1024)
    q, s = oracle.ptgq(d["x"], "fp16", 12, 1024, 128, False, code, "ue8m0", layout)
    xf = d["x"].view(np.float16).astype(np.float32)
    for out in OUTS:
        got = run(q, code, 12, 1024, 128, s, "ue8m0", layout, out)
        assert np.array_equal(as_f32(got, out), xf)


def test_full_headline_shape():
    """[16384, 7168] e4m3 codes with packed column-major UE8M0 scales to bf16,
    in the launch configuration the benchmark times, every element."""
    M, K, G = 16384, 7168, 128
    rng = np.random.default_rng(16384)
    q = rng.integers(0, 256, (M, K), dtype=np.uint8)
    s = random_scales(rng, M, K, G, "ue8m0", "col")
    got = run(q, "e4m3", M, K, G, s, "ue8m0", "col", "bf16")
    want = oracle.dequant(q, "e4m3", M, K, G, s, "ue8m0", "col", "bf16")
    compare("dequant full [16384, 7168] e4m3->bf16 ue8m0/col", got, want, "bf16")


@pytest.mark.parametrize("out", OUTS)
def test_uncapped_grid_ragged(out):
    """Enough tasks for the uncapped, XCD-chunked grid (more tasks than the
    chip holds waves) with rows that end mid-task and a last, partial span of
    blocks, every scale format and layout."""
    M, K, G = 2401, 7040, 128
    rng = np.random.default_rng(2401 + OSZ[out])
    q = rng.integers(0, 256, (M, K)).astype(np.uint8)
    for fmt, layout in LAYOUTS:
        s = random_scales(rng, M, K, G, fmt, layout)
        got = run(q, "e4m3", M, K, G, s, fmt, layout, out)
        want = oracle.dequant(q, "e4m3", M, K, G, s, fmt, layout, out)
        compare(f"dequant uncapped M={M} K={K} ->{out} {fmt}/{layout}", got, want, out)


def test_tuning_knobs_never_change_results():
    """Grid caps, task sizes and XCD chunks (including chunks that leave a
    ragged last span) change speed only."""
    M, K, G = 2401, 7040, 128
    rng = np.random.default_rng(77)
    q = rng.integers(0, 256, (M, K)).astype(np.uint8)
    s = random_scales(rng, M, K, G, "ue8m0", "col")
    want = oracle.dequant(q, "e4m3", M, K, G, s, "ue8m0", "col", "bf16")
    try:
        for knob, values in ((0, [1, 4]), (2, [1, 4, 100000]), (5, [0, 1, 3, 16, 1000])):
            for v in values:
                aq.ptgq_set_tuning(knob, v)
                got = run(q, "e4m3", M, K, G, s, "ue8m0", "col", "bf16")
                compare(f"dequant knob {knob}={v}", got, want, "bf16")
                aq.ptgq_set_tuning(knob, -1)
    finally:
        for k in range(8):
            aq.ptgq_set_tuning(k, -1)
