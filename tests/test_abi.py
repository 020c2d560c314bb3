"""CPU checks of the C ABI: the library loads, exports exactly the functions
that include/ptgq.h (the quantization interface) and include/ptgq_diag.h
(diagnostics) declare, and rejects invalid arguments on the host (no device is
touched, nothing is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import activation_quantization_amd as aq
import oracle
from activation_quantization_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if libbuild.is_stale():
        libbuild.build()
    return aq.load_library()


def declared_functions(header="ptgq.h"):
    with open(os.path.join(ROOT, "include", header)) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"PTGQ_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_headers_declare_the_binding_names():
    assert declared_functions("ptgq.h") == sorted(aq.EXPORTS)
    assert declared_functions("ptgq_diag.h") == sorted(aq.DIAG_EXPORTS)
    assert not set(aq.EXPORTS) & set(aq.DIAG_EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    both = sorted(declared_functions("ptgq.h") + declared_functions("ptgq_diag.h"))
    for name in both:
        assert hasattr(lib, name), name
    # nothing but the two headers' C ABI is visible
    out = os.popen(f"nm -D --defined-only {aq.LIB_PATH}").read()
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == both


def test_quantization_header_has_no_diagnostics():
    """The production header declares the quantization calls only: probes,
    tuning overrides and the geometry report live in ptgq_diag.h."""
    names = declared_functions("ptgq.h")
    assert not [n for n in names if "probe" in n or "tuning" in n or "plan" in n or "diag" in n]


def test_fastdiv_matches_integer_division(lib):
    """The multiply-high division the kernels use for task indices, for every
    divisor 1..4096 and selected large ones, on numerators spread over
    [0, 2^31) including every multiple boundary near the top."""
    rng = np.random.default_rng(1994)
    for d in list(range(1, 4097)) + [5000, 7 * 512, 65535, 65537, 1 << 20, (1 << 20) + 1,
                                      (1 << 30) - 1, 1 << 30, (1 << 31) - 1]:
        n = np.concatenate([rng.integers(0, 1 << 31, 256, dtype=np.int64),
                            np.arange(0, 64),
                            (1 << 31) - 1 - np.arange(0, 64),
                            ((((1 << 31) - 1) // d) * d + np.arange(-2, 1)).clip(0)]).astype(np.uint32)
        q = aq.ptgq_diag_fastdiv(d, n)
        assert np.array_equal(q, (n.astype(np.int64) // d).astype(np.uint32)), d


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5):
        assert aq.status_string(st)
    assert aq.status_string(7) == "unknown status"


@pytest.mark.parametrize("rows,K,G,fmt,lay", [
    (64, 2048, 128, "f32", "row"), (5, 7168, 128, "ue8m0", "col"), (1, 128, 128, "ue8m0", "col"),
    (7, 3584, 16, "f32", "col"), (9, 640, 64, "ue8m0", "row"), (0, 2048, 128, "f32", "col"),
    (384, 2048, 128, "ue8m0", "col"), (3, 96, 32, "ue8m0", "col")])
def test_scale_bytes_matches_the_oracle(lib, rows, K, G, fmt, lay):
    assert aq.ptgq_scale_bytes(rows, K, G, fmt, lay) == oracle.scale_bytes(rows, K, G, fmt, lay)


def test_scale_bytes_rejects_invalid(lib):
    assert aq.ptgq_scale_bytes(4, 100, 128, "f32", "row") == 0
    assert aq.ptgq_scale_bytes(4, 96, 48, "f32", "row") == 0
    assert aq.ptgq_scale_bytes(-1, 128, 128, "f32", "row") == 0
    assert aq.ptgq_scale_bytes(4, 128, 128, 7, 0) == 0


A16 = 0x10000          # a 16-byte aligned fake address (never dereferenced)


def quant(**kw):
    args = dict(x=A16, in_dtype="bf16", M=4, K=256, group_size=128, fuse_silu_mul=False,
                out_dtype="e4m3", scale_fmt="ue8m0", scale_layout="col", eps=1e-10, q=A16 * 2,
                s=A16 * 3, stream=0, check=False)
    args.update(kw)
    return aq.ptgq_quant(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(group_size=48), aq.PTGQ_EINVAL),
    (dict(group_size=256), aq.PTGQ_EINVAL),
    (dict(K=200), aq.PTGQ_EINVAL),
    (dict(M=-1), aq.PTGQ_EINVAL),
    (dict(K=-128), aq.PTGQ_EINVAL),
    (dict(in_dtype=2, fuse_silu_mul=True), aq.PTGQ_EUNSUPPORTED),   # fused: 16-bit only
    (dict(in_dtype=9), aq.PTGQ_EINVAL),
    (dict(out_dtype=3), aq.PTGQ_EINVAL),
    (dict(scale_fmt=2), aq.PTGQ_EINVAL),
    (dict(scale_layout=5), aq.PTGQ_EINVAL),
    (dict(eps=float("nan")), aq.PTGQ_EINVAL),
    (dict(eps=-1.0), aq.PTGQ_EINVAL),
    (dict(eps=float("inf")), aq.PTGQ_EINVAL),
    (dict(eps=-0.0), aq.PTGQ_EINVAL),
    (dict(x=0), aq.PTGQ_EINVAL),
    (dict(q=0), aq.PTGQ_EINVAL),
    (dict(s=0), aq.PTGQ_EINVAL),
    (dict(x=A16 + 8), aq.PTGQ_EALIGN),
    (dict(q=A16 + 4), aq.PTGQ_EALIGN),
    (dict(s=A16 + 2), aq.PTGQ_EALIGN),
    (dict(M=0, x=0, q=0, s=0), aq.PTGQ_OK),   # nothing to do: no launch
    (dict(K=0, x=0, q=0, s=0), aq.PTGQ_OK),
])
def test_ptgq_quant_validation(lib, kw, status):
    assert quant(**kw) == status


def test_fp32_group_input_passes_validation(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert quant(in_dtype="fp32") == aq.PTGQ_EDEVICE
    assert quant(in_dtype="fp32", scale_fmt="f32", scale_layout="row") == aq.PTGQ_EDEVICE


def padded(**kw):
    args = dict(x=A16, in_dtype="bf16", M=5, K=256, group_size=128, fuse_silu_mul=False,
                out_dtype="e4m3", scale_fmt="ue8m0", scale_layout="col", eps=1e-10, q=A16 * 2,
                q_rows=8, s=A16 * 3, stream=0, check=False)
    args.update(kw)
    return aq.ptgq_quant_padded(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q_rows=4), aq.PTGQ_EINVAL),               # fewer q rows than M
    (dict(q_rows=-1, M=0), aq.PTGQ_EINVAL),
    (dict(group_size=96), aq.PTGQ_EINVAL),
    (dict(x=0), aq.PTGQ_EINVAL),
    (dict(q=A16 + 8), aq.PTGQ_EALIGN),
    (dict(M=0, x=0, s=0, q=0), aq.PTGQ_EINVAL),     # zero fill still needs q
    (dict(M=0, x=0, s=0, q=A16 + 4), aq.PTGQ_EALIGN),
    (dict(q_rows=1 << 31), aq.PTGQ_EUNSUPPORTED),
    (dict(in_dtype="fp32", fuse_silu_mul=True), aq.PTGQ_EUNSUPPORTED),
    (dict(M=0, q_rows=0, x=0, s=0, q=0), aq.PTGQ_OK),
    (dict(K=0, x=0, s=0, q=0), aq.PTGQ_OK),
])
def test_ptgq_quant_padded_validation(lib, kw, status):
    assert padded(**kw) == status


def test_padded_zero_fill_alone_needs_no_input(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert padded(M=0, x=0, s=0) == aq.PTGQ_EDEVICE


def masked(**kw):
    args = dict(x=A16, in_dtype="bf16", E=4, tokens_pad=32, K=256, group_size=128,
                fuse_silu_mul=True, masked_m=A16 * 4, expected_m=0, out_dtype="e4m3",
                scale_fmt="ue8m0", scale_layout="col", eps=1e-10, q=A16 * 2, s=A16 * 3,
                stream=0, check=False)
    args.update(kw)
    return aq.ptgq_quant_masked(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(E=-1), aq.PTGQ_EINVAL),
    (dict(tokens_pad=-3), aq.PTGQ_EINVAL),
    (dict(masked_m=0), aq.PTGQ_EINVAL),
    (dict(masked_m=A16 + 2), aq.PTGQ_EALIGN),
    (dict(group_size=8), aq.PTGQ_EINVAL),
    (dict(x=A16 + 4), aq.PTGQ_EALIGN),
    (dict(E=4097), aq.PTGQ_EUNSUPPORTED),
    (dict(in_dtype="fp32"), aq.PTGQ_EUNSUPPORTED),  # fused fp32
    (dict(E=0, x=0, q=0, s=0, masked_m=0), aq.PTGQ_OK),
    (dict(tokens_pad=0, x=0, q=0, s=0, masked_m=0), aq.PTGQ_OK),
])
def test_ptgq_quant_masked_validation(lib, kw, status):
    assert masked(**kw) == status


def per_token(**kw):
    args = dict(x=A16, in_dtype="bf16", M=4, K=1076, q=A16 * 2, s=A16 * 3, stream=0, check=False)
    args.update(kw)
    return aq.ptq_quant_fp8(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(K=1074), aq.PTGQ_EINVAL),           # K % 4 != 0
    (dict(in_dtype=5), aq.PTGQ_EINVAL),
    (dict(M=-2), aq.PTGQ_EINVAL),
    (dict(x=0), aq.PTGQ_EINVAL),
    (dict(s=0), aq.PTGQ_EINVAL),
    (dict(q=A16 + 1), aq.PTGQ_EALIGN),
    (dict(s=A16 + 1), aq.PTGQ_EALIGN),
    (dict(M=0, x=0, q=0, s=0), aq.PTGQ_OK),
])
def test_ptq_quant_fp8_validation(lib, kw, status):
    assert per_token(**kw) == status


def test_probe_validation(lib):
    assert aq.ptgq_probe_e4m3(0, A16, 5, stream=0, check=False) == aq.PTGQ_EINVAL
    assert aq.ptgq_probe_e4m3(A16, A16, -1, stream=0, check=False) == aq.PTGQ_EINVAL
    assert aq.ptgq_probe_e4m3(0, 0, 0, stream=0, check=False) == aq.PTGQ_OK
    assert aq.ptgq_probe_silu_mul(A16, A16, 2, 0, A16, 4, stream=0, check=False) == aq.PTGQ_EINVAL
    assert aq.ptgq_probe_silu_mul(A16, A16, "fp16", 3, A16, 4, stream=0, check=False) == aq.PTGQ_EINVAL
    assert aq.ptgq_probe_silu_mul(A16, A16, "bf16", 2, A16, 4, stream=0, check=False) == aq.PTGQ_EINVAL
    with pytest.raises(aq.PtgqError):
        aq.ptgq_set_tuning(9, 1)
    assert aq.ptgq_probe_scale(0x7F800000, 1, 0.0, "e4m3", "ue8m0", A16, stream=0,
                               check=False) == aq.PTGQ_EINVAL          # +inf is no amax
    assert aq.ptgq_probe_scale(0, 4, -1.0, "e4m3", "f32", A16, stream=0,
                               check=False) == aq.PTGQ_EINVAL
    assert aq.ptgq_probe_scale(0, 4, 0.0, "e4m3", "f32", A16 + 2, stream=0,
                               check=False) == aq.PTGQ_EALIGN
    assert aq.ptgq_probe_scale(0, 0, 0.0, "e4m3", "f32", 0, stream=0, check=False) == aq.PTGQ_OK
    assert aq.ptgq_probe_int8(0, (1 << 32) + 1, A16, stream=0, check=False) == aq.PTGQ_EINVAL
    assert aq.ptgq_probe_int8(0, 4, 0, stream=0, check=False) == aq.PTGQ_EINVAL
    assert aq.ptgq_probe_stream(A16, 1000, A16 * 2, stream=0, check=False) == aq.PTGQ_EINVAL
    assert aq.ptgq_probe_stream(A16 + 8, 1024, A16 * 2, stream=0, check=False) == aq.PTGQ_EALIGN
    assert aq.ptgq_probe_stream(0, 0, 0, stream=0, check=False) == aq.PTGQ_OK


def test_binding_raises_on_error(lib):
    with pytest.raises(aq.PtgqError) as ei:
        aq.ptgq_quant(A16, "bf16", 4, 200, 128, False, "e4m3", "f32", "row", 1e-10, A16, A16,
                      stream=0)
    assert ei.value.status == aq.PTGQ_EINVAL


def test_without_gpu_a_valid_call_reports_no_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert quant() == aq.PTGQ_EDEVICE
    assert lib.ptgq_init(0) == aq.PTGQ_EDEVICE


def test_binding_refuses_undersized_tensors(lib):
    import torch
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    q = torch.zeros((4, 255), dtype=torch.uint8)
    s = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError):
        aq.ptgq_quant(x, "bf16", 4, 256, 128, False, "e4m3", "ue8m0", "col", 1e-10, q, s, stream=0)
    with pytest.raises(ValueError):
        aq.ptq_quant_fp8(x, "bf16", 5, 256, torch.zeros((5, 256), dtype=torch.uint8),
                         torch.zeros(5), stream=0)


def requant(**kw):
    args = dict(x=A16, E=4, T=48, K=3584, group_size=128, x_scale=A16 * 5,
                scale_strides=(28 * 48, 1, 48), masked_m=A16 * 4, expected_m=0,
                output_scale=A16 * 6, out=A16 * 2, stream=0, check=False)
    args.update(kw)
    return aq.ptgq_requant_fp8(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(K=3500), aq.PTGQ_EINVAL),
    (dict(group_size=96), aq.PTGQ_EINVAL),
    (dict(E=-1), aq.PTGQ_EINVAL),
    (dict(scale_strides=(1, -1, 1)), aq.PTGQ_EINVAL),
    (dict(x=0), aq.PTGQ_EINVAL),
    (dict(output_scale=0), aq.PTGQ_EINVAL),
    (dict(out=A16), aq.PTGQ_EINVAL),                # in place is refused
    (dict(x=A16 + 8), aq.PTGQ_EALIGN),
    (dict(x_scale=A16 + 2), aq.PTGQ_EALIGN),
    (dict(masked_m=A16 + 2), aq.PTGQ_EALIGN),
    (dict(E=5000), aq.PTGQ_EUNSUPPORTED),
    (dict(E=0, x=0, out=0, x_scale=0, output_scale=0), aq.PTGQ_OK),
])
def test_ptgq_requant_fp8_validation(lib, kw, status):
    assert requant(**kw) == status


def dequant(**kw):
    args = dict(q=A16, code_dtype="e4m3", M=8, K=1024, group_size=128, s=A16 * 3,
                scale_fmt="f32", scale_layout="col", out_dtype="bf16", y=A16 * 5, stream=0,
                check=False)
    args.update(kw)
    return aq.ptgq_dequant(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(K=1000), aq.PTGQ_EINVAL),
    (dict(group_size=256), aq.PTGQ_EINVAL),
    (dict(M=-1), aq.PTGQ_EINVAL),
    (dict(code_dtype=2), aq.PTGQ_EINVAL),
    (dict(out_dtype=3), aq.PTGQ_EINVAL),
    (dict(scale_fmt=2), aq.PTGQ_EINVAL),
    (dict(scale_layout=2), aq.PTGQ_EINVAL),
    (dict(q=0), aq.PTGQ_EINVAL),
    (dict(s=0), aq.PTGQ_EINVAL),
    (dict(y=A16), aq.PTGQ_EINVAL),                  # y aliasing q
    (dict(y=A16 * 3), aq.PTGQ_EINVAL),              # y aliasing s
    (dict(q=A16 + 8), aq.PTGQ_EALIGN),
    (dict(y=A16 * 5 + 4), aq.PTGQ_EALIGN),
    (dict(s=A16 * 3 + 2), aq.PTGQ_EALIGN),
    (dict(K=1 << 29), aq.PTGQ_EUNSUPPORTED),
    (dict(M=0, q=0, s=0, y=0), aq.PTGQ_OK),
    (dict(K=0, q=0, s=0, y=0), aq.PTGQ_OK),
])
def test_ptgq_dequant_validation(lib, kw, status):
    assert dequant(**kw) == status


def test_dequant_ue8m0_scales_need_no_alignment(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert dequant(s=A16 * 3 + 1, scale_fmt="ue8m0") == aq.PTGQ_EDEVICE
