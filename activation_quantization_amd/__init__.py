"""Python binding of libptgq (per-token-group 8-bit activation quantization on
MI355X / gfx950).

Argument marshalling only: every function below passes device pointers, sizes
and the current HIP stream straight to the C ABI declared in include/ptgq.h,
under the same names.  PyTorch supplies device memory and streams.  There is
no fallback: if the library was not built, importing this package's functions
raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libptgq.so")

PTGQ_OK, PTGQ_EINVAL, PTGQ_EALIGN, PTGQ_EUNSUPPORTED, PTGQ_ELAUNCH, PTGQ_EDEVICE = 0, -1, -2, -3, -4, -5
PTGQ_BF16, PTGQ_FP16, PTGQ_FP32 = 0, 1, 2
PTGQ_E4M3, PTGQ_INT8 = 0, 1
PTGQ_SCALE_F32, PTGQ_SCALE_UE8M0 = 0, 1
PTGQ_ROW_MAJOR, PTGQ_COL_MAJOR = 0, 1

IN_DTYPES = {"bf16": PTGQ_BF16, "fp16": PTGQ_FP16, "fp32": PTGQ_FP32}
OUT_DTYPES = {"e4m3": PTGQ_E4M3, "int8": PTGQ_INT8}
SCALE_FMTS = {"f32": PTGQ_SCALE_F32, "ue8m0": PTGQ_SCALE_UE8M0}
SCALE_LAYOUTS = {"row": PTGQ_ROW_MAJOR, "col": PTGQ_COL_MAJOR}

# include/ptgq.h: the quantization interface
EXPORTS = ("ptgq_quant", "ptgq_quant_padded", "ptgq_quant_masked", "ptq_quant_fp8", "ptgq_requant_fp8",
           "ptgq_dequant", "ptgq_scale_bytes", "ptgq_status_string", "ptgq_init")
# include/ptgq_diag.h: probes, the stream reference, the chooser's report and overrides
DIAG_EXPORTS = ("ptgq_probe_e4m3", "ptgq_probe_silu_mul", "ptgq_probe_scale", "ptgq_probe_int8",
                "ptgq_probe_stream", "ptgq_diag_fastdiv", "ptgq_plan_group", "ptgq_set_tuning")


class PtgqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libptgq.so (raises if it is missing: there is no other path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libptgq.so not built at {path}; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    i32, i64, f32, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.ptgq_quant.argtypes = [vp, i32, i64, i64, i32, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.ptgq_quant.restype = i32
    lib.ptgq_quant_padded.argtypes = [vp, i32, i64, i64, i32, i32, i32, i32, i32, f32, vp, i64,
                                      vp, vp]
    lib.ptgq_quant_padded.restype = i32
    lib.ptgq_quant_masked.argtypes = [vp, i32, i64, i64, i64, i32, i32, vp, i64, i32, i32, i32,
                                      f32, vp, vp, vp]
    lib.ptgq_quant_masked.restype = i32
    lib.ptq_quant_fp8.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    lib.ptq_quant_fp8.restype = i32
    lib.ptgq_requant_fp8.argtypes = [vp, i64, i64, i64, i32, vp, i64, i64, i64, vp, i64, vp, vp,
                                     vp]
    lib.ptgq_requant_fp8.restype = i32
    lib.ptgq_dequant.argtypes = [vp, i32, i64, i64, i32, vp, i32, i32, i32, vp, vp]
    lib.ptgq_dequant.restype = i32
    lib.ptgq_scale_bytes.argtypes = [i64, i64, i32, i32, i32]
    lib.ptgq_scale_bytes.restype = ctypes.c_size_t
    lib.ptgq_status_string.argtypes = [i32]
    lib.ptgq_status_string.restype = ctypes.c_char_p
    lib.ptgq_init.argtypes = [i32]
    lib.ptgq_init.restype = i32
    lib.ptgq_probe_e4m3.argtypes = [vp, vp, i64, vp]
    lib.ptgq_probe_e4m3.restype = i32
    lib.ptgq_probe_silu_mul.argtypes = [vp, vp, i32, i32, vp, i64, vp]
    lib.ptgq_probe_silu_mul.restype = i32
    lib.ptgq_set_tuning.argtypes = [i32, i64]
    lib.ptgq_set_tuning.restype = i32
    lib.ptgq_plan_group.argtypes = [i32, i64, i64, i64, i32, i32, i64, i64, i32, vp]
    lib.ptgq_plan_group.restype = i32
    u32 = ctypes.c_uint32
    lib.ptgq_probe_scale.argtypes = [u32, i64, f32, i32, i32, vp, vp, vp]
    lib.ptgq_probe_scale.restype = i32
    lib.ptgq_probe_int8.argtypes = [u32, i64, vp, vp]
    lib.ptgq_probe_int8.restype = i32
    lib.ptgq_probe_stream.argtypes = [vp, i64, vp, vp]
    lib.ptgq_probe_stream.restype = i32
    lib.ptgq_diag_fastdiv.argtypes = [u32, vp, vp, i64]
    lib.ptgq_diag_fastdiv.restype = i32
    _lib = lib
    return lib


def _ptr(t):
    """Device (or host) address of a tensor, or a raw integer address."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _enum(v, table):
    return table[v] if isinstance(v, str) else int(v)


_IN_SIZE = {PTGQ_BF16: 2, PTGQ_FP16: 2, PTGQ_FP32: 4}


def _need(t, nbytes, fn, name):
    """Host-side guard: a tensor argument must hold every byte the call touches
    (raw integer addresses are passed through unchecked)."""
    if t is None or isinstance(t, int):
        return
    if t.device.type != "cuda":
        raise ValueError(f"{fn}: {name} must be a device tensor, got one on {t.device}")
    have = t.numel() * t.element_size()
    if not t.is_contiguous() or have < nbytes:
        raise ValueError(f"{fn}: {name} needs {nbytes} contiguous bytes, has {have}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _check(fn, rc):
    if rc != PTGQ_OK:
        raise PtgqError(fn, rc)
    return rc


def status_string(status: int) -> str:
    return load_library().ptgq_status_string(int(status)).decode()


def ptgq_status_string(status: int) -> str:
    return status_string(status)


def ptgq_scale_bytes(rows, K, group_size, scale_fmt, scale_layout) -> int:
    return int(load_library().ptgq_scale_bytes(rows, K, group_size, _enum(scale_fmt, SCALE_FMTS),
                                               _enum(scale_layout, SCALE_LAYOUTS)))


def ptgq_init(device: int = 0) -> int:
    return _check("ptgq_init", load_library().ptgq_init(int(device)))


def ptgq_set_tuning(knob: int, value: int) -> int:
    return _check("ptgq_set_tuning", load_library().ptgq_set_tuning(int(knob), int(value)))


PLAN_FIELDS = ("grid", "block", "slabs_per_task", "tasks_per_row", "tasks", "xcd_chunk",
               "silu_table", "uncapped", "flat_slabs")


def ptgq_plan_group(in_dtype, E, rows, K, group_size, fuse_silu_mul, expected_m, q_rows, cus):
    """The launch geometry the chooser picks for a flat (E = 0) or masked
    (E >= 1) group call on a device of `cus` compute units, as a dict of
    PLAN_FIELDS.  Host only: no device is touched."""
    out = (ctypes.c_int64 * len(PLAN_FIELDS))()
    rc = load_library().ptgq_plan_group(_enum(in_dtype, IN_DTYPES), int(E), int(rows), int(K),
                                        int(group_size), int(bool(fuse_silu_mul)),
                                        int(expected_m), int(q_rows), int(cus),
                                        ctypes.cast(out, ctypes.c_void_p))
    _check("ptgq_plan_group", rc)
    return dict(zip(PLAN_FIELDS, (int(v) for v in out)))


def ptgq_quant(x, in_dtype, M, K, group_size, fuse_silu_mul, out_dtype, scale_fmt, scale_layout,
               eps, q, s, stream=None, check=True):
    ind, fmt, lay = _enum(in_dtype, IN_DTYPES), _enum(scale_fmt, SCALE_FMTS), _enum(scale_layout, SCALE_LAYOUTS)
    if M > 0 and K > 0 and ind in _IN_SIZE:
        _need(x, M * K * (2 if fuse_silu_mul else 1) * _IN_SIZE[ind], "ptgq_quant", "x")
        _need(q, M * K, "ptgq_quant", "q")
        _need(s, ptgq_scale_bytes(M, K, group_size, fmt, lay), "ptgq_quant", "s")
    rc = load_library().ptgq_quant(_ptr(x), _enum(in_dtype, IN_DTYPES), M, K, group_size,
                                   int(bool(fuse_silu_mul)), _enum(out_dtype, OUT_DTYPES),
                                   _enum(scale_fmt, SCALE_FMTS), _enum(scale_layout, SCALE_LAYOUTS),
                                   float(eps), _ptr(q), _ptr(s), _stream(stream))
    return _check("ptgq_quant", rc) if check else rc


def ptgq_quant_padded(x, in_dtype, M, K, group_size, fuse_silu_mul, out_dtype, scale_fmt,
                      scale_layout, eps, q, q_rows, s, stream=None, check=True):
    ind, fmt, lay = _enum(in_dtype, IN_DTYPES), _enum(scale_fmt, SCALE_FMTS), _enum(scale_layout, SCALE_LAYOUTS)
    if K > 0 and q_rows >= M >= 0:
        fn = "ptgq_quant_padded"
        _need(q, q_rows * K, fn, "q")
        if M > 0 and ind in _IN_SIZE:
            _need(x, M * K * (2 if fuse_silu_mul else 1) * _IN_SIZE[ind], fn, "x")
            _need(s, ptgq_scale_bytes(M, K, group_size, fmt, lay), fn, "s")
    rc = load_library().ptgq_quant_padded(_ptr(x), ind, M, K, group_size, int(bool(fuse_silu_mul)),
                                          _enum(out_dtype, OUT_DTYPES), fmt, lay, float(eps),
                                          _ptr(q), int(q_rows), _ptr(s), _stream(stream))
    return _check("ptgq_quant_padded", rc) if check else rc


def ptgq_quant_masked(x, in_dtype, E, tokens_pad, K, group_size, fuse_silu_mul, masked_m,
                      expected_m, out_dtype, scale_fmt, scale_layout, eps, q, s, stream=None,
                      check=True):
    ind, fmt, lay = _enum(in_dtype, IN_DTYPES), _enum(scale_fmt, SCALE_FMTS), _enum(scale_layout, SCALE_LAYOUTS)
    if E > 0 and tokens_pad > 0 and K > 0 and ind in _IN_SIZE:
        fn = "ptgq_quant_masked"
        _need(x, E * tokens_pad * K * (2 if fuse_silu_mul else 1) * _IN_SIZE[ind], fn, "x")
        _need(q, E * tokens_pad * K, fn, "q")
        _need(s, E * ptgq_scale_bytes(tokens_pad, K, group_size, fmt, lay), fn, "s")
        _need(masked_m, 4 * E, fn, "masked_m")
    rc = load_library().ptgq_quant_masked(
        _ptr(x), _enum(in_dtype, IN_DTYPES), E, tokens_pad, K, group_size,
        int(bool(fuse_silu_mul)), _ptr(masked_m), int(expected_m), _enum(out_dtype, OUT_DTYPES),
        _enum(scale_fmt, SCALE_FMTS), _enum(scale_layout, SCALE_LAYOUTS), float(eps), _ptr(q),
        _ptr(s), _stream(stream))
    return _check("ptgq_quant_masked", rc) if check else rc


def ptq_quant_fp8(x, in_dtype, M, K, q, s, stream=None, check=True):
    ind = _enum(in_dtype, IN_DTYPES)
    if M > 0 and K > 0 and ind in _IN_SIZE:
        _need(x, M * K * _IN_SIZE[ind], "ptq_quant_fp8", "x")
        _need(q, M * K, "ptq_quant_fp8", "q")
        _need(s, 4 * M, "ptq_quant_fp8", "s")
    rc = load_library().ptq_quant_fp8(_ptr(x), _enum(in_dtype, IN_DTYPES), M, K, _ptr(q), _ptr(s),
                                      _stream(stream))
    return _check("ptq_quant_fp8", rc) if check else rc


def ptgq_requant_fp8(x, E, T, K, group_size, x_scale, scale_strides, masked_m, expected_m,
                     output_scale, out, stream=None, check=True):
    """scale_strides = (stride_e, stride_t, stride_g) in elements."""
    se, st, sg = (int(v) for v in scale_strides)
    if E > 0 and T > 0 and K > 0 and group_size > 0 and K % group_size == 0 and min(se, st, sg) >= 0:
        fn = "ptgq_requant_fp8"
        _need(x, E * T * K, fn, "x")
        _need(out, E * T * K, fn, "out")
        _need(x_scale, 4 * ((E - 1) * se + (T - 1) * st + (K // group_size - 1) * sg + 1), fn,
              "x_scale")
        _need(output_scale, 4, fn, "output_scale")
        if masked_m is not None:
            _need(masked_m, 4 * E, fn, "masked_m")
    rc = load_library().ptgq_requant_fp8(_ptr(x), E, T, K, group_size, _ptr(x_scale), se, st, sg,
                                         _ptr(masked_m), int(expected_m), _ptr(output_scale),
                                         _ptr(out), _stream(stream))
    return _check("ptgq_requant_fp8", rc) if check else rc


def ptgq_dequant(q, code_dtype, M, K, group_size, s, scale_fmt, scale_layout, out_dtype, y,
                 stream=None, check=True):
    fmt, lay = _enum(scale_fmt, SCALE_FMTS), _enum(scale_layout, SCALE_LAYOUTS)
    outd = _enum(out_dtype, IN_DTYPES)
    if M > 0 and K > 0 and outd in _IN_SIZE:
        fn = "ptgq_dequant"
        _need(q, M * K, fn, "q")
        _need(s, ptgq_scale_bytes(M, K, group_size, fmt, lay), fn, "s")
        _need(y, M * K * _IN_SIZE[outd], fn, "y")
    rc = load_library().ptgq_dequant(_ptr(q), _enum(code_dtype, OUT_DTYPES), M, K, group_size,
                                     _ptr(s), fmt, lay, outd, _ptr(y), _stream(stream))
    return _check("ptgq_dequant", rc) if check else rc


def ptgq_probe_e4m3(v, out, n, stream=None, check=True):
    if n > 0:
        _need(v, 4 * n, "ptgq_probe_e4m3", "v")
        _need(out, n, "ptgq_probe_e4m3", "out")
    rc = load_library().ptgq_probe_e4m3(_ptr(v), _ptr(out), n, _stream(stream))
    return _check("ptgq_probe_e4m3", rc) if check else rc


def ptgq_probe_silu_mul(g, u, in_dtype, path, out, n, stream=None, check=True):
    if n > 0:
        _need(g, 2 * n, "ptgq_probe_silu_mul", "g")
        _need(u, 2 * n, "ptgq_probe_silu_mul", "u")
        _need(out, 4 * n, "ptgq_probe_silu_mul", "out")
    rc = load_library().ptgq_probe_silu_mul(_ptr(g), _ptr(u), _enum(in_dtype, IN_DTYPES),
                                            int(path), _ptr(out), n, _stream(stream))
    return _check("ptgq_probe_silu_mul", rc) if check else rc


def ptgq_probe_scale(first_bits, n, eps, out_dtype, scale_fmt, scale_out, inv_out=None,
                     stream=None, check=True):
    fmt = _enum(scale_fmt, SCALE_FMTS)
    if n > 0:
        _need(scale_out, n * (4 if fmt == PTGQ_SCALE_F32 else 1), "ptgq_probe_scale", "scale_out")
        if inv_out is not None:
            _need(inv_out, 4 * n, "ptgq_probe_scale", "inv_out")
    rc = load_library().ptgq_probe_scale(int(first_bits), int(n), float(eps),
                                         _enum(out_dtype, OUT_DTYPES), fmt, _ptr(scale_out),
                                         _ptr(inv_out), _stream(stream))
    return _check("ptgq_probe_scale", rc) if check else rc


def ptgq_probe_int8(first_bits, n, out, stream=None, check=True):
    if n > 0:
        _need(out, n, "ptgq_probe_int8", "out")
    rc = load_library().ptgq_probe_int8(int(first_bits), int(n), _ptr(out), _stream(stream))
    return _check("ptgq_probe_int8", rc) if check else rc


def ptgq_probe_stream(x, n, q, stream=None, check=True):
    if n > 0:
        _need(x, 2 * n, "ptgq_probe_stream", "x")
        _need(q, n, "ptgq_probe_stream", "q")
    rc = load_library().ptgq_probe_stream(_ptr(x), int(n), _ptr(q), _stream(stream))
    return _check("ptgq_probe_stream", rc) if check else rc


def ptgq_diag_fastdiv(d, n):
    """floor(n / d) for a host numpy array n (uint32, each < 2^31) by the
    kernels' multiply-high division.  Host only."""
    import numpy as np
    n = np.ascontiguousarray(n, dtype=np.uint32)
    q = np.empty_like(n)
    rc = load_library().ptgq_diag_fastdiv(int(d), ctypes.c_void_p(n.ctypes.data),
                                          ctypes.c_void_p(q.ctypes.data), n.size)
    _check("ptgq_diag_fastdiv", rc)
    return q
