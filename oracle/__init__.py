"""CPU oracle for per-token-group 8-bit activation quantization (numpy facade).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
does, and this package imports nothing from it: the two share no code.

The arithmetic lives in ``ptgq_oracle.c`` (plain single-threaded C, IEEE fp32);
this module only marshals numpy arrays into it.  Argument names follow the
pages: ``in_dtype`` in {"bf16", "fp16", "fp32"}, ``out_dtype`` in {"e4m3",
"int8"}, ``scale_fmt`` in {"f32", "ue8m0"}, ``scale_layout`` in {"row", "col"}.
Inputs are 16-bit patterns as ``numpy.uint16`` (bf16/fp16) or ``numpy.float32``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_IN = {"bf16": 0, "fp16": 1, "fp32": 2}
_OUT = {"e4m3": 0, "int8": 1}
_FMT = {"f32": 0, "ue8m0": 1}
_LAY = {"row": 0, "col": 1}

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        lib.oracle_ptgq.argtypes = [vp, i32, i64, i64, i32, i32, i32, i32, i32, f32, vp, vp]
        lib.oracle_ptgq.restype = i32
        lib.oracle_ptgq_masked.argtypes = [vp, i32, i64, i64, i64, i32, i32, vp, i32, i32, i32,
                                           f32, vp, vp]
        lib.oracle_ptgq_masked.restype = i32
        lib.oracle_ptq_fp8.argtypes = [vp, i32, i64, i64, vp, vp]
        lib.oracle_ptq_fp8.restype = i32
        lib.oracle_scale_bytes.argtypes = [i64, i64, i32, i32, i32]
        lib.oracle_scale_bytes.restype = ctypes.c_size_t
        for name in ("oracle_e4m3_vec", "oracle_int8_vec", "oracle_exp_vec"):
            getattr(lib, name).argtypes = [vp, vp, i64]
            getattr(lib, name).restype = None
        lib.oracle_silu_mul_vec.argtypes = [vp, vp, vp, i64]
        lib.oracle_silu_mul_vec.restype = None
        lib.oracle_decode_vec.argtypes = [vp, i32, vp, i64]
        lib.oracle_decode_vec.restype = None
        lib.oracle_requant_fp8.argtypes = [vp, i64, i64, i64, i32, vp, i64, i64, i64, vp, f32, vp]
        lib.oracle_requant_fp8.restype = i32
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = f32
        lib.oracle_dequant.argtypes = [vp, i32, i64, i64, i32, vp, i32, i32, i32, vp]
        lib.oracle_dequant.restype = i32
        for name in ("oracle_bf16_rne_vec", "oracle_fp16_rne_vec"):
            getattr(lib, name).argtypes = [vp, vp, i64]
            getattr(lib, name).restype = None
        lib.oracle_scale_vec.argtypes = [vp, i64, f32, i32, i32, vp, vp, vp]
        lib.oracle_scale_vec.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _check_input(x: np.ndarray, in_dtype: str):
    want = np.float32 if in_dtype == "fp32" else np.uint16
    if x.dtype != want:
        raise TypeError(f"{in_dtype} input must be a numpy {want.__name__} array")
    return np.ascontiguousarray(x)


def scale_bytes(rows: int, K: int, G: int, scale_fmt: str, scale_layout: str) -> int:
    return int(_load().oracle_scale_bytes(rows, K, G, _FMT[scale_fmt], _LAY[scale_layout]))


def ptgq(x, in_dtype, M, K, G, fuse, out_dtype, scale_fmt, scale_layout, eps=1e-10):
    """Flat per-token-group quantization; returns (codes uint8 [M,K], scale bytes uint8)."""
    x = _check_input(x, in_dtype)
    width = 2 * K if fuse else K
    assert x.size == M * width
    q = np.empty((M, K), dtype=np.uint8)
    s = np.zeros(scale_bytes(M, K, G, scale_fmt, scale_layout), dtype=np.uint8)
    rc = _load().oracle_ptgq(_ptr(x), _IN[in_dtype], M, K, G, int(bool(fuse)), _OUT[out_dtype],
                             _FMT[scale_fmt], _LAY[scale_layout], eps, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_ptgq rejected its arguments")
    return q, s


def ptgq_masked(x, in_dtype, E, T, K, G, fuse, masked_m, out_dtype, scale_fmt, scale_layout,
                eps=1e-10, q_init=None, s_init=None):
    """Masked MoE-layout quantization.  ``q_init``/``s_init`` are the caller's
    prefilled buffers (sentinels); rows past masked_m keep them."""
    x = _check_input(x, in_dtype)
    width = 2 * K if fuse else K
    assert x.size == E * T * width
    mm = np.ascontiguousarray(masked_m, dtype=np.int32)
    assert mm.size == E
    sb = scale_bytes(T, K, G, scale_fmt, scale_layout)
    q = np.array(q_init, dtype=np.uint8, copy=True).reshape(E, T, K) if q_init is not None \
        else np.zeros((E, T, K), dtype=np.uint8)
    s = np.array(s_init, dtype=np.uint8, copy=True).reshape(E * sb) if s_init is not None \
        else np.zeros(E * sb, dtype=np.uint8)
    rc = _load().oracle_ptgq_masked(_ptr(x), _IN[in_dtype], E, T, K, G, int(bool(fuse)),
                                    _ptr(mm), _OUT[out_dtype], _FMT[scale_fmt],
                                    _LAY[scale_layout], eps, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_ptgq_masked rejected its arguments")
    return q, s


def ptq_fp8(x, in_dtype, M, K):
    """Whole-row per-token e4m3; returns (codes uint8 [M,K], scales float32 [M])."""
    x = _check_input(x, in_dtype)
    assert x.size == M * K
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty(M, dtype=np.float32)
    rc = _load().oracle_ptq_fp8(_ptr(x), _IN[in_dtype], M, K, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_ptq_fp8 rejected its arguments")
    return q, s


def requant_fp8(x, E, T, K, G, x_scale, strides, masked_m, output_scale, out_init=None):
    """Per-token-group fp8 -> per-tensor fp8 requantization of x [E, T, K]
    (uint8 e4m3 codes) with group scales x_scale (float32, element (e, t, g) at
    e*strides[0] + t*strides[1] + g*strides[2]); rows past masked_m keep
    out_init (None: every row is live when masked_m is None)."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    assert x.size == E * T * K
    xs = np.ascontiguousarray(x_scale, dtype=np.float32)
    out = np.array(out_init, dtype=np.uint8, copy=True).reshape(E, T, K) if out_init is not None \
        else np.zeros((E, T, K), dtype=np.uint8)
    mm = None if masked_m is None else np.ascontiguousarray(masked_m, dtype=np.int32)
    rc = _load().oracle_requant_fp8(_ptr(x), E, T, K, G, _ptr(xs), int(strides[0]),
                                    int(strides[1]), int(strides[2]),
                                    None if mm is None else _ptr(mm), float(output_scale),
                                    _ptr(out))
    if rc != 0:
        raise ValueError("oracle_requant_fp8 rejected its arguments")
    return out


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    table = np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float32)
    return table[np.asarray(codes, dtype=np.uint8)]


def dequant(q, code_dtype, M, K, G, s, scale_fmt, scale_layout, out_dtype):
    """codes [M, K] (uint8, e4m3 or int8) x group scales -> y [M, K] as bf16 /
    fp16 bit patterns (uint16) or float32."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    assert q.size == M * K
    s = np.ascontiguousarray(s).view(np.uint8)
    y = np.empty((M, K), dtype=np.float32 if out_dtype == "fp32" else np.uint16)
    rc = _load().oracle_dequant(_ptr(q), _OUT[code_dtype], M, K, G, _ptr(s), _FMT[scale_fmt],
                                _LAY[scale_layout], _IN[out_dtype], _ptr(y))
    if rc != 0:
        raise ValueError("oracle_dequant rejected its arguments")
    return y


def bf16_rne(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_bf16_rne_vec(_ptr(v), _ptr(out), v.size)
    return out


def fp16_rne(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_fp16_rne_vec(_ptr(v), _ptr(out), v.size)
    return out


# ---- element helpers (for pinning single steps) ----

def e4m3(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().oracle_e4m3_vec(_ptr(v), _ptr(out), v.size)
    return out


def scale(amax, eps, out_dtype, scale_fmt):
    """The scale of groups with the given absmax values (float32 array):
    (r float32, UE8M0 byte uint8, multiplier float32), as the quantizer makes
    them (the byte is 0 for the fp32 format)."""
    a = np.ascontiguousarray(amax, dtype=np.float32)
    r = np.empty(a.shape, dtype=np.float32)
    e = np.empty(a.shape, dtype=np.uint8)
    inv = np.empty(a.shape, dtype=np.float32)
    _load().oracle_scale_vec(_ptr(a), a.size, float(eps), _OUT[out_dtype],
                             int(scale_fmt == "ue8m0"), _ptr(r), _ptr(e), _ptr(inv))
    return r, e, inv


def int8(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.int8)
    _load().oracle_int8_vec(_ptr(v), _ptr(out), v.size)
    return out


def exp_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.float32)
    _load().oracle_exp_vec(_ptr(x), _ptr(out), x.size)
    return out


def silu_mul(g, u) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    assert g.shape == u.shape
    out = np.empty(g.shape, dtype=np.float32)
    _load().oracle_silu_mul_vec(_ptr(g), _ptr(u), _ptr(out), g.size)
    return out


def decode(h, in_dtype: str) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    _load().oracle_decode_vec(_ptr(h), _IN[in_dtype], _ptr(out), h.size)
    return out


def lib_path() -> str:
    return os.path.abspath(_build.LIB)
