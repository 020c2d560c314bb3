"""Seeded synthetic inputs for the five quantization workloads.

This module holds no quantization arithmetic: it only draws random numbers and
rounds them to the input dtype.  Both the GPU tests/benchmark and the CPU
oracle take their inputs from here.

Generator (stated so it can be re-implemented anywhere):
  * SplitMix64 (Steele, Lea & Flood, 2014): output i of a stream with seed s is
    mix64(s + (i+1) * 0x9E3779B97F4A7C15) mod 2^64.  Sub-streams use the seed
    mix64(s ^ (k * 0xD1B54A32D192ED03)) for k = 1, 2, ...
  * uniform in (0, 1]: ((z >> 11) + 1) * 2^-53.
  * normal: Box-Muller in float64 on consecutive uniform pairs (u1, u2):
    sqrt(-2 ln u1) * (cos 2 pi u2, sin 2 pi u2), then rounded to float32 (RN)
    and to bf16 / fp16 (round-to-nearest-even).
  * seeds: 1000 * config + index of M in the config's M list (0-based).

Workloads (shapes and distributions of the activation-quantization configs):
  1  bf16 [64, 2048] N(0,1), 4 outlier channels x50, 2 all-zero (row, group)s
  2  bf16 [M, 7168] N(0,1), 72 outlier channels (1 % of 7168) x30,
     M in {1, 16, 256, 4096, 16384}; stands in for DeepSeek-V3 activations,
     whose real values need model weights this repository does not have
  3  bf16 [M, 2*4096] gate|up, each N(0,1), M in {1, 64, 2048, 8192}
  4  bf16 [32, 384, 2*2048] N(0,1); masked_m[0]=0, masked_m[1]=384, the
     others uniform integers in [0, 384]
  5  fp16 [8192, 3584] N(0,1);  5c: uniform integers in [-8, 8]
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_SUB = 0xD1B54A32D192ED03
_MASK64 = (1 << 64) - 1

CFG2_M = (1, 16, 256, 4096, 16384)
CFG3_M = (1, 64, 2048, 8192)
CHUNK = 1 << 22


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def substream(seed: int, k: int) -> int:
    return _mix64_int(seed ^ ((k * _SUB) & _MASK64))


def splitmix64(seed: int, start: int, n: int) -> np.ndarray:
    """Outputs start .. start+n-1 of the SplitMix64 stream with this seed."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed & _MASK64) + i * GAMMA
        return _mix64(z)


def uniform(seed: int, start: int, n: int) -> np.ndarray:
    z = splitmix64(seed, start, n)
    return ((z >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def distinct(seed: int, n: int, k: int) -> np.ndarray:
    """k distinct indices of range(n), by a partial Fisher-Yates shuffle."""
    z = splitmix64(seed, 0, k)
    idx = np.arange(n, dtype=np.int64)
    for i in range(k):
        j = i + int(z[i] % np.uint64(n - i))
        idx[i], idx[j] = idx[j], idx[i]
    return idx[:k].copy()


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64/float32 -> float32 (RN) -> bf16 bit patterns (RNE)."""
    f = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    with np.errstate(over="ignore"):
        r = (f + np.uint32(0x7FFF) + ((f >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def to_fp16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RN) -> fp16 bit patterns (RNE, numpy's cast)."""
    return np.asarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(seed, shape, scale_cols=None, factor=1.0):
    """N(0,1) in float64, optional column outlier factor, -> bf16 bits."""
    rows = int(np.prod(shape[:-1]))
    cols = shape[-1]
    out = np.empty((rows, cols), dtype=np.uint16)
    rows_per = max(1, CHUNK // cols)
    colmul = None
    if scale_cols is not None:
        colmul = np.ones(cols, dtype=np.float64)
        colmul[scale_cols] = factor
    for r0 in range(0, rows, rows_per):
        r1 = min(rows, r0 + rows_per)
        n0 = r0 * cols
        vals = _normal_range(seed, n0, (r1 - r0) * cols).reshape(r1 - r0, cols)
        if colmul is not None:
            vals = vals * colmul
        out[r0:r1] = to_bf16_bits(vals)
    return out.reshape(shape)


def _normal_range(seed: int, start: int, n: int) -> np.ndarray:
    """Normals start .. start+n-1 of the stream (start must be even)."""
    assert start % 2 == 0
    npairs = (n + 1) // 2
    u = uniform(seed, start, 2 * npairs)
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    t = 2.0 * np.pi * u[1::2]
    pair = np.empty(2 * npairs, dtype=np.float64)
    pair[0::2] = r * np.cos(t)
    pair[1::2] = r * np.sin(t)
    return pair[:n]


# ---------------------------------------------------------------- workloads

def cfg1(seed: int = 1000):
    """bf16 [64, 2048], 4 outlier channels x50, 2 zero (row, group) pairs."""
    M, K, G = 64, 2048, 128
    ch = distinct(substream(seed, 1), K, 4)
    x = _normal_bf16(seed, (M, K), scale_cols=ch, factor=50.0)
    zg = distinct(substream(seed, 2), M * (K // G), 2)
    for f in zg:
        m, g = divmod(int(f), K // G)
        x[m, g * G:(g + 1) * G] = 0
    return {"x": x, "M": M, "K": K, "G": G, "outlier_channels": ch, "zero_groups": zg,
            "in_dtype": "bf16", "eps": 1e-10}


def cfg2(M: int, seed: int = None):
    """bf16 [M, 7168] N(0,1) with 72 outlier channels x30."""
    K = 7168
    if seed is None:
        seed = 2000 + CFG2_M.index(M)
    ch = distinct(substream(seed, 1), K, 72)
    x = _normal_bf16(seed, (M, K), scale_cols=ch, factor=30.0)
    return {"x": x, "M": M, "K": K, "G": 128, "outlier_channels": ch, "in_dtype": "bf16",
            "eps": 1e-10}


def cfg3(M: int, seed: int = None):
    """bf16 [M, 2*4096] (gate | up), each N(0,1) i.i.d."""
    K = 4096
    if seed is None:
        seed = 3000 + CFG3_M.index(M)
    x = _normal_bf16(seed, (M, 2 * K))
    return {"x": x, "M": M, "K": K, "G": 128, "in_dtype": "bf16", "eps": 1e-10}


def cfg4(seed: int = 4000, E: int = 32, T: int = 384, K: int = 2048):
    """bf16 [E, T, 2K] gate|up N(0,1); masked_m with 0 and T forced in."""
    x = _normal_bf16(seed, (E, T, 2 * K))
    z = splitmix64(substream(seed, 1), 0, E)
    mm = (z % np.uint64(T + 1)).astype(np.int32)
    if E > 0:
        mm[0] = 0
    if E > 1:
        mm[1] = T
    return {"x": x, "E": E, "T": T, "K": K, "G": 128, "masked_m": mm, "in_dtype": "bf16",
            "eps": 1e-10}


def cfg5(seed: int = 5000, M: int = 8192, K: int = 3584):
    """fp16 [M, K] N(0,1) (K 128-aligned, not 1024-aligned)."""
    out = np.empty((M, K), dtype=np.uint16)
    rows_per = max(1, CHUNK // K)
    for r0 in range(0, M, rows_per):
        r1 = min(M, r0 + rows_per)
        out[r0:r1] = to_fp16_bits(_normal_range(seed, r0 * K, (r1 - r0) * K)).reshape(r1 - r0, K)
    return {"x": out, "M": M, "K": K, "in_dtype": "fp16", "eps": 1e-10}


def cfg5c(seed: int = 5002, M: int = 8192, K: int = 3584):
    """fp16 [M, K] of uniform integers in [-8, 8] (exactness family)."""
    z = splitmix64(seed, 0, M * K)
    v = (z % np.uint64(17)).astype(np.int64) - 8
    return {"x": to_fp16_bits(v.astype(np.float64)).reshape(M, K), "M": M, "K": K,
            "in_dtype": "fp16", "eps": 1e-10}


def normal_bf16(seed: int, shape, factor_cols=None, factor=1.0):
    """Generic N(0,1) bf16 tensor of any shape (parity cases at other sizes)."""
    return _normal_bf16(seed, tuple(shape), scale_cols=factor_cols, factor=factor)


def normal_fp16(seed: int, shape):
    n = int(np.prod(shape))
    return to_fp16_bits(_normal_range(seed, 0, n)).reshape(shape)


def normal_f32(seed: int, shape):
    n = int(np.prod(shape))
    return _normal_range(seed, 0, n).astype(np.float32).reshape(shape)


def fnv1a(b: np.ndarray) -> str:
    """FNV-1a 64-bit checksum of an array's bytes (recorded beside results)."""
    data = np.ascontiguousarray(b).view(np.uint8).ravel()
    h = 0xCBF29CE484222325
    # process 8 bytes per step via numpy is not FNV; keep it exact but cheap by
    # hashing a 64 KiB stride sample plus the length for large arrays.
    if data.size > (1 << 20):
        data = np.concatenate([data[:: max(1, data.size // 65536)], np.frombuffer(
            np.int64(data.size).tobytes(), dtype=np.uint8)])
    for byte in data.tobytes():
        h ^= byte
        h = (h * 0x100000001B3) & _MASK64
    return f"{h:016x}"
