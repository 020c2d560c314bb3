"""Invariants and closed forms that hold for the oracle's outputs at any size:
exactness family, dequantization error bound, layout equivalences, masked-row
sentinels, and per-token == group quantization with G = K and eps = 0."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

F8 = torch.float8_e4m3fn


def decode_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(F8).to(torch.float64).numpy()


def decode_codes(codes, out_dtype):
    if out_dtype == "e4m3":
        return decode_e4m3(codes)
    return codes.view(np.int8).astype(np.float64)


def scales_rowmajor(s, M, ng, fmt, layout):
    """Scale tensor -> float64 [M, ng] (independent of the oracle's own writer)."""
    if layout == "row":
        if fmt == "f32":
            return s.view(np.float32).reshape(M, ng).astype(np.float64)
        return np.ldexp(1.0, s.reshape(M, ng).astype(np.int64) - 127)
    Mp = (M + 3) // 4 * 4
    if fmt == "f32":
        return s.view(np.float32).reshape(ng, Mp)[:, :M].T.astype(np.float64)
    W_ = (ng + 3) // 4
    b = s.reshape(W_, Mp, 4)                  # word (c, m), byte j -> group 4c+j
    out = np.empty((M, ng), dtype=np.float64)
    for g in range(ng):
        out[:, g] = np.ldexp(1.0, b[g // 4, :M, g % 4].astype(np.int64) - 127)
    return out


def ulp_e4m3(a):
    a = np.abs(a)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)


@pytest.mark.parametrize("G", [16, 32, 64, 128])
@pytest.mark.parametrize("out_dtype", ["int8", "e4m3"])
def test_exactness_family(G, out_dtype):
    """Integers in [-8, 8] with power-of-two scales dequantize exactly
    (the technique of the sglang #35593 page's unit test)."""
    d = W.cfg5c(M=48, K=3584)
    x, M, K = d["x"], d["M"], d["K"]
    q, s = oracle.ptgq(x, "fp16", M, K, G, False, out_dtype, "ue8m0", "row")
    deq = decode_codes(q, out_dtype).reshape(M, K // G, G) * \
        scales_rowmajor(s, M, K // G, "ue8m0", "row")[:, :, None]
    xf = x.view(np.float16).astype(np.float64).reshape(M, K // G, G)
    assert np.array_equal(deq, xf)


CASES = [(fmt, lay, od) for fmt in ("f32", "ue8m0") for lay in ("row", "col")
         for od in ("e4m3", "int8")]


@pytest.mark.parametrize("fmt,layout,out_dtype", CASES)
@pytest.mark.parametrize("fuse", [False, True])
def test_dequant_error_bound(fmt, layout, out_dtype, fuse):
    """|decode(code) * scale - y| <= half an output ulp times the scale, plus,
    for fp32 scales, the drift of the two fp32 roundings in y * fl(1/scale)."""
    M, K, G = 37, 512, 128
    x = W.normal_bf16(77, (M, 2 * K if fuse else K), factor_cols=[3, 200], factor=40.0)
    q, s = oracle.ptgq(x, "bf16", M, K, G, fuse, out_dtype, fmt, layout)
    xf = W.bf16_bits_to_f32(x).reshape(M, -1)
    y = oracle.silu_mul(xf[:, :K], xf[:, K:]) if fuse else xf
    y = y.astype(np.float64).reshape(M, K // G, G)
    sc = scales_rowmajor(s, M, K // G, fmt, layout)[:, :, None]
    deq = decode_codes(q, out_dtype).reshape(M, K // G, G) * sc
    # v = fl(y * fl(1/s)) is within |y/s| * 2^-22 of y/s (two roundings), and the
    # code within half an output ulp of v; UE8M0 multipliers are exact.
    t = np.abs(y / sc)
    drift = t * 2.0 ** -22 if fmt == "f32" else 0.0 * t
    ulp = ulp_e4m3(t + drift) if out_dtype == "e4m3" else np.ones_like(t)
    bound = (0.5 * ulp + drift) * sc
    assert np.all(np.abs(deq - y) <= bound)
    # and the scale is the group absmax over the format maximum (rounded)
    qmax = 448.0 if out_dtype == "e4m3" else 127.0
    amax = np.maximum(np.abs(y).max(axis=2), 1e-10)
    r = (amax / qmax)[:, :, None]
    if fmt == "f32":
        assert np.all(np.abs(sc - r) <= r * 2.0 ** -23)
    else:
        assert np.all((sc >= r * (1 - 2.0 ** -23)) & (sc < 2 * r * (1 + 2.0 ** -23)))


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_layouts_hold_the_same_scales_and_pads_are_zero(fmt):
    for M in (1, 3, 4, 5, 18):
        for K, G in ((2048, 128), (384, 128), (640, 128), (96, 32)):
            x = W.normal_bf16(M * 1000 + K, (M, K))
            q1, s1 = oracle.ptgq(x, "bf16", M, K, G, False, "e4m3", fmt, "row")
            q2, s2 = oracle.ptgq(x, "bf16", M, K, G, False, "e4m3", fmt, "col")
            ng = K // G
            assert np.array_equal(q1, q2)
            assert np.array_equal(scales_rowmajor(s1, M, ng, fmt, "row"),
                                  scales_rowmajor(s2, M, ng, fmt, "col"))
            Mp = (M + 3) // 4 * 4
            if fmt == "f32":
                c = s2.view(np.float32).reshape(ng, Mp)
                assert np.all(c[:, M:] == 0)
            else:
                b = s2.reshape((ng + 3) // 4, Mp, 4)
                assert np.all(b[:, M:, :] == 0)
                for g in range(ng, (ng + 3) // 4 * 4):
                    assert np.all(b[g // 4, :, g % 4] == 0)


@pytest.mark.parametrize("fmt,layout", [("ue8m0", "col"), ("f32", "row"), ("f32", "col"),
                                        ("ue8m0", "row")])
def test_masked_matches_flat_on_live_rows_and_keeps_sentinels(fmt, layout):
    d = W.cfg4(seed=4100, E=6, T=21, K=256)
    x, E, T, K, mm = d["x"], d["E"], d["T"], d["K"], d["masked_m"].copy()
    mm[2] = -5          # negative counts as 0
    mm[3] = T + 40      # above T counts as T
    sb = oracle.scale_bytes(T, K, 128, fmt, layout)
    q0 = np.full((E, T, K), 0x7F, np.uint8)
    s0 = np.full(E * sb, 0xFF, np.uint8)
    q, s = oracle.ptgq_masked(x, "bf16", E, T, K, 128, True, mm, "e4m3", fmt, layout,
                              q_init=q0, s_init=s0)
    ng = K // 128
    for e in range(E):
        live = int(min(max(mm[e], 0), T))
        assert np.all(q[e, live:] == 0x7F)
        se = s[e * sb:(e + 1) * sb]
        if live:
            qf, sf = oracle.ptgq(np.ascontiguousarray(x[e, :live]), "bf16", live, K, 128, True,
                                 "e4m3", fmt, "row")
            assert np.array_equal(q[e, :live], qf)
            got = scales_rowmajor(se, T, ng, fmt, layout)[:live] if layout == "col" else \
                scales_rowmajor(se[: live * ng * (4 if fmt == "f32" else 1)], live, ng, fmt, "row")
            assert np.array_equal(got, scales_rowmajor(sf, live, ng, fmt, "row"))
        # every scale slot of a dead row is untouched
        per = 4 if fmt == "f32" else 1
        if layout == "row":
            assert np.all(se[live * ng * per:] == 0xFF)
        elif fmt == "f32":
            c = se.reshape(ng, -1, 4)
            assert np.all(c[:, live:, :] == 0xFF)
        else:
            c = se.reshape((ng + 3) // 4, -1, 4)
            assert np.all(c[:, live:, :] == 0xFF)


@pytest.mark.parametrize("in_dtype", ["bf16", "fp16"])
def test_per_token_equals_group_quant_with_G_equal_K_and_no_floor(in_dtype):
    M = 64
    x = W.normal_bf16(9, (M, 128)) if in_dtype == "bf16" else W.normal_fp16(9, (M, 128))
    x[5] = 0                                  # a zero row: scale 0, codes 0
    qt, st = oracle.ptq_fp8(x, in_dtype, M, 128)
    qg, sg = oracle.ptgq(x, in_dtype, M, 128, 128, False, "e4m3", "f32", "row", eps=0.0)
    assert np.array_equal(qt, qg)
    assert np.array_equal(st.view(np.uint32), sg.view(np.uint32))
    assert st[5] == 0 and np.all(qt[5] == 0)


def test_per_token_fp32_input_and_dequant_bound():
    M, K = 9, 1076
    x = W.normal_f32(5, (M, K)) * np.float32(3.0)
    q, s = oracle.ptq_fp8(x, "fp32", M, K)
    assert np.array_equal(s, (np.abs(x).max(axis=1) / np.float32(448.0)).astype(np.float32))
    deq = decode_e4m3(q) * s[:, None].astype(np.float64)
    t = np.abs(x.astype(np.float64) / s[:, None])
    bound = (0.5 * ulp_e4m3(t * (1 + 2.0 ** -22)) + t * 2.0 ** -22) * s[:, None]
    assert np.all(np.abs(deq - x) <= bound)


def test_rejects_bad_arguments():
    x = np.zeros((2, 100), np.uint16)
    with pytest.raises(ValueError):
        oracle.ptgq(x, "bf16", 2, 100, 128, False, "e4m3", "f32", "row")   # K % G != 0
    x = np.zeros((2, 96), np.uint16)
    with pytest.raises(ValueError):
        oracle.ptgq(x, "bf16", 2, 96, 48, False, "e4m3", "f32", "row")    # G not a power of 2


@pytest.mark.parametrize("fmt,layout", [("f32", "row"), ("ue8m0", "col")])
@pytest.mark.parametrize("out_dtype", ["e4m3", "int8"])
def test_fp32_input_equals_16bit_input_on_the_same_values(out_dtype, fmt, layout):
    """Decoding is the only step that depends on the input dtype: fp32 inputs
    holding bf16 (or fp16) values give the bf16 (fp16) results byte for byte."""
    M, K, G = 9, 640, 64
    xb = W.normal_bf16(91, (M, K), factor_cols=[3], factor=40.0)
    xh = W.normal_fp16(92, (M, K))
    for x, dt in ((xb, "bf16"), (xh, "fp16")):
        xf = oracle.decode(x, dt).reshape(M, K)
        assert np.array_equal(np.asarray(oracle.ptgq(xf, "fp32", M, K, G, False, out_dtype, fmt,
                                                     layout)[0]),
                              oracle.ptgq(x, dt, M, K, G, False, out_dtype, fmt, layout)[0])
        assert np.array_equal(oracle.ptgq(xf, "fp32", M, K, G, False, out_dtype, fmt, layout)[1],
                              oracle.ptgq(x, dt, M, K, G, False, out_dtype, fmt, layout)[1])


def test_fp32_input_keeps_what_16bit_inputs_cannot_hold():
    """An fp32 value between two bf16 values is quantized from its own value:
    with a unit UE8M0 scale (amax 448) 1.0625 (e4m3 tie between 1.0 and
    1.125 -> even 1.0) and the next fp32 above it (-> 1.125, no bf16 or fp16
    holds it) give different codes."""
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 448.0
    x[0, 1] = 1.0625
    x[0, 2] = np.nextafter(np.float32(1.0625), np.float32(2))
    q, s = oracle.ptgq(x, "fp32", 1, 128, 128, False, "e4m3", "ue8m0", "row")
    assert s[0] == 0x7F
    assert list(q[0, :3]) == [0x7E, 0x38, 0x39]


def test_fused_fp32_is_rejected():
    with pytest.raises(ValueError):
        oracle.ptgq(np.zeros((1, 256), np.float32), "fp32", 1, 128, 128, True, "e4m3", "f32",
                    "row")


@pytest.mark.parametrize("in_dtype", ["bf16", "fp16", "fp32"])
def test_masked_expert_equals_flat_call_on_its_rows(in_dtype):
    """Each expert's live rows are a flat call on that expert's slice (its own
    scale tensor of tokens_pad rows); other rows keep the sentinels."""
    E, T, K, G = 4, 9, 384, 128
    if in_dtype == "fp32":
        x = W.normal_f32(61, (E, T, K))
    elif in_dtype == "fp16":
        x = W.normal_fp16(62, (E, T, K))
    else:
        x = W.normal_bf16(63, (E, T, K))
    mm = np.array([9, 0, 4, 12], np.int32)
    sb = oracle.scale_bytes(T, K, G, "f32", "row")
    q, s = oracle.ptgq_masked(x, in_dtype, E, T, K, G, False, mm, "e4m3", "f32", "row",
                              q_init=np.full((E, T, K), 0x7F, np.uint8),
                              s_init=np.full(E * sb, 0xFF, np.uint8))
    for e in range(E):
        live = int(min(max(mm[e], 0), T))
        if live:
            fq, fs = oracle.ptgq(np.ascontiguousarray(x[e, :live]), in_dtype, live, K, G, False,
                                 "e4m3", "f32", "row")
            assert np.array_equal(q[e, :live], fq)
            assert np.array_equal(s[e * sb:e * sb + fs.size], fs)
        assert np.all(q[e, live:] == 0x7F)
        assert np.all(s[e * sb + live * (K // G) * 4:(e + 1) * sb] == 0xFF)


def tiny_rows(seed, M, K, in_dtype):
    """Rows whose largest magnitude lies in [1e-38, 4e-36] (normal fp32 and
    bf16 values included), a quarter of each row zeros of both signs, one row
    all zero and one row of ordinary size (its multiplier stays finite)."""
    rng = np.random.default_rng(seed)
    amax = np.exp(rng.uniform(np.log(1e-38), np.log(4e-36), M))
    y = rng.uniform(-1.0, 1.0, (M, K)) * amax[:, None]
    y[rng.random((M, K)) < 0.25] = 0.0
    y[rng.random((M, K)) < 0.1] = -0.0
    y[1] = 0.0
    y[2] = rng.normal(size=K)
    if in_dtype == "fp32":
        return y.astype(np.float32)
    return W.to_bf16_bits(y)


def codes_from_multiplier(y, inv, out_dtype):
    """Codes of y (float32) times a per-row or per-group multiplier: where the
    multiplier is infinite, zeros keep their sign and the rest saturate;
    elsewhere torch's saturating e4m3 cast / numpy rint of the fp32 product."""
    with np.errstate(invalid="ignore", over="ignore"):
        v = (y * inv).astype(np.float32)
    v = np.where(y == 0, y, v)
    if out_dtype == "e4m3":
        c = torch.from_numpy(np.clip(v, -448.0, 448.0)).to(F8).view(torch.uint8).numpy()
    else:
        c = np.clip(np.rint(v.astype(np.float64)), -128, 127).astype(np.int8).view(np.uint8)
    return c


@pytest.mark.parametrize("in_dtype", ["bf16", "fp32"])
def test_overflowed_multiplier_per_token(in_dtype):
    """Per-token rows with a maximum below ~1.3e-36: 1 / (max / 448) overflows
    to +inf (numpy's IEEE quotients decide where); zeros keep their sign, the
    other elements saturate to +-448."""
    M, K = 16, 256
    x = tiny_rows(71, M, K, in_dtype)
    y = x if in_dtype == "fp32" else oracle.decode(x, "bf16").reshape(M, K)
    q, s = oracle.ptq_fp8(x, in_dtype, M, K)
    r = (np.abs(y).max(axis=1) / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(s.view(np.uint32), r.view(np.uint32))
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.where(r == 0, np.float32(0), np.float32(1.0) / r).astype(np.float32)
    assert np.isinf(inv).sum() >= M // 2          # the corner is reached
    assert np.array_equal(q, codes_from_multiplier(y, inv[:, None], "e4m3"))
    neg_zero = (y == 0) & np.signbit(y)
    assert np.all(q[neg_zero] == 0x80) and np.all(q[(y == 0) & ~np.signbit(y)] == 0x00)


@pytest.mark.parametrize("out_dtype", ["e4m3", "int8"])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp32"])
def test_overflowed_multiplier_group_fp32_scale_eps0(in_dtype, out_dtype):
    M, K, G = 12, 512, 64
    x = tiny_rows(72, M, K, in_dtype)
    y = x if in_dtype == "fp32" else oracle.decode(x, "bf16").reshape(M, K)
    q, s = oracle.ptgq(x, in_dtype, M, K, G, False, out_dtype, "f32", "row", eps=0.0)
    qmax = np.float32(448.0 if out_dtype == "e4m3" else 127.0)
    r = (np.abs(y).reshape(M, K // G, G).max(axis=2) / qmax).astype(np.float32)
    assert np.array_equal(s.view(np.float32).reshape(M, K // G).view(np.uint32), r.view(np.uint32))
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.where(r == 0, np.float32(0), np.float32(1.0) / r).astype(np.float32)
    assert np.isinf(inv).any()
    want = codes_from_multiplier(y.reshape(M, K // G, G), inv[:, :, None], out_dtype)
    assert np.array_equal(q, want.reshape(M, K))


def test_overflowed_multiplier_requant():
    """An output scale whose reciprocal overflows (1e-39): zero products keep
    their sign, the others saturate."""
    E, T, K = 2, 5, 256
    rng = np.random.default_rng(73)
    x = rng.integers(0, 256, (E, T, K)).astype(np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x00
    x[:, :, :16] = 0x80                                          # -0
    s = rng.uniform(0.5, 2.0, (E, T, K // 128)).astype(np.float32)
    os_ = np.float32(1e-39)
    with np.errstate(divide="ignore", over="ignore"):
        assert np.isinf(np.float32(1.0) / os_)
    out = oracle.requant_fp8(x, E, T, K, 128, s, (T * (K // 128), K // 128, 1), None, os_)
    dec = torch.from_numpy(x).view(F8).to(torch.float32).numpy()
    h = (dec * np.repeat(s, 128, axis=2)).astype(np.float32)
    assert np.array_equal(out, codes_from_multiplier(h, np.float32(np.inf), "e4m3"))
    assert np.all(out[:, :, :16] == 0x80)
