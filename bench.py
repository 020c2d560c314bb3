"""Benchmark: per-token-group 8-bit activation quantization on one MI355X.

Headline workload: bf16 [16384, 7168] activations (the DeepSeek-V3 hidden
size, synthetic N(0,1) with 1 % outlier channels x30), G = 128, e4m3 codes and
UE8M0 scales packed column-major with M padded to 4.  A step is one
ptgq_quant call over that batch.  Inputs are resident in HBM before timing;
buffer sets totalling >= 1 GiB are rotated so that no set is still in the
256 MB Infinity Cache when it is reused.

Printed: one JSON line.  `value` = achieved GB/s at M = 16384, where bytes are
the algorithmic bytes (bf16 read + codes written + one UE8M0 byte per group);
`per_m` gives us/call, GB/s and fraction of the 8 TB/s HBM peak at every M of
the workload; `variants` measures the fused, masked, per-token,
requantization and dequantization entry points the same way; `roofline` gives
the dominant kernel's figures; `cpu_baseline` times the CPU oracle on whole
headline steps (one thread).  That CPU-baseline leg is the only part of this
script that calls the oracle: it also runs it on sampled rows of every measured
case, whose GPU outputs were copied to the host after timing, and
`parity_sample` / each variant's `parity` hold the mismatch counts and the worst
dequantization error over its bound (null with --no-cpu-baseline).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --profile-main   (only the headline loop, for rocprofv3)
    python bench.py --profile-dequant / --profile-requant / --profile-fused [--fp16] /
                    --profile-masked / --profile-fp32 / --profile-per-token /
                    --profile-int8 [--int8-group G] / --profile-stream
                    (only that loop; --graph: the variant loops in HIP graphs)
    ... --tuning KNOB=VALUE  (profile loops only, repeatable: a launch-geometry
                              override of ptgq_set_tuning, for comparing
                              geometries under the profiler)

`roofline.achievable_GBps` is the rate of a no-arithmetic stream with the
headline kernel's traffic and geometry (ptgq_probe_stream, 2 bytes read per
byte written) timed the same way; `stream_reference` gives the same stream at
the element counts of the smaller workloads (graph figures).
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
GIB = 1 << 30
METRIC = "achieved HBM GB/s and % of peak per M; us/call at M=1..16384, K=7168"


def alg_bytes_flat(M, K, G, in_size, fuse, scale_bytes_per_group):
    """Input read + codes written + real scale entries written (no pad slots)."""
    return M * K * in_size * (2 if fuse else 1) + M * K + M * (K // G) * scale_bytes_per_group


def kernel_source_digest():
    h = hashlib.sha256()
    for rel in ("activation_quantization_amd/csrc/ptgq_kernels.hip",
                "activation_quantization_amd/csrc/ptgq_api.cpp",
                "activation_quantization_amd/csrc/ptgq_internal.h"):
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(name):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != kernel_source_digest():
        return None
    return float(m_b.group(1))


class Timer:
    """Times a list of zero-argument launch closures, cycled, on the current
    stream: per-launch HIP events give the kernel's average duration, and one
    event pair around the whole region gives the per-step time."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, calls, steps, warmup, per_launch=True):
        """Timed passes over `steps` launches: one HIP event pair around the
        whole region (launches back to back, nothing between them: the average
        launch duration, inter-launch gaps included), then, with `per_launch`,
        an event pair around every launch (each launch then starts from a
        drained queue; the events themselves add about 2 us)."""
        torch = self.torch
        for i in range(warmup):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        region0 = torch.cuda.Event(enable_timing=True)
        region1 = torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        region0.record()
        for i in range(steps):
            calls[i % len(calls)]()
        region1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        if not per_launch:
            return {"region_ms": region0.elapsed_time(region1), "wall_s": wall}
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            starts[i].record()
            calls[i % len(calls)]()
            ends[i].record()
        torch.cuda.synchronize()
        per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
        return {"region_ms": region0.elapsed_time(region1), "launch_ms_mean": float(np.mean(per)),
                "launch_ms_median": float(np.median(per)), "wall_s": wall}

    def graph(self, calls, per_graph, replays, min_ms=50.0):
        """Device time per call of `per_graph` back-to-back launches captured in
        one HIP graph (launch overhead excluded): the latency-bound small-M
        figure.  The graph is replayed at least `replays` times and for at
        least `min_ms` of device time, so that short windows of a GPU that is
        still changing clocks do not decide the figure."""
        torch = self.torch
        for c in calls:
            c()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for i in range(per_graph):
                    calls[i % len(calls)]()
        torch.cuda.current_stream().wait_stream(st)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        replays = max(replays, math.ceil(min_ms / max(e0.elapsed_time(e1), 1e-3)))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (replays * per_graph)


def variant_entry(timer, calls, nbytes, steps=100):
    """us/call and GB/s of a variant: device time per call of back-to-back
    launches captured in a HIP graph (the pages time their kernels inside
    graphs too), with the eager back-to-back figure beside it."""
    r = timer.run(calls, steps, 10)
    per_graph = max(len(calls), min(200, max(8, math.ceil(1.2e10 / max(nbytes, 1)))))
    ms = timer.graph(calls, per_graph, 5)
    us = ms * 1e3
    return {"us_per_call": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
            "frac_of_peak": round(nbytes / us / 1e3 / PEAK_GBS, 4),
            "us_per_call_eager": round(r["region_ms"] * 1e3 / steps, 2)}


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def rotation_sets(footprint, cap=64):
    return int(max(2, min(cap, math.ceil(GIB / max(footprint, 1)))))


def make_flat_sets(torch, aq, x_host, M, K, G, fuse, out_dtype, fmt, layout, in_dtype, nsets):
    dev = "cuda"
    xt = torch.from_numpy(np.ascontiguousarray(x_host).view(np.int16)).to(dev)
    sets = []
    sb = aq.ptgq_scale_bytes(M, K, G, fmt, layout)
    for i in range(nsets):
        xi = xt if i == 0 else xt.clone()
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        s = torch.empty((max(sb, 1),), dtype=torch.uint8, device=dev)
        sets.append((xi, q, s))

    def mk(xi, q, s):
        return lambda: aq.ptgq_quant(xi, in_dtype, M, K, G, fuse, out_dtype, fmt, layout, 1e-10,
                                     q, s, check=False)
    return sets, [mk(*st) for st in sets]


def stream_calls(torch, aq, M, K, nsets):
    """The no-arithmetic stream with the plain quantization kernel's traffic and
    geometry (2 bytes read per byte written, two 512-element slabs per wave,
    uncapped grid, XCD chunks) over M x K 16-bit elements, rotated buffer
    sets.  Its rate is what the memory system gives the headline's access
    pattern."""
    n = M * K
    calls = []
    for _ in range(nsets):
        xi = torch.empty(n, dtype=torch.int16, device="cuda").fill_(0x3F80)
        qi = torch.empty(n, dtype=torch.uint8, device="cuda")
        calls.append(lambda xi=xi, qi=qi: aq.ptgq_probe_stream(xi, n, qi, check=False))
    return calls, 3 * n


def dequant_calls(torch, aq):
    """Dequantization of the headline output: e4m3 codes [16384, 7168] with
    packed column-major UE8M0 scales back to bf16, over rotated buffer sets."""
    Md, Kd = 16384, 7168
    rng = np.random.default_rng(7168)
    qh = rng.integers(0, 256, (Md, Kd), dtype=np.uint8)
    qh[(qh & 0x7F) == 0x7F] = 0x38
    sbd = aq.ptgq_scale_bytes(Md, Kd, 128, "ue8m0", "col")
    sd = torch.from_numpy(rng.integers(110, 135, sbd, dtype=np.uint8)).to("cuda")
    qd = torch.from_numpy(qh).to("cuda")
    fd = Md * Kd * (1 + 2) + Md * (Kd // 128)
    cd = []
    for i in range(rotation_sets(fd)):
        qi = qd if i == 0 else qd.clone()
        yi = torch.empty((Md, Kd), dtype=torch.bfloat16, device="cuda")
        cd.append((lambda qi=qi, yi=yi: aq.ptgq_dequant(qi, "e4m3", Md, Kd, 128, sd, "ue8m0",
                                                        "col", "bf16", yi, check=False)))

    def capture():
        """Sampled rows of set 0's output, kept for the oracle comparison."""
        rows = np.unique(np.linspace(0, Md - 1, 24).astype(np.int64))
        srow = np.ascontiguousarray(rows_of_scales(sd, Md, Kd, 128, "ue8m0", "col", rows))
        qs = np.ascontiguousarray(qh[rows])
        got = cd[0].__defaults__[1][rows].view(torch.int16).cpu().numpy().view(np.uint16)

        def check(oracle):
            ref = oracle.dequant(qs, "e4m3", len(rows), Kd, 128, srow, "ue8m0", "row", "bf16")
            # the exact product code * 2^(e - 127) against the bf16 output
            exact = oracle.e4m3_decode(qs).astype(np.float64) * np.repeat(
                np.ldexp(1.0, srow.astype(np.int64) - 127), 128, axis=1)
            return {"rows": int(len(rows)), "mismatches": int((got != ref).sum()),
                    "elements": int(got.size),
                    "past_strict_bound": bf16_past_half_ulp(exact, got)}
        return check
    return cd, fd, capture


def fused_calls(torch, aq, W, fp16=False):
    """Fused silu(gate)*up quantization, bf16 [8192, 2*4096] -> e4m3 [8192, 4096]
    (fp16: N(0,1) fp16 inputs of the same shape), G = 128, UE8M0 column-major
    scales, over rotated buffer sets."""
    d3 = dict(W.cfg3(8192))
    if fp16:
        d3["x"] = W.normal_fp16(3016, (8192, 2 * 4096))
    f3 = alg_bytes_flat(8192, 4096, 128, 2, True, 1)
    s3, c3 = make_flat_sets(torch, aq, d3["x"], 8192, 4096, 128, True, "e4m3", "ue8m0",
                            "col", "fp16" if fp16 else "bf16", rotation_sets(f3))
    return d3, s3, c3, f3


def masked_calls(torch, aq, W, masked_m=None):
    """Masked MoE layout, bf16 [32, 384, 2*2048] fused, the seeded masked_m of
    the workload (or `masked_m`, e.g. one live row per expert as in decoding),
    UE8M0 column-major scales per expert, over rotated buffer sets.  Returns
    the workload (with the masked_m used), the calls, the algorithmic bytes
    (live rows only, plus masked_m) and the live row count."""
    d4 = dict(W.cfg4())
    if masked_m is not None:
        d4["masked_m"] = np.asarray(masked_m, dtype=np.int32)
    E, T, K4, mm = d4["E"], d4["T"], d4["K"], d4["masked_m"]
    live = int(np.clip(mm, 0, T).sum())
    f4 = live * (2 * K4 * 2 + K4 + K4 // 128) + 4 * E
    x4 = torch.from_numpy(d4["x"].view(np.int16)).to("cuda")
    mm_d = torch.from_numpy(mm).to("cuda")
    sb4 = aq.ptgq_scale_bytes(T, K4, 128, "ue8m0", "col")
    c4 = []
    for i in range(rotation_sets(E * T * (4 * K4 + K4))):
        xi = x4 if i == 0 else x4.clone()
        q4 = torch.empty((E, T, K4), dtype=torch.uint8, device="cuda")
        s4 = torch.empty((E * sb4,), dtype=torch.uint8, device="cuda")
        c4.append((lambda xi=xi, q4=q4, s4=s4: aq.ptgq_quant_masked(
            xi, "bf16", E, T, K4, 128, True, mm_d, int(live // E), "e4m3", "ue8m0", "col",
            1e-10, q4, s4, check=False)))
    return d4, c4, f4, live


def fp32_calls(torch, aq, W):
    """fp32 input [8192, 7168] -> e4m3, G = 128, packed column-major UE8M0
    scales, over rotated buffer sets.  Returns the host input, the calls and
    the algorithmic bytes."""
    M32, K, G = 8192, 7168, 128
    x32h = W.normal_f32(32, (M32, K))
    x32 = torch.from_numpy(x32h).to("cuda")
    f32b = alg_bytes_flat(M32, K, G, 4, False, 1)
    sb32 = aq.ptgq_scale_bytes(M32, K, G, "ue8m0", "col")
    c32 = []
    for i in range(rotation_sets(f32b)):
        xi = x32 if i == 0 else x32.clone()
        qi = torch.empty((M32, K), dtype=torch.uint8, device="cuda")
        si = torch.empty((sb32,), dtype=torch.uint8, device="cuda")
        c32.append((lambda xi=xi, qi=qi, si=si: aq.ptgq_quant(
            xi, "fp32", M32, K, G, False, "e4m3", "ue8m0", "col", 1e-10, qi, si, check=False)))
    return x32h, c32, f32b


def per_token_calls(torch, aq, d5):
    """Whole-row per-token e4m3 of the fp16 [8192, 3584] workload tensor, over
    rotated buffer sets.  Returns the calls and the algorithmic bytes."""
    f5b = 8192 * 3584 * 2 + 8192 * 3584 + 8192 * 4
    x5 = torch.from_numpy(d5["x"].view(np.int16)).to("cuda")
    c5b = []
    for i in range(rotation_sets(f5b)):
        xi = x5 if i == 0 else x5.clone()
        q5 = torch.empty((8192, 3584), dtype=torch.uint8, device="cuda")
        s5 = torch.empty((8192,), dtype=torch.float32, device="cuda")
        c5b.append((lambda xi=xi, q5=q5, s5=s5: aq.ptq_quant_fp8(xi, "fp16", 8192, 3584, q5, s5,
                                                                check=False)))
    return c5b, f5b


def int8_fp16_calls(torch, aq, W, G=128):
    """fp16 [8192, 3584] -> int8, group size G, fp32 row-major scales, over
    rotated buffer sets.  Returns the calls and the algorithmic bytes."""
    d5 = W.cfg5()
    f5 = alg_bytes_flat(8192, 3584, G, 2, False, 4)
    _, c5 = make_flat_sets(torch, aq, d5["x"], 8192, 3584, G, False, "int8", "f32", "row",
                           "fp16", rotation_sets(f5))
    return c5, f5


def requant_calls(torch, aq, live):
    """fp8 requantization at the sglang #35593 page's timed shape: K = 3584,
    8 experts, tokens_pad 1024, `live` rows per expert, DeepEP column-major
    group scales, output scale 2."""
    E8, T8, K8 = 8, 1024, 3584
    rng = np.random.default_rng(35593)
    xq = torch.from_numpy(rng.integers(0, 127, (E8, T8, K8)).astype(np.uint8)).to("cuda")
    xs = torch.from_numpy(rng.uniform(0.5, 2.0, E8 * T8 * (K8 // 128)).astype(np.float32)).to("cuda")
    osd = torch.tensor([2.0], dtype=torch.float32, device="cuda")
    strides = (T8 * (K8 // 128), 1, T8)
    mmq = torch.full((E8,), live, dtype=torch.int32, device="cuda")
    nsets = rotation_sets(E8 * live * 7280)
    outs = [torch.empty((E8, T8, K8), dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    ins = [xq] + [xq.clone() for _ in range(nsets - 1)]
    cq = [(lambda xi=ins[i], oi=outs[i]: aq.ptgq_requant_fp8(
        xi, E8, T8, K8, 128, xs, strides, mmq, live, osd, oi, check=False))
        for i in range(nsets)]
    fq = E8 * live * (K8 + K8 + (K8 // 128) * 4) + 4 * E8 + 4

    def capture():
        """Sampled live rows of three experts of set 0's output, each row's
        group scales gathered from the column-major layout, kept for the
        oracle comparison."""
        xh = xq.cpu().numpy()
        sh = xs.cpu().numpy()
        ng = K8 // 128
        rows = np.unique(np.linspace(0, live - 1, 8).astype(np.int64))
        cases = []
        for e in (0, 3, E8 - 1):
            srow = np.stack([sh[e * strides[0] + t * strides[1] + np.arange(ng) * strides[2]]
                             for t in rows])
            cases.append((np.ascontiguousarray(xh[e, rows][None]), srow,
                          outs[0][e, rows].cpu().numpy()))

        def check(oracle):
            bad, worst, strict, n = 0, 0.0, 0, 0
            for xr, srow, got in cases:
                ref = oracle.requant_fp8(xr, 1, len(rows), K8, 128, srow,
                                         (len(rows) * ng, ng, 1), None, 2.0)
                bad += int((got != ref[0]).sum())
                # the exact dequantized input, against the output code times
                # the output scale (two fp32 roundings: the drift-aware bound)
                y = oracle.e4m3_decode(xr[0]).astype(np.float64) * np.repeat(
                    srow.astype(np.float64), 128, axis=1)
                w, st = error_stats(oracle, y, got, "e4m3", np.full(y.shape, 2.0), True)
                worst, strict, n = max(worst, w), strict + st, n + got.size
            return {"rows": len(cases) * len(rows), "mismatches": bad,
                    "max_error_over_bound": round(worst, 6), "elements": n,
                    "past_strict_bound": strict}
        return check
    return cq, fq, capture


def rows_of_scales(s_dev, M, K, G, fmt, layout, rows):
    """The scales of `rows` from a device scale tensor, as a row-major array
    ([len(rows), ng] float32 or uint8)."""
    ng = K // G
    Mp = (M + 3) // 4 * 4
    b = s_dev.cpu().numpy().view(np.uint8)
    if fmt == "f32":
        f = b.view(np.float32)
        return f.reshape(M, ng)[rows] if layout == "row" else f[:ng * Mp].reshape(ng, Mp)[:, rows].T
    if layout == "row":
        return b[:M * ng].reshape(M, ng)[rows]
    words = b.view(np.uint32)[:((ng + 3) // 4) * Mp].reshape((ng + 3) // 4, Mp)
    out = np.empty((len(rows), ng), dtype=np.uint8)
    for g in range(ng):
        out[:, g] = (words[g // 4, rows] >> (8 * (g % 4))) & 0xFF
    return out


def error_stats(oracle, y, gq, code, sc, fp32_scale):
    """Dequantization error of every element against two bounds.

    strict: |dequant(code) - y| <= ulp/2 * scale, half an output ulp of
    |y / scale| (e4m3 ulp, or 1 for int8) -- the bound the codes meet when the
    multiplier is exact (UE8M0 scales: v = y * 2^k exactly).
    drift-aware: with fp32 scales v = fl(y * fl(1/scale)) also drifts from
    y / scale by at most |y / scale| * 2^-22 (two roundings), so the bound is
    (ulp/2 + drift) * scale, with the ulp taken at |y / scale| + drift.
    Returns the worst error over the drift-aware bound and the number of
    elements past the strict bound.  `sc`: each element's scale (float64,
    broadcast over its group)."""
    vals = oracle.e4m3_decode(gq) if code == "e4m3" else gq.view(np.int8)
    dq = vals.astype(np.float64) * sc
    t = np.abs(y.astype(np.float64) / np.where(sc > 0, sc, 1.0))
    drift = t * 2.0 ** -22 if fp32_scale else np.zeros_like(t)

    def half_ulp(a):
        if code != "e4m3":
            return np.full_like(a, 0.5)
        _, ex = np.frexp(a)
        return 0.5 * np.where(a >= 2.0 ** -6, np.ldexp(1.0, ex - 4), 2.0 ** -9)

    err = np.abs(dq - y.astype(np.float64))
    bound = (half_ulp(t + drift) + drift) * sc
    r = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    strict = err > half_ulp(t) * sc
    return (float(r.max()) if r.size else 0.0), int(strict.sum())


def bf16_past_half_ulp(exact, got_bits):
    """Number of bf16 outputs (bit patterns `got_bits`) farther than half a
    bf16 ulp from the exact float64 values `exact` (finite, below the bf16
    maximum): the strict bound of a dequantization to bf16."""
    out = (np.asarray(got_bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.abs(exact)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    # |exact| in [2^(ex-1), 2^ex): ulp 2^(ex-1-7), subnormals 2^-133
    half = np.ldexp(1.0, np.maximum(ex - 1, -126) - 8)
    return int((np.abs(out - exact) > half).sum())


def error_fields(oracle, y, gq, code, sc, fp32_scale):
    worst, strict = error_stats(oracle, y, gq, code, sc, fp32_scale)
    return {"max_error_over_bound": round(worst, 6), "elements": int(gq.size),
            "past_strict_bound": strict}


def capture_flat(x_host, in_dtype, M, K, G, fuse, out_dtype, fmt, layout, q_dev, s_dev, rows):
    """Sampled rows of a timed flat (or one expert's masked) output, kept on the
    host; the returned check(oracle) counts code and scale mismatches against
    the oracle on the same rows and the worst dequantization error over its
    bound."""
    rows = np.asarray(rows, dtype=np.int64)
    xs = np.ascontiguousarray(x_host[rows])
    gq = q_dev[rows].cpu().numpy()
    gs = np.ascontiguousarray(rows_of_scales(s_dev, M, K, G, fmt, layout, rows))

    def check(oracle):
        n = len(rows)
        rq, rs = oracle.ptgq(xs, in_dtype, n, K, G, fuse, out_dtype, fmt, "row", eps=1e-10)
        rs = rs.view(np.float32 if fmt == "f32" else np.uint8).reshape(n, K // G)
        if in_dtype == "fp32":
            y = xs.astype(np.float32)
        elif fuse:
            y = oracle.silu_mul(oracle.decode(xs[:, :K], in_dtype),
                                oracle.decode(xs[:, K:], in_dtype))
        else:
            y = oracle.decode(xs, in_dtype)
        sc = gs.astype(np.float64) if fmt == "f32" else np.ldexp(1.0, gs.astype(np.int64) - 127)
        return dict({"rows": int(n), "code_mismatches": int((gq != rq).sum()),
                     "scale_mismatches": int((gs.view(np.uint8) != rs.view(np.uint8)).sum())},
                    **error_fields(oracle, y, gq, out_dtype, np.repeat(sc, G, axis=1),
                                   fmt == "f32"))
    return check


def merge_checks(parts):
    """One check(oracle) that sums the counts of several."""
    def check(oracle):
        res = [p(oracle) for p in parts]
        out = {k: sum(r[k] for r in res) for k in res[0] if k != "max_error_over_bound"}
        out["max_error_over_bound"] = max(r["max_error_over_bound"] for r in res)
        return out
    return check


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--profile-main", action="store_true")
    ap.add_argument("--profile-m", type=int, default=16384,
                    help="rows of the workload that --profile-main launches")
    ap.add_argument("--profile-dequant", action="store_true")
    ap.add_argument("--profile-requant", action="store_true")
    ap.add_argument("--profile-fused", action="store_true")
    ap.add_argument("--profile-masked", action="store_true")
    ap.add_argument("--profile-fp32", action="store_true")
    ap.add_argument("--profile-per-token", action="store_true")
    ap.add_argument("--profile-int8", action="store_true")
    ap.add_argument("--profile-stream", action="store_true",
                    help="only the no-arithmetic stream over the headline's element count")
    ap.add_argument("--int8-group", type=int, default=128, choices=[16, 32, 64, 128],
                    help="group size of the --profile-int8 loop")
    ap.add_argument("--fp16", action="store_true",
                    help="the --profile-fused loop on fp16 inputs")
    ap.add_argument("--graph", action="store_true",
                    help="variant profile loops: launch in HIP graphs of 200 launches")
    ap.add_argument("--tuning", action="append", default=[], metavar="KNOB=VALUE",
                    help="launch-geometry override for the profile loops (ptgq_set_tuning)")
    args = ap.parse_args()
    tuning = []
    for t in args.tuning:
        k, _, v = t.partition("=")
        tuning.append((int(k), int(v)))

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this quantization path needs no exchange between "
              f"GPUs (rows and experts are independent), and only --gpus 1 is supported "
              f"(got --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import activation_quantization_amd as aq
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    aq.load_library()
    aq.ptgq_init(0)
    timer = Timer(torch)

    profiling = (args.profile_main or args.profile_dequant or args.profile_requant or
                 args.profile_fused or args.profile_masked or args.profile_fp32 or
                 args.profile_per_token or args.profile_int8 or args.profile_stream)
    if tuning and not profiling:
        print("--tuning applies to the profile loops only", file=sys.stderr)
        sys.exit(2)
    for k, v in tuning:
        aq.ptgq_set_tuning(k, v)

    if (args.profile_dequant or args.profile_requant or args.profile_fused or args.profile_masked
            or args.profile_fp32 or args.profile_per_token or args.profile_int8):
        if args.profile_dequant:
            name, (calls, nbytes, _) = "dequant", dequant_calls(torch, aq)
        elif args.profile_requant:
            name, (calls, nbytes, _) = "requant", requant_calls(torch, aq, 1024)
        elif args.profile_fused:
            name, (_, _, calls, nbytes) = ("fused_fp16" if args.fp16 else "fused",
                                           fused_calls(torch, aq, W, fp16=args.fp16))
        elif args.profile_masked:
            name, (_, calls, nbytes, _) = "masked", masked_calls(torch, aq, W)
        elif args.profile_fp32:
            name, (_, calls, nbytes) = "fp32", fp32_calls(torch, aq, W)
        elif args.profile_per_token:
            name, (calls, nbytes) = "per_token", per_token_calls(torch, aq, W.cfg5())
        else:
            name, (calls, nbytes) = "int8", int8_fp16_calls(torch, aq, W, args.int8_group)
        if args.graph:
            # back-to-back launches in HIP graphs of 200, as the variant
            # figures are taken (launched one by one from Python, a kernel
            # shorter than the launch interval starts from an idle GPU)
            us = timer.graph(calls, 200, max(1, args.steps // 200), min_ms=0.0) * 1e3
        else:
            r = timer.run(calls, args.steps, args.warmup, per_launch=False)
            us = r["region_ms"] * 1e3 / args.steps
        print(json.dumps({"profile": name, "steps": args.steps, "bytes": nbytes,
                          "tuning": dict(tuning), "graph": args.graph, "us_per_launch": us}))
        return

    M, K, G = 16384, 7168, 128
    if args.profile_stream:
        calls, nbytes = stream_calls(torch, aq, M, K, rotation_sets(alg_bytes_flat(M, K, G, 2, False, 1)))
        r = timer.run(calls, args.steps, args.warmup, per_launch=False)
        print(json.dumps({"profile": "stream", "steps": args.steps, "bytes": nbytes,
                          "us_per_launch": r["region_ms"] * 1e3 / args.steps}))
        return
    if args.profile_main:
        M = args.profile_m
    d = W.cfg2(M)
    x_host = d["x"]
    foot = alg_bytes_flat(M, K, G, 2, False, 1)
    nsets = rotation_sets(foot)
    sets, calls = make_flat_sets(torch, aq, x_host, M, K, G, False, "e4m3", "ue8m0", "col",
                                 "bf16", nsets)

    if args.profile_main:
        r = timer.run(calls, args.steps, args.warmup, per_launch=False)
        print(json.dumps({"profile_main": True, "steps": args.steps,
                          "us_per_launch": r["region_ms"] * 1e3 / args.steps}))
        return

    main_res = timer.run(calls, args.steps, args.warmup)
    ms_per_step = main_res["region_ms"] / args.steps
    # the stream reference over the same element count, timed the same way
    # right after the headline (the same number of launches)
    s_calls, s_bytes = stream_calls(torch, aq, M, K, nsets)
    stream_res = timer.run(s_calls, args.steps, args.warmup, per_launch=False)
    stream_us = stream_res["region_ms"] * 1e3 / args.steps
    del s_calls
    torch.cuda.empty_cache()
    value = foot / (ms_per_step * 1e-3) / 1e9
    # the kernel's average launch duration: the event pair around the K
    # back-to-back launches on the stream they run on (gaps included, so a
    # lower bound on the kernel's own rate); one launch per step
    achieved = foot / (ms_per_step * 1e-3) / 1e9

    # Sampled outputs of every measured case are kept on the host; the oracle
    # runs on them only in the CPU-baseline leg at the end.
    checks = {}
    rows = sorted(set([0, 1, 2, M - 3, M - 2, M - 1] + list(range(5, M, 257))))
    checks["headline"] = capture_flat(x_host, "bf16", M, K, G, False, "e4m3", "ue8m0", "col",
                                      sets[0][1], sets[0][2], rows)

    # per-M sweep of the same workload
    per_m = []
    for Mi in W.CFG2_M:
        di = x_host if Mi == M else W.cfg2(Mi)["x"]
        fi = alg_bytes_flat(Mi, K, G, 2, False, 1)
        ns = rotation_sets(fi)
        _, ci = make_flat_sets(torch, aq, di, Mi, K, G, False, "e4m3", "ue8m0", "col", "bf16", ns)
        per_graph = max(ns, min(200, max(8, math.ceil(1.2e10 / max(fi, 1)))))
        t_cold = timer.graph(ci, per_graph, 5)
        t_warm = timer.graph(ci[:1], min(per_graph, 100), 5) if Mi <= 256 else None
        ent = {"M": Mi, "us_per_call": round(t_cold * 1e3, 3), "bytes": fi,
               "GBps": round(fi / (t_cold * 1e-3) / 1e9, 1),
               "frac_of_peak": round(fi / (t_cold * 1e-3) / 1e9 / PEAK_GBS, 4),
               "buffer_sets": ns}
        if t_warm is not None:
            ent["us_per_call_warm"] = round(t_warm * 1e3, 3)
        per_m.append(ent)
        del ci
        torch.cuda.empty_cache()

    # the stream reference at the smaller workloads' element counts (M x 7168
    # for M = 4096 equals fp16 [8192, 3584]; M = 2048 is the fused
    # workload's output count at M = 2048 x 2)
    stream_ref = []
    for Mi in (2048, 4096):
        sc_i, sb_i = stream_calls(torch, aq, Mi, K, rotation_sets(3 * Mi * K))
        per_graph = max(len(sc_i), min(200, max(8, math.ceil(1.2e10 / sb_i))))
        us = timer.graph(sc_i, per_graph, 5) * 1e3
        stream_ref.append({"elements": Mi * K, "bytes": sb_i, "us_per_call": round(us, 3),
                           "GBps": round(sb_i / us / 1e3, 1),
                           "frac_of_peak": round(sb_i / us / 1e3 / PEAK_GBS, 4)})
        del sc_i
        torch.cuda.empty_cache()

    variants = {}
    if not args.no_variants:
        def spread(n, k=24):
            return np.unique(np.linspace(0, n - 1, k).astype(np.int64))
        # the headline input to int8 codes with the same UE8M0 scales
        fi8 = alg_bytes_flat(M, K, G, 2, False, 1)
        si8, ci8 = make_flat_sets(torch, aq, x_host, M, K, G, False, "int8", "ue8m0", "col",
                                  "bf16", rotation_sets(fi8))
        variants["int8_ue8m0_bf16_M16384_K7168"] = dict(variant_entry(timer, ci8, fi8),
                                                        input_fnv1a=W.fnv1a(x_host))
        checks["int8_ue8m0_bf16_M16384_K7168"] = capture_flat(
            x_host, "bf16", M, K, G, False, "int8", "ue8m0", "col", si8[0][1], si8[0][2],
            spread(M))
        del ci8, si8
        # fp32 input [8192, 7168] -> e4m3, packed column-major UE8M0 scales
        M32 = 8192
        x32h, c32, f32b = fp32_calls(torch, aq, W)
        variants["fp32_input_M8192_K7168"] = dict(variant_entry(timer, c32, f32b),
                                                  input_fnv1a=W.fnv1a(x32h))
        checks["fp32_input_M8192_K7168"] = capture_flat(
            x32h, "fp32", M32, K, G, False, "e4m3", "ue8m0", "col", c32[0].__defaults__[1],
            c32[0].__defaults__[2], spread(M32))
        del c32
        torch.cuda.empty_cache()
        # fused silu(gate)*up, bf16 [8192, 2*4096]
        d3, s3, c3, f3 = fused_calls(torch, aq, W)
        variants["fused_silu_mul_M8192_K4096"] = dict(variant_entry(timer, c3, f3),
                                                      input_fnv1a=W.fnv1a(d3["x"]))
        checks["fused_silu_mul_M8192_K4096"] = capture_flat(
            d3["x"], "bf16", 8192, 4096, 128, True, "e4m3", "ue8m0", "col", s3[0][1], s3[0][2],
            spread(8192))
        del c3, s3
        # the rest of the fused workload's sizes, M = 1, 64 and 2048 (graph
        # figures; M <= 64 is latency-bound), each with every output row or
        # 24 sampled rows checked
        for M3 in W.CFG3_M:
            if M3 == 8192:
                continue
            d3m = W.cfg3(M3)
            f3m = alg_bytes_flat(M3, 4096, 128, 2, True, 1)
            s3m, c3m = make_flat_sets(torch, aq, d3m["x"], M3, 4096, 128, True, "e4m3", "ue8m0",
                                      "col", "bf16", rotation_sets(f3m))
            name = f"fused_silu_mul_M{M3}_K4096"
            variants[name] = dict(variant_entry(timer, c3m, f3m), input_fnv1a=W.fnv1a(d3m["x"]))
            checks[name] = capture_flat(d3m["x"], "bf16", M3, 4096, 128, True, "e4m3", "ue8m0",
                                        "col", s3m[0][1], s3m[0][2], spread(M3))
            del c3m, s3m
        # the same fused call on fp16 gates and ups (N(0,1)), which reads the
        # fp16 SiLU table
        d3h, s3h, c3h, _ = fused_calls(torch, aq, W, fp16=True)
        variants["fused_silu_mul_fp16_M8192_K4096"] = dict(variant_entry(timer, c3h, f3),
                                                           input_fnv1a=W.fnv1a(d3h["x"]))
        checks["fused_silu_mul_fp16_M8192_K4096"] = capture_flat(
            d3h["x"], "fp16", 8192, 4096, 128, True, "e4m3", "ue8m0", "col", s3h[0][1],
            s3h[0][2], spread(8192))
        del c3h, s3h, d3h
        # the plain workload: bf16 [64, 2048] -> e4m3, fp32 row-major scales
        # (latency-bound), every row checked
        d1 = W.cfg1()
        f1 = alg_bytes_flat(64, 2048, 128, 2, False, 4)
        s1, c1 = make_flat_sets(torch, aq, d1["x"], 64, 2048, 128, False, "e4m3", "f32", "row",
                                "bf16", rotation_sets(f1))
        variants["plain_fp32_rowmajor_M64_K2048"] = dict(variant_entry(timer, c1, f1),
                                                         input_fnv1a=W.fnv1a(d1["x"]))
        checks["plain_fp32_rowmajor_M64_K2048"] = capture_flat(
            d1["x"], "bf16", 64, 2048, 128, False, "e4m3", "f32", "row", s1[0][1], s1[0][2],
            np.arange(64))
        del c1, s1
        # masked MoE, E=32, tokens_pad=384, fused, K=2048
        d4, c4, f4, live = masked_calls(torch, aq, W)
        E, T, K4, mm = d4["E"], d4["T"], d4["K"], d4["masked_m"]
        sb4 = aq.ptgq_scale_bytes(T, K4, 128, "ue8m0", "col")
        variants["masked_E32_T384_K2048_fused"] = dict(variant_entry(timer, c4, f4),
                                                       live_rows=live,
                                                       input_fnv1a=W.fnv1a(d4["x"]))
        # every live row of four experts of set 0 (its other rows hold
        # whatever the buffer held: only live rows are checked)
        q40, s40 = c4[0].__defaults__[1], c4[0].__defaults__[2]
        checks["masked_E32_T384_K2048_fused"] = merge_checks([
            capture_flat(d4["x"][e], "bf16", T, K4, 128, True, "e4m3", "ue8m0", "col", q40[e],
                         s40[e * sb4:(e + 1) * sb4], np.arange(int(np.clip(mm[e], 0, T))))
            for e in (0, 1, 7, E - 1) if int(np.clip(mm[e], 0, T)) > 0])
        del c4
        # the same layout at one live row per expert (decoding): the waves
        # walk the 32 live rows only, never the 384-row padding
        d4d, c4d, f4d, live_d = masked_calls(torch, aq, W, masked_m=np.ones(32, np.int32))
        variants["masked_E32_T384_K2048_fused_1token"] = dict(variant_entry(timer, c4d, f4d),
                                                              live_rows=live_d)
        q4d, s4d = c4d[0].__defaults__[1], c4d[0].__defaults__[2]
        checks["masked_E32_T384_K2048_fused_1token"] = merge_checks([
            capture_flat(d4d["x"][e], "bf16", T, K4, 128, True, "e4m3", "ue8m0", "col", q4d[e],
                         s4d[e * sb4:(e + 1) * sb4], np.arange(1))
            for e in (0, 1, 7, E - 1)])
        del c4d
        # fp16 [8192, 3584] -> int8, fp32 row-major scales, G = 128; per-token e4m3
        d5 = W.cfg5()
        f5 = alg_bytes_flat(8192, 3584, 128, 2, False, 4)
        s5s, c5 = make_flat_sets(torch, aq, d5["x"], 8192, 3584, 128, False, "int8", "f32", "row",
                                 "fp16", rotation_sets(f5))
        variants["int8_fp16_M8192_K3584_G128"] = dict(variant_entry(timer, c5, f5),
                                                      input_fnv1a=W.fnv1a(d5["x"]))
        checks["int8_fp16_M8192_K3584_G128"] = capture_flat(
            d5["x"], "fp16", 8192, 3584, 128, False, "int8", "f32", "row", s5s[0][1], s5s[0][2],
            spread(8192))
        del c5, s5s
        # the rest of the group-size sweep of the same tensor
        for G5 in (16, 32, 64):
            f5g = alg_bytes_flat(8192, 3584, G5, 2, False, 4)
            s5g, c5g = make_flat_sets(torch, aq, d5["x"], 8192, 3584, G5, False, "int8", "f32",
                                      "row", "fp16", rotation_sets(f5g))
            name = f"int8_fp16_M8192_K3584_G{G5}"
            variants[name] = dict(variant_entry(timer, c5g, f5g), input_fnv1a=W.fnv1a(d5["x"]))
            checks[name] = capture_flat(d5["x"], "fp16", 8192, 3584, G5, False, "int8", "f32",
                                        "row", s5g[0][1], s5g[0][2], spread(8192, 8))
            del c5g, s5g
        c5b, f5b = per_token_calls(torch, aq, d5)
        variants["per_token_fp8_fp16_M8192_K3584"] = dict(variant_entry(timer, c5b, f5b),
                                                          input_fnv1a=W.fnv1a(d5["x"]))
        rows5 = spread(8192)
        x5s = np.ascontiguousarray(d5["x"][rows5])
        q50 = c5b[0].__defaults__[1][rows5].cpu().numpy()
        s50 = c5b[0].__defaults__[2][rows5].cpu().numpy()

        def check5(oracle):
            rq5, rs5 = oracle.ptq_fp8(x5s, "fp16", len(rows5), 3584)
            sc = np.repeat(s50.astype(np.float64)[:, None], 3584, axis=1)
            return dict({"rows": int(len(rows5)), "code_mismatches": int((q50 != rq5).sum()),
                         "scale_mismatches": int((s50.view(np.uint32) != rs5.view(np.uint32)).sum())},
                        **error_fields(oracle, oracle.decode(x5s, "fp16"), q50, "e4m3", sc, True))
        checks["per_token_fp8_fp16_M8192_K3584"] = check5
        del c5b
        torch.cuda.empty_cache()
        # fp8 requantization, the sglang #35593 page's timed shape: K = 3584,
        # 8 experts, 1024 live rows -- read both as 1024 rows in total (128 per
        # expert) and as 1024 rows per expert; tokens_pad 1024, DeepEP
        # column-major group scales, output scale 2
        for label, live in (("total", 128), ("per_expert", 1024)):
            cq, fq, capq = requant_calls(torch, aq, live)
            name = f"requant_fp8_E8_K3584_live1024_{label}"
            variants[name] = dict(variant_entry(timer, cq, fq), live_rows=8 * live,
                                  pages_context_us={"H200": 25.4, "B200": 14.6})
            checks[name] = capq()
            del cq, capq
        torch.cuda.empty_cache()
        cd, fd, capd = dequant_calls(torch, aq)
        variants["dequant_e4m3_to_bf16_M16384_K7168"] = variant_entry(timer, cd, fd)
        checks["dequant_e4m3_to_bf16_M16384_K7168"] = capd()
        del cd, capd
        torch.cuda.empty_cache()

    # The CPU-baseline leg: the oracle timed on whole headline steps, then
    # run on the sampled rows of every measured case (mismatch counts).
    cpu = None
    parity = {}
    if not args.no_cpu_baseline:
        import oracle
        # whole steps, repeated until about 10 s of CPU work (at most 4), the
        # process pinned to one host core (the oracle is single-threaded C)
        allowed = sorted(os.sched_getaffinity(0))
        core = allowed[-1]
        os.sched_setaffinity(0, {core})
        try:
            times, t0 = [], time.perf_counter()
            while len(times) < 4 and (not times or time.perf_counter() - t0 < 10.0):
                t1 = time.perf_counter()
                oracle.ptgq(x_host, "bf16", M, K, G, False, "e4m3", "ue8m0", "col", eps=1e-10)
                times.append(time.perf_counter() - t1)
            steps_cpu, dt = len(times), float(np.median(times))
        finally:
            os.sched_setaffinity(0, allowed)
        cpu = {"value": round(foot / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{steps_cpu} full steps of all {M} rows of the bf16 [{M},{K}] input "
                         f"({M * K} elements each), single-threaded, median {dt:.1f} s per step",
               "ns_per_element": round(dt / (M * K) * 1e9, 2),
               "host": {"cpu_model": host_cpu_model(), "cores_visible": len(allowed),
                        "pinned_core": core}}
        # context: the same oracle run rows-parallel, one contiguous row range
        # per thread on every visible core (at most 16), one whole step
        from concurrent.futures import ThreadPoolExecutor
        nth = min(16, len(allowed))
        bounds = np.linspace(0, M, nth + 1).astype(np.int64)
        with ThreadPoolExecutor(nth) as ex:
            t1 = time.perf_counter()
            list(ex.map(lambda i: oracle.ptgq(x_host[bounds[i]:bounds[i + 1]], "bf16",
                                              int(bounds[i + 1] - bounds[i]), K, G, False,
                                              "e4m3", "ue8m0", "col", eps=1e-10), range(nth)))
            dtp = time.perf_counter() - t1
        cpu["rows_parallel"] = {"value": round(foot / dtp / 1e9, 4), "unit": "GB/s", "cores": nth,
                                "sample": f"one full step, {nth} threads over contiguous row "
                                          f"ranges, {dtp:.2f} s"}
        parity = {name: check(oracle) for name, check in checks.items()}
    for name in variants:
        variants[name]["parity"] = parity.get(name)

    traffic = read_traffic("traffic_ptgq_flat_bf16_M16384_K7168.md")
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "bf16 [16384, 7168] -> e4m3, G=128, UE8M0 scales column-major "
                               "(M padded to 4), N(0,1) with 1% outlier channels x30",
                   "M": M, "K": K, "group_size": G, "eps": 1e-10, "buffer_sets": nsets,
                   "algorithmic_bytes_per_step": foot, "input_fnv1a": W.fnv1a(x_host)},
        "frac_of_peak": round(value / PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "ptgq_flat_kernel<bf16, G=128, no fuse, e4m3>",
                     "avg_launch_us": round(ms_per_step * 1e3, 3),
                     "avg_launch_us_isolated": round(main_res["launch_ms_mean"] * 1e3, 3),
                     "kernel_source_digest": kernel_source_digest(),
                     # what a no-arithmetic stream with this kernel's traffic
                     # and geometry reaches here (ptgq_probe_stream, the same
                     # launch count): the memory system's share of the gap
                     "achievable_GBps": round(s_bytes / stream_us / 1e3, 1),
                     "achievable_us_per_launch": round(stream_us, 3),
                     "frac_of_achievable": round(achieved / (s_bytes / stream_us / 1e3), 4)},
        "parity_sample": parity.get("headline"),
        "per_m": per_m,
        "stream_reference": stream_ref,
        "variants": variants,
        "cpu_baseline": cpu,
        "wall_s_timed_region": round(main_res["wall_s"], 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
