"""The entry points captured into one HIP graph and replayed (among them a
small fused call in chunk tasks and a large fp16 one reading the fp16 SiLU
table): every replay, with new inputs and freshly filled sentinels written
eagerly in between, gives the oracle's bytes (the calls are asynchronous,
allocate nothing and never synchronize, so they can be captured after one
ptgq_init)."""
import numpy as np
import pytest
import torch

import activation_quantization_amd as aq
import oracle
import workloads as W
from gpu_util import DEV, compare

pytestmark = pytest.mark.gpu


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def test_graph_replays_match_the_oracle():
    aq.ptgq_init(0)
    M, K, G = 37, 1152, 128                      # flat: ragged rows, packed pads
    E, T, K4 = 5, 45, 640                        # masked, fused
    QR = 40                                      # padded code buffer rows
    Mt, Kt = 9, 1076                             # per-token
    Ed, Td, Kd = 3, 20, 1152                     # requant
    xf = torch.empty((M, K), dtype=torch.int16, device=DEV)
    qf = torch.empty((QR, K), dtype=torch.uint8, device=DEV)
    sbf = aq.ptgq_scale_bytes(M, K, G, "ue8m0", "col")
    sf = torch.empty(sbf, dtype=torch.uint8, device=DEV)
    xm = torch.empty((E, T, 2 * K4), dtype=torch.int16, device=DEV)
    mm = torch.empty(E, dtype=torch.int32, device=DEV)
    qm = torch.empty((E, T, K4), dtype=torch.uint8, device=DEV)
    sbm = aq.ptgq_scale_bytes(T, K4, 64, "f32", "col")
    sm = torch.empty(E * sbm, dtype=torch.uint8, device=DEV)
    xt = torch.empty((Mt, Kt), dtype=torch.int16, device=DEV)
    qt = torch.empty((Mt, Kt), dtype=torch.uint8, device=DEV)
    st = torch.empty(Mt, dtype=torch.float32, device=DEV)
    xr = torch.empty((Ed, Td, Kd), dtype=torch.uint8, device=DEV)
    sr = torch.empty(Ed * Td * (Kd // 128), dtype=torch.float32, device=DEV)
    mr = torch.empty(Ed, dtype=torch.int32, device=DEV)
    osr = torch.empty(1, dtype=torch.float32, device=DEV)
    outr = torch.empty((Ed, Td, Kd), dtype=torch.uint8, device=DEV)
    yd = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    r_strides = (Td * (Kd // 128), 1, Td)
    Mc, Kc = 3, 640                              # fused, chunk tasks
    xc = torch.empty((Mc, 2 * Kc), dtype=torch.int16, device=DEV)
    qc = torch.empty((Mc, Kc), dtype=torch.uint8, device=DEV)
    sc = torch.empty(aq.ptgq_scale_bytes(Mc, Kc, 128, "ue8m0", "col"), dtype=torch.uint8,
                     device=DEV)
    Mh, Kh = 1030, 4096                          # fused fp16, the fp16 SiLU table
    xh = torch.empty((Mh, 2 * Kh), dtype=torch.int16, device=DEV)
    qh = torch.empty((Mh, Kh), dtype=torch.uint8, device=DEV)
    sh = torch.empty(aq.ptgq_scale_bytes(Mh, Kh, 128, "f32", "row"), dtype=torch.uint8,
                     device=DEV)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert aq.ptgq_plan_group("bf16", 0, Mc, Kc, 128, True, 0, Mc, cus)["flat_slabs"] == 4
    assert aq.ptgq_plan_group("fp16", 0, Mh, Kh, 128, True, 0, Mh, cus)["silu_table"] == 1

    def calls():
        aq.ptgq_quant_padded(xf, "bf16", M, K, G, False, "e4m3", "ue8m0", "col", 1e-10, qf, QR,
                             sf)
        aq.ptgq_quant_masked(xm, "bf16", E, T, K4, 64, True, mm, 16, "int8", "f32", "col",
                             1e-10, qm, sm)
        aq.ptq_quant_fp8(xt, "bf16", Mt, Kt, qt, st)
        aq.ptgq_requant_fp8(xr, Ed, Td, Kd, 128, sr, r_strides, mr, 0, osr, outr)
        aq.ptgq_dequant(qf, "e4m3", M, K, G, sf, "ue8m0", "col", "bf16", yd)
        aq.ptgq_quant(xc, "bf16", Mc, Kc, 128, True, "e4m3", "ue8m0", "col", 1e-10, qc, sc)
        aq.ptgq_quant(xh, "fp16", Mh, Kh, 128, True, "int8", "f32", "row", 1e-10, qh, sh)

    def fill(seed):
        """New inputs and sentinels, written eagerly; returns host copies."""
        h = {}
        h["xf"] = W.normal_bf16(seed, (M, K), factor_cols=[3], factor=40.0)
        h["xm"] = W.normal_bf16(seed + 1, (E, T, 2 * K4))
        z = W.splitmix64(seed + 2, 0, E)
        h["mm"] = (z % np.uint64(T + 8)).astype(np.int32) - 3
        h["xt"] = W.normal_bf16(seed + 3, (Mt, Kt))
        rng = np.random.default_rng(seed)
        h["xr"] = rng.integers(0, 256, (Ed, Td, Kd)).astype(np.uint8)
        h["xr"][(h["xr"] & 0x7F) == 0x7F] = 0x11
        h["sr"] = rng.uniform(0.1, 4.0, Ed * Td * (Kd // 128)).astype(np.float32)
        h["mr"] = np.array([Td, 0, 7], np.int32)
        h["os"] = np.float32(rng.uniform(0.5, 3.0))
        h["xc"] = W.normal_bf16(seed + 4, (Mc, 2 * Kc))
        h["xh"] = W.normal_fp16(seed + 5, (Mh, 2 * Kh))
        xf.copy_(dev16(h["xf"]))
        xm.copy_(dev16(h["xm"]))
        mm.copy_(torch.from_numpy(h["mm"]))
        xt.copy_(dev16(h["xt"]))
        xr.copy_(torch.from_numpy(h["xr"]))
        sr.copy_(torch.from_numpy(h["sr"]))
        mr.copy_(torch.from_numpy(h["mr"]))
        osr.fill_(float(h["os"]))
        xc.copy_(dev16(h["xc"]))
        xh.copy_(dev16(h["xh"]))
        for t, v in ((qf, 0x5C), (sf, 0x5C), (qm, 0x7F), (sm, 0xFF), (qt, 0x33), (outr, 0x2C),
                     (qc, 0x5C), (sc, 0x5C), (qh, 0x5C), (sh, 0x5C)):
            t.fill_(v)
        st.fill_(float("nan"))
        yd.fill_(7.0)
        torch.cuda.synchronize()
        return h

    def check(h, tag):
        torch.cuda.synchronize()
        rq, rs = oracle.ptgq(h["xf"], "bf16", M, K, G, False, "e4m3", "ue8m0", "col")
        q_all = qf.cpu().numpy()
        compare(f"{tag} padded", q_all[:M], sf.cpu().numpy(), rq, rs)
        assert np.all(q_all[M:] == 0)
        sbm_ = aq.ptgq_scale_bytes(T, K4, 64, "f32", "col")
        rqm, rsm = oracle.ptgq_masked(h["xm"], "bf16", E, T, K4, 64, True, h["mm"], "int8", "f32",
                                      "col", q_init=np.full((E, T, K4), 0x7F, np.uint8),
                                      s_init=np.full(E * sbm_, 0xFF, np.uint8))
        compare(f"{tag} masked", qm.cpu().numpy(), sm.cpu().numpy(), rqm, rsm)
        rqt, rst = oracle.ptq_fp8(h["xt"], "bf16", Mt, Kt)
        compare(f"{tag} per-token", qt.cpu().numpy(), st.cpu().numpy(), rqt, rst)
        ro = oracle.requant_fp8(h["xr"], Ed, Td, Kd, 128, h["sr"], r_strides, h["mr"], h["os"],
                                out_init=np.full((Ed, Td, Kd), 0x2C, np.uint8))
        compare(f"{tag} requant", outr.cpu().numpy(), np.zeros(0, np.uint8), ro,
                np.zeros(0, np.uint8))
        ry = oracle.dequant(rq, "e4m3", M, K, G, rs, "ue8m0", "col", "bf16")
        got = yd.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ry), f"{tag} dequant"
        compare(f"{tag} fused chunk tasks", qc.cpu().numpy(), sc.cpu().numpy(),
                *oracle.ptgq(h["xc"], "bf16", Mc, Kc, 128, True, "e4m3", "ue8m0", "col"))
        compare(f"{tag} fused fp16 table", qh.cpu().numpy(), sh.cpu().numpy(),
                *oracle.ptgq(h["xh"], "fp16", Mh, Kh, 128, True, "int8", "f32", "row"))

    # eager reference run (also makes the device ready for capture)
    h = fill(11)
    calls()
    check(h, "eager")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i, seed in enumerate((21, 31, 41)):
        h = fill(seed)
        g.replay()
        check(h, f"replay {i}")
