"""Helpers shared by the GPU tests: move seeded numpy inputs to the device,
run the C-ABI through the binding, and compare byte for byte with the oracle."""
import numpy as np
import torch

import activation_quantization_amd as aq

DEV = "cuda"


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def run_flat(x, in_dtype, M, K, G, fuse, out_dtype, fmt, layout, eps=1e-10, fill=0xCD,
             stream=None):
    xd = to_dev(x)
    q = torch.full((M, K), fill, dtype=torch.uint8, device=DEV)
    sb = aq.ptgq_scale_bytes(M, K, G, fmt, layout)
    s = torch.full((max(sb, 1),), fill, dtype=torch.uint8, device=DEV)
    aq.ptgq_quant(xd, in_dtype, M, K, G, fuse, out_dtype, fmt, layout, eps, q, s, stream=stream)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()[:sb]


def run_masked(x, in_dtype, E, T, K, G, fuse, masked_m, expected_m, out_dtype, fmt, layout,
               eps=1e-10, q_fill=0x7F, s_fill=0xFF):
    xd = to_dev(x)
    mm = torch.from_numpy(np.ascontiguousarray(masked_m, dtype=np.int32)).to(DEV)
    q = torch.full((E, T, K), q_fill, dtype=torch.uint8, device=DEV)
    sb = aq.ptgq_scale_bytes(T, K, G, fmt, layout)
    s = torch.full((max(E * sb, 1),), s_fill, dtype=torch.uint8, device=DEV)
    aq.ptgq_quant_masked(xd, in_dtype, E, T, K, G, fuse, mm, expected_m, out_dtype, fmt, layout,
                         eps, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()[:E * sb]


def run_per_token(x, in_dtype, M, K, fill=0xCD):
    xd = to_dev(x)
    q = torch.full((M, K), fill, dtype=torch.uint8, device=DEV)
    s = torch.full((max(M, 1),), float("nan"), dtype=torch.float32, device=DEV)
    aq.ptq_quant_fp8(xd, in_dtype, M, K, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()[:M]


def compare(tag, got_q, got_s, ref_q, ref_s):
    """Byte-exact comparison; prints the mismatch counts before asserting."""
    gq, rq = np.asarray(got_q).view(np.uint8), np.asarray(ref_q).view(np.uint8)
    gs, rs = np.asarray(got_s).view(np.uint8), np.asarray(ref_s).view(np.uint8)
    assert gq.shape == rq.shape and gs.shape == rs.shape, (gq.shape, rq.shape, gs.shape, rs.shape)
    nq = int((gq != rq).sum())
    ns = int((gs != rs).sum())
    print(f"[parity] {tag}: code mismatches {nq}/{rq.size}, scale byte mismatches "
          f"{ns}/{rs.size}", flush=True)
    if nq:
        i = int(np.flatnonzero(gq.ravel() != rq.ravel())[0])
        print(f"  first code mismatch at flat index {i}: got {gq.ravel()[i]:#04x} "
              f"want {rq.ravel()[i]:#04x}", flush=True)
    if ns:
        i = int(np.flatnonzero(gs.ravel() != rs.ravel())[0])
        print(f"  first scale mismatch at byte {i}: got {gs.ravel()[i]:#04x} "
              f"want {rs.ravel()[i]:#04x}", flush=True)
    assert nq == 0 and ns == 0
