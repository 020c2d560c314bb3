"""Helpers shared by the GPU tests: move seeded numpy inputs to the device,
run the C-ABI through the binding, and compare byte for byte with the oracle.

Every output the helpers allocate sits between two guard bands of sentinel
bytes, checked after each call: a write past either end of an output fails
the test that made it."""
import numpy as np
import torch

import activation_quantization_amd as aq

DEV = "cuda"
GUARD = 512          # sentinel bytes before and after every output (keeps 16-byte alignment)
GUARD_BYTE = 0xA5


class Guarded:
    """A device output of `shape` and `dtype` between two GUARD-byte bands of
    GUARD_BYTE; `fill` (a byte value) pre-fills the output itself."""

    def __init__(self, shape, dtype, fill=None):
        shape = tuple(int(d) for d in (shape if isinstance(shape, (tuple, list)) else (shape,)))
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((2 * GUARD + n,), GUARD_BYTE, dtype=torch.uint8, device=DEV)
        if fill is not None and n:
            self.raw[GUARD:GUARD + n] = fill
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self, tag=""):
        h = self.raw.cpu().numpy()
        before = int((h[:GUARD] != GUARD_BYTE).sum())
        after = int((h[GUARD + self.n:] != GUARD_BYTE).sum())
        assert before == 0 and after == 0, \
            f"{tag}: {before} guard bytes changed before the output, {after} after it"

    def host(self):
        return self.t.cpu().numpy()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def run_flat(x, in_dtype, M, K, G, fuse, out_dtype, fmt, layout, eps=1e-10, fill=0xCD,
             stream=None):
    xd = to_dev(x)
    q = Guarded((M, K), torch.uint8, fill)
    sb = aq.ptgq_scale_bytes(M, K, G, fmt, layout)
    s = Guarded((sb,), torch.uint8, fill)
    aq.ptgq_quant(xd, in_dtype, M, K, G, fuse, out_dtype, fmt, layout, eps, q.t, s.t,
                  stream=stream)
    torch.cuda.synchronize()
    q.check("ptgq_quant q")
    s.check("ptgq_quant s")
    return q.host(), s.host()


def run_masked(x, in_dtype, E, T, K, G, fuse, masked_m, expected_m, out_dtype, fmt, layout,
               eps=1e-10, q_fill=0x7F, s_fill=0xFF):
    xd = to_dev(x)
    mm = torch.from_numpy(np.ascontiguousarray(masked_m, dtype=np.int32)).to(DEV)
    q = Guarded((E, T, K), torch.uint8, q_fill)
    sb = aq.ptgq_scale_bytes(T, K, G, fmt, layout)
    s = Guarded((E * sb,), torch.uint8, s_fill)
    aq.ptgq_quant_masked(xd, in_dtype, E, T, K, G, fuse, mm, expected_m, out_dtype, fmt, layout,
                         eps, q.t, s.t)
    torch.cuda.synchronize()
    q.check("ptgq_quant_masked q")
    s.check("ptgq_quant_masked s")
    return q.host(), s.host()


def run_per_token(x, in_dtype, M, K, fill=0xCD, extra_rows=0):
    """ptq_quant_fp8 into outputs of M + extra_rows rows (serving pads its
    buffers): the rows past M must keep their fill."""
    xd = to_dev(x)
    q = Guarded((M + extra_rows, K), torch.uint8, fill)
    s = Guarded((M + extra_rows,), torch.float32, 0xFF)          # NaN pattern
    aq.ptq_quant_fp8(xd, in_dtype, M, K, q.t, s.t)
    torch.cuda.synchronize()
    q.check("ptq_quant_fp8 q")
    s.check("ptq_quant_fp8 s")
    qh, sh = q.host(), s.host()
    assert np.all(qh[M:] == fill), "ptq_quant_fp8 wrote code rows past M"
    assert np.all(sh[M:].view(np.uint32) == 0xFFFFFFFF), "ptq_quant_fp8 wrote scales past M"
    return qh[:M], sh[:M]


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
