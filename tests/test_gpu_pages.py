"""The pages' own correctness matrices, run against the oracle (bit-exact
codes and scales):

* sglang #27449 PR body, validation: 96 flat cases (plain and fused
  silu+mul x bf16 / fp16 x tokens {1, 7, 64, 333} x hidden {128, 2048, 4096}
  x fp32 / UE8M0 scales) and 8 masked cases (UE8M0, fused, [experts,
  tokens_pad, hidden*2] x experts {2, 5} x hidden {2048, 4096} x tokens_pad
  {128, 384}); group size 128, e4m3 codes.
* sglang #34257 review page, key source snippets (the bit-exact test): per-token
  e4m3 of uniform [0, 1) inputs in fp16 / bf16 / fp32, hidden {1076, 1368},
  39 tokens (one block per row) and compute-units x 16 tokens (the page's
  warp-dispatch threshold).

Inputs are seeded synthetic stand-ins for the pages' torch.randn / torch.rand
draws.  Scale layouts: fp32 scales row-major, UE8M0 scales packed column-major
(the DeepGEMM layout the UE8M0 trait serves)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import compare, run_flat, run_masked, run_per_token

pytestmark = pytest.mark.gpu


def randn(seed, shape, in_dtype):
    return W.normal_bf16(seed, shape) if in_dtype == "bf16" else W.normal_fp16(seed, shape)


@pytest.mark.parametrize("scale", ["f32", "ue8m0"])
@pytest.mark.parametrize("hidden", [128, 2048, 4096])
@pytest.mark.parametrize("tokens", [1, 7, 64, 333])
@pytest.mark.parametrize("in_dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("fuse", [False, True])
def test_sglang27449_flat_matrix(fuse, in_dtype, tokens, hidden, scale):
    layout = "row" if scale == "f32" else "col"
    seed = 27449 + 7 * tokens + hidden + 3 * fuse + (in_dtype == "fp16")
    x = randn(seed, (tokens, 2 * hidden if fuse else hidden), in_dtype)
    args = (x, in_dtype, tokens, hidden, 128, fuse, "e4m3", scale, layout)
    compare(f"#27449 fuse={fuse} {in_dtype} tokens={tokens} hidden={hidden} {scale}",
            *run_flat(*args), *oracle.ptgq(*args, eps=1e-10))


@pytest.mark.parametrize("tokens_pad", [128, 384])
@pytest.mark.parametrize("hidden", [2048, 4096])
@pytest.mark.parametrize("experts", [2, 5])
def test_sglang27449_masked_matrix(experts, hidden, tokens_pad):
    rng = np.random.default_rng(27449 + experts + hidden + tokens_pad)
    mm = rng.integers(0, tokens_pad + 1, experts).astype(np.int32)
    x = W.normal_bf16(27450 + experts * hidden + tokens_pad, (experts, tokens_pad, 2 * hidden))
    E, T, K = experts, tokens_pad, hidden
    gq, gs = run_masked(x, "bf16", E, T, K, 128, True, mm, int(mm.mean()), "e4m3", "ue8m0", "col")
    sb = oracle.scale_bytes(T, K, 128, "ue8m0", "col")
    rq, rs = oracle.ptgq_masked(x, "bf16", E, T, K, 128, True, mm, "e4m3", "ue8m0", "col",
                                q_init=np.full((E, T, K), 0x7F, np.uint8),
                                s_init=np.full(E * sb, 0xFF, np.uint8))
    compare(f"#27449 masked experts={E} hidden={K} tokens_pad={T} masked_m={list(mm)}",
            gq, gs, rq, rs)


def rand01(seed, shape, in_dtype):
    """Uniform [0, 1) in the given dtype (round to nearest even)."""
    u = 1.0 - W.uniform(seed, 0, int(np.prod(shape))).reshape(shape)
    if in_dtype == "fp32":
        return u.astype(np.float32)
    return W.to_bf16_bits(u) if in_dtype == "bf16" else W.to_fp16_bits(u)


@pytest.mark.parametrize("hidden", [1076, 1368])
@pytest.mark.parametrize("dispatch", ["cta", "warp"])
@pytest.mark.parametrize("in_dtype", ["fp16", "bf16", "fp32"])
def test_sglang34257_per_token_matrix(in_dtype, dispatch, hidden):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tokens = 39 if dispatch == "cta" else cus * 16
    x = rand01(34257 + hidden + tokens, (tokens, hidden), in_dtype)
    compare(f"#34257 {in_dtype} {dispatch} tokens={tokens} hidden={hidden}",
            *run_per_token(x, in_dtype, tokens, hidden, extra_rows=2),
            *oracle.ptq_fp8(x, in_dtype, tokens, hidden))
