"""bi_sdpa_ex_noalloc (bi.h): the attention entry point that allocates nothing, with the split partials in
the library's per-GPU scratch array.  Called through the C ABI, it must give the bits of bi_sdpa_ex with a
caller workspace (the same kernels run), on two calls in a row where the second is smaller, with and
without masks and sinks, and in fp32 as well as bf16."""
import pytest
import torch

import invariant_deterministic_gemm_amd as bi
import synthetic
from helpers import assert_bits_equal

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(B, Hq, Hkv, Lq, S, dt, seed):
    q = synthetic.randn((B, Hq, Lq, 128), seed, 1.0, dt).to(DEV)
    k = synthetic.randn((B, Hkv, S, 128), seed + 1, 1.0, dt).to(DEV)
    v = synthetic.randn((B, Hkv, S, 128), seed + 2, 1.0, dt).to(DEV)
    return q, k, v


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_noalloc_equals_workspace_call_twice_shrinking(dt):
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F32
    lib = bi._native.load()
    # first call: a decode batch whose partials fill much of the scratch; second: a smaller one
    for (B, Hq, Hkv, Lq, S, seed) in [(8, 32, 8, 4, 5000, 0x5EEDA0), (2, 32, 8, 1, 3000, 0x5EEDA4)]:
        need = lib.bi_sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, 128, BI)
        assert 0 < need <= lib.bi_sdpa_scratch_limit()
        q, k, v = _inputs(B, Hq, Hkv, Lq, S, dt, seed)
        ref = bi.bi_sdpa(q, k, v, causal=True)
        out = bi.bi_sdpa_noalloc(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert_bits_equal(out, ref, f"B={B} S={S} Lq={Lq}: noalloc vs workspace call")


def test_noalloc_masks_sinks_and_limit():
    lib = bi._native.load()
    q, k, v = _inputs(4, 32, 8, 1, 4100, torch.bfloat16, 0x5EEDA8)
    gen = torch.Generator(device="cpu").manual_seed(0x5EEDA9)
    keep = (torch.rand((4, 1, 1, 4100), generator=gen) > 0.2).to(DEV)
    madd = torch.where(keep, torch.randn((4, 1, 1, 4100), generator=gen).to(DEV),
                       torch.full((), float("-inf"), device=DEV)).to(torch.bfloat16)
    sinks = torch.randn((32,), generator=gen).to(DEV)
    for mask in (keep, madd):
        ref = bi.bi_sdpa(q, k, v, mask=mask, sinks=sinks)
        out = bi.bi_sdpa_noalloc(q, k, v, mask=mask, sinks=sinks)
        assert_bits_equal(out, ref, f"mask {mask.dtype} + sinks: noalloc vs workspace call")
    # shapes served without partials use no scratch and still match
    qp, kp, vp = _inputs(1, 32, 8, 400, 1200, torch.bfloat16, 0x5EEDAA)
    assert lib.bi_sdpa_workspace_bytes(1, 32, 8, 400, 1200, 128, bi.BI_BF16) == 0
    assert_bits_equal(bi.bi_sdpa_noalloc(qp, kp, vp, causal=True), bi.bi_sdpa(qp, kp, vp, causal=True), "prefill")
    # a call above the limit raises before anything is enqueued
    B, S = 64, 65536
    assert lib.bi_sdpa_workspace_bytes(B, 32, 8, 1, S, 128, bi.BI_BF16) > lib.bi_sdpa_scratch_limit()
    qb = torch.zeros((B, 32, 1, 128), dtype=torch.bfloat16, device=DEV)
    kb = torch.zeros((1, 8, S, 128), dtype=torch.bfloat16, device=DEV).expand(B, 8, S, 128)
    with pytest.raises(NotImplementedError, match="scratch"):
        bi.bi_sdpa_noalloc(qb, kb, kb, causal=True)
