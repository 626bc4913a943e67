"""GPU tests of the attention forms beyond the boolean mask: additive masks, attention sinks, and head
dims that are multiples of 32 (README, section "How the kernels work", attention paragraph: the mask
forms of the single-pass kernel; section "Limitations": sinks, head dims).

* oracle tolerance (fp32 1e-5, bf16 / fp16 2e-2) against the float64 oracle on every kernel path:
  the quad kernel for small grids, one launch for other short caches, split + combine for long ones,
  the prefill kernel for long query chunks, and the generic split kernel for fp32 and head dims above
  128;
* equivalences on raw bits: an additive mask of 0 / -inf equals the boolean mask, -inf sinks equal
  no sinks;
* invariance on raw bits: every token of a prefill chunk equals its own decode call (K / V truncated
  after it, its mask row), batch neighbours do not matter, and keys appended with -inf (or masked
  off) leave every result unchanged as the cache grows past split boundaries.
"""
import math

import numpy as np
import pytest
import torch

import invariant_deterministic_gemm_amd as bi
import oracle
import synthetic
from helpers import assert_bits_equal, assert_close_to_oracle, round_ref

pytestmark = pytest.mark.gpu
DEV = "cuda"
DTS = [torch.float32, torch.bfloat16, torch.float16]
# (B, Hq, Hkv, Lq, S) for 16-bit D = 128: quad + combine (at most 256 workgroups of one split and row
# tile), one launch (more, S <= 1024), split + combine (more, S > 1024), prefill (Lq >= 384)
PATHS = [(2, 8, 2, 5, 700), (4, 32, 8, 17, 900), (4, 32, 8, 3, 2085), (1, 4, 2, 400, 900)]
PATH_IDS = ["quad", "fused", "split", "prefill"]


def _ids(d):
    return str(d).split(".")[-1]


def _qkv(B, Hq, Hkv, Lq, S, D, dt, seed):
    q = synthetic.randn((B, Hq, Lq, D), seed, 1.0, dt)
    k = synthetic.randn((B, Hkv, S, D), seed + 1, 1.0, dt)
    v = synthetic.randn((B, Hkv, S, D), seed + 2, 1.0, dt)
    return q, k, v


def _gpu(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _additive(shape, seed, dt, frac_inf=0.2):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(shape, generator=g) * 2
    a[torch.rand(shape, generator=g) < frac_inf] = float("-inf")
    return a.to(dt)


@pytest.mark.parametrize("shape", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("dt", DTS, ids=_ids)
def test_additive_mask_against_oracle_and_boolean(dt, shape):
    B, Hq, Hkv, Lq, S = shape
    q, k, v = _qkv(B, Hq, Hkv, Lq, S, 128, dt, 300 + Lq)
    amask = _additive((B, 1, Lq, S), 301 + Lq, dt)
    amask[..., S - Lq] = 0.0                            # every row keeps at least one key
    qg, kg, vg, ag = _gpu(q, k, v, amask)
    o = bi.bi_sdpa(qg, kg, vg, causal=True, mask=ag)
    want = oracle.sdpa(q, k, v, causal=True, mask=amask.to(torch.float64))
    assert_close_to_oracle(o, want, f"additive mask {dt} {shape}")
    # 0 / -inf is the boolean mask, bit for bit
    bm = torch.isfinite(amask)
    zero_inf = torch.where(bm, torch.zeros((), dtype=dt), torch.full((), float("-inf"), dtype=dt))
    assert_bits_equal(bi.bi_sdpa(qg, kg, vg, causal=True, mask=zero_inf.to(DEV)),
                      bi.bi_sdpa(qg, kg, vg, causal=True, mask=bm.to(DEV)), "0 / -inf vs boolean")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=_ids)
def test_additive_mask_tokens_equal_their_decode_and_ignore_neighbours(dt):
    B, Hq, Hkv, Lq, S, D = 3, 8, 2, 24, 1300, 128
    q, k, v = _gpu(*_qkv(B, Hq, Hkv, Lq, S, D, dt, 310))
    amask = _additive((B, Hq, Lq, S), 311, dt).to(DEV)
    amask[..., :8] = 0.0
    full = bi.bi_sdpa(q, k, v, causal=True, mask=amask)
    for i in (0, 7, 23):
        p = S - Lq + i
        dec = bi.bi_sdpa(q[:, :, i:i + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True,
                         mask=amask[:, :, i:i + 1, :p + 1])
        assert_bits_equal(dec[:, :, 0], full[:, :, i], f"token {i} vs its decode")
    one = bi.bi_sdpa(q[1:2], k[1:2], v[1:2], causal=True, mask=amask[1:2])
    assert_bits_equal(one, full[1:2], "batch element alone")


@pytest.mark.parametrize("dt", DTS, ids=_ids)
def test_keys_appended_with_minus_inf_change_nothing(dt):
    B, Hq, Hkv, Lq, S0, D = 1, 8, 2, 4, 1000, 128
    q, k, v = _qkv(B, Hq, Hkv, Lq, S0 + 600, D, dt, 320)
    amask = _additive((B, Hq, Lq, S0 + 600), 321, dt, frac_inf=0.1)
    amask[..., :4] = 0.0
    q, k, v, amask = _gpu(q, k, v, amask)
    base = bi.bi_sdpa(q, k[:, :, :S0], v[:, :, :S0], mask=amask[..., :S0])
    for S in (S0 + 24, S0 + 300, S0 + 600):            # 4 -> 5, 6, 7 splits
        grown = amask[..., :S].clone()
        grown[..., S0:] = float("-inf")
        o = bi.bi_sdpa(q, k[:, :, :S], v[:, :, :S], mask=grown)
        assert_bits_equal(o, base, f"cache {S0} -> {S}, new keys at -inf")


@pytest.mark.parametrize("shape", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("dt", DTS, ids=_ids)
def test_sinks_against_oracle_and_minus_inf(dt, shape):
    B, Hq, Hkv, Lq, S = shape
    q, k, v = _qkv(B, Hq, Hkv, Lq, S, 128, dt, 330 + Lq)
    sinks = synthetic.randn((Hq,), 331, 2.0)
    qg, kg, vg = _gpu(q, k, v)
    o = bi.bi_sdpa(qg, kg, vg, causal=True, sinks=sinks.to(DEV))
    want = oracle.sdpa(q, k, v, causal=True, sinks=sinks)
    assert_close_to_oracle(o, want, f"sinks {dt} {shape}")
    none = torch.full((Hq,), float("-inf"), device=DEV)
    assert_bits_equal(bi.bi_sdpa(qg, kg, vg, causal=True, sinks=none), bi.bi_sdpa(qg, kg, vg, causal=True),
                      "-inf sinks vs no sinks")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=_ids)
def test_sinks_invariance(dt):
    B, Hq, Hkv, Lq, S, D = 2, 8, 2, 20, 1100, 128
    q, k, v = _gpu(*_qkv(B, Hq, Hkv, Lq, S + 400, D, dt, 340))
    sinks = synthetic.randn((Hq,), 341, 2.0).to(DEV)
    full = bi.bi_sdpa(q, k[:, :, :S], v[:, :, :S], causal=True, sinks=sinks)
    for i in (0, 19):
        p = S - Lq + i
        dec = bi.bi_sdpa(q[:, :, i:i + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True, sinks=sinks)
        assert_bits_equal(dec[:, :, 0], full[:, :, i], f"token {i} vs its decode, sinks")
    assert_bits_equal(bi.bi_sdpa(q[:1], k[:1, :, :S], v[:1, :, :S], causal=True, sinks=sinks), full[:1],
                      "batch element alone, sinks")
    # the cache grows by masked keys: the sink's place in the fold (first) does not move
    m = torch.ones(1, 1, Lq, S + 400, dtype=torch.bool, device=DEV)
    m[..., S:] = False
    qd = q[:, :, :1]
    base = bi.bi_sdpa(qd, k[:, :, :S], v[:, :, :S], sinks=sinks)
    grown = bi.bi_sdpa(qd, k, v, mask=m[:, :, :1], sinks=sinks)
    assert_bits_equal(grown, base, "cache growth with masked keys, sinks")
    # a query that sees no key gives zeros, sink or not
    none = torch.zeros(1, 1, 1, S, dtype=torch.bool, device=DEV)
    z = bi.bi_sdpa(qd, k[:, :, :S], v[:, :, :S], mask=none, sinks=sinks)
    assert_bits_equal(z, torch.zeros_like(z), "no visible key with a sink")


@pytest.mark.parametrize("D", [32, 96, 160, 192, 224, 256])
@pytest.mark.parametrize("dt", DTS, ids=_ids)
def test_head_dims_multiple_of_32(dt, D):
    B, Hq, Hkv, Lq, S = 2, 4, 2, 9, 300              # two splits, ragged last block
    q, k, v = _qkv(B, Hq, Hkv, Lq, S, D, dt, 350 + D)
    qg, kg, vg = _gpu(q, k, v)
    o = bi.bi_sdpa(qg, kg, vg, causal=True)
    assert_close_to_oracle(o, oracle.sdpa(q, k, v, causal=True), f"D={D} {dt}")
    for i in (0, Lq - 1):
        p = S - Lq + i
        dec = bi.bi_sdpa(qg[:, :, i:i + 1], kg[:, :, :p + 1], vg[:, :, :p + 1], causal=True)
        assert_bits_equal(dec[:, :, 0], o[:, :, i], f"D={D}: token {i} vs its decode")
    assert_bits_equal(bi.bi_sdpa(qg[1:], kg[1:], vg[1:], causal=True), o[1:], f"D={D}: batch element alone")
    # zero queries: weights exp2(0) = 1, integer values -> the correctly rounded mean
    q0 = torch.zeros(1, Hq, S, D, dtype=dt)
    vi = synthetic.randint((1, Hkv, S, D), 352, -8, 8, dt)
    z = bi.bi_sdpa(q0.to(DEV), kg[:1], vi.to(DEV), causal=True).cpu()
    assert_bits_equal(z, round_ref(oracle.sdpa(q0, k[:1], vi, causal=True), dt), f"D={D}: zero-query means")


@pytest.mark.parametrize("D", [32, 64, 96])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_small_head_dims_agree_across_kernels(dt, D):
    """16-bit D < 128: the prefill kernel and the split kernels take the head dim's own D / 32 score
    chunks and D / 16 output tiles (D = 64 on the 16-bit split kernel with 128-byte key rows, D = 32 and 96
    on the generic one), the quad and one-launch kernels run on rows zero-padded to 128 (the zero
    products only add exact zeros), so every path gives the same bits.  Prefill chunk (prefill kernel) vs
    the decode of its tokens (quad kernel) and vs the oracle, a masked prefill vs the same rows called
    few at a time (split kernel), and one batch element alone (quad kernel) vs inside a batch of 40 (one
    launch at S <= 1024, a split kernel above)."""
    B, Hq, Hkv, Lq, S = 1, 16, 4, 400, 1500
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    qc, kc, vc = _qkv(B, Hq, Hkv, Lq, S, D, dt, 370 + D)
    q, k, v = _gpu(qc, kc, vc)
    lib = bi._native.load()
    name = lambda *a: lib.bi_sdpa_kernel_name(*a, D, BI).decode()
    assert name(B, Hq, Hkv, Lq, S) == "sdpa_prefill16"
    full = bi.bi_sdpa(q, k, v, causal=True)
    for i in (0, 150, 399):
        p = S - Lq + i
        assert name(B, Hq, Hkv, 1, p + 1) == "sdpa_quad16+combine"
        dec = bi.bi_sdpa(q[:, :, i:i + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True)
        assert_bits_equal(dec[:, :, 0], full[:, :, i], f"D={D}: prefill token {i} vs its quad-kernel decode")
    rows = slice(390, 400)
    ref = oracle.sdpa(qc[:, :, rows], kc[:, :, :S - Lq + 400], vc[:, :, :S - Lq + 400], causal=True)
    assert_close_to_oracle(full[:, :, rows], ref, f"D={D} prefill rows 390-399")
    gen = torch.Generator(device="cpu").manual_seed(380 + D)
    mask = (torch.rand((1, 1, Lq, S), generator=gen) > 0.2).to(DEV)
    masked = bi.bi_sdpa(q, k, v, mask=mask)
    for a in (0, 200, 396):
        assert name(B, Hq, Hkv, 4, S) != "sdpa_prefill16"
        part = bi.bi_sdpa(q[:, :, a:a + 4], k, v, mask=mask[:, :, a:a + 4])
        assert_bits_equal(part, masked[:, :, a:a + 4], f"D={D}: masked prefill rows {a}.. vs four at a time")
    split_kernel = "sdpa_split16+combine" if D == 64 else "sdpa_split+combine"
    for S2, big_kernel in ((900, "sdpa_fused16"), (1500, split_kernel)):
        qd, kd, vd = q[:, :, :2], k[:, :, :S2], v[:, :, :S2]
        assert name(1, Hq, Hkv, 2, S2) == "sdpa_quad16+combine" and name(40, Hq, Hkv, 2, S2) == big_kernel
        one = bi.bi_sdpa(qd, kd, vd, causal=True)
        rep = lambda t: t.expand(40, -1, -1, -1).contiguous()
        big = bi.bi_sdpa(rep(qd), rep(kd), rep(vd), causal=True)
        assert_bits_equal(big[:1], one, f"D={D} S={S2}: {big_kernel} vs the quad kernel")
        assert_bits_equal(big[39:], one, f"D={D} S={S2}: last batch element, {big_kernel} vs the quad kernel")


@pytest.mark.parametrize("D", [160, 192, 256])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_wide_head_dims_prefill(dt, D):
    """16-bit D > 128 with query chunks of >= 384 rows: the wide prefill kernel (rows zero-padded to
    256, all output columns of a row tile in one workgroup).  Oracle tolerance on sampled
    rows; every sampled token equals its own decode (generic split kernel) on raw bits, also under an
    additive mask with sinks; eager and graph-captured launches agree."""
    B, Hq, Hkv, Lq, S = 1, 8, 2, 400, 1300
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    q, k, v = _qkv(B, Hq, Hkv, Lq, S, D, dt, 390 + D)
    qg, kg, vg = _gpu(q, k, v)
    lib = bi._native.load()
    assert lib.bi_sdpa_kernel_name(B, Hq, Hkv, Lq, S, D, BI).decode() == "sdpa_prefill16w"
    assert lib.bi_sdpa_kernel_name(B, Hq, Hkv, 1, S, D, BI).decode() == (
        "sdpa_split16w+combine" if D == 256 else "sdpa_split+combine")
    assert bi.sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D, dt) == 0
    full = bi.bi_sdpa(qg, kg, vg, causal=True)
    rows = [0, 1, 200, 399]
    want = oracle.sdpa(q[:, :, rows[-1:]], k, v, causal=True)
    assert_close_to_oracle(full[:, :, rows[-1:]], want, f"D={D}: last row vs oracle")
    for i in rows:
        p = S - Lq + i
        ref = oracle.sdpa(q[:, :, i:i + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True)
        assert_close_to_oracle(full[:, :, i:i + 1], ref, f"D={D}: row {i} vs oracle")
        dec = bi.bi_sdpa(qg[:, :, i:i + 1], kg[:, :, :p + 1], vg[:, :, :p + 1], causal=True)
        assert_bits_equal(dec[:, :, 0], full[:, :, i], f"D={D}: prefill token {i} vs its split-kernel decode")
    amask = _additive((B, Hq, Lq, S), 391 + D, dt).to(DEV)
    amask[..., 0] = 0.0
    sinks = synthetic.randn((Hq,), 392 + D, 2.0).to(DEV)
    fm = bi.bi_sdpa(qg, kg, vg, causal=True, mask=amask, sinks=sinks)
    for i in rows:
        p = S - Lq + i
        dec = bi.bi_sdpa(qg[:, :, i:i + 1], kg[:, :, :p + 1], vg[:, :, :p + 1], causal=True,
                         mask=amask[:, :, i:i + 1, :p + 1], sinks=sinks)
        assert_bits_equal(dec[:, :, 0], fm[:, :, i], f"D={D}: masked prefill token {i} vs its decode")
    fn = lambda: bi.bi_sdpa(qg, kg, vg, causal=True, mask=amask, sinks=sinks)
    _graph_replays_equal_eager(fn, fm, f"D={D} wide prefill")


@pytest.mark.parametrize("D", [160, 192, 224, 256])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_wide_prefill_batch_switch_keeps_bits(dt, D):
    """The wide prefill kernel takes 16-bit D > 128 calls from 64 query rows once the batch holds 192 rows
    or more, so whether a row runs there or on the split kernels depends on the batch: B = 4 x 64 rows
    (wide prefill) against each element alone (split kernels), and B = 3 (192 rows, wide prefill) against
    B = 2 (128 rows, split kernels); causal, with an additive mask, and with sinks; raw bits, plus the
    oracle on one element."""
    Hq, Hkv, Lq, S = 8, 2, 64, 700
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    lib = bi._native.load()
    assert lib.bi_sdpa_kernel_name(4, Hq, Hkv, Lq, S, D, BI).decode() == "sdpa_prefill16w"
    assert lib.bi_sdpa_kernel_name(3, Hq, Hkv, Lq, S, D, BI).decode() == "sdpa_prefill16w"
    assert lib.bi_sdpa_kernel_name(2, Hq, Hkv, Lq, S, D, BI).decode() != "sdpa_prefill16w"
    assert lib.bi_sdpa_kernel_name(1, Hq, Hkv, Lq, S, D, BI).decode() != "sdpa_prefill16w"
    q, k, v = _qkv(4, Hq, Hkv, Lq, S, D, dt, 410 + D)
    amask = _additive((4, 1, Lq, S), 411 + D, dt)
    amask[..., 0] = 0.0
    sinks = synthetic.randn((Hq,), 412 + D, 2.0)
    qg, kg, vg, ag, sg = _gpu(q, k, v, amask, sinks)
    forms = (("causal", lambda b0, b1: dict(causal=True)),
             ("additive", lambda b0, b1: dict(mask=ag[b0:b1])),
             ("causal+sinks", lambda b0, b1: dict(causal=True, sinks=sg)))
    for what, kw in forms:
        four = bi.bi_sdpa(qg, kg, vg, **kw(0, 4))
        for e in range(4):
            one = bi.bi_sdpa(qg[e:e + 1], kg[e:e + 1], vg[e:e + 1], **kw(e, e + 1))
            assert_bits_equal(four[e:e + 1], one, f"D={D} {what}: element {e} in B=4 vs alone")
        three = bi.bi_sdpa(qg[:3], kg[:3], vg[:3], **kw(0, 3))
        two = bi.bi_sdpa(qg[:2], kg[:2], vg[:2], **kw(0, 2))
        assert_bits_equal(three[:2], two, f"D={D} {what}: B=3 vs B=2")
    want = oracle.sdpa(q[:1], k[:1], v[:1], causal=True, sinks=sinks)
    assert_close_to_oracle(bi.bi_sdpa(qg[:1], kg[:1], vg[:1], causal=True, sinks=sg), want, f"D={D}: vs oracle")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_wide_split_matches_generic_split(dt):
    """16-bit D = 256 decode: the wide split kernel (512-byte rows, moderate grids) and the generic split
    kernel (larger grids) give the same bits: one batch element alone against the same element inside a
    batch of 40, causal, with an additive mask and sinks, and with a ragged cache; the wide kernel also
    matches the oracle."""
    Hq, Hkv, D, NB = 8, 2, 256, 40
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    lib = bi._native.load()
    for Lq, S in ((1, 7000), (3, 6500)):
        q, k, v = _qkv(1, Hq, Hkv, Lq, S, D, dt, 400 + Lq)
        amask = _additive((1, 1, Lq, S), 401 + Lq, dt)
        amask[..., 0] = 0.0
        sinks = synthetic.randn((Hq,), 402 + Lq, 2.0)
        assert lib.bi_sdpa_kernel_name(1, Hq, Hkv, Lq, S, D, BI).decode() == "sdpa_split16w+combine"
        assert lib.bi_sdpa_kernel_name(NB, Hq, Hkv, Lq, S, D, BI).decode() == "sdpa_split+combine"
        qg, kg, vg, ag, sg = _gpu(q, k, v, amask, sinks)
        rep = lambda t: t.expand(NB, *t.shape[1:]).contiguous()
        for what, kw in (("causal", dict(causal=True)), ("additive+sinks", dict(causal=True, mask=ag, sinks=sg))):
            one = bi.bi_sdpa(qg, kg, vg, **kw)
            kwb = dict(kw)
            if "mask" in kw:
                kwb["mask"] = rep(kw["mask"])
            many = bi.bi_sdpa(rep(qg), rep(kg), rep(vg), **kwb)
            for e in (0, NB - 1):
                assert_bits_equal(many[e:e + 1], one, f"Lq={Lq} S={S} {what}: generic element {e} vs wide")
        want = oracle.sdpa(q, k, v, causal=True, mask=amask.to(torch.float64), sinks=sinks)
        assert_close_to_oracle(bi.bi_sdpa(qg, kg, vg, causal=True, mask=ag, sinks=sg), want, f"Lq={Lq}: wide vs oracle")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_d64_split_matches_quad(dt):
    """16-bit D = 64 decode: the 16-bit split kernel on 128-byte key rows (large grids) and the quad kernel
    on rows zero-padded to 128 (small grids) give the same bits: one batch element alone against the same
    element inside a batch of 40, causal, with an additive mask and sinks, with a ragged cache and three
    query rows; the split kernel also matches the oracle."""
    Hq, Hkv, D, NB = 8, 2, 64, 40
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    lib = bi._native.load()
    for Lq, S in ((1, 7000), (3, 6500)):
        q, k, v = _qkv(1, Hq, Hkv, Lq, S, D, dt, 410 + Lq)
        amask = _additive((1, 1, Lq, S), 411 + Lq, dt)
        amask[..., 0] = 0.0
        sinks = synthetic.randn((Hq,), 412 + Lq, 2.0)
        assert lib.bi_sdpa_kernel_name(1, Hq, Hkv, Lq, S, D, BI).decode() == "sdpa_quad16+combine"
        assert lib.bi_sdpa_kernel_name(NB, Hq, Hkv, Lq, S, D, BI).decode() == "sdpa_split16+combine"
        qg, kg, vg, ag, sg = _gpu(q, k, v, amask, sinks)
        rep = lambda t: t.expand(NB, *t.shape[1:]).contiguous()
        for what, kw in (("causal", dict(causal=True)), ("additive+sinks", dict(causal=True, mask=ag, sinks=sg))):
            one = bi.bi_sdpa(qg, kg, vg, **kw)
            kwb = dict(kw)
            if "mask" in kw:
                kwb["mask"] = rep(kw["mask"])
            many = bi.bi_sdpa(rep(qg), rep(kg), rep(vg), **kwb)
            for e in (0, NB - 1):
                assert_bits_equal(many[e:e + 1], one, f"Lq={Lq} S={S} {what}: split element {e} vs quad")
        want = oracle.sdpa(q, k, v, causal=True, mask=amask.to(torch.float64), sinks=sinks)
        many = bi.bi_sdpa(rep(qg), rep(kg), rep(vg), causal=True, mask=rep(ag), sinks=sg)
        assert_close_to_oracle(many[:1], want, f"Lq={Lq}: split vs oracle")


def test_forms_together_and_bad_arguments():
    B, Hq, Hkv, Lq, S, D = 1, 8, 4, 6, 520, 64
    dt = torch.bfloat16
    q, k, v = _qkv(B, Hq, Hkv, Lq, S, D, dt, 360)
    amask = _additive((1, 1, Lq, S), 361, dt)
    amask[..., 0] = 0.0
    sinks = synthetic.randn((Hq,), 362, 2.0)
    qg, kg, vg, ag = _gpu(q, k, v, amask)
    o = bi.bi_sdpa(qg, kg, vg, causal=True, mask=ag, sinks=sinks)
    want = oracle.sdpa(q, k, v, causal=True, mask=amask.to(torch.float64), sinks=sinks)
    assert_close_to_oracle(o, want, "additive mask, causal and sinks together")
    with pytest.raises(ValueError):                     # an additive mask must share q's dtype
        bi.bi_sdpa(qg, kg, vg, mask=ag.float())
    with pytest.raises(ValueError):                     # one sink per query head
        bi.bi_sdpa(qg, kg, vg, sinks=sinks[:3])
    with pytest.raises(NotImplementedError):            # head dims are multiples of 32
        bi.bi_sdpa(qg[..., :48], kg[..., :48], vg[..., :48])


def _graph_replays_equal_eager(fn, eager, what, reps=4):
    """Capture fn in a graph, replay it several times with eager work and synchronisations in between,
    and compare every replay with the eager result on raw bits (the output is poisoned before each)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    for rep in range(reps):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(out, eager, f"{what}: graph replay {rep}")
        fn()
        torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(1, 8, 2, 9, 1500), (1, 32, 8, 64, 1024), (1, 8, 2, 5, 200), (1, 8, 2, 400, 900)],
                         ids=["quad", "quad-two-tiles", "quad-one-split", "prefill"])
def test_forms_graph_replay_equals_eager(shape):
    """Eager vs graph-captured launch give the same bits, for the additive mask, sinks and a padded
    head dim (workspace, when the path needs one, allocated inside the captured call)."""
    B, Hq, Hkv, Lq, S = shape
    dt = torch.bfloat16
    q, k, v = _gpu(*_qkv(B, Hq, Hkv, Lq, S, 128, dt, 380 + Lq))
    amask = _additive((B, 1, Lq, S), 381, dt).to(DEV)
    amask[..., 0] = 0.0
    sinks = synthetic.randn((Hq,), 382, 2.0).to(DEV)
    fn = lambda: bi.bi_sdpa(q, k, v, causal=True, mask=amask, sinks=sinks)
    _graph_replays_equal_eager(fn, fn(), f"additive mask + sinks {shape}")
    q64, k64, v64 = _gpu(*_qkv(B, Hq, Hkv, Lq, S, 64, dt, 383 + Lq))
    fn64 = lambda: bi.bi_sdpa(q64, k64, v64, causal=True)
    _graph_replays_equal_eager(fn64, fn64(), f"D=64 {shape}")
