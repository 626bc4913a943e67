"""GPU tests of the invariant attention entry point (bi_sdpa).

* exact pins: zero queries make every weight exp2(0) = 1, so with integer
  values the output is the correctly rounded mean; a row that sees one key
  returns that key's value row;
* oracle tolerance on the seeded workloads;
* invariance on raw bit patterns: every token of a prefill chunk equals its
  own decode call (K / V truncated after it) and the full-cache decode with a
  mask, for every query length of the sweep; growing the KV cache with masked
  keys (crossing 4096) leaves results unchanged; batch neighbours, GQA vs
  repeated-KV MHA, causal and masked-key invariants; repeats and graph replay.
"""
import math

import numpy as np
import pytest
import torch

import invariant_deterministic_gemm_amd as bi
import oracle
import synthetic
from helpers import assert_bits_equal, assert_close_to_oracle, n_bit_diff, round_ref

pytestmark = pytest.mark.gpu
DEV = "cuda"
DTS = [torch.float32, torch.bfloat16, torch.float16]


def _ids(d):
    return str(d).split(".")[-1]


@pytest.mark.parametrize("dt", DTS, ids=_ids)
@pytest.mark.parametrize("D", [64, 128])
def test_zero_query_gives_exact_mean(dt, D):
    B, Hq, Hkv, S = 1, 4, 2, 700                 # three splits, ragged last block
    q = torch.zeros(B, Hq, S, D, dtype=dt)
    k = synthetic.randn((B, Hkv, S, D), 51, 1.0, dt)
    v = synthetic.randint((B, Hkv, S, D), 52, -8, 8, dt)
    o = bi.bi_sdpa(q.to(DEV), k.to(DEV), v.to(DEV), causal=True).cpu()
    ref = oracle.sdpa(q, k, v, causal=True)
    assert_bits_equal(o, round_ref(ref, dt), f"zero-query means {dt} D={D}")


@pytest.mark.parametrize("dt", DTS, ids=_ids)
def test_single_visible_key_returns_its_value(dt):
    B, Hq, Hkv, S, D = 2, 8, 2, 300, 128
    q = synthetic.randn((B, Hq, S, D), 61, 1.0, dt)
    k = synthetic.randn((B, Hkv, S, D), 62, 1.0, dt)
    v = synthetic.randn((B, Hkv, S, D), 63, 1.0, dt)
    o = bi.bi_sdpa(q.to(DEV), k.to(DEV), v.to(DEV), causal=True).cpu()
    for h in range(Hq):
        assert_bits_equal(o[:, h, 0], v[:, h * Hkv // Hq, 0], f"row 0 sees only key 0 (h={h})")
    mask = torch.zeros(1, 1, 1, S, dtype=torch.bool)
    mask[..., 123] = True
    o = bi.bi_sdpa(q[:, :, :3].to(DEV), k.to(DEV), v.to(DEV), mask=mask.to(DEV)).cpu()
    for h in range(Hq):
        for i in range(3):
            assert_bits_equal(o[:, h, i], v[:, h * Hkv // Hq, 123], "mask with one key")


def test_rows_without_visible_keys_are_zero():
    q = synthetic.randn((1, 4, 2, 128), 71, 1.0, torch.bfloat16).to(DEV)
    k = synthetic.randn((1, 2, 50, 128), 72, 1.0, torch.bfloat16).to(DEV)
    mask = torch.zeros(1, 1, 2, 50, dtype=torch.bool, device=DEV)
    o = bi.bi_sdpa(q, k, k, mask=mask)
    assert_bits_equal(o, torch.zeros_like(o), "no visible key")
    o = bi.bi_sdpa(q, k[:, :, :0], k[:, :, :0])
    assert_bits_equal(o, torch.zeros_like(o), "empty cache")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_single_split_finished_in_the_quad_kernel(dt):
    """At most 256 keys (one split) the quad kernel applies the combine's fold itself (no workspace, no
    second launch): the same bits as the one-launch kernel, or the prefill kernel once a KV head has 64
    query rows (the element inside a batch of 160), for every mask form, sinks and ragged cache lengths,
    and the oracle's values."""
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    Hq, Hkv, D, NB = 8, 2, 128, 160
    for S, Lq in ((256, 1), (200, 3), (70, 17), (1, 1)):
        q = synthetic.randn((1, Hq, Lq, D), 91 + S, 1.0, dt)
        k = synthetic.randn((1, Hkv, S, D), 92 + S, 1.0, dt)
        v = synthetic.randn((1, Hkv, S, D), 93 + S, 1.0, dt)
        g = torch.Generator().manual_seed(94 + S)
        bmask = torch.rand((1, Hq, Lq, S), generator=g) > 0.3
        bmask[..., 0] = True
        amask = (torch.randn((1, 1, Lq, S), generator=g) * 2).to(dt)
        amask[..., S // 2:] = float("-inf")
        amask[..., 0] = 0.0
        sinks = synthetic.randn((Hq,), 95 + S, 2.0)
        assert lib.bi_sdpa_kernel_name(1, Hq, Hkv, Lq, S, D, BI).decode() == "sdpa_quad16"
        assert lib.bi_sdpa_kernel_name(NB, Hq, Hkv, Lq, S, D, BI).decode() == (
            "sdpa_prefill16" if Hq // Hkv * Lq >= 64 else "sdpa_fused16")
        assert bi.sdpa_workspace_bytes(1, Hq, Hkv, Lq, S, D, dt) == 0
        rep = lambda t: t.expand(NB, *t.shape[1:]).contiguous()
        qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
        forms = {"causal": dict(causal=True), "bool": dict(mask=bmask.to(DEV)),
                 "additive+sinks": dict(mask=amask.to(DEV), causal=True, sinks=sinks.to(DEV)),
                 "sinks": dict(sinks=sinks.to(DEV))}
        for fname, kw in forms.items():
            one = bi.bi_sdpa(qg, kg, vg, **kw)
            kwb = dict(kw)
            if "mask" in kw:
                kwb["mask"] = rep(kw["mask"])
            many = bi.bi_sdpa(rep(qg), rep(kg), rep(vg), **kwb)
            for e in (0, NB - 1):
                assert_bits_equal(many[e:e + 1], one, f"S={S} Lq={Lq} {fname}: one-launch element {e} vs quad")
        want = oracle.sdpa(q, k, v, causal=True, mask=amask.to(torch.float64), sinks=sinks)
        assert_close_to_oracle(bi.bi_sdpa(qg, kg, vg, causal=True, mask=amask.to(DEV), sinks=sinks.to(DEV)).cpu(),
                               want, f"S={S} Lq={Lq}: quad vs oracle")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_edge_rows_on_every_16bit_kernel(dt):
    """A row that sees one key returns that key's value row, and a row that sees none returns zeros, on
    the quad kernel (one batch element) and on the one-launch and split kernels (the same element
    repeated 80 times), with and without sinks (a sink with no visible key still gives zeros)."""
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    Hq, Hkv, D, NB = 8, 2, 128, 80
    for S, big in ((300, "sdpa_fused16"), (2000, "sdpa_split16+combine")):
        q = synthetic.randn((1, Hq, 3, D), 81 + S, 1.0, dt).to(DEV)
        k = synthetic.randn((1, Hkv, S, D), 82 + S, 1.0, dt).to(DEV)
        v = synthetic.randn((1, Hkv, S, D), 83 + S, 1.0, dt).to(DEV)
        one_key = torch.zeros(1, 1, 3, S, dtype=torch.bool, device=DEV)
        one_key[..., S - 7] = True
        one_key[:, :, 2] = False                          # the third row sees nothing
        sinks = synthetic.randn((Hq,), 84 + S, 2.0).to(DEV)
        assert lib.bi_sdpa_kernel_name(1, Hq, Hkv, 3, S, D, BI).decode() == "sdpa_quad16+combine"
        assert lib.bi_sdpa_kernel_name(NB, Hq, Hkv, 3, S, D, BI).decode() == big
        rep = lambda t: t.expand(NB, *t.shape[1:]).contiguous()
        for b_, (qq, kk, vv, mm) in (("quad", (q, k, v, one_key)), (big, (rep(q), rep(k), rep(v), rep(one_key)))):
            o = bi.bi_sdpa(qq, kk, vv, mask=mm)
            for h in range(Hq):
                for i in range(2):
                    assert_bits_equal(o[:, h, i], vv[:, h * Hkv // Hq, S - 7], f"{b_} S={S}: one visible key")
            assert_bits_equal(o[:, :, 2], torch.zeros_like(o[:, :, 2]), f"{b_} S={S}: no visible key")
            os_ = bi.bi_sdpa(qq, kk, vv, mask=mm, sinks=sinks)
            assert_bits_equal(os_[:, :, 2], torch.zeros_like(os_[:, :, 2]), f"{b_} S={S}: no visible key, sinks")
            # one key and a sink: weights e^(s - m) / (e^(s - m) + e^(sink - m)); only the key carries a value
            assert torch.isfinite(os_.float()).all()


@pytest.mark.parametrize("B", [1, 2])
def test_config3_prefill_tokens_equal_their_decode(B):
    S = 1024
    d = synthetic.cfg3_inputs(B=max(B, 1), S=S + 64)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(128)
    # decode references for the last 64 positions of S = 1024, two ways
    dec = {}
    for p in range(S - 64, S):
        dec[p] = bi.bi_sdpa(q[:, :, p:p + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True, scale=scale)
        m = torch.zeros(1, 1, 1, S, dtype=torch.bool, device=DEV)
        m[..., :p + 1] = True
        dm = bi.bi_sdpa(q[:, :, p:p + 1], k[:, :, :S], v[:, :, :S], mask=m, scale=scale)
        assert_bits_equal(dm, dec[p], f"decode p={p}: truncated cache vs full cache + mask")
    for L in synthetic.CFG3["Lq_values"] + [3, 33]:
        o = bi.bi_sdpa(q[:, :, S - L:S], k[:, :, :S], v[:, :, :S], causal=True, scale=scale)
        for i in range(L):
            p = S - L + i
            assert_bits_equal(o[:, :, i:i + 1], dec[p], f"q_len={L}, token {i} (position {p})")
    # the same chunks against a cache of 1024 + L (chunk at the end)
    for L in (1, 9, 64):
        SS = S + L
        o = bi.bi_sdpa(q[:, :, SS - L:SS], k[:, :, :SS], v[:, :, :SS], causal=True, scale=scale)
        for i in range(L):
            p = SS - L + i
            ref = bi.bi_sdpa(q[:, :, p:p + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True, scale=scale)
            assert_bits_equal(o[:, :, i:i + 1], ref, f"cache {SS}, q_len={L}, token {i}")


def test_config3_accuracy_against_oracle():
    S = 1024
    d = synthetic.cfg3_inputs(B=1, S=S)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    for L in (1, 9, 64):
        o = bi.bi_sdpa(q[:, :, S - L:], k, v, causal=True)
        ref = oracle.sdpa(d["q"][:, :, S - L:], d["k"], d["v"], causal=True)
        assert_close_to_oracle(o.cpu(), ref, f"config 3 q_len={L}")


def test_batch_neighbours_and_gqa_equal_mha():
    S = 1024
    d = synthetic.cfg3_inputs(B=4, S=S)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    L = 16
    full = bi.bi_sdpa(q[:, :, S - L:], k, v, causal=True)
    for b in range(4):
        one = bi.bi_sdpa(q[b:b + 1, :, S - L:], k[b:b + 1], v[b:b + 1], causal=True)
        assert_bits_equal(full[b:b + 1], one, f"batch element {b} alone vs in a batch of 4")
    # neighbours replaced by NaN
    q2, k2, v2 = (torch.full_like(t, float("nan")) for t in (q, k, v))
    q2[2], k2[2], v2[2] = q[2], k[2], v[2]
    o2 = bi.bi_sdpa(q2[:, :, S - L:], k2, v2, causal=True)
    assert_bits_equal(o2[2], full[2], "NaN batch neighbours")
    # GQA == MHA with K/V repeated per group
    G = 4
    krep = k.repeat_interleave(G, dim=1).contiguous()
    vrep = v.repeat_interleave(G, dim=1).contiguous()
    mha = bi.bi_sdpa(q[:, :, S - L:], krep, vrep, causal=True)
    assert_bits_equal(mha, full, "GQA vs repeated-KV MHA")
    # a single head of a group called alone (G = 1)
    h = 5
    solo = bi.bi_sdpa(q[:, h:h + 1, S - L:], k[:, h // G:h // G + 1], v[:, h // G:h // G + 1], causal=True)
    assert_bits_equal(solo, full[:, h:h + 1], "one query head alone")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=_ids)
def test_config4_context_growth_with_masked_keys(dt):
    d = synthetic.cfg4_inputs(dt, S=4200)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    lo, hi = synthetic.CFG4["S_lo"], synthetic.CFG4["S_hi"]
    for n0 in (4000, 4095, 4096, 4097):
        base = bi.bi_sdpa(q, k[:, :, :n0], v[:, :, :n0])
        ref = oracle.sdpa(d["q"], d["k"][:, :, :n0], d["v"][:, :, :n0])
        assert_close_to_oracle(base.cpu(), ref, f"config 4 {dt} S={n0}")
        for n in range(n0, hi + 1, 7 if n0 == 4000 else 1):
            m = torch.zeros(1, 1, 1, n, dtype=torch.bool, device=DEV)
            m[..., :n0] = True
            o = bi.bi_sdpa(q, k[:, :, :n], v[:, :, :n], mask=m)
            assert_bits_equal(o, base, f"{dt}: S={n} with keys >= {n0} masked vs S={n0}")
    prev = bi.bi_sdpa(q, k[:, :, :lo - 1], v[:, :, :lo - 1])
    for n in range(lo, hi + 1):
        m = torch.ones(1, 1, 1, n, dtype=torch.bool, device=DEV)
        m[..., n - 1] = False
        o = bi.bi_sdpa(q, k[:, :, :n], v[:, :, :n], mask=m)
        assert_bits_equal(o, prev, f"{dt}: S={n} with its newest key masked vs S={n - 1}")
        prev = bi.bi_sdpa(q, k[:, :, :n], v[:, :, :n])


@pytest.mark.parametrize("dt", DTS, ids=_ids)
def test_context_growth_across_split_counts(dt):
    """Masked keys appended past 256, 512, 768 and 1024 keys (where the number
    of 256-key splits, and with it the launch shape, changes) leave the bits
    unchanged; decode and a 5-token chunk both."""
    S_max = 1100
    q = synthetic.randn((2, 16, 5, 128), 0x5EED40, 1.0, dt).to(DEV)
    k = synthetic.randn((2, 8, S_max, 128), 0x5EED41, 1.0, dt).to(DEV)
    v = synthetic.randn((2, 8, S_max, 128), 0x5EED42, 1.0, dt).to(DEV)
    for n0 in (250, 256, 500, 700, 1000, 1024):
        for L in (1, 5):
            base = bi.bi_sdpa(q[:, :, :L], k[:, :, :n0], v[:, :, :n0], causal=True)
            for n in sorted({n0 + 1, n0 + 7, 257, 513, 769, 1025, 1100}):
                if n <= n0:
                    continue
                m = torch.zeros(1, 1, L, n, dtype=torch.bool, device=DEV)
                for i in range(L):
                    m[..., i, :n0 - L + 1 + i] = True
                o = bi.bi_sdpa(q[:, :, :L], k[:, :, :n], v[:, :, :n], mask=m)
                assert_bits_equal(o, base, f"{dt} q_len={L}: S={n} with keys >= {n0} masked vs S={n0}")


def test_causal_and_masked_key_values_are_never_read():
    B, Hq, Hkv, L, S, D = 1, 8, 2, 40, 600, 128
    q = synthetic.randn((B, Hq, L, D), 81, 1.0, torch.bfloat16).to(DEV)
    k = synthetic.randn((B, Hkv, S, D), 82, 1.0, torch.bfloat16).to(DEV)
    v = synthetic.randn((B, Hkv, S, D), 83, 1.0, torch.bfloat16).to(DEV)
    base = bi.bi_sdpa(q, k, v, causal=True)
    for i in (0, 17, 39):
        p = S - L + i
        k2, v2 = k.clone(), v.clone()
        k2[:, :, p + 1:] = 1e4
        v2[:, :, p + 1:] = -3e3
        assert_bits_equal(bi.bi_sdpa(q, k2, v2, causal=True)[:, :, i], base[:, :, i], f"causal row {i}")
    mask = torch.ones(1, 1, L, S, dtype=torch.bool, device=DEV)
    mask[..., 100:130] = False
    mask[..., 7] = False
    mb = bi.bi_sdpa(q, k, v, mask=mask)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 100:130] = 5e3
    v2[:, :, 7] = -7e3
    assert_bits_equal(bi.bi_sdpa(q, k2, v2, mask=mask), mb, "masked key values are not read")
    ref = oracle.sdpa(q.cpu(), k.cpu(), v.cpu(), mask=mask.cpu())
    assert_close_to_oracle(mb.cpu(), ref, "boolean mask")
    # per-head mask equal to the broadcast one
    mfull = mask.expand(B, Hq, L, S).contiguous()
    assert_bits_equal(bi.bi_sdpa(q, k, v, mask=mfull), mb, "expanded mask")


@pytest.mark.parametrize("dt", DTS, ids=_ids)
@pytest.mark.parametrize("D", [64, 128])
def test_accuracy_small_shapes(dt, D):
    B, Hq, Hkv, L, S = 2, 6, 3, 20, 333
    q = synthetic.randn((B, Hq, L, D), 91, 1.0, dt)
    k = synthetic.randn((B, Hkv, S, D), 92, 1.0, dt)
    v = synthetic.randn((B, Hkv, S, D), 93, 1.0, dt)
    for causal in (False, True):
        o = bi.bi_sdpa(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
        assert_close_to_oracle(o.cpu(), oracle.sdpa(q, k, v, causal=causal), f"{dt} D={D} causal={causal}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_quad_fused_and_split_kernels_agree(dt):
    """16-bit D = 128: the kernel follows the size of the grid (splits x row tiles x B x KV heads), so
    the same batch element runs the quad kernel alone and the one-launch (S <= 1024), split (S > 1024)
    or prefill (64 query rows per KV head) kernel inside a batch of 48.  Every mask form, sinks, ragged S and several query lengths give
    the same bits either way, and the quad results match the oracle."""
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    Hq, Hkv, NB = 8, 2, 48
    for S, Lq, big in ((700, 1, "sdpa_fused16"), (1024, 5, "sdpa_fused16"), (1000, 17, "sdpa_prefill16"),
                       (2085, 2, "sdpa_split16+combine"), (4100, 9, "sdpa_split16+combine")):
        seed = 0x5EED70 + S + Lq
        q = synthetic.randn((1, Hq, Lq, 128), seed, 1.0, dt)
        k = synthetic.randn((1, Hkv, S, 128), seed + 1, 1.0, dt)
        v = synthetic.randn((1, Hkv, S, 128), seed + 2, 1.0, dt)
        g = torch.Generator().manual_seed(seed + 3)
        bmask = torch.rand((1, Hq, Lq, S), generator=g) > 0.25
        bmask[..., 0] = True
        amask = (torch.randn((1, 1, Lq, S), generator=g) * 2).to(dt)
        amask[torch.rand((1, 1, Lq, S), generator=g) < 0.2] = float("-inf")
        amask[..., 0] = 0.0
        sinks = synthetic.randn((Hq,), seed + 4, 2.0)
        assert lib.bi_sdpa_kernel_name(1, Hq, Hkv, Lq, S, 128, BI).decode() == "sdpa_quad16+combine"
        assert lib.bi_sdpa_kernel_name(NB, Hq, Hkv, Lq, S, 128, BI).decode() == big
        rep = lambda t: t.expand(NB, *t.shape[1:]).contiguous()
        qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
        qb, kb, vb = rep(qg), rep(kg), rep(vg)
        forms = {"causal": dict(causal=True), "bool": dict(mask=bmask.to(DEV)),
                 "additive+causal": dict(mask=amask.to(DEV), causal=True),
                 "sinks+causal": dict(causal=True, sinks=sinks.to(DEV))}
        for fname, kw in forms.items():
            one = bi.bi_sdpa(qg, kg, vg, **kw)
            kwb = dict(kw)
            if "mask" in kw:
                kwb["mask"] = kw["mask"].expand(NB, *kw["mask"].shape[1:]).contiguous()
            many = bi.bi_sdpa(qb, kb, vb, **kwb)
            for e in (0, 17, NB - 1):
                assert_bits_equal(many[e:e + 1], one, f"S={S} Lq={Lq} {fname}: {big} element {e} vs quad")
            if fname in ("causal", "sinks+causal"):
                want = oracle.sdpa(q, k, v, causal=True, sinks=sinks if fname == "sinks+causal" else None)
                assert_close_to_oracle(one.cpu(), want, f"S={S} Lq={Lq} {fname}: quad vs oracle")


def test_strided_qkv_views():
    S, D = 512, 128
    qkv = synthetic.randn((1, 300, 3 * 4, D), 95, 1.0, torch.bfloat16).to(DEV)   # (B, L, 3H, D)
    q = qkv[:, :, 0:4].transpose(1, 2)
    k = qkv[:, :, 4:8:2].transpose(1, 2)
    v = qkv[:, :, 8:12:2].transpose(1, 2)
    o = bi.bi_sdpa(q, k, v, causal=True)
    oc = bi.bi_sdpa(q.contiguous(), k.contiguous(), v.contiguous(), causal=True)
    assert_bits_equal(o, oc, "strided views vs contiguous copies")
    assert S > 0


def test_repeat_and_graph_replay():
    d = synthetic.cfg3_inputs(B=1, S=1024)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    eager = bi.bi_sdpa(q[:, :, -9:], k, v, causal=True)
    for _ in range(20):
        assert_bits_equal(bi.bi_sdpa(q[:, :, -9:], k, v, causal=True), eager, "repeat")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bi.bi_sdpa(q[:, :, -9:], k, v, causal=True)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = bi.bi_sdpa(q[:, :, -9:], k, v, causal=True)
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(out, eager, f"graph replay {rep}")
        bi.bi_sdpa(q[:, :, -1:], k, v, causal=True)
        torch.cuda.synchronize()


def test_readme_style_call():
    d = synthetic.cfg3_inputs(B=1, S=256)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    assert_bits_equal(bi.scaled_dot_product_attention(q[:, :, -4:], k, v, mask="causal"),
                      bi.bi_sdpa(q[:, :, -4:], k, v, causal=True), "mask='causal'")
    assert np.isfinite(bi.scaled_dot_product_attention(q[:, :, -4:], k, v).float().cpu().numpy()).all()


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
def test_prefill_path_matches_split_path_and_decode(dt):
    """Query chunks of >= 384 rows run the workspace-free prefill kernel, and so do chunks of 383 (at
    least 64 rows per KV head); chunks of fewer than 64 rows per KV head run the quad, split + combine or
    one-launch kernels.  The tokens such chunks share must have the same bits, and sampled tokens must
    equal their own decode call."""
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    for (B, Hq, Hkv, S) in [(2, 32, 8, 2085), (1, 16, 8, 1500), (1, 16, 16, 1100), (1, 32, 8, 1000), (2, 8, 8, 700)]:
        q = synthetic.randn((B, Hq, 500, 128), 0x5EED50 + S, 1.0, dt).to(DEV)
        k = synthetic.randn((B, Hkv, S, 128), 0x5EED51 + S, 1.0, dt).to(DEV)
        v = synthetic.randn((B, Hkv, S, 128), 0x5EED52 + S, 1.0, dt).to(DEV)
        Ls = 64 // (Hq // Hkv) - 1                       # rows of a chunk below the prefill kernel's range
        assert lib.bi_sdpa_kernel_name(B, Hq, Hkv, 384, S, 128, BI).decode() == "sdpa_prefill16"
        assert lib.bi_sdpa_kernel_name(B, Hq, Hkv, 383, S, 128, BI).decode() == "sdpa_prefill16"
        assert lib.bi_sdpa_kernel_name(B, Hq, Hkv, Ls, S, 128, BI).decode() != "sdpa_prefill16"
        shifted = bi.bi_sdpa(q[:, :, -383:], k, v, causal=True)
        split = bi.bi_sdpa(q[:, :, -Ls:], k, v, causal=True)
        for L in (384, 390, 500):
            pre = bi.bi_sdpa(q[:, :, -L:], k, v, causal=True)
            assert_bits_equal(pre[:, :, -383:], shifted, f"S={S} Hq={Hq}: q_len {L} vs 383 (row tiles shifted)")
            assert_bits_equal(pre[:, :, -Ls:], split, f"S={S} Hq={Hq}: q_len {L} (prefill) vs {Ls} (split)")
            for i in (0, L // 2, L - 1):
                p = S - L + i
                dec = bi.bi_sdpa(q[:, :, 500 - L + i:500 - L + i + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True)
                assert_bits_equal(pre[:, :, i:i + 1], dec, f"S={S} q_len {L} token {i} vs its decode")
        # no causal mask, boolean mask with holes
        mask = torch.ones(1, 1, 1, S, dtype=torch.bool, device=DEV)
        mask[..., 50:300] = False
        a = bi.bi_sdpa(q[:, :, -384:], k, v, mask=mask)
        c = bi.bi_sdpa(q[:, :, -Ls:], k, v, mask=mask)
        assert_bits_equal(a[:, :, -Ls:], c, f"S={S}: masked, prefill vs split")
        ref = oracle.sdpa(q[:1, :, -384:].cpu(), k[:1].cpu(), v[:1].cpu(), mask=mask.cpu())
        assert_close_to_oracle(a[:1].cpu(), ref, f"S={S}: masked prefill vs oracle")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=_ids)
@pytest.mark.parametrize("B,Hq,Hkv,S", [(2, 16, 8, 1000), (1, 32, 8, 1337), (3, 8, 2, 777)])
def test_every_prefill_token_matches_split_chunks(dt, B, Hq, Hkv, S):
    """Every token of a causal prefill (query chunk = the whole cache, the prefill kernel) equals the same
    token computed by the quad, split + combine or one-launch kernels in chunks of fewer than 64 query
    rows per KV head against the cache truncated after the chunk: ragged row-tile groups, caches that
    end inside a block, GQA factors 2 and 4, batch neighbours."""
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    q = synthetic.randn((B, Hq, S, 128), 0x5EED53 + S, 1.0, dt).to(DEV)
    k = synthetic.randn((B, Hkv, S, 128), 0x5EED54 + S, 1.0, dt).to(DEV)
    v = synthetic.randn((B, Hkv, S, 128), 0x5EED55 + S, 1.0, dt).to(DEV)
    assert lib.bi_sdpa_kernel_name(B, Hq, Hkv, S, S, 128, BI).decode() == "sdpa_prefill16"
    full = bi.bi_sdpa(q, k, v, causal=True)
    cs = 64 // (Hq // Hkv) - 1
    a = 0
    while a < S:
        e = min(a + cs, S)
        assert lib.bi_sdpa_kernel_name(B, Hq, Hkv, e - a, e, 128, BI).decode() != "sdpa_prefill16"
        part = bi.bi_sdpa(q[:, :, a:e], k[:, :, :e], v[:, :, :e], causal=True)
        assert_bits_equal(full[:, :, a:e], part, f"tokens {a}..{e - 1}")
        a = e
    ref = oracle.sdpa(q[:1, :, -64:].cpu(), k[:1].cpu(), v[:1].cpu(), causal=True)
    assert_close_to_oracle(full[:1, :, -64:].cpu(), ref, "last 64 tokens vs oracle")


def test_long_causal_prefill_needs_no_workspace():
    """A 4096-token causal prefill against its own 4096-key cache (the split path would need a
    multi-GB workspace): no workspace is requested, sampled rows match the oracle and equal a decode."""
    S = 4096
    q = synthetic.randn((1, 32, S, 128), 0x5EED60, 1.0, torch.bfloat16).to(DEV)
    k = synthetic.randn((1, 8, S, 128), 0x5EED61, 1.0, torch.bfloat16).to(DEV)
    v = synthetic.randn((1, 8, S, 128), 0x5EED62, 1.0, torch.bfloat16).to(DEV)
    assert bi.sdpa_workspace_bytes(1, 32, 8, S, S, 128, torch.bfloat16) == 0
    o = bi.bi_sdpa(q, k, v, causal=True)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for p in (0, 1, 255, 256, 1000, 2047, 4095):
        ref = oracle.sdpa(qc[:, :, p:p + 1], kc[:, :, :p + 1], vc[:, :, :p + 1], causal=True)
        assert_close_to_oracle(o[:, :, p:p + 1].cpu(), ref, f"row {p}")
        dec = bi.bi_sdpa(q[:, :, p:p + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True)
        assert_bits_equal(o[:, :, p:p + 1], dec, f"row {p} vs its decode")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=_ids)
def test_variant_attention_is_accurate_but_batch_variant(dt):
    """The batch-variant attention comparator (split length from G * q_len and S, one pass up to 4096 keys):
    within the oracle gate, but a token's bits move with its query count (GQA factor 2: decode runs 32
    splits, a chunk of two tokens 64) and when a fully masked key takes the cache past 4096 keys -- the
    three switches the page lists -- while the invariant path does not move."""
    lib = bi._native.load()
    assert lib.bi_variant_sdpa_split_len(2, 1, 8192) == 256 and lib.bi_variant_sdpa_split_len(2, 2, 8192) == 128
    assert lib.bi_variant_sdpa_split_len(4, 1, 4096) == 4096 and lib.bi_variant_sdpa_split_len(4, 1, 4097) == 128
    S = 6000
    q = synthetic.randn((1, 16, 2, 128), 0x5EEDB0, 1.0, dt).to(DEV)
    k = synthetic.randn((1, 8, S, 128), 0x5EEDB1, 1.0, dt).to(DEV)
    v = synthetic.randn((1, 8, S, 128), 0x5EEDB2, 1.0, dt).to(DEV)
    chunk = bi.bi_variant_sdpa(q, k, v, causal=True)
    dec = bi.bi_variant_sdpa(q[:, :, 1:], k, v, causal=True)
    ref = oracle.sdpa(q.cpu(), k.cpu(), v.cpu(), causal=True)
    assert_close_to_oracle(chunk.cpu(), ref, "variant chunk vs oracle")
    assert_close_to_oracle(dec.cpu(), ref[:, :, 1:], "variant decode vs oracle")
    assert n_bit_diff(chunk[:, :, 1:], dec) > 0, "q_len 2 vs 1 changed no bit"
    assert_bits_equal(bi.bi_sdpa(q, k, v, causal=True)[:, :, 1:], bi.bi_sdpa(q[:, :, 1:], k, v, causal=True),
                      "invariant path, q_len 2 vs 1")
    # context growth: 4096 keys vs 4097 with the newest fully masked
    qd = q[:, :, 1:]
    base = bi.bi_variant_sdpa(qd, k[:, :, :4096], v[:, :, :4096])
    mask = torch.ones(1, 1, 1, 4097, dtype=torch.bool, device=DEV)
    mask[..., 4096] = False
    grown = bi.bi_variant_sdpa(qd, k[:, :, :4097], v[:, :, :4097], mask=mask)
    assert n_bit_diff(base, grown) > 0, "crossing 4096 keys changed no bit"
    assert_close_to_oracle(grown.cpu(), oracle.sdpa(qd.cpu(), k[:, :, :4096].cpu(), v[:, :, :4096].cpu()),
                           "variant grown vs oracle")
    assert_bits_equal(bi.bi_sdpa(qd, k[:, :, :4097], v[:, :, :4097], mask=mask),
                      bi.bi_sdpa(qd, k[:, :, :4096], v[:, :, :4096]), "invariant path across 4096")


def test_workspace_stays_bounded_for_long_calls():
    """Calls whose split partials would exceed 256 MiB (fp32 long prefill, 16-bit multi-row calls against
    long caches) run in query-row chunks, so the workspace query stays bounded; every sampled row keeps the
    bits of its own single-row call and the oracle gate holds."""
    lib = bi._native.load()
    cap = 256 * 2 ** 20
    # fp32 causal prefill, 4096 tokens (the whole-call partials would need ~1.1 GB)
    S = 4096
    q = synthetic.randn((1, 32, S, 128), 0x5EEDC0, 1.0, torch.float32).to(DEV)
    k = synthetic.randn((1, 8, S, 128), 0x5EEDC1, 1.0, torch.float32).to(DEV)
    v = synthetic.randn((1, 8, S, 128), 0x5EEDC2, 1.0, torch.float32).to(DEV)
    assert 0 < bi.sdpa_workspace_bytes(1, 32, 8, S, S, 128, torch.float32) <= cap
    o = bi.bi_sdpa(q, k, v, causal=True)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for p in (0, 1000, 2047, 2048, 3333, 4095):
        dec = bi.bi_sdpa(q[:, :, p:p + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True)
        assert_bits_equal(o[:, :, p:p + 1], dec, f"fp32 row {p} vs its decode")
        ref = oracle.sdpa(qc[:, :, p:p + 1], kc[:, :, :p + 1], vc[:, :, :p + 1], causal=True)
        assert_close_to_oracle(o[:, :, p:p + 1].cpu(), ref, f"fp32 row {p}")
    # fp32 with a boolean mask, not causal: chunks keep every key and start their mask rows at the chunk
    Lq, S2 = 2048, 3000
    gen = torch.Generator(device="cpu").manual_seed(0x5EEDC3)
    mask = (torch.rand((1, 1, Lq, S2), generator=gen) > 0.3).to(DEV)
    assert 0 < bi.sdpa_workspace_bytes(1, 32, 8, Lq, S2, 128, torch.float32) <= cap
    om = bi.bi_sdpa(q[:, :, :Lq], k[:, :, :S2], v[:, :, :S2], mask=mask)
    for i in (0, 700, 1500, 2047):
        one = bi.bi_sdpa(q[:, :, i:i + 1], k[:, :, :S2], v[:, :, :S2], mask=mask[:, :, i:i + 1])
        assert_bits_equal(om[:, :, i:i + 1], one, f"fp32 masked row {i} vs alone")
    # bf16: 15 query rows per sequence (60 per KV head: the split kernel) against a 20000-key cache, batch 16
    B, L3, S3 = 16, 15, 20000
    assert lib.bi_sdpa_kernel_name(B, 32, 8, L3, S3, 128, bi.BI_BF16).decode() == "sdpa_split16+combine"
    assert 0 < bi.sdpa_workspace_bytes(B, 32, 8, L3, S3, 128, torch.bfloat16) <= cap
    q3 = synthetic.randn((B, 32, L3, 128), 0x5EEDC4, 1.0, torch.bfloat16).to(DEV)
    k3 = synthetic.randn((B, 8, S3, 128), 0x5EEDC5, 1.0, torch.bfloat16).to(DEV)
    v3 = synthetic.randn((B, 8, S3, 128), 0x5EEDC6, 1.0, torch.bfloat16).to(DEV)
    o3 = bi.bi_sdpa(q3, k3, v3, causal=True)
    for i in (0, 7, 14):
        p = S3 - L3 + i
        dec = bi.bi_sdpa(q3[:, :, i:i + 1], k3[:, :, :p + 1], v3[:, :, :p + 1], causal=True)
        assert_bits_equal(o3[:, :, i:i + 1], dec, f"bf16 row {i} vs its decode")


@pytest.mark.parametrize("dt", DTS, ids=_ids)
@pytest.mark.parametrize("D", [64, 128, 256])
def test_many_split_fold_matches_aligned_windows(dt, D):
    """Decode rows over caches of 17 to 129 splits (the fold of many partials runs through LDS, 64 splits
    at a time): a row whose visible keys all lie in a window starting at a multiple of 256 equals, bit
    for bit, the same window called as a short cache of its own -- every split before and after it is
    empty and skipped; the first visible split may sit in the second or third 64-split chunk.  With a
    sink, and against the oracle."""
    Hq, Hkv = 8, 2
    S_max = 33000
    q = synthetic.randn((1, Hq, 1, D), 0x5EEDD0 + D, 1.0, dt).to(DEV)
    k = synthetic.randn((1, Hkv, S_max, D), 0x5EEDD1 + D, 1.0, dt).to(DEV)
    v = synthetic.randn((1, Hkv, S_max, D), 0x5EEDD2 + D, 1.0, dt).to(DEV)
    sinks = synthetic.randn((Hq,), 0x5EEDD3, 2.0).to(DEV)
    for S, lo, hi in ((4097, 256, 700), (4352, 4096, 4352), (16385, 0, 300), (16385, 16384, 16385),
                      (20000, 16384 + 100, 16384 + 500), (33000, 32768 - 256, 33000), (33000, 5000, 30000)):
        w0 = lo // 256 * 256
        m = torch.zeros(1, 1, 1, S, dtype=torch.bool, device=DEV)
        m[..., lo:hi] = True
        mw = m[..., w0:hi].contiguous()
        for sk in (None, sinks):
            o = bi.bi_sdpa(q, k[:, :, :S], v[:, :, :S], mask=m, sinks=sk)
            ow = bi.bi_sdpa(q, k[:, :, w0:hi], v[:, :, w0:hi], mask=mw, sinks=sk)
            assert_bits_equal(o, ow, f"{dt} D={D} S={S} keys [{lo}, {hi}) sinks={sk is not None}")
    S, lo, hi = 33000, 5000, 30000
    m = torch.zeros(1, 1, 1, S, dtype=torch.bool)
    m[..., lo:hi] = True
    o = bi.bi_sdpa(q, k[:, :, :S], v[:, :, :S], mask=m.to(DEV), sinks=sinks)
    ref = oracle.sdpa(q.cpu(), k[:, :, :S].cpu(), v[:, :, :S].cpu(), mask=m, sinks=sinks.cpu())
    assert_close_to_oracle(o.cpu(), ref, f"{dt} D={D} S={S}")
