"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * exact rational arithmetic (fractions.Fraction) and correctly rounded
    sums (math.fsum) on tiny and medium shapes;
  * integer-valued inputs, where numpy's int64 matmul is exact;
  * closed forms (identity / permutation / one-hot weights, zero queries,
    single visible key) and the hand-worked examples in tests/golden;
  * invariants of attention (causality, masked keys, GQA == repeated-KV MHA,
    shift invariance of softmax).
Each pin group is also run against deliberately broken copies of oracle.c
(a transposed operand, a dropped term, an off-by-one mask, ...) to show that
the pins would catch such a mistake.
"""
import json
import math
import os
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "worked_examples.json")


def _vals(t):
    return t.to(torch.float64).numpy()


# ------------------------------------------------------------------ GEMM pins
def exact_gemm(A, B, b_is_nk, C, alpha, beta):
    """Fraction-exact alpha*A@B + beta*C, rounded once to double."""
    M, K = A.shape
    N = B.shape[0] if b_is_nk else B.shape[1]
    out = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                b = B[n, k] if b_is_nk else B[k, n]
                s += Fraction(float(A[m, k])) * Fraction(float(b))
            r = Fraction(float(alpha)) * s
            if C is not None and beta != 0:
                c = C[n] if C.ndim == 1 else C[m, n]
                r += Fraction(float(beta)) * Fraction(float(c))
            out[m, n] = float(r)
    return out


def pin_gemm_fraction():
    for dt, seed in ((torch.float32, 1), (torch.bfloat16, 2), (torch.float16, 3)):
        M, N, K = 3, 5, 7
        A = synthetic.randn((M, K), seed, 1.0, dt)
        W = synthetic.randn((N, K), seed + 10, 1.0, dt)
        bias = synthetic.randn((N,), seed + 20, 1.0, dt)
        Cfull = synthetic.randn((M, N), seed + 30, 1.0, dt)
        An, Wn, bn, Cn = map(_vals, (A, W, bias, Cfull))
        got = oracle.linear(A, W, bias)
        np.testing.assert_allclose(got, exact_gemm(An, Wn, True, bn, 1.0, 1.0), rtol=1e-13, atol=1e-13)
        Bkn = W.t().contiguous()
        got = oracle.addmm(Cfull, A, Bkn, alpha=0.75, beta=-2.0)
        np.testing.assert_allclose(got, exact_gemm(An, _vals(Bkn), False, Cn, 0.75, -2.0),
                                   rtol=1e-13, atol=1e-13)
        got = oracle.addmm(bias, A, Bkn, alpha=-1.5, beta=0.25)
        np.testing.assert_allclose(got, exact_gemm(An, _vals(Bkn), False, bn, -1.5, 0.25),
                                   rtol=1e-13, atol=1e-13)
        got = oracle.matmul(A, Bkn)
        np.testing.assert_allclose(got, exact_gemm(An, _vals(Bkn), False, None, 1.0, 0.0),
                                   rtol=1e-13, atol=1e-13)


def pin_gemm_fsum_medium():
    M, N, K = 4, 6, 300
    A = synthetic.randn((M, K), 41, 1.0, torch.bfloat16)
    W = synthetic.randn((N, K), 42, 0.02, torch.bfloat16)
    An, Wn = _vals(A), _vals(W)
    got = oracle.linear(A, W)
    ref = np.array([[math.fsum(An[m, k] * Wn[n, k] for k in range(K)) for n in range(N)]
                    for m in range(M)])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def pin_gemm_integer_exact():
    M, N, K = 9, 13, 64
    A = synthetic.randint((M, K), 51, -3, 3, torch.bfloat16)
    W = synthetic.randint((N, K), 52, -3, 3, torch.bfloat16)
    b = synthetic.randint((N,), 53, -5, 5, torch.bfloat16)
    Ai, Wi, bi_ = (t.to(torch.int64).numpy() for t in (A, W, b))
    ref = Ai @ Wi.T + bi_[None, :]
    assert np.array_equal(oracle.linear(A, W, b), ref.astype(np.float64))
    assert np.array_equal(oracle.matmul(A, W.t().contiguous()), (Ai @ Wi.T).astype(np.float64))


def pin_gemm_closed_forms():
    K = 16
    x = synthetic.randint((5, K), 61, -8, 8, torch.float32)
    b = synthetic.randint((K,), 62, -4, 4, torch.float32)
    eye = torch.eye(K)
    assert np.array_equal(oracle.linear(x, eye, b), _vals(x) + _vals(b)[None, :])
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(63))
    P = eye[perm]                       # row n of W selects input column perm[n]
    assert np.array_equal(oracle.linear(x, P), _vals(x)[:, perm.numpy()])
    W = synthetic.randn((7, K), 64)
    onehot = torch.zeros(3, K)
    onehot[0, 2] = 1
    onehot[1, 0] = 1
    onehot[2, K - 1] = 1
    got = oracle.linear(onehot, W)
    assert np.array_equal(got, _vals(W)[:, [2, 0, K - 1]].T)
    # beta == 0 never reads C, even when C is NaN.
    cnan = torch.full((5, 7), float("nan"))
    got = oracle.addmm(cnan, x, W.t().contiguous(), alpha=1.0, beta=0.0)
    assert np.isfinite(got).all()


def pin_gemm_golden():
    with open(GOLDEN) as f:
        cases = json.load(f)["gemm"]
    for c in cases:
        if c["op"] == "linear":
            got = oracle.linear(np.array(c["x"], float), np.array(c["w"], float),
                                np.array(c["bias"], float))
        elif c["op"] == "matmul":
            got = oracle.matmul(np.array(c["a"], float), np.array(c["b"], float))
        else:
            got = oracle.addmm(np.array(c["c"], float), np.array(c["a"], float),
                               np.array(c["b"], float), c["alpha"], c["beta"])
        assert np.array_equal(got, np.array(c["expected"], float)), c["name"]


GEMM_PINS = [pin_gemm_fraction, pin_gemm_fsum_medium, pin_gemm_integer_exact,
             pin_gemm_closed_forms, pin_gemm_golden]


# ------------------------------------------------------------------ SDPA pins
def brute_sdpa(q, k, v, causal, mask, scale, amask=None, sinks=None):
    """Plain-Python attention: exact dot products, math.exp, math.fsum.  amask (full shape) is added
    to the scaled scores, -inf dropping the key; sinks[h] is an extra softmax term with no value."""
    B, Hq, Lq, D = q.shape
    _, Hkv, S, _ = k.shape
    out = np.zeros((B, Hq, Lq, D))
    for b in range(B):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            for i in range(Lq):
                p = S - Lq + i
                vis = [j for j in range(S)
                       if (not causal or j <= p) and (mask is None or mask[b, h, i, j])
                       and (amask is None or amask[b, h, i, j] != -math.inf)]
                if not vis:
                    continue
                s = {j: float(Fraction(scale) * sum(Fraction(float(q[b, h, i, d])) * Fraction(float(k[b, g, j, d]))
                                                   for d in range(D))) for j in vis}
                if amask is not None:
                    s = {j: s[j] + float(amask[b, h, i, j]) for j in vis}
                m = max(s.values())
                extra = []
                if sinks is not None:
                    m = max(m, float(sinks[h]))
                    extra = [math.exp(float(sinks[h]) - m)]
                w = {j: math.exp(s[j] - m) for j in vis}
                den = math.fsum(list(w.values()) + extra)
                for d in range(D):
                    out[b, h, i, d] = math.fsum(w[j] * float(v[b, g, j, d]) for j in vis) / den
    return out


def _mask_full(mask, shape):
    return None if mask is None else np.broadcast_to(mask, shape)


def pin_sdpa_bruteforce():
    B, Hq, Hkv, Lq, S, D = 2, 4, 2, 3, 6, 5
    for dt, seed in ((torch.float32, 71), (torch.bfloat16, 72)):
        q = synthetic.randn((B, Hq, Lq, D), seed, 1.0, dt)
        k = synthetic.randn((B, Hkv, S, D), seed + 1, 1.0, dt)
        v = synthetic.randn((B, Hkv, S, D), seed + 2, 1.0, dt)
        qn, kn, vn = map(_vals, (q, k, v))
        g = torch.Generator().manual_seed(seed + 3)
        mask = (torch.rand((B, 1, Lq, S), generator=g) > 0.3).numpy()
        for causal in (False, True):
            for m in (None, mask):
                scale = 0.4472135954999579
                got = oracle.sdpa(q, k, v, causal=causal, mask=m, scale=scale)
                ref = brute_sdpa(qn, kn, vn, causal, _mask_full(m, (B, Hq, Lq, S)), scale)
                np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def pin_sdpa_default_scale():
    q = synthetic.randn((1, 2, 2, 8), 81)
    k = synthetic.randn((1, 1, 4, 8), 82)
    v = synthetic.randn((1, 1, 4, 8), 83)
    ref = brute_sdpa(_vals(q), _vals(k), _vals(v), True, None, 1.0 / math.sqrt(8))
    np.testing.assert_allclose(oracle.sdpa(q, k, v, causal=True), ref, rtol=1e-12, atol=1e-13)


def pin_sdpa_closed_forms():
    B, Hq, Hkv, S, D = 1, 4, 2, 9, 8
    v = synthetic.randint((B, Hkv, S, D), 91, -6, 6, torch.float32)
    k = synthetic.randn((B, Hkv, S, D), 92)
    vn = _vals(v)
    # q = 0: every score is 0, so each row is the mean of the values it sees.
    q0 = torch.zeros(B, Hq, S, D)
    got = oracle.sdpa(q0, k, v, causal=True)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        for i in range(S):
            np.testing.assert_allclose(got[0, h, i], vn[0, g, : i + 1].mean(axis=0), rtol=1e-14, atol=1e-14)
    # One visible key: the output is that key's value row, exactly.
    q = synthetic.randn((B, Hq, S, D), 93)
    got = oracle.sdpa(q, k, v, causal=True)
    for h in range(Hq):
        assert np.array_equal(got[0, h, 0], vn[0, (h * Hkv) // Hq, 0])
    # No visible key gives 0.
    mask = np.zeros((1, 1, 1, S), dtype=bool)
    got = oracle.sdpa(q[:, :, :1], k, v, mask=mask)
    assert np.array_equal(got, np.zeros_like(got))


def pin_sdpa_invariants():
    B, Hq, Hkv, Lq, S, D = 1, 4, 2, 4, 11, 8
    q = synthetic.randn((B, Hq, Lq, D), 101)
    k = synthetic.randn((B, Hkv, S, D), 102)
    v = synthetic.randn((B, Hkv, S, D), 103)
    base = oracle.sdpa(q, k, v, causal=True)
    # Causality: keys after a query's position cannot change its row.
    for i in range(Lq):
        p = S - Lq + i
        k2, v2 = k.clone(), v.clone()
        k2[:, :, p + 1:] = synthetic.randn(k2[:, :, p + 1:].shape, 104 + i)
        v2[:, :, p + 1:] = synthetic.randn(v2[:, :, p + 1:].shape, 204 + i)
        assert np.array_equal(oracle.sdpa(q, k2, v2, causal=True)[:, :, i], base[:, :, i])
        # Truncating the cache after p gives the decode result of that token.
        dec = oracle.sdpa(q[:, :, i:i + 1], k[:, :, :p + 1], v[:, :, :p + 1], causal=True)
        assert np.array_equal(dec[:, :, 0], base[:, :, i])
    # Masked keys: their values are never read.
    mask = np.ones((1, 1, 1, S), dtype=bool)
    mask[..., [1, 5, 7]] = False
    m1 = oracle.sdpa(q, k, v, mask=mask)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, [1, 5, 7]] = 77.0
    v2[:, :, [1, 5, 7]] = -55.0
    assert np.array_equal(oracle.sdpa(q, k2, v2, mask=mask), m1)
    # Masking a suffix equals truncating the cache.
    msuf = np.ones((1, 1, 1, S), dtype=bool)
    msuf[..., 8:] = False
    assert np.array_equal(oracle.sdpa(q, k, v, mask=msuf), oracle.sdpa(q, k[:, :, :8], v[:, :, :8]))
    # GQA == MHA on K/V repeated per group.
    G = Hq // Hkv
    krep = k.repeat_interleave(G, dim=1)
    vrep = v.repeat_interleave(G, dim=1)
    assert np.array_equal(oracle.sdpa(q, krep, vrep, causal=True), base)
    # Shift invariance: adding u to every key adds q.u to every score of a row.
    u = synthetic.randn((D,), 105)
    shifted = oracle.sdpa(q, k.double() + u.double(), v, causal=True)
    np.testing.assert_allclose(shifted, base, rtol=1e-11, atol=1e-12)
    # The mask broadcasts: a per-head mask equal for all heads equals the broadcast one.
    mfull = np.broadcast_to(mask, (B, Hq, Lq, S)).copy()
    assert np.array_equal(oracle.sdpa(q, k, v, mask=mfull), m1)


def pin_sdpa_additive_mask():
    B, Hq, Hkv, Lq, S, D = 2, 4, 2, 3, 7, 5
    q = synthetic.randn((B, Hq, Lq, D), 121)
    k = synthetic.randn((B, Hkv, S, D), 122)
    v = synthetic.randn((B, Hkv, S, D), 123)
    qn, kn, vn = map(_vals, (q, k, v))
    g = torch.Generator().manual_seed(124)
    amask = (torch.randn((B, Hq, Lq, S), generator=g, dtype=torch.float64) * 2).numpy()
    amask[0, 1, 2, [0, 3]] = -math.inf
    amask[1, :, 0, :] = -math.inf                      # rows with no visible key
    for causal in (False, True):
        got = oracle.sdpa(q, k, v, causal=causal, mask=amask, scale=0.37)
        ref = brute_sdpa(qn, kn, vn, causal, None, 0.37, amask=amask)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    assert np.array_equal(oracle.sdpa(q, k, v, mask=amask)[1, :, 0], np.zeros((Hq, D)))
    # a mask of zeros is no mask; -inf where a boolean mask says no is that boolean mask
    base = oracle.sdpa(q, k, v, causal=True)
    assert np.array_equal(oracle.sdpa(q, k, v, causal=True, mask=np.zeros((1, 1, Lq, S))), base)
    bm = (torch.rand((B, 1, Lq, S), generator=g) > 0.4).numpy()
    assert np.array_equal(oracle.sdpa(q, k, v, mask=np.where(bm, 0.0, -math.inf)), oracle.sdpa(q, k, v, mask=bm))
    # q = 0: every scaled score is 0, so the weights are exp(mask); with mask = log(w) they are w
    w = synthetic.randint((1, 1, Lq, S), 125, 1, 9, torch.float64).numpy()
    q0 = torch.zeros(1, Hq, Lq, D)
    got = oracle.sdpa(q0, k[:1], v[:1], mask=np.log(w))
    for h in range(Hq):
        gk = (h * Hkv) // Hq
        for i in range(Lq):
            want = (w[0, 0, i][:, None] * vn[0, gk]).sum(axis=0) / w[0, 0, i].sum()
            np.testing.assert_allclose(got[0, h, i], want, rtol=1e-13, atol=1e-14)
    # a constant added to a whole row changes nothing; the mask broadcasts like the boolean one
    shifted = amask + 5.25
    np.testing.assert_allclose(oracle.sdpa(q, k, v, mask=shifted), oracle.sdpa(q, k, v, mask=amask),
                               rtol=1e-12, atol=1e-13)
    row = amask[:1, :1]
    assert np.array_equal(oracle.sdpa(q, k, v, mask=row),
                          oracle.sdpa(q, k, v, mask=np.broadcast_to(row, (B, Hq, Lq, S)).copy()))


def pin_sdpa_sinks():
    B, Hq, Hkv, Lq, S, D = 2, 4, 2, 3, 6, 5
    q = synthetic.randn((B, Hq, Lq, D), 131)
    k = synthetic.randn((B, Hkv, S, D), 132)
    v = synthetic.randn((B, Hkv, S, D), 133)
    qn, kn, vn = map(_vals, (q, k, v))
    sinks = np.array([-0.5, 1.25, 0.0, 2.5])            # one per query head, all different
    for causal in (False, True):
        got = oracle.sdpa(q, k, v, causal=causal, scale=0.41, sinks=sinks)
        ref = brute_sdpa(qn, kn, vn, causal, None, 0.41, sinks=sinks)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # -inf sinks are no sinks
    base = oracle.sdpa(q, k, v, causal=True)
    assert np.array_equal(oracle.sdpa(q, k, v, causal=True, sinks=np.full(Hq, -math.inf)), base)
    # q = 0, causal: row i sees n = S - Lq + i + 1 keys of weight 1 and the sink of weight e^sink
    q0 = torch.zeros(1, Hq, Lq, D)
    got = oracle.sdpa(q0, k[:1], v[:1], causal=True, sinks=sinks)
    for h in range(Hq):
        gk = (h * Hkv) // Hq
        for i in range(Lq):
            n = S - Lq + i + 1
            want = vn[0, gk, :n].sum(axis=0) / (n + math.exp(sinks[h]))
            np.testing.assert_allclose(got[0, h, i], want, rtol=1e-13, atol=1e-14)
    # a dominant sink takes all the weight (exp(-1000) is 0 in float64); no visible key stays 0
    assert np.array_equal(oracle.sdpa(q0, k[:1], v[:1], sinks=np.full(Hq, 1000.0)), np.zeros((1, Hq, Lq, D)))
    none = np.zeros((1, 1, Lq, S), dtype=bool)
    assert np.array_equal(oracle.sdpa(q, k, v, mask=none, sinks=sinks), np.zeros((B, Hq, Lq, D)))


def pin_sdpa_golden():
    with open(GOLDEN) as f:
        cases = json.load(f)["sdpa"]
    for c in cases:
        got = oracle.sdpa(np.array(c["q"], float), np.array(c["k"], float), np.array(c["v"], float),
                          causal=c["causal"], scale=c["scale"],
                          mask=np.array(c["mask"], float) if "mask" in c else None,
                          sinks=np.array(c["sinks"], float) if "sinks" in c else None)
        exp = np.array(c["expected"], float)
        if "rtol" in c:
            np.testing.assert_allclose(got, exp, rtol=c["rtol"], atol=0, err_msg=c["name"])
        else:
            assert np.array_equal(got, exp), c["name"]


SDPA_PINS = [pin_sdpa_bruteforce, pin_sdpa_default_scale, pin_sdpa_closed_forms,
             pin_sdpa_invariants, pin_sdpa_additive_mask, pin_sdpa_sinks, pin_sdpa_golden]


def pin_rowsum_exact():
    # integers: every order of summation is exact
    x = synthetic.randint((7, 300), 111, -50, 50, torch.float32)
    xi = x.to(torch.int64).numpy()
    assert np.array_equal(oracle.rowsum(x), xi.sum(axis=1).astype(np.float64))
    assert np.array_equal(oracle.rowsum(x, mean=True), xi.sum(axis=1) / 300.0)
    # correctly rounded sums of random doubles (math.fsum)
    y = synthetic.randn((5, 1000), 112, 1.0, torch.float32)
    got = oracle.rowsum(y)
    for r in range(5):
        exact = math.fsum(float(v) for v in _vals(y)[r])
        assert abs(got[r] - exact) <= 1e-12 * np.abs(_vals(y)[r]).sum()
    # closed forms: constant rows, one nonzero element, empty rows
    c = torch.full((3, 17), 0.25)
    assert np.array_equal(oracle.rowsum(c, mean=True), np.full(3, 0.25))
    one = torch.zeros(2, 9)
    one[0, 8] = 3.0
    one[1, 0] = -2.0
    assert np.array_equal(oracle.rowsum(one), np.array([3.0, -2.0]))
    assert np.array_equal(oracle.rowsum(torch.zeros(4, 0)), np.zeros(4))
    assert np.isnan(oracle.rowsum(torch.zeros(2, 0), mean=True)).all()
    # leading dims are batch: (2, 3, N) reduces to (2, 3)
    z = synthetic.randint((2, 3, 11), 113, -9, 9, torch.float32)
    assert np.array_equal(oracle.rowsum(z), z.to(torch.int64).sum(-1).numpy().astype(np.float64))


ROWSUM_PINS = [pin_rowsum_exact]


# ------------------------------------------------------------ quantized weights
def _pack(q, bits):
    """Pack integer fields (N, K) into uint32 words, 32 / bits per word, lowest bits first (plain
    Python integers: an independent inverse of the oracle's unpacking)."""
    per = 32 // bits
    N, K = q.shape
    words = np.zeros((N, K // per), dtype=np.uint32)
    for n in range(N):
        for w in range(K // per):
            v = 0
            for j in range(per):
                v |= int(q[n, w * per + j]) << (j * bits)
            words[n, w] = v
    return words


def pin_dequant_golden():
    with open(GOLDEN) as f:
        cases = json.load(f)["quantized"]
    for c in cases:
        got = oracle.dequantize(np.array(c["words"], dtype=np.uint32), np.array(c["scales"], float),
                                np.array(c["biases"], float), c["bits"], c["group_size"], c["K"])
        assert np.array_equal(got, np.array(c["expected"], float)), c["name"]


def pin_dequant_roundtrip():
    rng = np.random.default_rng(7)
    for bits in (2, 4, 8):
        for gs in (32, 64, 128):
            N, K = 3, 256
            q = rng.integers(0, 1 << bits, size=(N, K))
            words = _pack(q, bits)
            ones, zeros = np.ones((N, K // gs)), np.zeros((N, K // gs))
            # scale 1, bias 0: the fields come back unchanged
            assert np.array_equal(oracle.dequantize(words, ones, zeros, bits, gs), q.astype(float))
            # every field 1: w = scale + bias of the field's own group
            words1 = _pack(np.ones((N, K), dtype=np.int64), bits)
            sc = rng.integers(1, 9, size=(N, K // gs)) / 4.0
            bi = rng.integers(-9, 9, size=(N, K // gs)) / 2.0
            want = np.repeat(sc + bi, gs, axis=1)
            assert np.array_equal(oracle.dequantize(words1, sc, bi, bits, gs), want)
            # largest field: w = (2^bits - 1) * scale + bias
            wordsmax = _pack(np.full((N, K), (1 << bits) - 1), bits)
            want = np.repeat(((1 << bits) - 1) * sc + bi, gs, axis=1)
            assert np.array_equal(oracle.dequantize(wordsmax, sc, bi, bits, gs), want)


def pin_qlinear_integer_exact():
    rng = np.random.default_rng(8)
    for bits, gs in ((4, 64), (8, 32), (2, 128)):
        M, N, K = 5, 7, 256
        q = rng.integers(0, 1 << bits, size=(N, K))
        sc = rng.integers(1, 4, size=(N, K // gs)).astype(float)
        bi = rng.integers(-5, 5, size=(N, K // gs)).astype(float)
        x = rng.integers(-6, 7, size=(M, K))
        bias = rng.integers(-9, 9, size=N)
        w_int = q * np.repeat(sc.astype(np.int64), gs, axis=1) + np.repeat(bi.astype(np.int64), gs, axis=1)
        want = (x @ w_int.T + bias).astype(float)          # int64 arithmetic: exact
        got = oracle.quantized_linear(x.astype(float), _pack(q, bits), sc, bi, bits, gs, bias.astype(float))
        assert np.array_equal(got, want)


QUANT_PINS = [pin_dequant_golden, pin_dequant_roundtrip, pin_qlinear_integer_exact]


@pytest.mark.parametrize("pin", GEMM_PINS + SDPA_PINS + ROWSUM_PINS + QUANT_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


# ------------------------------------------------------------ planted mistakes
MUTANTS = {
    "gemm_transposed_B": ("b_is_nk ? B[n * ldb + k] : B[k * ldb + n]",
                          "b_is_nk ? B[k * ldb + n] : B[n * ldb + k]", GEMM_PINS),
    "gemm_dropped_C": ("r = r + beta * c;", "r = r;", GEMM_PINS),
    "gemm_wrong_sign": ("acc[j] = acc[j] + a * b;", "acc[j] = acc[j] - a * b;", GEMM_PINS),
    "gemm_bias_broadcast_index": ("(ldc == 0 ? 0 : m * ldc)", "(ldc == 0 ? m : m * ldc)", GEMM_PINS),
    "gemm_dropped_alpha": ("double r = alpha * acc[j];", "double r = acc[j];", GEMM_PINS),
    "gemm_last_k_dropped": ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k < K - 1; ++k) {",
                            GEMM_PINS),
    "sdpa_causal_off_by_one": ("if (causal && j > p) ok = 0;", "if (causal && j >= p) ok = 0;", SDPA_PINS),
    "sdpa_causal_top_left": ("const int64_t p = S - Lq + i;", "const int64_t p = i;", SDPA_PINS),
    "sdpa_gqa_interleaved": ("const int64_t g = (h * Hkv) / Hq;", "const int64_t g = h % Hkv;", SDPA_PINS),
    "sdpa_unnormalised": ("orow[d] = num[d] / den;", "orow[d] = num[d];", SDPA_PINS),
    "sdpa_no_max_shift": ("exp(s[j] - m)", "exp(s[j])", SDPA_PINS),
    "sdpa_scale_dropped": ("s[j] = scale * dot + add;", "s[j] = dot + add;", SDPA_PINS),
    "sdpa_additive_sign": ("s[j] = scale * dot + add;", "s[j] = scale * dot - add;", SDPA_PINS),
    "sdpa_additive_key_index": ("i * as[2] + j * as[3]]", "i * as[2] + 0 * as[3]]", SDPA_PINS),
    "sdpa_additive_inf_visible": ("if (add == -INFINITY) ok = 0;", "if (add != add) ok = 0;", SDPA_PINS),
    "sdpa_sink_dropped": ("den = den + exp(sk - m);", "den = den;", SDPA_PINS),
    "sdpa_sink_kv_head": ("const double sk = sinks[h];", "const double sk = sinks[g];", SDPA_PINS),
    "sdpa_mask_polarity": ("ms[3]] != 0;", "ms[3]] == 0;", SDPA_PINS),
    "sdpa_value_from_key": ("const double *vrow = v + b * vs[0] + g * vs[1] + j * vs[2];",
                            "const double *vrow = k + b * ks[0] + g * ks[1] + j * ks[2];", SDPA_PINS),
    "rowsum_last_dropped": ("for (int64_t n = 0; n < N; ++n) s = s + row[n];",
                            "for (int64_t n = 0; n + 1 < N; ++n) s = s + row[n];", ROWSUM_PINS),
    "rowsum_mean_undivided": ("out[m] = mean ? s / (double)N : s;", "out[m] = s;", ROWSUM_PINS),
    "rowsum_row_pitch": ("const double *row = x + m * ldx;", "const double *row = x + m;", ROWSUM_PINS),
    "dequant_bit_order": ("(word >> ((k % per) * bits))", "(word >> ((per - 1 - k % per) * bits))", QUANT_PINS),
    "dequant_group_off_by_one": ("const int64_t grp = k / gs;", "const int64_t grp = (k + 1) / gs % (K / gs);",
                                 QUANT_PINS),
    "dequant_scale_bias_swapped": ("scales[n * ldsb + grp] * (double)q + biases[n * ldsb + grp]",
                                   "biases[n * ldsb + grp] * (double)q + scales[n * ldsb + grp]", QUANT_PINS),
    "dequant_word_index": ("const uint32_t word = wq[n * ldwq + k / per];",
                           "const uint32_t word = wq[n * ldwq + k / bits % ldwq];", QUANT_PINS),
}


def _run_pins_with(lib_path: str, group: str) -> list:
    """Run one pin group against another build of oracle.c; return the pins that failed."""
    pins = {"gemm": GEMM_PINS, "sdpa": SDPA_PINS, "rowsum": ROWSUM_PINS, "quant": QUANT_PINS}[group]
    failed = []
    with oracle.use_library(lib_path):
        for pin in pins:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new, pins = MUTANTS[name]
    group = {id(GEMM_PINS): "gemm", id(SDPA_PINS): "sdpa", id(ROWSUM_PINS): "rowsum", id(QUANT_PINS): "quant"}[id(pins)]
    root = os.path.dirname(HERE)
    src = open(os.path.join(root, "oracle", "oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not unique in oracle.c: {old!r}"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(mut), "-o", str(lib), "-lm"], check=True)
    # A planted out-of-range index may crash the process, so the mutant runs
    # in a child; a crash counts as caught, like a failed pin.
    code = ("import sys; sys.path[:0] = [%r, %r]; import test_oracle as t; "
            "print('FAILED=' + ','.join(t._run_pins_with(%r, %r)))" % (root, HERE, str(lib), group))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    if r.returncode == 0:
        line = [l for l in r.stdout.splitlines() if l.startswith("FAILED=")][-1]
        failed = [x for x in line[len("FAILED="):].split(",") if x]
        assert failed, f"no pin caught the planted mistake {name}"
    else:
        assert r.returncode < 0 or r.returncode > 128, r.stderr[-2000:]


def test_oracle_threads_positive():
    assert oracle.threads() >= 1
