"""GPU tests of the PyTorch routing mode (batch_invariant_mode).

Routed calls must equal the direct library calls bit for bit (the mode only
marshals), rows must not depend on the batch through ordinary nn.Linear code,
torch's top-left is_causal semantics must be kept, and strict mode must raise
where the kernels cannot serve a call while non-strict mode falls back and
counts.  The last test sweeps the row-wise torch ops the mode leaves alone
(softmax, norms, reductions) for batch invariance on this GPU."""
import math

import pytest
import torch
import torch.nn.functional as F

import invariant_deterministic_gemm_amd as bi
import synthetic
from helpers import assert_bits_equal, bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _r(shape, seed, std=1.0, dt=torch.bfloat16):
    return synthetic.randn(shape, seed, std, dt).to(DEV)


def test_routed_matmuls_equal_direct_calls():
    x, w, b = _r((37, 256), 1), _r((96, 256), 2, 0.02), _r((96,), 3)
    C = _r((37, 96), 4)
    with bi.batch_invariant_mode() as m:
        lin = F.linear(x, w, b)
        mm = torch.mm(x, w.t())
        mat = x @ w.t()
        add1 = torch.addmm(b, x, w.t())
        add2 = torch.addmm(C, x, w.t(), beta=0.5, alpha=2.0)
        x3 = x.reshape(1, 37, 256)
        m3 = torch.matmul(x3, w.t())
        mv = torch.matmul(x, w[0])
        vm = torch.matmul(x[0], w.t())
        bat = torch.matmul(_r((2, 3, 16, 64), 5), _r((2, 3, 64, 24), 6))
        bmm = torch.bmm(_r((3, 16, 64), 7), _r((3, 64, 24), 8))
    assert m.routed["linear"] == 1 and not m.fallbacks
    assert_bits_equal(lin, bi.bi_linear(x, w, b), "F.linear")
    assert_bits_equal(mm, bi.bi_matmul(x, w.t()), "torch.mm")
    assert_bits_equal(mat, bi.bi_matmul(x, w.t()), "@")
    assert_bits_equal(add1, bi.bi_addmm(b, x, w.t()), "addmm, 1-D bias")
    assert_bits_equal(add2, bi.bi_addmm(C, x, w.t(), 2.0, 0.5), "addmm, alpha / beta")
    assert_bits_equal(m3, bi.bi_matmul(x, w.t()).reshape(1, 37, 96), "3-D x 2-D")
    assert_bits_equal(mv, bi.bi_linear(x, w[:1]).reshape(37), "matrix x vector")
    assert_bits_equal(vm, bi.bi_matmul(x[:1], w.t()).reshape(96), "vector x matrix")
    a4, b4 = _r((2, 3, 16, 64), 5), _r((2, 3, 64, 24), 6)
    for i in range(2):
        for j in range(3):
            assert_bits_equal(bat[i, j], bi.bi_matmul(a4[i, j], b4[i, j]), f"batched matmul element {i},{j}")
    a3, b3 = _r((3, 16, 64), 7), _r((3, 64, 24), 8)
    for i in range(3):
        assert_bits_equal(bmm[i], bi.bi_matmul(a3[i], b3[i]), f"bmm element {i}")
    ref = (x.float() @ w.float().t() + b.float())
    assert (lin.float() - ref).abs().max() / ref.abs().max() < 2e-2


def test_broadcast_batched_matmuls_equal_per_element_calls():
    """torch's broadcasting matmul forms run one batched launch; each element equals bi_matmul on it."""
    a, b = _r((2, 3, 40, 64), 41), _r((2, 3, 64, 24), 42)
    bb, v = _r((3, 64, 24), 43), _r((64,), 44)
    with bi.batch_invariant_mode() as m:
        ybc = a @ bb                      # b broadcast over the first batch dim (a copy when dims merge)
        yab = a[0, 0] @ b                 # a 2-D left operand shared by every element (batch stride 0)
        yv = torch.matmul(v, b)           # (K,) x (2, 3, K, N) -> (2, 3, N)
        ybt = torch.matmul(a, b.transpose(-1, -2).contiguous().transpose(-1, -2))   # column-major b views
    assert not m.fallbacks
    assert ybc.shape == (2, 3, 40, 24) and yab.shape == (2, 3, 40, 24) and yv.shape == (2, 3, 24)
    for i in range(2):
        for j in range(3):
            assert_bits_equal(ybc[i, j], bi.bi_matmul(a[i, j], bb[j]), f"b broadcast, element {i},{j}")
            assert_bits_equal(yab[i, j], bi.bi_matmul(a[0, 0], b[i, j]), f"a broadcast, element {i},{j}")
            assert_bits_equal(yv[i, j], bi.bi_matmul(v.reshape(1, 64), b[i, j])[0], f"vector, element {i},{j}")
            assert_bits_equal(ybt[i, j], bi.bi_matmul(a[i, j], b[i, j]), f"column-major b, element {i},{j}")


def test_nn_linear_rows_do_not_depend_on_batch():
    torch.manual_seed(0)
    net = torch.nn.Sequential(torch.nn.Linear(512, 1024), torch.nn.GELU(), torch.nn.Linear(1024, 512))
    net = net.to(DEV, torch.bfloat16).eval()
    x = _r((256, 512), 11)
    with torch.no_grad(), bi.batch_invariant_mode() as m:
        full = net(x)
        for M in (1, 2, 7, 33, 100):
            assert_bits_equal(net(x[:M]), full[:M], f"MLP rows, batch {M}")
        for r in (0, 77, 255):
            assert_bits_equal(net(x[r:r + 1]), full[r:r + 1], f"row {r} alone")
    assert m.routed["linear"] > 0 and not m.fallbacks


def test_sdpa_routing_keeps_torch_semantics():
    q, k, v = _r((2, 8, 40, 128), 21), _r((2, 2, 40, 128), 22), _r((2, 2, 40, 128), 23)
    with bi.batch_invariant_mode():
        same = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
        mask = torch.rand(2, 1, 40, 40, device=DEV) > 0.3
        mask[..., 0] = True
        masked = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, enable_gqa=True)
        # query shorter than the keys: torch's is_causal is top-left aligned
        tl = F.scaled_dot_product_attention(q[:, :, :9], k, v, is_causal=True, enable_gqa=True, scale=0.1)
    assert_bits_equal(same, bi.bi_sdpa(q, k, v, causal=True), "is_causal, Lq == S")
    assert_bits_equal(masked, bi.bi_sdpa(q, k, v, mask=mask), "boolean mask")
    tri = torch.ones(9, 40, dtype=torch.bool, device=DEV).tril()
    assert_bits_equal(tl, bi.bi_sdpa(q[:, :, :9], k, v, mask=tri, scale=0.1), "is_causal, Lq < S")
    kr, vr = k.float().repeat_interleave(4, 1), v.float().repeat_interleave(4, 1)
    ref = F.scaled_dot_product_attention(q[:, :, :9].float(), kr, vr, attn_mask=tri, scale=0.1)
    assert (tl.float() - ref).abs().max() / ref.abs().max() < 2e-2
    # a float mask of q's dtype is added to the scaled scores, torch's meaning and the library's
    # additive form; other head dims that are multiples of 32 are routed too
    amask = (torch.randn(2, 1, 40, 40, device=DEV) * 2).to(torch.bfloat16)
    amask[..., 5] = float("-inf")
    q96, k96, v96 = _r((1, 4, 12, 96), 24), _r((1, 2, 40, 96), 25), _r((1, 2, 40, 96), 26)
    with bi.batch_invariant_mode() as m:
        added = F.scaled_dot_product_attention(q, k, v, attn_mask=amask, enable_gqa=True)
        d96 = F.scaled_dot_product_attention(q96, k96, v96, enable_gqa=True)
    assert not m.fallbacks, dict(m.fallbacks)
    assert_bits_equal(added, bi.bi_sdpa(q, k, v, mask=amask), "additive mask")
    assert_bits_equal(d96, bi.bi_sdpa(q96, k96, v96), "head dim 96")
    ref = F.scaled_dot_product_attention(q.float(), k.float().repeat_interleave(4, 1),
                                         v.float().repeat_interleave(4, 1), attn_mask=amask.float())
    assert (added.float() - ref).abs().max() / ref.abs().max() < 2e-2


def test_strict_mode_raises_and_lenient_mode_falls_back():
    x64 = torch.randn(4, 16, dtype=torch.float64, device=DEV)
    xb, wb = _r((4, 64), 31), _r((8, 64), 32)
    q = _r((1, 4, 8, 48), 33)                                 # head dim not a multiple of 32
    fmask = torch.zeros(1, 1, 8, 8, device=DEV, dtype=torch.bfloat16)
    with bi.batch_invariant_mode():
        with pytest.raises(NotImplementedError):
            x64 @ x64.t()
        with pytest.raises(NotImplementedError):
            F.scaled_dot_product_attention(q, q, q, attn_mask=fmask)
        with pytest.raises(NotImplementedError):
            F.scaled_dot_product_attention(q, q, q, dropout_p=0.1)
        with pytest.raises(NotImplementedError):
            F.linear(xb.requires_grad_(), wb)
        with pytest.raises(NotImplementedError):
            torch.matmul(_r((2, 4, 64), 34), _r((3, 64, 8), 35))     # batch dims that do not broadcast
    with bi.batch_invariant_mode(strict=False) as m:
        y = x64 @ x64.t()
        z = F.scaled_dot_product_attention(q, q, q, attn_mask=fmask)
        w = xb.detach() @ wb.t()
    assert torch.equal(y, x64 @ x64.t())
    assert sum(m.fallbacks.values()) == 2 and m.fallbacks["scaled_dot_product_attention"] == 1, dict(m.fallbacks)
    assert sum(m.routed.values()) == 1, dict(m.routed)
    assert_bits_equal(w, bi.bi_matmul(xb.detach(), wb.t()), "routed in lenient mode")
    assert z.shape == q.shape


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["float32", "bfloat16"])
def test_rowwise_ops_left_to_torch_are_batch_invariant(dt):
    """The mode leaves these row-wise ops to torch because on this GPU each row gets the same bits
    at every batch size (a model built from them and the routed ops stays invariant end to end)."""
    x = _r((1024, 4096), 41, 1.0, dt)
    wn = _r((4096,), 42, 1.0, dt)
    ops = {
        "softmax": lambda t: torch.softmax(t, dim=-1),
        "log_softmax": lambda t: torch.log_softmax(t, dim=-1),
        "layer_norm": lambda t: F.layer_norm(t, (4096,), wn, None, 1e-5),
        "rms_norm": lambda t: F.rms_norm(t, (4096,), wn, 1e-6),
        "amax": lambda t: t.amax(dim=-1),
        "vector_norm": lambda t: torch.linalg.vector_norm(t.float(), dim=-1),
    }
    bad = []
    for name, op in ops.items():
        full = op(x)
        for M in (1, 3, 64, 257):
            if not torch.equal(bits(op(x[:M])), bits(full[:M])):
                bad.append((name, M))
    assert not bad, f"row-wise ops that are not batch invariant on this GPU: {bad}"


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["float32", "bfloat16"])
def test_mode_makes_last_dim_sum_and_mean_invariant(dt):
    """Stock fp32 sum / mean over the last dimension change their order with the number of rows on
    this GPU; under the mode they run bi_rowsum, whose rows do not depend on M."""
    x = _r((1024, 4099), 43, 1.0, dt)
    with bi.batch_invariant_mode() as m:
        full_s, full_m = x.sum(dim=-1), torch.mean(x, -1, keepdim=True)
        for M in (1, 3, 64, 257):
            assert_bits_equal(x[:M].sum(-1), full_s[:M], f"sum, M={M}")
            assert_bits_equal(torch.mean(x[:M], dim=[-1], keepdim=True), full_m[:M], f"mean, M={M}")
        assert_bits_equal(x.sum(-1), bi.bi_rowsum(x), "routed sum == bi_rowsum")
        total = x.sum()                               # full reduction: not row-wise, left to torch
        cols = x.sum(dim=0)                           # over the batch: left to torch
    assert m.routed["sum"] >= 5 and m.routed["mean"] >= 4 and not m.fallbacks
    assert total.shape == () and cols.shape == (4099,)



def test_other_threads_and_nested_calls_run_stock_pytorch():
    """The mode belongs to the thread that entered it: a linear on another thread runs PyTorch's own kernel
    (not counted), the same call on this thread is routed and equals the direct library call."""
    import threading
    x, w = _r((48, 256), 21), _r((80, 256), 22, 0.02)
    other = []
    with bi.batch_invariant_mode() as m:
        t = threading.Thread(target=lambda: other.append(F.linear(x, w)))
        t.start()
        t.join()
        assert not m.routed
        y = F.linear(x, w)
        assert m.routed["linear"] == 1
    assert_bits_equal(y, bi.bi_linear(x, w), "routed linear vs direct call")
    torch.testing.assert_close(other[0].float(), y.float(), rtol=2e-2, atol=2e-2)
