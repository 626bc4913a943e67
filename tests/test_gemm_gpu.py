"""GPU tests of the invariant GEMM entry points (bi_linear, bi_matmul, bi_addmm).

* exact pins: integer-valued inputs make every summation order exact, so the
  GPU must equal the oracle rounded once to the output dtype, bit for bit;
* oracle tolerance on the seeded workloads (fp32: 1e-5, bf16/fp16: 2e-2);
* invariance on raw bit patterns across batch size (every M of each sweep
  and every tile-switch boundary), batch neighbours (other rows redrawn or
  NaN), repeated calls, call form (linear / addmm / matmul) and HIP-graph
  replay;
* the negative control: the split-K comparator must NOT be invariant.
"""
import numpy as np
import pytest
import torch

import invariant_deterministic_gemm_amd as bi
import oracle
import synthetic
from helpers import assert_bits_equal, assert_close_to_oracle, n_bit_diff, round_ref

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAIRS = [(torch.float32, torch.float32), (torch.bfloat16, torch.bfloat16), (torch.float16, torch.float16),
         (torch.bfloat16, torch.float32), (torch.float16, torch.float32)]
# M values that cross every kernel switch: strip / skinny row-fragment counts (4/16/32/48/64),
# strip -> ring tiles (64/65) and the ring tile choices.
M_EDGES = [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def ints(shape, seed, dt, lo=-3, hi=3):
    return synthetic.randint(shape, seed, lo, hi, dt)


@pytest.mark.parametrize("ind,outd", PAIRS, ids=lambda d: str(d).split(".")[-1])
def test_integer_inputs_are_exact_for_every_layout(ind, outd):
    K = 136 if ind != torch.float32 else 132        # ragged last k step
    N = 72
    M = 300
    x = ints((M, K), 11, ind)
    w = ints((N, K), 12, ind)
    b = ints((N,), 13, outd, -5, 5)
    C = ints((M, N), 14, outd, -5, 5)
    ref_lin = oracle.linear(x, w, b)
    ref_mm = oracle.matmul(x, w.t().contiguous())
    ref_add = oracle.addmm(C, x, w.t().contiguous(), 2.0, -1.0)
    xg, wg, bg, Cg = (t.to(DEV) for t in (x, w, b, C))
    wt = wg.t().contiguous()
    for m in (1, 5, 16, 17, 64, 65, 200, 300):
        assert_bits_equal(bi.bi_linear(xg[:m], wg, bg, out_dtype=outd).cpu(), round_ref(ref_lin[:m], outd),
                          f"linear M={m}")
        assert_bits_equal(bi.bi_matmul(xg[:m], wt, out_dtype=outd).cpu(), round_ref(ref_mm[:m], outd),
                          f"matmul M={m}")
        assert_bits_equal(bi.bi_addmm(Cg[:m], xg[:m], wt, 2.0, -1.0, out_dtype=outd).cpu(),
                          round_ref(ref_add[:m], outd), f"addmm M={m}")
        # the same operand as a transposed view (column-major (K, N)) takes the (N, K) kernels
        assert_bits_equal(bi.bi_matmul(xg[:m], wg.t(), out_dtype=outd).cpu(), round_ref(ref_mm[:m], outd),
                          f"matmul, transposed view, M={m}")
        assert_bits_equal(bi.bi_addmm(Cg[:m], xg[:m], wg.t(), 2.0, -1.0, out_dtype=outd).cpu(),
                          round_ref(ref_add[:m], outd), f"addmm, transposed view, M={m}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_small_m_strip_configs_are_exact_with_tails(dt):
    """Every small-M strip configuration (A rows per stage 4 / 16 / 32 / 64) on integer inputs:
    N ragged for the 16-column strip, K ragged for the 128-k stage and the 32-k step."""
    lib = bi._native.load()
    K, N = 1000, 4100
    x = ints((64, K), 51, dt)
    w = ints((N, K), 52, dt)
    b = ints((N,), 53, dt, -5, 5)
    ref = oracle.linear(x, w, b)
    xg, wg, bg = x.to(DEV), w.to(DEV), b.to(DEV)
    seen = set()
    for m in (1, 3, 4, 5, 8, 16, 17, 31, 32, 33, 64):
        for n in (N, 4096, 72):
            seen.add(lib.bi_gemm_kernel_name(m, n, K, bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16, 0).decode())
            y = bi.bi_linear(xg[:m], wg[:n], bg[:n]).cpu()
            assert_bits_equal(y, round_ref(ref[:m, :n], dt), f"M={m} N={n}")
    assert len([k for k in seen if "strip" in k]) >= 4, seen


def test_identity_permutation_and_onehot_weights():
    K = 64
    x = ints((40, K), 21, torch.bfloat16, -100, 100)
    eye = torch.eye(K, dtype=torch.bfloat16)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(22))
    y = bi.bi_linear(x.to(DEV), eye.to(DEV)).cpu()
    assert_bits_equal(y, x, "identity weight")
    y = bi.bi_linear(x.to(DEV), eye[perm].contiguous().to(DEV)).cpu()
    assert_bits_equal(y, x[:, perm], "permutation weight")
    w = synthetic.randn((24, K), 23, 1.0, torch.float32)
    onehot = torch.zeros(3, K)
    onehot[0, 5] = 1
    onehot[1, 0] = 1
    onehot[2, K - 1] = 1
    y = bi.bi_linear(onehot.to(DEV), w.to(DEV)).cpu()
    assert_bits_equal(y, w[:, [5, 0, K - 1]].t().contiguous(), "one-hot rows select columns of W")


def test_config1_fp32_linear_invariant_and_accurate():
    d = synthetic.cfg1_inputs()
    x, w, b = (t.to(DEV) for t in (d["x"], d["w"], d["b"]))
    ref = oracle.linear(d["x"], d["w"], d["b"])
    full = bi.bi_linear(x, w, b)
    assert_close_to_oracle(full.cpu(), ref, "config 1 fp32")
    for m in range(1, 9):
        y = bi.bi_linear(x[:m], w, b)
        assert_bits_equal(y, full[:m], f"config 1, M={m}")
        assert_close_to_oracle(y.cpu(), ref[:m], f"config 1, M={m}")
    for r in range(8):
        assert_bits_equal(bi.bi_linear(x[r:r + 1], w, b), full[r:r + 1], f"config 1 single row {r}")


@pytest.mark.parametrize("N", [4096, 14336])
def test_config2_bf16_linear_addmm_sweep(N):
    d = synthetic.cfg2_inputs(N, M_max=257)
    x, w, b, c = (d[k].to(DEV) for k in ("x", "w", "b", "c"))
    wt = w.t().contiguous()
    full = bi.bi_linear(x, w, b)
    full_add = bi.bi_addmm(b, x, wt, 1.0, 1.0)
    assert_bits_equal(full_add, full, "addmm(b row, x, W^T) == linear(x, W, b)")
    assert_bits_equal(bi.bi_addmm(b, x, w.t(), 1.0, 1.0), full, "addmm(b row, x, W.t() view) == linear")
    assert_bits_equal(bi.bi_matmul(x, w.t()), bi.bi_matmul(x, wt), "matmul: view == row-major copy")
    full_c = bi.bi_addmm(c, x, wt, 1.0, 1.0)
    for m in sorted(set(synthetic.CFG2["M_values"] + M_EDGES)):
        assert_bits_equal(bi.bi_linear(x[:m], w, b), full[:m], f"linear N={N} M={m}")
        assert_bits_equal(bi.bi_addmm(b, x[:m], wt, 1.0, 1.0), full[:m], f"addmm N={N} M={m}")
        assert_bits_equal(bi.bi_addmm(b, x[:m], w.t(), 1.0, 1.0), full[:m], f"addmm view N={N} M={m}")
        assert_bits_equal(bi.bi_addmm(c[:m], x[:m], wt, 1.0, 1.0), full_c[:m], f"addmm full C N={N} M={m}")
    # single-row calls
    for r in (0, 1, 17, 100, 255):
        assert_bits_equal(bi.bi_linear(x[r:r + 1], w, b), full[r:r + 1], f"row {r} alone")
    # oracle on a row subset (full N)
    rows = [0, 3, 16, 64, 129, 256] if N == 4096 else [0, 33, 200]
    ref = oracle.linear(d["x"][rows], d["w"], d["b"])
    assert_close_to_oracle(full[rows].cpu(), ref, f"config 2 N={N}")
    refc = oracle.addmm(d["c"][rows], d["x"][rows], d["w"].t().contiguous(), 1.0, 1.0)
    assert_close_to_oracle(full_c[rows].cpu(), refc, f"config 2 addmm full C N={N}")


def test_neighbour_rows_cannot_move_a_row():
    d = synthetic.cfg2_inputs(4096, M_max=64)
    x, w, b = (d[k].to(DEV) for k in ("x", "w", "b"))
    base = bi.bi_linear(x, w, b)
    other = synthetic.randn((64, 4096), 999, 1.0, torch.bfloat16).to(DEV)
    for r in (0, 5, 31, 63):
        for fill in ("redraw", "nan", "inf", "zero"):
            x2 = other.clone() if fill == "redraw" else torch.full_like(x, {"nan": float("nan"),
                                                                             "inf": float("inf"),
                                                                             "zero": 0.0}[fill])
            x2[r] = x[r]
            for m in (r + 1, 64):
                y = bi.bi_linear(x2[:m], w, b)
                assert_bits_equal(y[r], base[r], f"row {r}, neighbours {fill}, M={m}")
    # large M through the tiled kernel
    d = synthetic.cfg2_inputs(4096, M_max=512)
    x, w = d["x"].to(DEV), d["w"].to(DEV)
    base = bi.bi_linear(x, w)
    x2 = torch.full_like(x, float("nan"))
    x2[300] = x[300]
    assert_bits_equal(bi.bi_linear(x2, w)[300], base[300], "row 300 among NaN rows, M=512")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_config5_logits_rows_match_their_m1_call(dt):
    d = synthetic.cfg5_inputs(dt)
    h, w = d["h"].to(DEV), d["w"].to(DEV)
    singles = torch.stack([bi.bi_linear(h[r:r + 1], w)[0] for r in range(64)])
    singles32 = torch.stack([bi.bi_linear(h[r:r + 1], w, out_dtype=torch.float32)[0] for r in (0, 63)])
    for m in range(1, 65):
        y = bi.bi_linear(h[:m], w)
        assert_bits_equal(y, singles[:m], f"logits {dt} M={m}")
    y32 = bi.bi_linear(h, w, out_dtype=torch.float32)
    assert_bits_equal(y32[[0, 63]], singles32, "fp32-output logits")
    ref = oracle.linear(d["h"][[0, 31, 63]], d["w"])
    assert_close_to_oracle(singles[[0, 31, 63]].cpu(), ref, f"logits {dt}")


def test_bias_is_rounded_once():
    d = synthetic.cfg2_inputs(4096, M_max=8)
    x, w, b = (d[k].to(DEV) for k in ("x", "w", "b"))
    y = bi.bi_linear(x, w, b)
    y_twice = (bi.bi_linear(x, w).float() + b.float()).to(torch.bfloat16)   # round, add, round again
    assert n_bit_diff(y, y_twice) > 0, "one rounding must differ from rounding twice somewhere"
    ref = oracle.linear(d["x"], d["w"], d["b"])
    e1 = np.abs(y.cpu().double().numpy() - ref).max()
    e2 = np.abs(y_twice.cpu().double().numpy() - ref).max()
    assert e1 <= e2


def test_beta_zero_ignores_nan_c():
    d = synthetic.cfg2_inputs(4096, M_max=4)
    x, w = d["x"].to(DEV), d["w"].to(DEV)
    cnan = torch.full((4, 4096), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = bi.bi_addmm(cnan, x, w.t().contiguous(), 1.0, 0.0)
    assert torch.isfinite(y).all()
    assert_bits_equal(y, bi.bi_matmul(x, w.t().contiguous()), "beta = 0 equals matmul")


def test_ragged_and_empty_shapes():
    x = synthetic.randn((37, 104), 31, 1.0, torch.bfloat16)
    w = synthetic.randn((45, 104), 32, 1.0, torch.bfloat16)
    b = synthetic.randn((45,), 33, 1.0, torch.bfloat16)
    y = bi.bi_linear(x.to(DEV), w.to(DEV), b.to(DEV))
    assert_close_to_oracle(y.cpu(), oracle.linear(x, w, b), "ragged 37x45x104")
    assert bi.bi_linear(x[:0].to(DEV), w.to(DEV)).shape == (0, 45)
    assert bi.bi_linear(x.to(DEV), w[:0].to(DEV)).shape == (37, 0)
    y0 = bi.bi_linear(x[:, :0].contiguous().to(DEV), w[:, :0].contiguous().to(DEV), b.to(DEV))
    assert_bits_equal(y0.cpu(), b.expand(37, 45).contiguous(), "K = 0 leaves only the bias")
    # leading batch dims are flattened into M
    x3 = synthetic.randn((2, 3, 104), 34, 1.0, torch.bfloat16).to(DEV)
    y3 = bi.bi_linear(x3, w.to(DEV))
    assert y3.shape == (2, 3, 45)
    assert_bits_equal(y3.reshape(6, 45), bi.bi_linear(x3.reshape(6, 104), w.to(DEV)), "3-D input")


def test_strided_inputs():
    base = synthetic.randn((20, 256), 41, 1.0, torch.bfloat16).to(DEV)
    w = synthetic.randn((64, 128), 42, 1.0, torch.bfloat16).to(DEV)
    xs = base[:, 64:192]                    # row pitch 256 elements
    y = bi.bi_linear(xs, w)
    assert_bits_equal(y, bi.bi_linear(xs.contiguous(), w), "strided rows")


def test_repeat_calls_are_bitwise_identical():
    d = synthetic.cfg2_inputs(4096, M_max=256)
    x, w, b = (d[k].to(DEV) for k in ("x", "w", "b"))
    for m in (1, 64, 256):
        first = bi.bi_linear(x[:m], w, b)
        for _ in range(20):
            assert_bits_equal(bi.bi_linear(x[:m], w, b), first, f"repeat M={m}")


def test_graph_replay_matches_eager():
    d = synthetic.cfg2_inputs(4096, M_max=128)
    x, w, b = (d[k].to(DEV) for k in ("x", "w", "b"))
    eager = {m: bi.bi_linear(x[:m], w, b) for m in (1, 8, 128)}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for m in (1, 8, 128):                # warm-up on the capture stream
            bi.bi_linear(x[:m], w, b)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = {m: bi.bi_linear(x[:m], w, b) for m in (1, 8, 128)}
    for rep in range(4):
        outs_prev = {m: o.clone() for m, o in outs.items()}
        for o in outs.values():
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for m in outs:
            assert_bits_equal(outs[m], eager[m], f"graph replay {rep}, M={m}")
        _ = bi.bi_linear(x[:3], w, b)        # eager work between replays
        torch.cuda.synchronize()
        assert outs_prev is not None


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("K", [1000, 136])
def test_ragged_k_random_rows_across_kernel_families(dt, K):
    """K not a multiple of 64: 16-bit linear runs the strip kernel up to M = 64 and the generic tiled kernel
    from M = 65.  Random N(0, 1) inputs (every summation order gives different bits, unlike integer
    inputs), so the two families must run the same chain and treat the ragged tail alike: every row of
    each M equals the same row of the M = 300 call, for the (N, K) weight and for the (K, N) layout."""
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    N = 200
    x = synthetic.randn((300, K), 0x5EED3D + K, 1.0, dt).to(DEV)
    w = synthetic.randn((N, K), 0x5EED3E + K, 1.0, dt).to(DEV)
    b = synthetic.randn((N,), 0x5EED3F + K, 1.0, dt).to(DEV)
    wkn = w.t().contiguous()
    names = {lib.bi_gemm_kernel_name(m, N, K, BI, 0).decode() for m in (64, 65)}
    assert any(n.startswith("gemm16_strip") for n in names) and any(n.startswith("gemm_tiled") for n in names), names
    full = bi.bi_linear(x, w, b)
    full_kn = bi.bi_matmul(x, wkn)
    for m in (1, 16, 63, 64, 65, 129, 300):
        assert_bits_equal(bi.bi_linear(x[:m], w, b), full[:m], f"K={K} linear M={m}")
        assert_bits_equal(bi.bi_matmul(x[:m], wkn), full_kn[:m], f"K={K} (K, N) matmul M={m}")
        assert_bits_equal(bi.bi_matmul(x[:m], w.t()), bi.bi_linear(x[:m], w), f"K={K} transposed view M={m}")
    ref = oracle.linear(x[:8].cpu(), w.cpu(), b.cpu())
    assert_close_to_oracle(full[:8].cpu(), ref, f"K={K} vs oracle")


def test_splitk_comparator_is_correct_but_batch_variant():
    d = synthetic.cfg2_inputs(4096, M_max=256)
    x, w, b = (d[k].to(DEV) for k in ("x", "w", "b"))
    ref = oracle.linear(d["x"][:4], d["w"], d["b"])
    diffs = 0
    v_full = bi.bi_variant_linear(x, w, b)            # M = 256 -> 1 split
    for m in (1, 16, 17, 64, 65, 128):
        v = bi.bi_variant_linear(x[:m], w, b)
        if m >= 4:
            assert_close_to_oracle(v[:4].cpu(), ref, f"variant M={m}")
        diffs += n_bit_diff(v, v_full[:m])
    assert diffs > 0, "negative control: M-keyed split-K must change some bits"
    # and with one split it is the invariant kernel itself
    assert_bits_equal(bi.bi_variant_linear(x[:8], w, b, splits=1), bi.bi_linear(x[:8], w, b), "splits=1")


@pytest.mark.parametrize("K", [1024, 960])
def test_splitk_comparator_runs_the_invariant_kernels_exactly(K):
    """The comparator cuts K into ranges on the very kernels bi_linear picks (strip, pipelined and ring
    tiles).  With integer inputs every summation order is exact, so any split count must give the oracle
    rounded once, bit for bit: no stage of K may be dropped or counted twice at any split boundary."""
    lib = bi._native.load()
    Ns = (72, 4100)
    Ms = (1, 5, 16, 33, 64, 65, 128, 129, 256, 300, 1024)
    x = ints((max(Ms), K), 71, torch.bfloat16)
    w = ints((max(Ns), K), 72, torch.bfloat16)
    b = ints((max(Ns),), 73, torch.bfloat16, -5, 5)
    xg, wg, bg = x.to(DEV), w.to(DEV), b.to(DEV)
    seen = set()
    for n in Ns:
        ref = round_ref(oracle.linear(x, w[:n], b[:n]), torch.bfloat16)
        for m in Ms:
            seen.add(lib.bi_gemm_kernel_name(m, n, K, bi.BI_BF16, 0).decode())
            for sp in (1, 2, 3, 8):
                v = bi.bi_variant_linear(xg[:m], wg[:n], bg[:n], splits=sp)
                assert_bits_equal(v.cpu(), ref[:m], f"K={K} N={n} M={m} splits={sp}")
    assert any(k.startswith("gemm16_strip") for k in seen) and any(k.startswith("gemm16_ring") for k in seen)
    assert any(k.startswith("gemm16_pipe") for k in seen) or K % 128 != 0, seen


def test_splitk_comparator_cost_shapes_match_oracle():
    """The bf16 linear workload's shapes (K = 4096, N = 14336) through the comparator's default M-keyed
    split counts: within the oracle gate, and different bits from bi_linear at every M that splits."""
    d = synthetic.cfg2_inputs(14336, M_max=256)
    x, w, b = (d[k].to(DEV) for k in ("x", "w", "b"))
    ref = oracle.linear(d["x"][:8], d["w"], d["b"])
    lib = bi._native.load()
    for m in (8, 33, 128):
        assert lib.bi_variant_splits(m) > 1
        v = bi.bi_variant_linear(x[:m], w, b)
        assert_close_to_oracle(v[:8].cpu(), ref[:min(m, 8)], f"variant M={m}")
        assert n_bit_diff(v, bi.bi_linear(x[:m], w, b)) > 0, f"M={m}: split-K changed no bit"


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=lambda d: str(d).split(".")[-1])
@pytest.mark.parametrize("N", [4096, 14336])
def test_large_m_rows_match_small_m_calls(N, dt):
    """Rows of big-M calls (256x256 / 256x224 / 128x128 / 64x64 tiles) equal the same rows computed
    by small-M calls (strip kernel) and stay within the oracle gate, in bf16 and fp16 with a bias (the
    fp16 case pins that every kernel rounds its fmaf result to fp32 before fp16: a fused fma-and-convert
    in some kernels had made a few elements differ)."""
    K = 4096
    x = synthetic.randn((4096, K), 0x5EED3A, 1.0, dt).to(DEV)
    w = synthetic.randn((N, K), 0x5EED3B, 0.02, dt).to(DEV)
    b = synthetic.randn((N,), 0x5EED3C, 1.0, dt).to(DEV)
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    full = bi.bi_linear(x, w, b)
    seen = set()
    for m in (4096, 2048, 1024, 777, 512, 300, 200, 129, 65, 64, 16, 1):
        seen.add(lib.bi_gemm_kernel_name(m, N, K, BI, 0).decode())
        y = bi.bi_linear(x[:m], w, b)
        assert_bits_equal(y, full[:m], f"{dt} N={N} M={m}")
    for r0 in (0, 255, 256, 1000, 4095):
        assert_bits_equal(bi.bi_linear(x[r0:r0 + 1], w, b), full[r0:r0 + 1], f"{dt} N={N} row {r0} alone")
    assert len(seen) >= 3, seen
    rows = [0, 255, 256, 2049, 4095]
    ref = oracle.linear(x[rows].cpu(), w.cpu(), b.cpu())
    assert_close_to_oracle(full[rows].cpu(), ref, f"large M, {dt}, N={N}")


@pytest.mark.parametrize("K", [1024, 960])
def test_every_tile_configuration_is_exact(K):
    """Integer inputs through every large-M tile configuration (the two-stage ring tiles and the
    pipelined tiles, with 128-k or 64-k stages), M and N ragged: sampled rows equal the oracle
    rounded once, and every row equals the same row of the largest call."""
    lib = bi._native.load()
    Ns = (72, 1000, 4100, 14336)
    Ms = (65, 100, 128, 129, 200, 256, 257, 300, 700, 1024, 2048)
    x = ints((max(Ms), K), 61, torch.bfloat16)
    w = ints((max(Ns), K), 62, torch.bfloat16)
    b = ints((max(Ns),), 63, torch.bfloat16, -5, 5)
    xg, wg, bg = x.to(DEV), w.to(DEV), b.to(DEV)
    seen = set()
    for n in Ns:
        full = bi.bi_linear(xg, wg[:n], bg[:n])
        rows = [0, 1, 63, 64, 127, 128, 255, 256, 1000, max(Ms) - 1]
        ref = oracle.linear(x[rows], w[:n], b[:n])
        assert_bits_equal(full[rows].cpu(), round_ref(ref, torch.bfloat16), f"N={n} sampled rows vs oracle")
        for m in Ms:
            seen.add(lib.bi_gemm_kernel_name(m, n, K, bi.BI_BF16, 0).decode())
            assert_bits_equal(bi.bi_linear(xg[:m], wg[:n], bg[:n]), full[:m], f"K={K} N={n} M={m}")
    expect = {"gemm16_ring_nk/256x256", "gemm16_ring_nk/256x128", "gemm16_pipe_nk/128x128",
              "gemm16_pipe_nk/128x64", "gemm16_ring_nk/128x64"}
    expect |= {"gemm16_pipe_nk/64x64", "gemm16_pipe_nk/32x64"} if K % 128 == 0 else {"gemm16_ring_nk/64x64"}
    assert expect <= seen, (sorted(expect - seen), sorted(seen))


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=lambda d: str(d).split(".")[-1])
def test_rows_across_the_tile_count_switch(dt):
    """K = 2048, N = 5632: M = 2048 gives 176 tiles of 256x256 (the plan takes the largest tile with at
    least 160), M = 1279 gives 5 x 44 = 220 tiles of 256x128 and smaller M smaller tiles or the strip
    kernel: every row equals the same row of the M = 2048 call, and the oracle gate holds."""
    K, N = 2048, 5632
    x = synthetic.randn((2048, K), 0x5EED3D, 1.0, dt).to(DEV)
    w = synthetic.randn((N, K), 0x5EED3E, 0.02, dt).to(DEV)
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    assert lib.bi_gemm_kernel_name(2048, N, K, BI, 0).decode() == "gemm16_ring_nk/256x256"
    full = bi.bi_linear(x, w)
    seen = set()
    for m in (2048, 1280, 1279, 1024, 300, 64, 3):
        seen.add(lib.bi_gemm_kernel_name(m, N, K, BI, 0).decode())
        assert_bits_equal(bi.bi_linear(x[:m], w), full[:m], f"{dt} M={m}")
    assert len(seen) >= 4, seen
    rows = [0, 1279, 2047]
    assert_close_to_oracle(full[rows].cpu(), oracle.linear(x[rows].cpu(), w.cpu()), f"{dt} K=2048 N=5632")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=lambda d: str(d).split(".")[-1])
def test_kn_strip_equals_nk_strip(dt):
    """Row-major (K, N) weights up to M = 64 run the strip kernel's (K, N) form (16-column strips dealt
    XCD by XCD, transposing LDS reads): every strip configuration, N ragged (strip counts not a multiple
    of 8, a last strip of 8 columns), K ragged and tiny; random inputs, so the bits equal the (N, K) path
    only if the chain is the same; matmul, addmm with a broadcast row and fp32 output."""
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    for N, K in ((8, 8), (24, 136), (1000, 4104), (4104, 1000), (4096, 4096)):
        x = synthetic.randn((64, K), 0x5EED40 + K, 1.0, dt).to(DEV)
        w = synthetic.randn((N, K), 0x5EED41 + N, 0.05, dt).to(DEV)
        c = synthetic.randn((N,), 0x5EED42 + N, 1.0, dt).to(DEV)
        wkn = w.t().contiguous()
        for m in (1, 4, 5, 8, 9, 16, 17, 32, 33, 64):
            assert lib.bi_gemm_kernel_name(m, N, K, BI, 1).decode().startswith("gemm16_strip_kn/"), (m, N, K)
            want = bi.bi_linear(x[:m], w)
            assert_bits_equal(bi.bi_matmul(x[:m], wkn), want, f"N={N} K={K} M={m}: (K, N) vs (N, K)")
            assert_bits_equal(bi.bi_addmm(c, x[:m], wkn), bi.bi_linear(x[:m], w, c), f"N={N} K={K} M={m}: addmm")
            assert_bits_equal(bi.bi_matmul(x[:m], wkn, out_dtype=torch.float32),
                              bi.bi_linear(x[:m], w, out_dtype=torch.float32), f"N={N} K={K} M={m}: fp32 out")
    ref = oracle.linear(x[:4].cpu(), w.cpu())
    assert_close_to_oracle(bi.bi_matmul(x[:4], wkn).cpu(), ref, "(K, N) strip vs oracle")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=lambda d: str(d).split(".")[-1])
def test_kn_pipe_equals_nk(dt):
    """Row-major (K, N) weights above 64 rows with K a multiple of 64 run the 128x128 pipelined kernel's
    (K, N) form (transposing LDS reads of 256-byte k-rows): ragged M and N, random inputs, bitwise equal
    to the (N, K) path (whatever tile that takes), for matmul, addmm with a broadcast row and fp32 out."""
    lib = bi._native.load()
    BI = bi.BI_BF16 if dt == torch.bfloat16 else bi.BI_F16
    for N, K in ((1000, 4096), (4104, 1024), (72, 192), (4096, 4096)):
        x = synthetic.randn((1100, K), 0x5EED43 + K, 1.0, dt).to(DEV)
        w = synthetic.randn((N, K), 0x5EED44 + N, 0.05, dt).to(DEV)
        c = synthetic.randn((N,), 0x5EED45 + N, 1.0, dt).to(DEV)
        wkn = w.t().contiguous()
        for m in (65, 128, 129, 300, 1100):
            assert lib.bi_gemm_kernel_name(m, N, K, BI, 1).decode() == "gemm16_pipe_kn/128x128", (m, N, K)
            assert_bits_equal(bi.bi_matmul(x[:m], wkn), bi.bi_linear(x[:m], w), f"N={N} K={K} M={m}: (K, N) vs (N, K)")
            assert_bits_equal(bi.bi_addmm(c, x[:m], wkn), bi.bi_linear(x[:m], w, c), f"N={N} K={K} M={m}: addmm")
        assert_bits_equal(bi.bi_matmul(x[:300], wkn, out_dtype=torch.float32),
                          bi.bi_linear(x[:300], w, out_dtype=torch.float32), f"N={N} K={K}: fp32 out")
    ref = oracle.linear(x[[0, 1099]].cpu(), w.cpu())
    assert_close_to_oracle(bi.bi_matmul(x, wkn)[[0, 1099]].cpu(), ref, "(K, N) pipe vs oracle")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16, torch.float32], ids=lambda d: str(d).split(".")[-1])
def test_batched_matmul_equals_per_element_calls(dt):
    """bi_matmul_batched runs every batch element in one launch (the grid's third dimension); each element's
    bits equal bi_matmul on that element alone, for every kernel family the shapes reach (strip, pipelined
    and ring tiles, the generic tiled kernel), row-major and column-major b, a shared operand (batch stride
    0), a strided slice of a larger batch, and fp32 output."""
    Z = 3
    shapes = ((1, 72, 136), (17, 264, 256), (100, 520, 520), (300, 1000, 1024), (1100, 256, 4096))
    for M, N, K in shapes:
        a = synthetic.randn((Z + 1, M, K), 0x5EED61 + M, 1.0, dt).to(DEV)[1:]      # storage offset: one element
        w = synthetic.randn((Z, N, K), 0x5EED62 + N, 0.05, dt).to(DEV)
        bkn = w.transpose(1, 2).contiguous()          # (Z, K, N) row-major
        bnk = w.transpose(1, 2)                       # column-major views of the (N, K) rows
        for name, b in (("(K, N)", bkn), ("(N, K)", bnk)):
            y = bi.bi_matmul_batched(a, b)
            assert y.shape == (Z, M, N)
            for z in range(Z):
                assert_bits_equal(y[z], bi.bi_matmul(a[z], b[z]), f"M={M} N={N} K={K} b {name} element {z}")
        shared = bkn[1:2].expand(Z, K, N)             # batch stride 0: one weight for every element
        y = bi.bi_matmul_batched(a, shared)
        for z in range(Z):
            assert_bits_equal(y[z], bi.bi_matmul(a[z], bkn[1]), f"M={M} N={N} K={K} shared b element {z}")
        if dt != torch.float32:
            y = bi.bi_matmul_batched(a, bkn, out_dtype=torch.float32)
            assert_bits_equal(y[2], bi.bi_matmul(a[2], bkn[2], out_dtype=torch.float32), f"M={M}: fp32 out")
        rows = [0, M - 1]
        ref = oracle.matmul(a[1, rows].cpu(), bkn[1].cpu())
        assert_close_to_oracle(bi.bi_matmul_batched(a, bkn)[1, rows].cpu(), ref, f"M={M} N={N} K={K} vs oracle")


def test_batched_matmul_past_one_grid_of_elements():
    """More than 65535 elements take several launches; integer inputs make every element exact."""
    Z, M, N, K = 70001, 2, 8, 16
    a = ints((Z, M, K), 0x5EED63, torch.bfloat16).to(DEV)
    b = ints((Z, K, N), 0x5EED64, torch.bfloat16).to(DEV)
    y = bi.bi_matmul_batched(a, b).cpu()
    ref = torch.bmm(a.cpu().double(), b.cpu().double()).to(torch.bfloat16)
    assert_bits_equal(y, ref, "70001 integer-valued elements")
