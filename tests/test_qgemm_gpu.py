"""GPU tests of the quantized linear (bi_quantized_linear), README section "Quantized models".

* bitwise identity with bi_linear on the dequantised weight: the weight is dequantised on the host in
  float64 (exact), rounded once to fp32 (what one fmaf gives) and once to the input dtype, and the
  result of bi_linear on it must equal the quantized kernel bit for bit -- the same chain, only the
  weight's storage differs;
* oracle tolerance (bf16 / fp16 outputs: 2e-2) against the float64 oracle's quantized_linear;
* invariance on raw bit patterns across batch size and batch neighbours;
* shapes with ragged N, a partial last stage of the K loop, every bit width and group size, and the three
  paths (up to 64 rows: unpacked inside the strip kernel's K loop; more rows with K a multiple of 128:
  dequantised on the way into the tile kernel's LDS; other K: dequantised by chunks into a workspace for
  bi_linear's kernels), whose rows must agree bit for bit;
* scale / bias rows padded past K / group_size (through the C ABI), and scales of 2^118 and 2^119 beside
  ordinary ones.
"""
import numpy as np
import pytest
import torch

import invariant_deterministic_gemm_amd as bi
from invariant_deterministic_gemm_amd import _native
import oracle
import synthetic
from helpers import assert_bits_equal, assert_close_to_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


def make(N, K, bits, gs, dt, seed):
    w = synthetic.randn((N, K), seed, 0.02, dt)
    wq, sc, sb = bi.quantize(w, bits, gs)
    return wq, sc, sb


def host_dequant(wq, sc, sb, bits, gs, K, dt):
    """The kernel's weight, built on the host: exact float64 value -> fp32 -> dt (each step RNE)."""
    exact = oracle.dequantize(wq, sc, sb, bits, gs, K)
    return torch.from_numpy(exact.astype(np.float32)).to(dt)


CASES = [  # M, N, K, bits, gs
    (1, 4096, 4096, 4, 64), (4, 300, 384, 4, 128), (7, 513, 256, 8, 32), (16, 257, 96, 2, 32),
    (33, 1000, 1024, 4, 32), (64, 128, 640, 8, 128), (100, 96, 512, 2, 64), (200, 72, 4096, 4, 64),
    (70, 8200, 256, 4, 64),   # more than 64 rows: dequantised in two chunks of columns (8192 + 8)
    # one row and few rows, with partial last stages (512-k stages for one strip per workgroup)
    (1, 100, 352, 8, 32), (1, 33, 160, 2, 32), (2, 77, 4160, 4, 64), (5, 200, 800, 2, 32),
    (9, 2000, 1536, 8, 128), (1, 4200, 768, 8, 64), (1, 4500, 1056, 2, 32),
    # wide N (more than 256 strips of 16 columns): two strips per workgroup, ragged last pair
    (2, 4200, 512, 4, 64), (16, 4113, 288, 8, 32), (17, 5000, 384, 2, 128), (40, 4500, 640, 4, 32),
    (64, 4104, 256, 8, 64),
    # more than 64 rows, K a multiple of 128: the dequantising tile kernel (64 x 64 tiles; 128 x 128 tiles
    # from 192 of them), every bit width; other K: the workspace path
    (150, 500, 1024, 8, 128), (65, 33, 384, 4, 32), (200, 12288, 256, 4, 64), (300, 1000, 640, 2, 128),
    (80, 300, 224, 4, 32), (130, 200, 352, 8, 32),
    # few rows of 4-bit weights at every group size, ragged N, K past a 1024-k boundary
    (3, 1000, 1024, 4, 32), (4, 300, 1280, 4, 128), (2, 4113, 2048, 4, 64), (4, 4096, 4096, 4, 64),
    (1, 16, 256, 4, 32),
]


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("M,N,K,bits,gs", CASES)
def test_equals_linear_on_dequantised_weight_and_oracle(M, N, K, bits, gs, dt):
    seed = M * 7 + N * 13 + K + bits
    wq, sc, sb = make(N, K, bits, gs, dt, seed)
    x = synthetic.randn((M, K), seed + 1, 1.0, dt)
    bias = synthetic.randn((N,), seed + 2, 1.0, dt)
    wd = host_dequant(wq, sc, sb, bits, gs, K, dt)
    y = bi.bi_quantized_linear(x.to(DEV), wq.to(DEV), sc.to(DEV), sb.to(DEV), bits, gs, bias.to(DEV))
    ref = bi.bi_linear(x.to(DEV), wd.to(DEV), bias.to(DEV))
    assert_bits_equal(y, ref, f"M={M} N={N} K={K} bits={bits} gs={gs}: quantized vs linear on dequantised W")
    want = oracle.quantized_linear(x, wq, sc, sb, bits, gs, bias)
    assert_close_to_oracle(y, want, f"M={M} N={N} K={K} bits={bits} gs={gs}")


@pytest.mark.parametrize("bits,gs,N", [(4, 64, 1536), (8, 32, 1536), (2, 128, 1536), (4, 64, 4500)])
def test_rows_do_not_depend_on_batch(bits, gs, N):
    dt = torch.bfloat16
    K, Mmax = 2048, 200
    wq, sc, sb = (t.to(DEV) for t in make(N, K, bits, gs, dt, 99 + bits))
    x = synthetic.randn((Mmax, K), 98, 1.0, dt).to(DEV)
    full = bi.bi_quantized_linear(x, wq, sc, sb, bits, gs)
    for M in (1, 2, 3, 15, 16, 17, 32, 33, 63, 64, 65, 129):
        part = bi.bi_quantized_linear(x[:M], wq, sc, sb, bits, gs)
        assert_bits_equal(part, full[:M], f"bits={bits} gs={gs} M={M} vs M={Mmax}")
    # batch neighbours: the other rows replaced by NaN
    noisy = x.clone()
    noisy[1:] = float("nan")
    one = bi.bi_quantized_linear(noisy[:40], wq, sc, sb, bits, gs)
    assert_bits_equal(one[:1], full[:1], "row 0 with NaN neighbours")


def test_zero_k_gives_bias_and_errors_raise():
    dt = torch.bfloat16
    bias = synthetic.randn((40,), 5, 1.0, dt).to(DEV)
    x = torch.empty((3, 0), dtype=dt, device=DEV)
    wq = torch.empty((40, 0), dtype=torch.int32, device=DEV)
    sc = torch.empty((40, 0), dtype=dt, device=DEV)
    y = bi.bi_quantized_linear(x, wq, sc, sc, 4, 64, bias)
    assert_bits_equal(y, bias[None].expand(3, 40).contiguous(), "K = 0")
    wq3, sc3, sb3 = (t.to(DEV) for t in make(16, 256, 4, 64, dt, 6))
    with pytest.raises(NotImplementedError):                      # 3-bit packings are refused, never guessed
        bi.bi_quantized_linear(torch.zeros((2, 256), dtype=dt, device=DEV), wq3, sc3, sb3, 3, 64)


@pytest.mark.parametrize("M", [1, 16, 100])
def test_graph_replay_equals_eager(M):
    """Eager vs graph-captured launch (the workspace of the M > 64 path allocated inside the capture):
    every replay, with eager calls and synchronisations in between, gives the eager bits."""
    dt = torch.bfloat16
    wq, sc, sb = (t.to(DEV) for t in make(1000, 768, 4, 64, dt, 390 + M))
    x = synthetic.randn((M, 768), 391, 1.0, dt).to(DEV)
    fn = lambda: bi.bi_quantized_linear(x, wq, sc, sb, 4, 64)
    eager = fn()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(out, eager, f"M={M}: graph replay {rep}")
        fn()
        torch.cuda.synchronize()


def _qlinear_raw(x, wq, sc, sb, ldsb, gs, N, K):
    """bi_quantized_linear through the C ABI with an explicit scale / bias row pitch (4-bit, bf16)."""
    lib = _native.load()
    M = x.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    st = lib.bi_quantized_linear(x.data_ptr(), x.stride(0), wq.data_ptr(), wq.stride(0), sc.data_ptr(),
                                 sb.data_ptr(), ldsb, 4, gs, None, y.data_ptr(), N, M, N, K, _native.BI_BF16,
                                 None, 0, torch.cuda.current_stream().cuda_stream)
    assert st == _native.BI_OK, lib.bi_last_error().decode()
    return y


def test_padded_scale_rows_and_huge_scales():
    """Few rows of 4-bit weights, equal bit for bit to bi_linear on the host's dequantised weight: (a)
    scale / bias rows padded to 8 entries for 3 groups (K = 96, a partial stage); (b) groups whose scale
    is 2^119 or 2^118 beside ordinary ones, with x small on those groups so every product stays finite."""
    dt = torch.bfloat16
    N, K, gs = 50, 96, 32
    wq, sc, sb = make(N, K, 4, gs, dt, 7)
    scp = torch.zeros((N, 8), dtype=dt)
    sbp = torch.zeros((N, 8), dtype=dt)
    scp[:, :3] = sc
    sbp[:, :3] = sb
    wd = host_dequant(wq, sc, sb, 4, gs, K, dt).to(DEV)
    for M in (1, 3, 4):
        x = synthetic.randn((M, K), 8 + M, 1.0, dt).to(DEV)
        y = _qlinear_raw(x, wq.to(DEV), scp.to(DEV), sbp.to(DEV), 8, gs, N, K)
        assert_bits_equal(y, bi.bi_linear(x, wd), f"padded scale rows, M={M}")
    N, K, gs = 64, 1024, 64
    wq, sc, sb = make(N, K, 4, gs, dt, 11)
    sc, sb = sc.clone(), sb.clone()
    sc[0::2, 1] = 2.0 ** 119
    sb[0::2, 1] = 0.0
    sc[0::3, 9] = 2.0 ** 118
    sb[0::3, 9] = 1.0
    x = synthetic.randn((4, K), 12, 1.0, dt)
    x[:, 64:128] *= 2.0 ** -124
    x[:, 576:640] *= 2.0 ** -123
    wd = host_dequant(wq, sc, sb, 4, gs, K, dt).to(DEV)
    for M in (1, 2, 4):
        xm = x[:M].contiguous().to(DEV)
        y = bi.bi_quantized_linear(xm, wq.to(DEV), sc.to(DEV), sb.to(DEV), 4, gs)
        ref = bi.bi_linear(xm, wd)
        assert torch.isfinite(ref.float()).all()
        assert_bits_equal(y, ref, f"scales of 2^118 and 2^119, M={M}")
