"""GPU tests of bi_rowsum, the row sum / mean over the last dimension.

* exact pins: integer inputs make every summation order exact, so the result
  equals the oracle rounded once;
* a rigorous bound against the float64 oracle on random inputs: each row is
  summed by a chain of at most ceil(N / 256) + 8 fp32 additions, so
  |y - ref| <= (ceil(N / 256) + 8) * 2^-24 * sum|x| + u_out * |ref|;
* invariance on raw bit patterns across the number of rows and against NaN
  neighbours; edge cases (one element, empty rows, no rows, strided rows).
"""
import math

import numpy as np
import pytest
import torch

import invariant_deterministic_gemm_amd as bi
import oracle
import synthetic
from helpers import assert_bits_equal, round_ref

pytestmark = pytest.mark.gpu
DEV = "cuda"
DTS = [torch.float32, torch.bfloat16, torch.float16]
U_OUT = {torch.float32: 2.0 ** -24, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def _ids(d):
    return str(d).split(".")[-1]


@pytest.mark.parametrize("dt", DTS, ids=_ids)
def test_integer_rows_are_exact(dt):
    x = synthetic.randint((300, 5000), 201, -8, 8, dt)
    y = bi.bi_rowsum(x.to(DEV)).cpu()
    assert_bits_equal(y, round_ref(oracle.rowsum(x), dt), f"sum {dt}")
    if dt == torch.float32:
        ym = bi.bi_rowsum(x.to(DEV), mean=True).cpu()
        assert_bits_equal(ym, round_ref(oracle.rowsum(x, mean=True), dt), "mean fp32")


@pytest.mark.parametrize("dt", DTS, ids=_ids)
@pytest.mark.parametrize("N", [1, 255, 256, 4099, 70000])
def test_error_bound_against_oracle(dt, N):
    x = synthetic.randn((64, N), 202 + N, 1.0, dt)
    for mean in (False, True):
        y = bi.bi_rowsum(x.to(DEV), mean=mean).cpu().double().numpy()
        ref = oracle.rowsum(x, mean=mean)
        absum = np.abs(x.double().numpy()).sum(axis=1) / (N if mean else 1)
        chain = math.ceil(N / 256) + 8 + (1 if mean else 0)
        bound = chain * 2.0 ** -24 * absum + U_OUT[dt] * np.abs(ref) * 1.0001 + 1e-30
        assert (np.abs(y - ref) <= bound).all(), f"N={N} mean={mean}: max excess {(np.abs(y - ref) / bound).max():.3f}"


@pytest.mark.parametrize("dt", DTS, ids=_ids)
def test_rows_do_not_depend_on_batch_or_neighbours(dt):
    x = synthetic.randn((1024, 4099), 203, 1.0, dt).to(DEV)
    full = bi.bi_rowsum(x)
    fullm = bi.bi_rowsum(x, mean=True)
    for M in (1, 2, 3, 7, 64, 255, 256, 257, 1000):
        assert_bits_equal(bi.bi_rowsum(x[:M]), full[:M], f"sum M={M}")
        assert_bits_equal(bi.bi_rowsum(x[:M], mean=True), fullm[:M], f"mean M={M}")
    x2 = torch.full_like(x, float("nan"))
    x2[500] = x[500]
    assert_bits_equal(bi.bi_rowsum(x2)[500:501], full[500:501], "NaN neighbours")
    for r in (0, 511, 1023):
        assert_bits_equal(bi.bi_rowsum(x[r:r + 1]), full[r:r + 1], f"row {r} alone")


def test_edge_cases_and_strided_rows():
    x = synthetic.randn((5, 3, 40), 204, 1.0, torch.bfloat16).to(DEV)
    y = bi.bi_rowsum(x)
    assert y.shape == (5, 3)
    assert_bits_equal(y.reshape(-1), bi.bi_rowsum(x.reshape(15, 40)), "leading dims are batch")
    wide = synthetic.randn((6, 96), 205, 1.0, torch.float32).to(DEV)
    assert_bits_equal(bi.bi_rowsum(wide[:, :64]), bi.bi_rowsum(wide[:, :64].contiguous()), "row pitch 96")
    one = bi.bi_rowsum(wide[:, :1])
    assert_bits_equal(one, wide[:, 0].contiguous(), "one element")
    empty = bi.bi_rowsum(wide[:, :0])
    assert torch.equal(empty, torch.zeros(6, device=DEV))
    assert torch.isnan(bi.bi_rowsum(wide[:, :0], mean=True)).all()
    assert bi.bi_rowsum(wide[:0]).shape == (0,)
