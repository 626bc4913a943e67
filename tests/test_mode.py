"""CPU checks of the PyTorch routing mode's decisions (no GPU call is made)."""
import pytest
import torch

import invariant_deterministic_gemm_amd as bi
from invariant_deterministic_gemm_amd import mode


def test_routed_functions():
    assert mode.routed_functions() == sorted(["__matmul__", "__rmatmul__", "addmm", "bmm", "linear", "matmul", "mm",
                                              "scaled_dot_product_attention", "sum", "mean"])


@pytest.mark.parametrize("a,b,kind", [((4, 5), (5, 3), "mm"), ((2, 4, 5), (5, 3), "mm"), ((5,), (5, 3), "vm"),
                                      ((4, 5), (5,), "mv"), ((5,), (5,), "dot"), ((2, 4, 5), (2, 5, 3), "batched"),
                                      ((2, 3, 4, 5), (2, 3, 5, 6), "batched")])
def test_plan_matmul(a, b, kind):
    assert mode.plan_matmul(a, b) == kind


@pytest.mark.parametrize("a,b", [((), (3,)), ((2, 4, 5), (1, 5, 3)), ((2, 4, 5), (3, 2, 5, 3)), ((4, 5), (2, 5, 3))])
def test_plan_matmul_refuses_broadcasts_and_scalars(a, b):
    with pytest.raises(mode.Unsupported):
        mode.plan_matmul(a, b)


def test_cpu_tensors_pass_through_in_strict_mode():
    a = torch.randn(3, 8, dtype=torch.float64)
    w = torch.randn(5, 8, dtype=torch.float64)
    with bi.batch_invariant_mode() as m:
        y = torch.nn.functional.linear(a, w)
        z = a @ w.t()
    assert torch.equal(y, torch.nn.functional.linear(a, w)) and torch.equal(z, a @ w.t())
    assert not m.routed and not m.fallbacks
