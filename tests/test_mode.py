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
                                      ((2, 3, 4, 5), (2, 3, 5, 6), "batched"), ((2, 4, 5), (1, 5, 3), "batched"),
                                      ((2, 4, 5), (3, 2, 5, 3), "batched"), ((4, 5), (2, 5, 3), "batched"),
                                      ((5,), (2, 5, 3), "batched")])
def test_plan_matmul(a, b, kind):
    assert mode.plan_matmul(a, b) == kind


@pytest.mark.parametrize("a,b", [((), (3,)), ((3, 4), ()), ((2, 4, 5), (3, 5, 3)), ((2, 3, 4, 5), (4, 5, 6))])
def test_plan_matmul_refuses_scalars_and_batch_dims_that_do_not_broadcast(a, b):
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


_PATCHED = [(torch.nn.functional, "linear"), (torch, "mm"), (torch.Tensor, "mm"), (torch, "addmm"),
            (torch.Tensor, "addmm"), (torch, "matmul"), (torch.Tensor, "matmul"), (torch.Tensor, "__matmul__"),
            (torch.Tensor, "__rmatmul__"), (torch, "bmm"), (torch.Tensor, "bmm"),
            (torch.nn.functional, "scaled_dot_product_attention"), (torch, "sum"), (torch.Tensor, "sum"),
            (torch, "mean"), (torch.Tensor, "mean")]


def _current():
    return [getattr(o, n) for o, n in _PATCHED], [n in vars(o) for o, n in _PATCHED]


def test_functions_are_restored_after_nested_modes_and_errors():
    before = _current()
    with bi.batch_invariant_mode():
        inside = _current()
        assert all(a is not b for a, b in zip(inside[0], before[0]))
        with bi.batch_invariant_mode(strict=False):
            assert _current()[0] == inside[0]
        assert _current()[0] == inside[0]              # the inner exit leaves the outer mode's wrappers
    after = _current()
    assert all(a is b for a, b in zip(after[0], before[0])) and after[1] == before[1]
    with pytest.raises(RuntimeError):
        with bi.batch_invariant_mode():
            raise RuntimeError("boom")
    assert all(a is b for a, b in zip(_current()[0], before[0]))


def test_wrappers_keep_names_and_cpu_results():
    a = torch.randn(4, 6, dtype=torch.float32)
    b = torch.randn(6, 3, dtype=torch.float32)
    want = (a @ b, torch.mm(a, b), a.sum(-1), a.mean(0), torch.nn.functional.linear(a, b.t()))
    with bi.batch_invariant_mode() as m:
        assert torch.mm.__name__ == "mm" and torch.Tensor.sum.__name__ == "sum"
        got = (a @ b, torch.mm(a, b), a.sum(-1), a.mean(0), torch.nn.functional.linear(a, b.t()))
        assert not m.routed and not m.fallbacks
    assert all(torch.equal(x, y) for x, y in zip(got, want))


def test_modes_are_per_thread():
    import threading
    seen = []
    with bi.batch_invariant_mode():
        t = threading.Thread(target=lambda: seen.append(list(getattr(mode._tls, "stack", None) or [])))
        t.start()
        t.join()
        assert len(mode._tls.stack) == 1
    assert seen == [[]]
