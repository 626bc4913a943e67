"""Comparison helpers shared by the GPU tests.

Invariance is judged on raw bit patterns (mlx-batch-invariant README,
section 'What "batch-invariant" means here': uint32 / uint16 patterns, never
allclose or float ==).  Correctness against the float64 oracle uses the
normwise relative error max|y - ref| / max|ref| with the gates below.
"""
import numpy as np
import torch

# Oracle gates: fp32 outputs 1e-5, bf16 / fp16 outputs (fp32 accumulation) 2e-2.
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 2e-2}

_INT = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16}


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(_INT[t.dtype])


def n_bit_diff(a: torch.Tensor, b: torch.Tensor) -> int:
    """Number of elements whose bit patterns differ (0 means bitwise identical)."""
    assert a.shape == b.shape, (a.shape, b.shape)
    assert a.dtype == b.dtype
    return int((bits(a) != bits(b)).sum().item())


def assert_bits_equal(a: torch.Tensor, b: torch.Tensor, what: str = ""):
    n = n_bit_diff(a, b)
    assert n == 0, f"{what}: {n} of {a.numel()} elements differ in their bits"


def rel_err(y: torch.Tensor, ref: np.ndarray) -> float:
    yn = y.detach().to("cpu", torch.float64).numpy()
    assert yn.shape == ref.shape, (yn.shape, ref.shape)
    assert np.isfinite(yn).all(), "non-finite output where the reference is finite"
    den = np.abs(ref).max()
    return float(np.abs(yn - ref).max() / (den if den > 0 else 1.0))


def assert_close_to_oracle(y: torch.Tensor, ref: np.ndarray, what: str = ""):
    e = rel_err(y, ref)
    tol = TOL[y.dtype]
    assert e <= tol, f"{what}: relative error {e:.3e} exceeds {tol:g}"
    return e


def round_ref(ref: np.ndarray, dtype) -> torch.Tensor:
    """Round the float64 oracle once to the output dtype (RNE), for exact pins."""
    return torch.from_numpy(ref).to(dtype)
