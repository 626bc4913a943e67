"""Seeded synthetic inputs for the batch-invariant GEMM and attention workloads.

This module only draws random numbers and names shapes; it holds none of the
arithmetic of the method.  Both the GPU path's tests / benchmark and the CPU
oracle are fed from it, so they always see identical values.

Recipe: torch.Generator('cpu').manual_seed(seed), torch.randn in float32,
multiplied by a standard deviation, then cast to the target dtype with
round-to-nearest-even.  Large base tensors are drawn once at the largest
size of a sweep and sliced (prefix rows), so "row r is identical across
batch sizes" holds by construction.

The pages measure on real models (logits of a chat model, a 0.94B model);
these seeded normal draws stand in for them with the same shapes: hidden
size 4096, MLP width 14336, vocabulary 32000, 32 query / 8 KV heads of
width 128, and so on.
"""
from __future__ import annotations

import hashlib

import torch

SEED_BASE = 0x5EED00

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def seed_for(config: int, sub: int = 0) -> int:
    return SEED_BASE + 16 * config + sub


def randn(shape, seed: int, std: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) draw on the CPU, cast (RNE) to dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t = t * std
    return t.to(dtype)


def randint(shape, seed: int, lo: int, hi: int, dtype=torch.float32) -> torch.Tensor:
    """Integer values uniform in [lo, hi], stored in a float dtype (exact)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randint(lo, hi + 1, tuple(shape), generator=g, dtype=torch.int64).to(dtype)


def sha256(t: torch.Tensor) -> str:
    """Fingerprint of a tensor's bytes, logged to detect input drift."""
    b = t.detach().to("cpu").contiguous().view(torch.uint8).numpy().tobytes()
    return hashlib.sha256(b).hexdigest()[:16]


# ---------------------------------------------------------------- configs
# 1: fp32 linear, x (M,256) with M in 1..8, W (512,256), b (512), all N(0,1).
CFG1 = dict(K=256, N=512, M_values=list(range(1, 9)), dtype="f32")
# 2: bf16 linear / addmm, K=4096, N in {4096, 14336}; x ~ N(0,1), W ~ N(0,0.02).
CFG2 = dict(K=4096, N_values=[4096, 14336],
            M_values=[1, 2, 3, 4, 7, 8, 16, 33, 64, 128, 256], dtype="bf16", w_std=0.02)
# 3: bf16 causal GQA attention, Hq=32, Hkv=8, D=128, KV cache 1024, q_len sweep.
CFG3 = dict(Hq=32, Hkv=8, D=128, S=1024, Lq_values=[1, 2, 4, 8, 9, 16, 64], dtype="bf16")
# 4: context growth, Hq=16, Hkv=8, D=128, single-token decode, S from 4000 to 4200.
CFG4 = dict(Hq=16, Hkv=8, D=128, S_lo=4000, S_hi=4200, dtypes=["f32", "bf16"])
# 5: logits projection, hidden (M,4096) x W (32000,4096)^T, M in 1..64, bf16 and fp16.
CFG5 = dict(K=4096, N=32000, M_max=64, dtypes=["bf16", "f16"], w_std=0.02)


def cfg1_inputs():
    s = seed_for(1)
    return dict(x=randn((8, 256), s), w=randn((512, 256), s + 1), b=randn((512,), s + 2))


def cfg2_inputs(N: int, M_max: int = 256, dtype=torch.bfloat16):
    s = seed_for(2, 0 if N == 4096 else 4)
    return dict(x=randn((M_max, 4096), s, 1.0, dtype),
                w=randn((N, 4096), s + 1, 0.02, dtype),
                b=randn((N,), s + 2, 1.0, dtype),
                c=randn((M_max, N), s + 3, 1.0, dtype))


def cfg3_inputs(B: int = 1, S: int = 1024, dtype=torch.bfloat16):
    s = seed_for(3)
    return dict(q=randn((B, 32, S, 128), s, 1.0, dtype),
                k=randn((B, 8, S, 128), s + 1, 1.0, dtype),
                v=randn((B, 8, S, 128), s + 2, 1.0, dtype))


def cfg4_inputs(dtype=torch.float32, S: int = 4200):
    s = seed_for(4)
    return dict(q=randn((1, 16, 1, 128), s, 1.0, dtype),
                k=randn((1, 8, S, 128), s + 1, 1.0, dtype),
                v=randn((1, 8, S, 128), s + 2, 1.0, dtype))


def cfg5_inputs(dtype=torch.bfloat16, M_max: int = 64):
    s = seed_for(5, 0 if dtype == torch.bfloat16 else 4)
    return dict(h=randn((M_max, 4096), s, 1.0, dtype),
                w=randn((32000, 4096), s + 1, 0.02, dtype))
