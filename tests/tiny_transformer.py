"""A small decoder-only transformer with seeded random weights, used as an
end-to-end workload for the routing mode (no trained weights are involved).

Llama-style: token embedding, pre-norm blocks of RMSNorm -> grouped-query
attention with rotary position embedding -> residual, RMSNorm -> SwiGLU MLP ->
residual, final RMSNorm and a vocabulary projection.  Written with plain torch
ops so that the same code runs as stock PyTorch or, inside
batch_invariant_mode(), on the batch-invariant kernels (linear layers,
attention, last-dim sums); everything else is element-wise or a row-wise op
the mode leaves alone.

Sequences of a batch share one length (prefill) and one position (decode),
so no padding mask is needed; attention in decode sees every cached key.
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F


class TinyConfig:
    def __init__(self, vocab=32000, hidden=2048, layers=4, heads=16, kv_heads=4, head_dim=128, mlp=5632,
                 rope_theta=10000.0, eps=1e-6):
        self.vocab, self.hidden, self.layers = vocab, hidden, layers
        self.heads, self.kv_heads, self.head_dim, self.mlp = heads, kv_heads, head_dim, mlp
        self.rope_theta, self.eps = rope_theta, eps


def make_weights(cfg: TinyConfig, seed: int, device, dtype=torch.bfloat16) -> dict:
    """Seeded normal weights (std 0.02, norms at 1) drawn on the CPU generator, then moved."""
    g = torch.Generator("cpu").manual_seed(seed)

    def w(*shape):
        return (torch.randn(*shape, generator=g) * 0.02).to(dtype).to(device)

    H, D, Hk = cfg.heads, cfg.head_dim, cfg.kv_heads
    W = {"embed": w(cfg.vocab, cfg.hidden), "norm": torch.ones(cfg.hidden, dtype=dtype, device=device),
         "lm_head": w(cfg.vocab, cfg.hidden), "layers": []}
    for _ in range(cfg.layers):
        W["layers"].append({
            "ln1": torch.ones(cfg.hidden, dtype=dtype, device=device),
            "wq": w(H * D, cfg.hidden), "wk": w(Hk * D, cfg.hidden), "wv": w(Hk * D, cfg.hidden),
            "wo": w(cfg.hidden, H * D),
            "ln2": torch.ones(cfg.hidden, dtype=dtype, device=device),
            "wg": w(cfg.mlp, cfg.hidden), "wu": w(cfg.mlp, cfg.hidden), "wd": w(cfg.hidden, cfg.mlp),
        })
    return W


def _rope(x, pos, theta):
    """Rotary embedding on (B, H, L, D) at integer positions pos (L,), computed in fp32."""
    D = x.shape[-1]
    inv = 1.0 / (theta ** (torch.arange(0, D, 2, device=x.device, dtype=torch.float32) / D))
    ang = pos.to(torch.float32)[:, None] * inv[None, :]
    cos, sin = ang.cos(), ang.sin()
    xf = x.float()
    x1, x2 = xf[..., 0::2], xf[..., 1::2]
    out = torch.stack((x1 * cos - x2 * sin, x1 * sin + x2 * cos), dim=-1).flatten(-2)
    return out.to(x.dtype)


def forward(cfg: TinyConfig, W: dict, tokens: torch.Tensor, cache: list | None, start: int):
    """Logits (B, L, vocab) for tokens (B, L) at positions start .. start + L - 1; `cache` is a list of
    (k, v) per layer with start keys each (None for a prefill from position 0).  Returns (logits, cache)."""
    B, L = tokens.shape
    H, Hk, D = cfg.heads, cfg.kv_heads, cfg.head_dim
    pos = torch.arange(start, start + L, device=tokens.device)
    x = W["embed"][tokens]
    new_cache = []
    for li, lw in enumerate(W["layers"]):
        h = F.rms_norm(x, (cfg.hidden,), lw["ln1"], cfg.eps)
        q = F.linear(h, lw["wq"]).view(B, L, H, D).transpose(1, 2)
        k = F.linear(h, lw["wk"]).view(B, L, Hk, D).transpose(1, 2)
        v = F.linear(h, lw["wv"]).view(B, L, Hk, D).transpose(1, 2)
        q, k = _rope(q, pos, cfg.rope_theta), _rope(k, pos, cfg.rope_theta)
        if cache is not None:
            k = torch.cat((cache[li][0], k), dim=2)
            v = torch.cat((cache[li][1], v), dim=2)
        new_cache.append((k, v))
        # prefill from 0: causal (query length == key length); decode: every cached key is visible
        a = F.scaled_dot_product_attention(q, k, v, is_causal=cache is None, enable_gqa=True,
                                           scale=1.0 / math.sqrt(D))
        x = x + F.linear(a.transpose(1, 2).reshape(B, L, H * D), lw["wo"])
        h = F.rms_norm(x, (cfg.hidden,), lw["ln2"], cfg.eps)
        x = x + F.linear(F.silu(F.linear(h, lw["wg"])) * F.linear(h, lw["wu"]), lw["wd"])
    x = F.rms_norm(x, (cfg.hidden,), W["norm"], cfg.eps)
    return F.linear(x, W["lm_head"]), new_cache


def greedy_decode(cfg: TinyConfig, W: dict, prompt: torch.Tensor, steps: int):
    """Prefill the prompt (B, L), then `steps` greedy decode steps; returns the logits of every step
    (B, steps + 1, vocab): the last prompt position, then each decoded token's."""
    logits, cache = forward(cfg, W, prompt, None, 0)
    out = [logits[:, -1]]
    tok = logits[:, -1].float().argmax(-1, keepdim=True)
    pos = prompt.shape[1]
    for _ in range(steps):
        logits, cache = forward(cfg, W, tok, cache, pos)
        out.append(logits[:, -1])
        tok = logits[:, -1].float().argmax(-1, keepdim=True)
        pos += 1
    return torch.stack(out, dim=1)
