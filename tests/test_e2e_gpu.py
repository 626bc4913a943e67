"""End-to-end batch invariance of a small random-weight decoder under batch_invariant_mode.

A sequence decoded on its own and the same sequence decoded inside batches of
other sequences must produce bit-identical logits at every step (the README's
headline check, section "What batch-invariant means here": logits differing
from batch 1, 0 of 32000).  Stock PyTorch on the same model is the negative
control: its logits move with the batch.  Accuracy: the mode's logits stay
close to stock PyTorch's on the same inputs, and within the oracle gate of the
same decoder composed from the float64 oracle (prefill and teacher-forced
decode steps)."""
import os
import sys

import pytest
import torch

import invariant_deterministic_gemm_amd as bi
import synthetic

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import tiny_transformer as tt  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def model():
    cfg = tt.TinyConfig(layers=2)
    return cfg, tt.make_weights(cfg, 0x5EEDE2, DEV)


def _prompts(cfg, B, L, seed):
    return synthetic.randint((B, L), seed, 0, cfg.vocab, torch.int64).to(DEV)


def test_logits_do_not_depend_on_the_batch(model):
    cfg, W = model
    prompts = _prompts(cfg, 8, 37, 0x5EEDE3)
    with torch.no_grad(), bi.batch_invariant_mode() as m:
        full = tt.greedy_decode(cfg, W, prompts, steps=12)            # (8, 13, vocab)
        for b in (0, 3, 7):
            one = tt.greedy_decode(cfg, W, prompts[b:b + 1], steps=12)
            n = int((one[0].view(torch.int16) != full[b].view(torch.int16)).sum())
            assert n == 0, f"sequence {b}: {n} of {one.numel()} logits differ from its batch-of-8 run"
        three = tt.greedy_decode(cfg, W, prompts[2:5], steps=12)
        assert torch.equal(three.view(torch.int16), full[2:5].view(torch.int16)), "batch of 3 vs batch of 8"
    assert not m.fallbacks and m.routed["linear"] > 0 and m.routed["scaled_dot_product_attention"] > 0


def test_stock_pytorch_is_the_negative_control(model):
    cfg, W = model
    prompts = _prompts(cfg, 8, 37, 0x5EEDE3)
    with torch.no_grad():
        full = tt.forward(cfg, W, prompts, None, 0)[0][:, -1]
        one = tt.forward(cfg, W, prompts[:1], None, 0)[0][:, -1]
    n = int((one[0].view(torch.int16) != full[0].view(torch.int16)).sum())
    print(f"stock PyTorch: {n} of {cfg.vocab} last-position logits of sequence 0 differ between batch 1 and 8")
    assert n > 0, "stock PyTorch happened to be batch invariant here; the control shows nothing"


def test_mode_logits_close_to_stock(model):
    cfg, W = model
    prompts = _prompts(cfg, 4, 64, 0x5EEDE4)
    with torch.no_grad():
        ref = tt.forward(cfg, W, prompts, None, 0)[0].float()
        with bi.batch_invariant_mode():
            got = tt.forward(cfg, W, prompts, None, 0)[0].float()
    rel = float((got - ref).abs().max() / ref.abs().max())
    assert rel < 3e-2, f"logits relative difference {rel:.3e}"


# ---------------------------------------------------------------- the decoder against a float64 oracle
def _bf16(a):
    """Round a float64 array to bf16 (round to nearest even) and return it as float64 again: the model keeps
    every activation in bf16, so the oracle composition rounds at the same points."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).double().numpy()


def _oracle_forward(cfg, Wc, tokens, cache, start):
    """tiny_transformer.forward in float64 on the CPU: oracle.linear and oracle.sdpa for the routed ops,
    RMSNorm, rotary embedding, SiLU and the residual adds written out here, activations rounded to bf16
    where the model stores them."""
    import numpy as np
    import oracle
    B, L = tokens.shape
    H, Hk, D = cfg.heads, cfg.kv_heads, cfg.head_dim

    def rms(x, w):
        return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + cfg.eps) * w.double().numpy()

    def lin(x, w):
        return _bf16(oracle.linear(x.reshape(-1, x.shape[-1]), w)).reshape(*x.shape[:-1], w.shape[0])

    pos = np.arange(start, start + L, dtype=np.float64)
    inv = 1.0 / (cfg.rope_theta ** (np.arange(0, D, 2, dtype=np.float64) / D))
    ang = pos[:, None] * inv[None, :]
    cos, sin = np.cos(ang), np.sin(ang)

    def rope(x):
        x1, x2 = x[..., 0::2], x[..., 1::2]
        return _bf16(np.stack((x1 * cos - x2 * sin, x1 * sin + x2 * cos), axis=-1).reshape(x.shape))

    x = Wc["embed"][tokens].double().numpy()
    new_cache = []
    for li, lw in enumerate(Wc["layers"]):
        h = _bf16(rms(x, lw["ln1"]))
        q = rope(lin(h, lw["wq"]).reshape(B, L, H, D).transpose(0, 2, 1, 3))
        k = rope(lin(h, lw["wk"]).reshape(B, L, Hk, D).transpose(0, 2, 1, 3))
        v = lin(h, lw["wv"]).reshape(B, L, Hk, D).transpose(0, 2, 1, 3)
        if cache is not None:
            k = np.concatenate((cache[li][0], k), axis=2)
            v = np.concatenate((cache[li][1], v), axis=2)
        new_cache.append((k, v))
        a = _bf16(oracle.sdpa(q, k, v, causal=cache is None, scale=1.0 / np.sqrt(D)))
        x = _bf16(x + lin(a.transpose(0, 2, 1, 3).reshape(B, L, H * D), lw["wo"]))
        h = _bf16(rms(x, lw["ln2"]))
        g = lin(h, lw["wg"])
        u = lin(h, lw["wu"])
        x = _bf16(x + lin(_bf16(_bf16(g / (1.0 + np.exp(-g))) * u), lw["wd"]))
    x = _bf16(rms(x, Wc["norm"]))
    logits = oracle.linear(x.reshape(B * L, -1), Wc["lm_head"]).reshape(B, L, -1)
    return logits, new_cache


def test_mode_logits_match_float64_oracle_composition(model):
    """Prefill of 12 tokens and 3 teacher-forced decode steps of the decoder under batch_invariant_mode
    against the same decoder composed from the float64 oracle (linear, attention) and float64 RMSNorm,
    rotary embedding and SwiGLU: every step's logits within the 2e-2 gate."""
    from helpers import assert_close_to_oracle
    cfg, W = model
    Wc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in W.items() if k != "layers"}
    Wc["layers"] = [{k: v.cpu() for k, v in lw.items()} for lw in W["layers"]]
    prompts = _prompts(cfg, 2, 12, 0x5EEDE8)
    steps = _prompts(cfg, 2, 3, 0x5EEDE9)
    with torch.no_grad(), bi.batch_invariant_mode():
        logits, cache = tt.forward(cfg, W, prompts, None, 0)
        ref, rcache = _oracle_forward(cfg, Wc, prompts.cpu(), None, 0)
        assert_close_to_oracle(logits.cpu(), ref, "prefill logits")
        for s in range(3):
            tok = steps[:, s:s + 1]
            logits, cache = tt.forward(cfg, W, tok, cache, 12 + s)
            ref, rcache = _oracle_forward(cfg, Wc, tok.cpu(), rcache, 12 + s)
            assert_close_to_oracle(logits.cpu(), ref, f"decode step {s} logits")
