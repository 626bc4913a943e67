"""Batch-invariant GEMM and attention for AMD MI355X (gfx950).

Python binding of libbi.so: argument marshalling only.  Every step of the
computation runs in the library's HIP kernels; PyTorch provides device
memory and the current stream.  There is no fallback: a call the library
cannot serve invariantly raises (mlx-batch-invariant README, section "Use":
unsupported cases raise NotImplementedError rather than silently falling
back).

Entry points (same names as the C ABI, plus the README's short names):
    bi_linear(x, w, bias=None)              y = x w^T + bias, w is (N, K)
    bi_matmul(a, b)                         y = a b, b is (K, N)
    bi_matmul_batched(a, b)                 y[z] = a[z] b[z], 3-D operands, one launch
    bi_addmm(c, a, b, alpha=1, beta=1)      y = alpha a b + beta c
    bi_sdpa(q, k, v, causal=False, mask=None, scale=None)
    bi_sdpa_noalloc(q, k, v, ...)           bi_sdpa with no workspace allocation (per-GPU scratch)
    bi_rowsum(x, mean=False)                row sum / mean over the last dim
    bi_variant_linear(x, w, bias=None, splits=None)   batch-VARIANT comparator
    bi_variant_sdpa(q, k, v, causal=False, mask=None)  batch-VARIANT attention comparator
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _native
from ._native import BI_BF16, BI_F16, BI_F32

__all__ = ["bi_linear", "bi_matmul", "bi_matmul_batched", "bi_addmm", "bi_sdpa", "bi_sdpa_noalloc", "bi_rowsum", "bi_variant_linear",
           "bi_variant_sdpa", "bi_quantized_linear", "quantize",
           "linear", "matmul", "addmm", "scaled_dot_product_attention",
           "abi_version", "library_path", "BiError"]

_DT = {torch.float32: BI_F32, torch.float16: BI_F16, torch.bfloat16: BI_BF16}


class BiError(RuntimeError):
    """The library reported a device error or a workspace problem."""


def library_path() -> str:
    return _native.LIB_PATH


def abi_version() -> int:
    return int(_native.load().bi_abi_version())


def _raise(status: int, fn: str):
    lib = _native.load()
    msg = (lib.bi_last_error() or b"").decode()
    name = lib.bi_status_name(status).decode()
    text = f"{fn}: {name}: {msg}"
    if status == _native.BI_ERR_UNSUPPORTED:
        raise NotImplementedError(text)
    if status == _native.BI_ERR_INVALID:
        raise ValueError(text)
    raise BiError(text)


def _check(status: int, fn: str):
    if status != _native.BI_OK:
        _raise(status, fn)


def _dt(t: torch.Tensor, what: str) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise NotImplementedError(f"{what}: dtype {t.dtype} is not supported") from None


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors are on different devices")
    return dev


def _rows(t: torch.Tensor) -> torch.Tensor:
    """View a (..., K) tensor as (M, K) with a unit inner stride (copies only if it must: exact)."""
    t2 = t.reshape(math.prod(t.shape[:-1]), t.shape[-1])
    if t2.stride(-1) != 1:
        t2 = t2.contiguous()
    return t2


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.dim() == 2 and t.shape[0] > 1 else max(t.shape[-1], 1)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _aligned_ld(t: torch.Tensor) -> torch.Tensor:
    """Row pitch must be a multiple of 16 bytes; compact copies satisfy that whenever K allows."""
    epc = 16 // t.element_size()
    if t.dim() == 2 and t.shape[0] > 1 and t.stride(0) % epc != 0:
        return t.contiguous()
    return t


def _kn_operand(b: torch.Tensor) -> torch.Tensor:
    """A (K, N) operand as given when one of its strides is 1 (row- or column-major), else a copy."""
    if b.dim() != 2:
        raise NotImplementedError("batched right operands are not supported")
    K, N = b.shape
    epc = 16 // b.element_size()
    if b.stride(1) == 1 and (K <= 1 or (b.stride(0) >= N and b.stride(0) % epc == 0)):
        return b
    if b.stride(0) == 1 and (N <= 1 or (b.stride(1) >= K and b.stride(1) % epc == 0)):
        return b
    return b.contiguous()


def bi_linear(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
              out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """y = x w^T + bias with w in the (N, K) nn.Linear layout; leading dims of x are batch."""
    dev = _on_gpu(x, w, bias)
    if x.dtype != w.dtype:
        raise ValueError("x and w must share a dtype")
    out_dtype = out_dtype or x.dtype
    lead = x.shape[:-1]
    x2 = _aligned_ld(_rows(x))
    w2 = _aligned_ld(_rows(w))
    M, K = x2.shape
    N = w2.shape[0]
    if w2.shape[1] != K:
        raise ValueError(f"inner dims differ: x has K={K}, w has K={w2.shape[1]}")
    b = None
    if bias is not None:
        if bias.shape != (N,) or bias.dtype != out_dtype:
            raise ValueError("bias must be (N,) in the output dtype")
        b = bias.contiguous()
    y = torch.empty((M, N), dtype=out_dtype, device=dev)
    lib = _native.load()
    st = lib.bi_linear(_ptr(x2), _ld(x2), _ptr(w2), _ld(w2), _ptr(b), _ptr(y), max(N, 1),
                       M, N, K, _dt(x2, "bi_linear"), _dt(y, "bi_linear"), _stream(dev))
    _check(st, "bi_linear")
    return y.reshape(*lead, N)


def bi_matmul(a: torch.Tensor, b: torch.Tensor, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """y = a b with b in the (K, N) layout; leading dims of a are batch."""
    dev = _on_gpu(a, b)
    if a.dtype != b.dtype:
        raise ValueError("a and b must share a dtype")
    if b.dim() != 2:
        raise NotImplementedError("bi_matmul: batched right operands are not supported")
    out_dtype = out_dtype or a.dtype
    lead = a.shape[:-1]
    a2 = _aligned_ld(_rows(a))
    b2 = _kn_operand(b)
    M, K = a2.shape
    if b2.shape[0] != K:
        raise ValueError("inner dims differ")
    N = b2.shape[1]
    y = torch.empty((M, N), dtype=out_dtype, device=dev)
    lib = _native.load()
    st = lib.bi_matmul(_ptr(a2), _ld(a2), _ptr(b2), b2.stride(0), b2.stride(1), _ptr(y), max(N, 1), M, N, K,
                       _dt(a2, "bi_matmul"), _dt(y, "bi_matmul"), _stream(dev))
    _check(st, "bi_matmul")
    return y.reshape(*lead, N)


def bi_matmul_batched(a: torch.Tensor, b: torch.Tensor, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """y[z] = a[z] b[z] for 3-D a (batch, M, K) and b (batch, K, N), one launch; every element has the bits
    bi_matmul(a[z], b[z]) gives."""
    dev = _on_gpu(a, b)
    if a.dtype != b.dtype:
        raise ValueError("a and b must share a dtype")
    if a.dim() != 3 or b.dim() != 3 or a.shape[0] != b.shape[0] or a.shape[2] != b.shape[1]:
        raise ValueError(f"bi_matmul_batched: shapes {tuple(a.shape)} and {tuple(b.shape)} do not match")
    out_dtype = out_dtype or a.dtype
    Z, M, K = a.shape
    N = b.shape[2]
    epc = 16 // a.element_size()
    # strides the kernels take as they are (a zero batch stride broadcasts one operand); else a copy
    if not (a.stride(2) == 1 and (M <= 1 or (a.stride(1) >= K and a.stride(1) % epc == 0))
            and a.stride(0) % epc == 0 and a.data_ptr() % 16 == 0):
        a = a.clone(memory_format=torch.contiguous_format)
    lda = a.stride(1) if M > 1 else max(K, 1)
    row_major = b.stride(2) == 1 and (K <= 1 or (b.stride(1) >= N and b.stride(1) % epc == 0))
    col_major = b.stride(1) == 1 and (N <= 1 or (b.stride(2) >= K and b.stride(2) % epc == 0))
    if not ((row_major or col_major) and b.stride(0) % epc == 0 and b.data_ptr() % 16 == 0):
        b = b.clone(memory_format=torch.contiguous_format)
    y = torch.empty((Z, M, N), dtype=out_dtype, device=dev)
    if Z == 0 or M == 0 or N == 0:
        return y
    lib = _native.load()
    st = lib.bi_matmul_batched(_ptr(a), lda, a.stride(0), _ptr(b), b.stride(1), b.stride(2), b.stride(0),
                               _ptr(y), max(N, 1), M * N, Z, M, N, K, _dt(a, "bi_matmul_batched"),
                               _dt(y, "bi_matmul_batched"), _stream(dev))
    _check(st, "bi_matmul_batched")
    return y


def bi_addmm(c: torch.Tensor | None, a: torch.Tensor, b: torch.Tensor, alpha: float = 1.0,
             beta: float = 1.0, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """alpha (a b) + beta c, b in (K, N); c is (M, N) or a broadcast (N,) row."""
    dev = _on_gpu(a, b, c)
    if a.dtype != b.dtype:
        raise ValueError("a and b must share a dtype")
    if a.dim() != 2 or b.dim() != 2:
        raise NotImplementedError("bi_addmm: 2-D operands only")
    out_dtype = out_dtype or a.dtype
    a2 = _aligned_ld(_rows(a))
    b2 = _kn_operand(b)
    M, K = a2.shape
    if b2.shape[0] != K:
        raise ValueError("inner dims differ")
    N = b2.shape[1]
    c2, ldc = None, 0
    if beta != 0.0:
        if c is None:
            raise ValueError("c is required when beta != 0")
        if c.dtype != out_dtype:
            raise ValueError("c must have the output dtype")
        if c.dim() == 1 or (c.dim() == 2 and c.shape[0] == 1 and M != 1):
            c2 = c.reshape(-1).contiguous()
            if c2.shape[0] != N:
                raise ValueError("broadcast c must have N elements")
            ldc = 0
        else:
            if tuple(c.shape) != (M, N):
                raise ValueError("c must be (M, N) or (N,)")
            c2 = c if c.stride(-1) == 1 else c.contiguous()
            ldc = c2.stride(0) if M > 1 else N
    y = torch.empty((M, N), dtype=out_dtype, device=dev)
    lib = _native.load()
    st = lib.bi_addmm(_ptr(c2), ldc, _ptr(a2), _ld(a2), _ptr(b2), b2.stride(0), b2.stride(1), _ptr(y),
                      max(N, 1), M, N, K,
                      float(alpha), float(beta), _dt(a2, "bi_addmm"), _dt(y, "bi_addmm"), _stream(dev))
    _check(st, "bi_addmm")
    return y


def sdpa_workspace_bytes(B: int, Hq: int, Hkv: int, Lq: int, S: int, D: int, dtype: torch.dtype) -> int:
    """Bytes of workspace bi_sdpa needs for these sizes and dtype (0 when the path taken needs none)."""
    return int(_native.load().bi_sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D, _DT[dtype]))


def _mask_strides(mask: torch.Tensor, shape) -> tuple:
    m = mask
    while m.dim() < 4:
        m = m.unsqueeze(0)
    st = []
    for d, want in enumerate(shape):
        if m.shape[d] == want:
            st.append(m.stride(d) if want > 1 else 0)
        elif m.shape[d] == 1:
            st.append(0)
        else:
            raise ValueError(f"mask dim {d} is {m.shape[d]}, expected 1 or {want}")
    return m, st


MASK_NONE, MASK_BOOL, MASK_ADD = 0, 1, 2


def bi_sdpa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
            mask: torch.Tensor | None = None, scale: float | None = None,
            workspace: torch.Tensor | None = None, sinks: torch.Tensor | None = None) -> torch.Tensor:
    """Softmax attention, q (B, Hq, Lq, D), k / v (B, Hkv, S, D), bottom-right causal.

    mask: boolean (True = attend) or additive in q's dtype (added to the scaled scores, -inf removes
    a key), broadcastable to (B, Hq, Lq, S).  sinks: None or Hq logits, one extra softmax term per
    query head that carries no value (bi.h, bi_sdpa_ex)."""
    return _sdpa(q, k, v, causal, mask, scale, workspace, sinks, noalloc=False)


def bi_sdpa_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                    mask: torch.Tensor | None = None, scale: float | None = None,
                    sinks: torch.Tensor | None = None) -> torch.Tensor:
    """bi_sdpa through bi_sdpa_ex_noalloc: no workspace is allocated; the library's per-GPU scratch array
    holds the split partials (bi.h: calls that overlap on one GPU race; sizes above
    bi_sdpa_scratch_limit() raise NotImplementedError).  The output tensor is still allocated here."""
    return _sdpa(q, k, v, causal, mask, scale, None, sinks, noalloc=True)


def _sdpa(q, k, v, causal, mask, scale, workspace, sinks, noalloc):
    dev = _on_gpu(q, k, v, mask)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be (B, Hq, Lq, D) and k, v (B, Hkv, S, D)")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, S, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("k / v batch or head dim differ from q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qs = q if q.stride(-1) == 1 else q.contiguous()
    ks = k if k.stride(-1) == 1 else k.contiguous()
    vs = v if v.stride(-1) == 1 else v.contiguous()
    o = torch.empty((B, Hq, Lq, D), dtype=q.dtype, device=dev)
    mptr, mstr, kind = None, None, MASK_NONE
    m8 = None
    if mask is not None:
        if mask.dtype in (torch.bool, torch.uint8):
            m8, st = _mask_strides(mask.to(torch.uint8) if mask.dtype == torch.bool else mask, (B, Hq, Lq, S))
            kind = MASK_BOOL
        elif mask.dtype == q.dtype:
            m8, st = _mask_strides(mask, (B, Hq, Lq, S))
            kind = MASK_ADD
        else:
            raise ValueError("an additive mask must have q's dtype (or use a boolean mask)")
        mptr, mstr = _ptr(m8), _native.i64x4(st)
    sk = None
    if sinks is not None:
        if torch.as_tensor(sinks).numel() != Hq:
            raise ValueError("sinks must hold one logit per query head")
        sk = torch.as_tensor(sinks).reshape(Hq).to(device=dev, dtype=torch.float32).contiguous()
    lib = _native.load()
    if noalloc:
        st = lib.bi_sdpa_ex_noalloc(_ptr(qs), _native.i64x4(qs.stride()), _ptr(ks), _native.i64x4(ks.stride()),
                                    _ptr(vs), _native.i64x4(vs.stride()), _ptr(o), _native.i64x4(o.stride()),
                                    B, Hq, Hkv, Lq, S, D, float(scale), 1 if causal else 0, kind, mptr, mstr,
                                    _ptr(sk), _dt(q, "bi_sdpa"), _stream(dev))
        _check(st, "bi_sdpa_ex_noalloc")
        return o
    need = int(lib.bi_sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D, _dt(q, "bi_sdpa")))
    ws = workspace
    if need > 0 and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib.bi_sdpa_ex(_ptr(qs), _native.i64x4(qs.stride()), _ptr(ks), _native.i64x4(ks.stride()),
                        _ptr(vs), _native.i64x4(vs.stride()), _ptr(o), _native.i64x4(o.stride()),
                        B, Hq, Hkv, Lq, S, D, float(scale), 1 if causal else 0, kind, mptr, mstr, _ptr(sk),
                        _dt(q, "bi_sdpa"), _ptr(ws) if ws is not None else None,
                        need if ws is not None else 0, _stream(dev))
    _check(st, "bi_sdpa_ex")
    return o


def bi_rowsum(x: torch.Tensor, mean: bool = False) -> torch.Tensor:
    """Sum (or mean) of x over its last dimension, in an order fixed by the row length alone."""
    dev = _on_gpu(x)
    lead = x.shape[:-1]
    N = x.shape[-1]
    x2 = _rows(x)
    M = x2.shape[0]
    y = torch.empty((M,), dtype=x.dtype, device=dev)
    lib = _native.load()
    st = lib.bi_rowsum(_ptr(x2), x2.stride(0) if M > 1 else max(N, 1), _ptr(y), M, N, 1 if mean else 0,
                       _dt(x2, "bi_rowsum"), _stream(dev))
    _check(st, "bi_rowsum")
    return y.reshape(lead)


def bi_variant_linear(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
                      splits: int | None = None, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """Batch-VARIANT comparator: bi_linear's kernels with M-keyed split-K (not invariant)."""
    dev = _on_gpu(x, w, bias)
    out_dtype = out_dtype or x.dtype
    x2 = _aligned_ld(_rows(x))
    w2 = _aligned_ld(_rows(w))
    M, K = x2.shape
    N = w2.shape[0]
    lib = _native.load()
    if splits is None:
        splits = int(lib.bi_variant_splits(M))
    b = bias.contiguous() if bias is not None else None
    y = torch.empty((M, N), dtype=out_dtype, device=dev)
    need = int(lib.bi_variant_workspace_bytes(M, N, splits))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.bi_variant_linear(_ptr(x2), _ld(x2), _ptr(w2), _ld(w2), _ptr(b), _ptr(y), max(N, 1),
                               M, N, K, _dt(x2, "bi_variant_linear"), _dt(y, "bi_variant_linear"),
                               int(splits), _ptr(ws), need, _stream(dev))
    _check(st, "bi_variant_linear")
    return y.reshape(*x.shape[:-1], N)


def bi_variant_sdpa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                    mask: torch.Tensor | None = None, scale: float | None = None) -> torch.Tensor:
    """Batch-VARIANT attention comparator (bi.h, bi_variant_sdpa): the split length follows the GQA factor
    times the query count and the cache length, so bits move with them.  Measurement only."""
    dev = _on_gpu(q, k, v, mask)
    B, Hq, Lq, D = q.shape
    _, Hkv, S, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qs = q if q.stride(-1) == 1 else q.contiguous()
    ks = k if k.stride(-1) == 1 else k.contiguous()
    vs = v if v.stride(-1) == 1 else v.contiguous()
    o = torch.empty((B, Hq, Lq, D), dtype=q.dtype, device=dev)
    mptr, mstr = None, None
    if mask is not None:
        if mask.dtype not in (torch.bool, torch.uint8):
            raise ValueError("bi_variant_sdpa takes a boolean mask")
        m8, st = _mask_strides(mask.to(torch.uint8) if mask.dtype == torch.bool else mask, (B, Hq, Lq, S))
        mptr, mstr = _ptr(m8), _native.i64x4(st)
    lib = _native.load()
    need = int(lib.bi_variant_sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.bi_variant_sdpa(_ptr(qs), _native.i64x4(qs.stride()), _ptr(ks), _native.i64x4(ks.stride()),
                             _ptr(vs), _native.i64x4(vs.stride()), _ptr(o), _native.i64x4(o.stride()),
                             B, Hq, Hkv, Lq, S, D, float(scale), 1 if causal else 0, mptr, mstr,
                             _dt(q, "bi_variant_sdpa"), _ptr(ws), need, _stream(dev))
    _check(st, "bi_variant_sdpa")
    return o


# README, section "Use": the short names.
linear = bi_linear
matmul = bi_matmul
addmm = bi_addmm


def quantize(w: torch.Tensor, bits: int = 4, group_size: int = 64):
    """Group-wise affine quantisation of an (N, K) weight (offline weight preparation in plain torch, not
    part of the kernel path): per group of group_size values along K, scale = (max - min) / (2^bits - 1)
    and bias = min, both rounded to w's dtype; q = round((w - bias) / scale) clamped to [0, 2^bits - 1].
    Returns (wq, scales, biases): wq is (N, K * bits / 32) int32 holding the packed uint32 words (32 / bits
    fields per word, lowest bits first), scales / biases are (N, K / group_size) in w's dtype."""
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    N, K = w.shape
    if K % group_size or K % 32:
        raise ValueError("K must be a multiple of group_size and of 32")
    g = w.float().reshape(N, K // group_size, group_size)
    lo, hi = g.amin(dim=-1), g.amax(dim=-1)
    levels = (1 << bits) - 1
    scale = ((hi - lo) / levels).clamp_min(1e-8).to(w.dtype)
    bias = lo.to(w.dtype)
    q = torch.round((g - bias.float()[..., None]) / scale.float()[..., None]).clamp_(0, levels).to(torch.int64)
    per = 32 // bits
    q = q.reshape(N, K // per, per)
    shifts = torch.arange(per, device=w.device, dtype=torch.int64) * bits
    words = (q << shifts).sum(dim=-1)                            # < 2^32
    words = torch.where(words >= 2**31, words - 2**32, words).to(torch.int32)
    return words.contiguous(), scale.contiguous(), bias.contiguous()


def bi_quantized_linear(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                        bits: int, group_size: int, bias: torch.Tensor | None = None) -> torch.Tensor:
    """y = x W^T + bias with W the group-wise affine dequantisation of wq (see `quantize` and bi.h):
    equal bit for bit to bi_linear(x, W, bias) with W[n, k] = round(fmaf(scale, q, bias_group))."""
    dev = _on_gpu(x, wq, scales, biases, bias)
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("x must be bf16 or fp16")
    if scales.dtype != x.dtype or biases.dtype != x.dtype:
        raise ValueError("scales / biases must share x's dtype")
    if wq.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise ValueError("wq must hold 32-bit words (int32 or uint32)")
    lead = x.shape[:-1]
    x2 = _aligned_ld(_rows(x))
    M, K = x2.shape
    N = wq.shape[0]
    w2 = wq.contiguous()
    s2, b2 = scales.contiguous(), biases.contiguous()
    if s2.shape != b2.shape or s2.shape[0] != N:
        raise ValueError("scales / biases must be (N, K / group_size)")
    bb = None
    if bias is not None:
        if bias.shape != (N,) or bias.dtype != x.dtype:
            raise ValueError("bias must be (N,) in x's dtype")
        bb = bias.contiguous()
    y = torch.empty((M, N), dtype=x.dtype, device=dev)
    lib = _native.load()
    dt = _dt(x2, "bi_quantized_linear")
    need = lib.bi_quantized_linear_workspace_bytes(M, N, K, dt)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None
    st = lib.bi_quantized_linear(_ptr(x2), _ld(x2), _ptr(w2), w2.shape[1], _ptr(s2), _ptr(b2), s2.shape[1],
                                 int(bits), int(group_size), _ptr(bb), _ptr(y), max(N, 1), M, N, K, dt,
                                 _ptr(ws), need, _stream(dev))
    _check(st, "bi_quantized_linear")
    return y.reshape(*lead, N)


def scaled_dot_product_attention(q, k, v, mask=None, scale=None, sinks=None):
    """README-style call: mask is None, "causal", a boolean tensor or an additive tensor; sinks
    optional (one logit per query head)."""
    if isinstance(mask, str):
        if mask != "causal":
            raise ValueError("mask must be None, 'causal' or a tensor")
        return bi_sdpa(q, k, v, causal=True, scale=scale, sinks=sinks)
    return bi_sdpa(q, k, v, causal=False, mask=mask, scale=scale, sinks=sinks)


# README, section "Use": route the framework's matmul and attention through these kernels.
from .mode import batch_invariant_mode  # noqa: E402

__all__ += ["batch_invariant_mode"]
