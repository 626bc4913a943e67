"""Route PyTorch's matmul family and scaled-dot-product attention through the
batch-invariant kernels (mlx-batch-invariant README, section "Use": a context
that patches the framework's matmul and attention, strict by default).

    with batch_invariant_mode():          # strict: unsupported calls raise
        y = model(x)

    with batch_invariant_mode(strict=False) as m:
        y = model(x)                      # unsupported calls run stock PyTorch
    m.fallbacks                           # how many did, by function name

Intercepted at the Python API, for GPU tensors (while a mode is active the functions below are
replaced by thin wrappers; a wrapper hands the call to the innermost mode of the calling thread, and
with no mode active on that thread, or for calls made from inside a routed call, it calls PyTorch's
function unchanged; the originals come back when the last mode exits):
    torch.nn.functional.linear, torch.mm, torch.addmm, torch.matmul, torch.bmm,
    the Tensor methods mm / addmm / matmul / bmm and the @ operator,
    torch.nn.functional.scaled_dot_product_attention,
    torch.sum / torch.mean and the Tensor methods, when they reduce floating
    point tensors over the last dimension alone (full reductions and other
    dims are not row-wise and pass through).  On this GPU PyTorch's fp32
    last-dim sum and mean change their order with the number of rows, so
    they are routed too; softmax, log_softmax, layer_norm, rms_norm and max
    were measured invariant and are left alone.
Every routed call runs the library's kernels through the C ABI binding, so
results equal bi_linear / bi_matmul / bi_addmm / bi_sdpa / bi_rowsum bit for
bit and no row depends on the batch.  A batched matmul runs bi_matmul_batched (every element's bits
those of bi_matmul on it).
Calls whose tensors are all on the CPU are not the library's business and
pass through untouched in either mode.  Every call of these functions is routed, including calls
made inside other PyTorch Python functions (nn.Linear.forward, for example); calls made from C++
inside PyTorch, and references to the functions taken before the mode was entered, are not.

Not routed (raises NotImplementedError when strict; runs stock PyTorch and
is counted otherwise): dtypes other than fp32 / fp16 / bf16, mixed dtypes,
inputs that require gradients while grad mode is on (the kernels are
forward-only), out= arguments, matmul batch dims that do not broadcast, attention
with dropout, a float mask of another dtype than the query, head dims that
are not a multiple of 32 up to 256, a causal flag together with a mask, and
anything the library itself refuses
(for example K not a multiple of 8 for 16-bit inputs).  torch's is_causal
aligns the mask to the top-left corner; it is passed on as the library's
causal flag when the query and key lengths are equal (the two alignments
coincide) and as the equivalent boolean mask otherwise.
"""
from __future__ import annotations

import contextlib
import functools
import threading
from collections import Counter

import torch
import torch.nn.functional as F

from . import bi_addmm, bi_linear, bi_matmul, bi_matmul_batched, bi_rowsum, bi_sdpa

_SUPPORTED = (torch.float32, torch.float16, torch.bfloat16)


class Unsupported(Exception):
    """A call the invariant kernels cannot serve (raised inside the mode only)."""


class _NotOurs(Exception):
    """A call of a routed function that is not a row-wise operation (passed to torch, not counted)."""


def _need(cond: bool, why: str):
    if not cond:
        raise Unsupported(why)


def _check_tensors(*ts):
    dt = None
    for t in ts:
        if t is None:
            continue
        _need(isinstance(t, torch.Tensor), "non-tensor operand")
        _need(t.dtype in _SUPPORTED, f"dtype {t.dtype}")
        _need(not (torch.is_grad_enabled() and t.requires_grad), "operand requires grad (forward-only kernels)")
        dt = dt or t.dtype
        _need(t.dtype == dt, "mixed dtypes")


def plan_matmul(a_shape, b_shape) -> str:
    """How torch.matmul(a, b) maps onto the kernels, from the shapes alone:
    'mm'  a (..., K) x b (K, N): one GEMM over the flattened rows of a;
    'mv'  a (..., K) x b (K,); 'vm' a (K,) x b (K, N); 'dot' a (K,) x b (K,);
    'batched' a (*Ba, M, K) or (K,) x b (*Bb, K, N) with at least one batch dim in b: the batch dims
    broadcast (torch's rule) and one launch runs a GEMM per element.
    Raises Unsupported otherwise (scalars, batch dims that do not broadcast)."""
    da, db = len(a_shape), len(b_shape)
    if da == 0 or db == 0:
        raise Unsupported("scalar operand")
    if db == 1:
        return "mv" if da >= 2 else "dot"
    if db == 2:
        return "vm" if da == 1 else "mm"
    try:
        torch.broadcast_shapes(tuple(a_shape[:-2]), tuple(b_shape[:-2]))
    except RuntimeError:
        raise Unsupported(f"matmul of shapes {tuple(a_shape)} and {tuple(b_shape)} (batch dims do not broadcast)")
    return "batched"


def _matmul(input, other):
    a, b = input, other
    _check_tensors(a, b)
    kind = plan_matmul(tuple(a.shape), tuple(b.shape))
    if kind == "mm":
        return bi_matmul(a, b)
    if kind == "mv":
        return bi_linear(a, b.reshape(1, -1)).squeeze(-1)
    if kind == "vm":
        return bi_matmul(a.reshape(1, -1), b).squeeze(0)
    if kind == "dot":
        return bi_linear(a.reshape(1, -1), b.reshape(1, -1)).reshape(())
    vec = a.dim() == 1                    # (K,) x (*B, K, N): a one-row matrix, the row dim dropped after
    if vec:
        a = a.reshape(1, -1)
    lead = torch.broadcast_shapes(a.shape[:-2], b.shape[:-2])
    M, K, N = a.shape[-2], a.shape[-1], b.shape[-1]
    _need(b.shape[-2] == K, f"inner dims differ ({K} vs {b.shape[-2]})")
    # a broadcast operand keeps batch stride 0 where the batch dims merge; a copy otherwise (exact)
    a3 = a.expand(*lead, M, K).reshape(-1, M, K)
    b3 = b.expand(*lead, K, N).reshape(-1, K, N)
    y = bi_matmul_batched(a3, b3).reshape(*lead, M, N)
    return y.squeeze(-2) if vec else y


def _rmatmul(input, other):               # Tensor.__rmatmul__(self, other) computes other @ self
    return _matmul(other, input)


def _linear(input, weight, bias=None):
    _check_tensors(input, weight, bias)
    _need(weight.dim() == 2, "weight must be 2-D")
    _need(bias is None or bias.dim() == 1, "bias must be 1-D")
    return bi_linear(input, weight, bias)


def _mm(input, mat2):
    _check_tensors(input, mat2)
    _need(input.dim() == 2 and mat2.dim() == 2, "mm needs 2-D operands")
    return bi_matmul(input, mat2)


def _bmm(input, mat2):
    _need(input.dim() == 3 and mat2.dim() == 3, "bmm needs 3-D operands")
    return _matmul(input, mat2)


def _addmm(input, mat1, mat2, beta=1, alpha=1):
    _check_tensors(input, mat1, mat2)
    _need(mat1.dim() == 2 and mat2.dim() == 2, "addmm needs 2-D operands")
    M, N = mat1.shape[0], mat2.shape[1]
    c = input
    if c.dim() == 2 and tuple(c.shape) == (1, N) and M != 1:
        c = c.reshape(N)
    _need((c.dim() == 1 and c.shape[0] == N) or (c.dim() == 2 and tuple(c.shape) == (M, N)),
          f"addmm input of shape {tuple(input.shape)} does not broadcast the library's way")
    return bi_addmm(c, mat1, mat2, float(alpha), float(beta))


def _sdpa(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None, enable_gqa=False):
    q, k, v = query, key, value
    _check_tensors(q, k, v)
    _need(dropout_p == 0.0, "dropout")
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D")
    D = q.shape[-1]
    _need(D % 32 == 0 and 0 < D <= 256 and k.shape[-1] == D and v.shape[-1] == D, "head dim")
    Hq, Hkv = q.shape[1], k.shape[1]
    _need(Hq == Hkv or (enable_gqa and Hq % Hkv == 0), "query / key head counts")
    Lq, S = q.shape[2], k.shape[2]
    if attn_mask is not None:
        _need(not is_causal, "causal flag together with a mask")
        # torch adds a float mask to the scaled scores, as the library's additive form does
        _need(attn_mask.dtype == torch.bool or attn_mask.dtype == q.dtype, "mask of another dtype than q")
        return bi_sdpa(q, k, v, mask=attn_mask, scale=scale)
    if is_causal:
        if Lq == S:
            return bi_sdpa(q, k, v, causal=True, scale=scale)
        # torch aligns is_causal to the top-left corner: query i sees keys 0 .. i
        top_left = torch.ones(Lq, S, dtype=torch.bool, device=q.device).tril()
        return bi_sdpa(q, k, v, mask=top_left, scale=scale)
    return bi_sdpa(q, k, v, scale=scale)


def _last_dim_only(x, dim) -> bool:
    if isinstance(dim, (list, tuple)):
        if len(dim) != 1:
            return False
        dim = dim[0]
    return isinstance(dim, int) and x.dim() > 0 and dim in (-1, x.dim() - 1)


def _reduce(input, dim=None, keepdim=False, dtype=None, mean=False):
    # only a reduction over the last dimension alone is row-wise; anything else is not the mode's
    if not (isinstance(input, torch.Tensor) and input.is_floating_point() and dim is not None
            and _last_dim_only(input, dim)):
        raise _NotOurs
    _need(dtype is None or dtype == input.dtype, "dtype= conversion")
    _check_tensors(input)
    y = bi_rowsum(input, mean=mean)
    return y.unsqueeze(-1) if keepdim else y


def _sum(input, dim=None, keepdim=False, dtype=None):
    return _reduce(input, dim, keepdim, dtype, mean=False)


def _mean(input, dim=None, keepdim=False, dtype=None):
    return _reduce(input, dim, keepdim, dtype, mean=True)


# torch function -> (handler, names of torch's parameters in order); handlers use the same names
_ROUTES = {
    F.linear: (_linear, ("input", "weight", "bias")),
    torch.mm: (_mm, ("input", "mat2")),
    torch.Tensor.mm: (_mm, ("input", "mat2")),
    torch.addmm: (_addmm, ("input", "mat1", "mat2", "beta", "alpha")),
    torch.Tensor.addmm: (_addmm, ("input", "mat1", "mat2", "beta", "alpha")),
    torch.matmul: (_matmul, ("input", "other")),
    torch.Tensor.matmul: (_matmul, ("input", "other")),
    torch.Tensor.__matmul__: (_matmul, ("input", "other")),
    torch.Tensor.__rmatmul__: (_rmatmul, ("input", "other")),
    torch.bmm: (_bmm, ("input", "mat2")),
    torch.Tensor.bmm: (_bmm, ("input", "mat2")),
    F.scaled_dot_product_attention: (_sdpa, ("query", "key", "value", "attn_mask", "dropout_p", "is_causal",
                                             "scale", "enable_gqa")),
    torch.sum: (_sum, ("input", "dim", "keepdim", "dtype")),
    torch.Tensor.sum: (_sum, ("input", "dim", "keepdim", "dtype")),
    torch.mean: (_mean, ("input", "dim", "keepdim", "dtype")),
    torch.Tensor.mean: (_mean, ("input", "dim", "keepdim", "dtype")),
}


def routed_functions():
    """Names of the torch functions the mode intercepts."""
    return sorted({getattr(f, "__name__", str(f)) for f in _ROUTES})


def _call(route, args, kwargs):
    fn, names = route
    _need("out" not in kwargs, "out= argument")
    _need(len(args) <= len(names), "too many arguments")
    kw = dict(zip(names, args))
    for k, v in kwargs.items():
        _need(k in names and k not in kw, f"argument {k}")
        kw[k] = v
    return fn(**kw)


def _tensors_in(args, kwargs):
    for x in list(args) + list(kwargs.values()):
        if isinstance(x, torch.Tensor):
            yield x


# (owner, attribute) of every routed function; the wrappers replace these attributes while any mode is
# active in any thread
_TARGETS = ((F, "linear"), (torch, "mm"), (torch.Tensor, "mm"), (torch, "addmm"), (torch.Tensor, "addmm"),
            (torch, "matmul"), (torch.Tensor, "matmul"), (torch.Tensor, "__matmul__"),
            (torch.Tensor, "__rmatmul__"), (torch, "bmm"), (torch.Tensor, "bmm"),
            (F, "scaled_dot_product_attention"), (torch, "sum"), (torch.Tensor, "sum"), (torch, "mean"),
            (torch.Tensor, "mean"))
# the route of each target, looked up once on the functions PyTorch defines
_TARGET_ROUTES = tuple((owner, name, _ROUTES[getattr(owner, name)], getattr(getattr(owner, name), "__name__", name))
                       for owner, name in _TARGETS)
_tls = threading.local()               # .stack: this thread's active modes; .busy: inside a routed call
_lock = threading.Lock()
_active_count = 0                      # modes active over all threads
_saved = []                            # (owner, name, original, owner held it in its own __dict__)


def _wrapper(orig, route, name):
    @functools.wraps(orig)
    def call(*args, **kwargs):
        stack = getattr(_tls, "stack", None)
        if not stack or getattr(_tls, "busy", False):
            return orig(*args, **kwargs)
        return stack[-1]._dispatch(orig, route, name, args, kwargs)
    return call


def _install():
    try:
        for owner, name, route, fname in _TARGET_ROUTES:
            orig = getattr(owner, name)
            _saved.append((owner, name, orig, name in vars(owner)))
            setattr(owner, name, _wrapper(orig, route, fname))
    except BaseException:
        _uninstall()
        raise


def _uninstall():
    while _saved:
        owner, name, orig, own = _saved.pop()
        if own:
            setattr(owner, name, orig)
        else:
            delattr(owner, name)       # the attribute is inherited again (Tensor methods of the C base)


class _InvariantMode:
    def __init__(self, strict: bool):
        self.strict = strict
        self.fallbacks = Counter()
        self.routed = Counter()

    def __enter__(self):
        global _active_count
        with _lock:
            if _active_count == 0:
                _install()
            _active_count += 1
        if getattr(_tls, "stack", None) is None:
            _tls.stack = []
        _tls.stack.append(self)
        return self

    def __exit__(self, *exc):
        global _active_count
        _tls.stack.remove(self)
        with _lock:
            _active_count -= 1
            if _active_count == 0:
                _uninstall()
        return False

    def _dispatch(self, orig, route, name, args, kwargs):
        if not any(t.is_cuda for t in _tensors_in(args, kwargs)):
            return orig(*args, **kwargs)
        _tls.busy = True
        try:
            try:
                out = _call(route, args, kwargs)
            except _NotOurs:
                return orig(*args, **kwargs)
            except (Unsupported, NotImplementedError) as e:
                if self.strict:
                    raise NotImplementedError(f"batch_invariant_mode: {name}: {e}") from None
                self.fallbacks[name] += 1
                return orig(*args, **kwargs)
        finally:
            _tls.busy = False
        self.routed[name] += 1
        return out


@contextlib.contextmanager
def batch_invariant_mode(strict: bool = True):
    """Route torch matmuls and attention on GPU tensors through the batch-invariant kernels.

    strict=True: a call the kernels cannot serve raises NotImplementedError, so nothing silently
    runs a batch-variant kernel.  strict=False: such calls run stock PyTorch and are counted in the
    yielded object's `fallbacks`; routed calls are counted in `routed`."""
    mode = _InvariantMode(strict)
    with mode:
        yield mode


__all__ = ["batch_invariant_mode", "plan_matmul", "routed_functions", "Unsupported"]
