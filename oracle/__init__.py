"""CPU oracle for batch-invariant GEMM and attention (float64, plain C).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The library under
test never imports it, and it imports nothing from the library.

The definitions follow the mlx-batch-invariant README:
  * section "Use" -- linear(x, w, bias) with w in (N, K), matmul(a, b) with
    b in (K, N), addmm(c, a, b, alpha, beta) and
    scaled_dot_product_attention(q, k, v, mask="causal");
  * section "Accuracy" -- results are judged against a float64 reference;
  * section "Quantized models" -- 2, 4 and 8-bit group-wise affine weights
    (dequantize, quantized_linear).
Inputs may be torch tensors (any dtype, any device-less CPU tensor) or numpy
arrays; they are converted exactly to float64 before the C code sees them.
Outputs are unrounded float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


class use_library:
    """Context manager that points this module at another build of oracle.c.

    Used only by the tests that plant mistakes in a copy of the oracle to show
    that the pins catch them.
    """

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _bind(lib):
    d, i64, p = ctypes.c_double, ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm_f64.argtypes = [p, i64, p, i64, ctypes.c_int, p, i64, d, d, p, i64, i64, i64, i64]
    lib.oracle_gemm_f64.restype = None
    lib.oracle_sdpa_f64.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, d,
                                    ctypes.c_int, p, p, p, p, p]
    lib.oracle_sdpa_f64.restype = None
    lib.oracle_rowsum_f64.argtypes = [p, i64, i64, i64, ctypes.c_int, p]
    lib.oracle_rowsum_f64.restype = None
    lib.oracle_dequant_f64.argtypes = [p, i64, p, p, i64, ctypes.c_int, i64, i64, i64, p]
    lib.oracle_dequant_f64.restype = None
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    return lib


def threads() -> int:
    """Number of OpenMP threads the oracle will use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def _f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor / numpy array to C-contiguous float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def gemm(a, b, b_is_nk: bool, c=None, alpha: float = 1.0, beta: float = 1.0) -> np.ndarray:
    """alpha * (a @ B) + beta * c, with B = b.T when b_is_nk (b is (N, K)), else B = b (K, N).

    c may be None, a length-N row (broadcast over rows) or an (M, N) matrix.
    With beta == 0 c is not read.
    """
    A = _f64(a)
    Bm = _f64(b)
    M, K = A.shape
    if b_is_nk:
        N, Kb = Bm.shape
    else:
        Kb, N = Bm.shape
    if Kb != K:
        raise ValueError(f"inner dims differ: {K} vs {Kb}")
    out = np.empty((M, N), dtype=np.float64)
    cptr, ldc = None, 0
    Cm = None
    if c is not None and beta != 0.0:
        Cm = _f64(c)
        if Cm.ndim == 1:
            if Cm.shape[0] != N:
                raise ValueError("bias length must be N")
            ldc = 0
        else:
            if Cm.shape != (M, N):
                raise ValueError("C must be (M, N)")
            ldc = N
        cptr = _ptr(Cm)
    _load().oracle_gemm_f64(_ptr(A), K, _ptr(Bm), Bm.shape[1], 1 if b_is_nk else 0,
                            cptr, ldc, float(alpha), float(beta), _ptr(out), N, M, N, K)
    return out


def linear(x, w, bias=None) -> np.ndarray:
    """y = x @ w.T + bias, w in the (N, K) layout (README, section "Use")."""
    return gemm(x, w, True, bias, 1.0, 1.0)


def matmul(a, b) -> np.ndarray:
    """y = a @ b, b in the (K, N) layout (README, section "Use")."""
    return gemm(a, b, False, None, 1.0, 0.0)


def addmm(c, a, b, alpha: float = 1.0, beta: float = 1.0) -> np.ndarray:
    """alpha * (a @ b) + beta * c, b in (K, N) (README, section "Use")."""
    return gemm(a, b, False, c, alpha, beta)


def sdpa(q, k, v, causal: bool = False, mask=None, scale: float | None = None, sinks=None) -> np.ndarray:
    """Softmax attention over (B, Hq, Lq, D) queries and (B, Hkv, S, D) keys / values.

    Bottom-right causal alignment, query head h reads KV head floor(h*Hkv/Hq).
    mask is broadcastable to (B, Hq, Lq, S): boolean or integer (nonzero = attend), or floating
    point, added to the scaled scores (-inf removes a key) -- the README's mask forms (section
    "How the kernels work", attention paragraph).  sinks: None or Hq logits, one extra softmax
    term per query head that carries no value (section "Limitations").  scale defaults to 1/sqrt(D).
    """
    Q, Kt, V = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, D = Q.shape
    Bk, Hkv, S, Dk = Kt.shape
    if V.shape != Kt.shape or Bk != B or Dk != D:
        raise ValueError("k / v shapes do not match q")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    out = np.empty((B, Hq, Lq, D), dtype=np.float64)
    i64x4 = ctypes.c_int64 * 4

    def strides(a):
        return i64x4(*[s // a.itemsize for s in a.strides])

    def bcast(a, name):
        while a.ndim < 4:
            a = a[None]
        a = np.ascontiguousarray(a)
        st = []
        for dim, want in zip(range(4), (B, Hq, Lq, S)):
            if a.shape[dim] == want:
                st.append(a.strides[dim] // a.itemsize)
            elif a.shape[dim] == 1:
                st.append(0)
            else:
                raise ValueError(f"{name} dim {dim} is {a.shape[dim]}, expected 1 or {want}")
        return a, i64x4(*st)

    mptr, mstr = None, i64x4(0, 0, 0, 0)
    aptr, astr = None, i64x4(0, 0, 0, 0)
    M8 = A64 = None
    if mask is not None:
        if hasattr(mask, "detach"):
            mask = mask.detach().to("cpu")
            mask = mask.float().numpy() if mask.is_floating_point() else mask.numpy()
        mask = np.asarray(mask)
        if np.issubdtype(mask.dtype, np.floating):
            A64, astr = bcast(mask.astype(np.float64), "mask")
            aptr = _ptr(A64)
        else:
            M8, mstr = bcast(mask.astype(np.uint8), "mask")
            mptr = _ptr(M8)
    sptr, S64 = None, None
    if sinks is not None:
        S64 = np.ascontiguousarray(_f64(sinks).reshape(-1))
        if S64.shape != (Hq,):
            raise ValueError(f"sinks must hold Hq={Hq} values")
        sptr = _ptr(S64)
    _load().oracle_sdpa_f64(_ptr(Q), strides(Q), _ptr(Kt), strides(Kt), _ptr(V), strides(V),
                            _ptr(out), B, Hq, Hkv, Lq, S, D, float(scale), 1 if causal else 0,
                            mptr, mstr, aptr, astr, sptr)
    return out


def rowsum(x, mean: bool = False) -> np.ndarray:
    """Sum (or mean) of x over its last dimension, in float64 (README, section "Why MLX is not
    invariant": sum and mean among the ops a batch-invariant stack relies on)."""
    X = _f64(x)
    lead = X.shape[:-1]
    N = X.shape[-1]
    X2 = np.ascontiguousarray(X.reshape(int(np.prod(lead)), N))
    out = np.empty((X2.shape[0],), dtype=np.float64)
    if X2.shape[0] > 0:
        with np.errstate(invalid="ignore"):
            _load().oracle_rowsum_f64(_ptr(X2), N, X2.shape[0], N, 1 if mean else 0, _ptr(out))
    return out.reshape(lead)


def _u32(w) -> np.ndarray:
    """Packed weight words as C-contiguous uint32 (torch int32 / uint32 or numpy), bits unchanged."""
    if hasattr(w, "detach"):
        import torch
        w = w.detach().to("cpu")
        if w.dtype == torch.int32:
            w = w.numpy().view(np.uint32)
        else:
            w = w.numpy()
    return np.ascontiguousarray(np.asarray(w).astype(np.uint32, copy=False))


def dequantize(wq, scales, biases, bits: int, group_size: int, K: int | None = None) -> np.ndarray:
    """(N, K) float64 weights from group-wise affine quantisation (README, section "Quantized models"):
    w[n, k] = scale[n, k // group_size] * q[n, k] + bias[n, k // group_size], q the bits-wide field
    k mod (32 / bits) of word k // (32 / bits) of row n, lowest bits first.  Exact in float64."""
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    W = _u32(wq)
    Sc, Bi = _f64(scales), _f64(biases)
    N = W.shape[0]
    if K is None:
        K = W.shape[1] * (32 // bits)
    if Sc.shape != Bi.shape or Sc.shape[0] != N or Sc.shape[1] * group_size < K:
        raise ValueError("scales / biases must be (N, >= K / group_size)")
    out = np.empty((N, K), dtype=np.float64)
    if N and K:
        _load().oracle_dequant_f64(_ptr(W), W.shape[1], _ptr(Sc), _ptr(Bi), Sc.shape[1], int(bits),
                                   int(group_size), N, K, _ptr(out))
    return out


def quantized_linear(x, wq, scales, biases, bits: int, group_size: int, bias=None) -> np.ndarray:
    """y = x @ dequantize(w).T + bias in float64 (README, section "Quantized models": the quantized
    layer is a linear layer on the dequantised weight)."""
    X = _f64(x)
    Wd = dequantize(wq, scales, biases, bits, group_size, X.shape[1])
    return gemm(X, Wd, True, bias, 1.0, 1.0)

