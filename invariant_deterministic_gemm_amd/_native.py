"""ctypes view of libbi.so (the C ABI in include/bi.h).

Loading never falls back to anything: if the library is missing or does not
export a symbol, this raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbi.so")

BI_OK, BI_ERR_INVALID, BI_ERR_UNSUPPORTED, BI_ERR_WORKSPACE, BI_ERR_DEVICE = range(5)
BI_F32, BI_F16, BI_BF16 = 0, 1, 2

# name -> (restype, argtypes); mirrors include/bi.h
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_i64p = ctypes.POINTER(ctypes.c_int64)
SIGNATURES = {
    "bi_linear": (_i, [_p, _i64, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _i, _i, _p]),
    "bi_matmul": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _i, _i, _p]),
    "bi_matmul_batched": (_i, [_p, _i64, _i64, _p, _i64, _i64, _i64, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i, _i,
                               _p]),
    "bi_addmm": (_i, [_p, _i64, _p, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _f, _f, _i, _i, _p]),
    "bi_sdpa": (_i, [_p, _i64p, _p, _i64p, _p, _i64p, _p, _i64p, _i64, _i64, _i64, _i64, _i64, _i64,
                     _f, _i, _p, _i64p, _i, _p, _sz, _p]),
    "bi_sdpa_ex": (_i, [_p, _i64p, _p, _i64p, _p, _i64p, _p, _i64p, _i64, _i64, _i64, _i64, _i64, _i64,
                        _f, _i, _i, _p, _i64p, _p, _i, _p, _sz, _p]),
    "bi_sdpa_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64, _i]),
    "bi_sdpa_ex_noalloc": (_i, [_p, _i64p, _p, _i64p, _p, _i64p, _p, _i64p, _i64, _i64, _i64, _i64, _i64, _i64,
                                _f, _i, _i, _p, _i64p, _p, _i, _p]),
    "bi_sdpa_scratch_limit": (_sz, []),
    "bi_rowsum": (_i, [_p, _i64, _p, _i64, _i64, _i, _i, _p]),
    "bi_quantized_linear": (_i, [_p, _i64, _p, _i64, _p, _p, _i64, _i, _i64, _p, _p, _i64, _i64, _i64, _i64, _i,
                                 _p, _sz, _p]),
    "bi_quantized_linear_workspace_bytes": (_sz, [_i64, _i64, _i64, _i]),
    "bi_variant_linear": (_i, [_p, _i64, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _i, _i, _i, _p, _sz, _p]),
    "bi_variant_workspace_bytes": (_sz, [_i64, _i64, _i]),
    "bi_variant_splits": (_i, [_i64]),
    "bi_variant_sdpa": (_i, [_p, _i64p, _p, _i64p, _p, _i64p, _p, _i64p, _i64, _i64, _i64, _i64, _i64, _i64,
                             _f, _i, _p, _i64p, _i, _p, _sz, _p]),
    "bi_variant_sdpa_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "bi_variant_sdpa_split_len": (_i64, [_i64, _i64, _i64]),
    "bi_gemm_kernel_name": (ctypes.c_char_p, [_i64, _i64, _i64, _i, _i]),
    "bi_sdpa_kernel_name": (ctypes.c_char_p, [_i64, _i64, _i64, _i64, _i64, _i64, _i]),
    "bi_status_name": (ctypes.c_char_p, [_i]),
    "bi_last_error": (ctypes.c_char_p, []),
    "bi_abi_version": (_i, []),
    # include/bi_measure.h: measured ceilings for the benchmark
    "bi_measure_stream_read": (_i, [_p, _sz, _p, _i, _p]),
    "bi_measure_mfma": (ctypes.c_double, [_p, _i, _i, _p]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libbi.so and bind every exported entry point (raises if anything is missing)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libbi.so not found at {path}; build it with "
                          f"`python -m invariant_deterministic_gemm_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)          # AttributeError if the symbol is not exported
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def i64x4(vals):
    return (ctypes.c_int64 * 4)(*[int(v) for v in vals])
