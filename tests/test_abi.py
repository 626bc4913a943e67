"""C-ABI checks that need no GPU: the library loads, exports every function
the headers under include/ declare, and rejects malformed or unsupported
arguments on the host before touching the device (no compute call is made
here)."""
import ctypes
import glob
import os
import re

import pytest

from invariant_deterministic_gemm_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

F32, F16, BF16 = _native.BI_F32, _native.BI_F16, _native.BI_BF16
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3

# Fake, never-dereferenced device addresses: validation must reject the call
# before any of them is used.
P16 = ctypes.c_void_p(0x7f0000000000)
P16b = ctypes.c_void_p(0x7f0000100000)
P_MIS = ctypes.c_void_p(0x7f0000000002)


@pytest.fixture(scope="module")
def lib():
    return _native.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(bi_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_headers_found():
    assert any(h.endswith("bi.h") for h in HEADERS) and any(h.endswith("bi_measure.h") for h in HEADERS)


def test_header_declares_what_the_binding_binds():
    assert declared_functions() == sorted(_native.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_exported_symbols_with_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _native.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (bi_\w+)", out))
    assert set(declared_functions()) <= exported


def test_sdpa_noalloc_host_checks(lib):
    # sizes whose partials exceed the scratch limit are refused on the host, before any device call
    lim = lib.bi_sdpa_scratch_limit()
    assert lim == 64 * 2 ** 20
    st4 = (ctypes.c_int64 * 4)(32 * 1 * 128, 1 * 128, 128, 1)
    kv4 = (ctypes.c_int64 * 4)(8 * 65536 * 128, 65536 * 128, 128, 1)
    need = lib.bi_sdpa_workspace_bytes(64, 32, 8, 1, 65536, 128, BF16)
    assert need > lim
    s = lib.bi_sdpa_ex_noalloc(P16, st4, P16b, kv4, P16b, kv4, P16, st4, 64, 32, 8, 1, 65536, 128, 0.088, 1,
                               0, None, None, None, BF16, None)
    assert s == UNSUPPORTED and b"scratch" in lib.bi_last_error()
    # malformed arguments that need no scratch are refused as by bi_sdpa_ex
    s = lib.bi_sdpa_ex_noalloc(P16, st4, P16b, kv4, P16b, kv4, P16, st4, 1, 30, 8, 1, 64, 128, 0.088, 1,
                               0, None, None, None, BF16, None)
    assert s == INVALID


def test_measure_validation(lib):
    # bad arguments are refused on the host, before any launch
    assert lib.bi_measure_stream_read(None, 1024, P16, 4, None) == 1
    assert lib.bi_measure_stream_read(P16, 1000, P16b, 4, None) == 1
    assert lib.bi_measure_stream_read(P_MIS, 1024, P16b, 4, None) == 1
    assert lib.bi_measure_stream_read(P16, 1024, P16b, 0, None) == 1
    assert lib.bi_measure_mfma(None, 4, 10, None) < 0
    assert lib.bi_measure_mfma(P16, 0, 10, None) < 0
    assert lib.bi_measure_mfma(P16, 4, 0, None) < 0


def test_abi_version_and_status_names(lib):
    v = lib.bi_abi_version()
    assert v >> 16 == 2 and (v & 0xffff) >= 1
    names = [lib.bi_status_name(s).decode() for s in range(5)]
    assert names == ["BI_OK", "BI_ERR_INVALID", "BI_ERR_UNSUPPORTED", "BI_ERR_WORKSPACE", "BI_ERR_DEVICE"]
    assert lib.bi_status_name(99).decode() == "BI_UNKNOWN_STATUS"


def linear(lib, M=4, N=32, K=64, ind=BF16, outd=BF16, x=P16, w=P16b, ldx=None, ldw=None, ldy=None, bias=None):
    return lib.bi_linear(x, K if ldx is None else ldx, w, K if ldw is None else ldw, bias, P16,
                         N if ldy is None else ldy, M, N, K, ind, outd, None)


def test_gemm_validation(lib):
    assert linear(lib, ind=F32, outd=BF16) == UNSUPPORTED
    assert linear(lib, ind=BF16, outd=F16) == UNSUPPORTED
    assert "not supported" in lib.bi_last_error().decode()
    assert linear(lib, ind=7) == INVALID
    assert linear(lib, M=-1) == INVALID
    assert linear(lib, K=60) == UNSUPPORTED          # K % 8 for 16-bit inputs
    assert linear(lib, x=P_MIS) == UNSUPPORTED
    assert linear(lib, ldx=63) == INVALID
    assert linear(lib, ldx=68) == UNSUPPORTED        # row pitch not a multiple of 16 bytes
    assert linear(lib, ldy=16) == INVALID
    assert linear(lib, x=None) == INVALID
    # empty problems succeed without doing anything
    assert linear(lib, M=0) == OK
    assert linear(lib, N=0) == OK
    assert lib.bi_last_error().decode() == ""


def test_matmul_batched_validation(lib):
    # every call fails validation or is empty, so nothing is launched on the placeholder pointers
    def bat(batch=2, sa=4096, sb=4096, sc=2048, b_k=32, b_n=1, M=64, N=32, K=64, ind=BF16, outd=BF16, c=P16):
        return lib.bi_matmul_batched(P16, 64, sa, P16b, b_k, b_n, sb, c, 32, sc, batch, M, N, K, ind, outd, None)
    assert bat(batch=-1) == INVALID
    assert bat(batch=1 << 31) == UNSUPPORTED
    assert bat(sa=-8) == INVALID
    assert bat(sc=-32) == INVALID
    assert bat(sc=2047) == INVALID                   # element z's last row overlaps element z+1's first
    assert bat(sa=4100) == UNSUPPORTED                # 16-bit batch strides: multiples of 8 elements
    assert bat(sb=12) == UNSUPPORTED
    assert bat(b_k=2, b_n=128) == UNSUPPORTED         # no unit stride in b
    assert bat(c=None) == INVALID
    assert bat(ind=F32, outd=BF16) == UNSUPPORTED
    # empty problems succeed without a launch
    assert bat(batch=0) == OK
    assert bat(M=0) == OK
    assert bat(N=0, b_k=0) == OK
    assert lib.bi_last_error().decode() == ""


def test_matmul_addmm_validation(lib):
    # row-major (K, N) operand: N must be a multiple of 8 for 16-bit inputs
    assert lib.bi_matmul(P16, 64, P16b, 36, 1, P16, 36, 4, 36, 64, BF16, BF16, None) == UNSUPPORTED
    assert lib.bi_matmul(P16, 64, P16b, 16, 1, P16, 32, 4, 32, 64, BF16, BF16, None) == INVALID  # rows overlap
    assert lib.bi_matmul(P16, 64, P16b, 1, 32, P16, 32, 4, 32, 64, BF16, BF16, None) == INVALID  # cols overlap
    assert lib.bi_matmul(P16, 64, P16b, 2, 128, P16, 32, 4, 32, 64, BF16, BF16, None) == UNSUPPORTED
    assert lib.bi_matmul(P16, 64, P16b, 1, 68, P16, 32, 4, 32, 64, BF16, BF16, None) == UNSUPPORTED  # pitch
    # beta != 0 needs cin; ldcin must be 0 or >= N
    assert lib.bi_addmm(None, 0, P16, 64, P16b, 32, 1, P16, 32, 4, 32, 64, 1.0, 1.0, BF16, BF16, None) == INVALID
    assert lib.bi_addmm(P16, 8, P16, 64, P16b, 32, 1, P16, 32, 4, 32, 64, 1.0, 1.0, BF16, BF16, None) == INVALID
    assert lib.bi_addmm(P16, 0, P16, 64, P16b, 32, 1, P16, 32, 4, 32, 64, float("nan"), 1.0, BF16, BF16,
                        None) == INVALID
    assert lib.bi_addmm(None, 0, P16, 64, P16b, 32, 1, P16, 32, 0, 32, 64, 1.0, 1.0, BF16, BF16, None) == OK


def strides(shape):
    s = [1] * 4
    for d in (2, 1, 0):
        s[d] = s[d + 1] * shape[d + 1]
    return _native.i64x4(s)


def sdpa(lib, B=1, Hq=4, Hkv=2, Lq=1, S=16, D=128, dt=BF16, causal=1, ws=P16, wsb=1 << 30, qstr=None,
         scale=0.088):
    qs = qstr or strides((B, Hq, Lq, D))
    kv = strides((B, Hkv, S, D))
    return lib.bi_sdpa(P16, qs, P16b, kv, P16b, kv, P16, strides((B, Hq, Lq, D)), B, Hq, Hkv, Lq, S, D,
                       scale, causal, None, None, dt, ws, wsb, None)


def test_sdpa_validation(lib):
    assert sdpa(lib, Hq=6, Hkv=4) == INVALID
    assert sdpa(lib, Hkv=0) == INVALID
    assert sdpa(lib, D=48) == UNSUPPORTED               # head dims: multiples of 32 up to 256
    assert sdpa(lib, D=288) == UNSUPPORTED
    assert sdpa(lib, D=0) == INVALID
    for D in (32, 96, 160, 256):                          # accepted: fp32 stops at the missing workspace
        assert sdpa(lib, D=D, ws=None, dt=F32) == WORKSPACE, D
    assert sdpa(lib, Lq=17, S=16, causal=1) == INVALID  # causal needs Lq <= S
    assert sdpa(lib, dt=9) == INVALID
    assert sdpa(lib, scale=float("inf")) == INVALID
    # fp32 runs the split path, which needs a workspace
    assert sdpa(lib, dt=F32, ws=None) == WORKSPACE
    need = lib.bi_sdpa_workspace_bytes(1, 4, 2, 1, 16, 128, F32)
    assert need > 0
    assert sdpa(lib, dt=F32, wsb=need - 4) == WORKSPACE
    assert sdpa(lib, dt=F32, ws=ctypes.c_void_p(0x7f0000000010)) == UNSUPPORTED   # workspace 256-byte aligned
    bad = strides((1, 4, 1, 128))
    bad[3] = 2
    assert sdpa(lib, qstr=bad) == UNSUPPORTED
    bad = strides((1, 4, 1, 128))
    bad[2] = 100                                          # not a multiple of 8 elements
    assert sdpa(lib, qstr=bad) == UNSUPPORTED
    assert sdpa(lib, B=0) == OK
    assert sdpa(lib, Lq=0) == OK


def sdpa_ex(lib, kind=0, mask=None, mstr=None, sinks=None, dt=BF16, ws=None, D=64):
    B, Hq, Hkv, Lq, S = 1, 4, 2, 1, 16
    qs, kv = strides((B, Hq, Lq, D)), strides((B, Hkv, S, D))
    return lib.bi_sdpa_ex(P16, qs, P16b, kv, P16b, kv, P16, strides((B, Hq, Lq, D)), B, Hq, Hkv, Lq, S, D,
                          0.125, 1, kind, mask, mstr, sinks, dt, ws, 0, None)


def test_sdpa_ex_validation(lib):
    m4 = strides((1, 1, 1, 16))
    assert sdpa_ex(lib, kind=3, mask=P16, mstr=m4) == INVALID                   # unknown mask kind
    assert sdpa_ex(lib, kind=1, mask=None, mstr=m4) == INVALID                  # kind without a mask
    assert sdpa_ex(lib, kind=2, mask=ctypes.c_void_p(0x7f0000000001), mstr=m4) == UNSUPPORTED   # bf16 alignment
    assert sdpa_ex(lib, sinks=ctypes.c_void_p(0x7f0000000002)) == UNSUPPORTED  # fp32 sinks alignment
    neg = strides((1, 1, 1, 16))
    neg[3] = -1
    assert sdpa_ex(lib, kind=2, mask=P16, mstr=neg) == INVALID
    # every form accepted together: fp32 always runs the split path, so each call stops at the missing
    # workspace, after every other check and before anything is launched
    assert sdpa_ex(lib, kind=2, mask=P16, mstr=m4, sinks=P16b, dt=F32) == WORKSPACE
    assert sdpa_ex(lib, kind=1, mask=P16, mstr=m4, sinks=P16b, dt=F32) == WORKSPACE
    assert sdpa_ex(lib, kind=0, mask=ctypes.c_void_p(0x7f0000000001), mstr=None, dt=F32) == WORKSPACE  # ignored


def test_sdpa_workspace_formula(lib):
    # split and quad paths: (rows * nsplit * 2 floats, padded to 256 B) + rows * nsplit * D floats
    def split_bytes(B, Hq, Lq, S, D):
        rows, nsplit = B * Hq * Lq, (S + 255) // 256
        return (rows * nsplit * 8 + 255) // 256 * 256 + rows * nsplit * D * 4
    ws = lib.bi_sdpa_workspace_bytes
    assert ws(2, 32, 8, 3, 1000, 128, F32) == split_bytes(2, 32, 3, 1000, 128)
    assert ws(2, 32, 8, 3, 2000, 64, BF16) == split_bytes(2, 32, 3, 2000, 64)     # quad, as D = 128
    assert ws(2, 32, 8, 3, 1000, 160, BF16) == split_bytes(2, 32, 3, 1000, 160)
    assert ws(2, 32, 8, 3, 2000, 128, F16) == split_bytes(2, 32, 3, 2000, 128)
    # 16-bit D <= 128: the quad grid (splits x row tiles x B x Hkv) decides between the quad kernel
    # (<= 256 workgroups, workspace) and the one-launch kernel (S <= 1024, none) or the split kernel
    assert ws(8, 32, 8, 1, 1024, 128, BF16) == split_bytes(8, 32, 1, 1024, 128)    # 4 x 1 x 8 x 8 = 256
    assert ws(9, 32, 8, 1, 1024, 128, BF16) == 0                                   # 288: one launch
    assert ws(2, 32, 8, 3, 1000, 64, BF16) == split_bytes(2, 32, 3, 1000, 64)
    assert ws(16, 32, 8, 3, 1000, 64, BF16) == 0
    assert ws(16, 32, 8, 3, 1024, 128, BF16) == 0
    assert ws(16, 32, 8, 3, 1025, 128, BF16) == split_bytes(16, 32, 3, 1025, 128)
    assert ws(1, 32, 8, 1, 8192, 128, BF16) == split_bytes(1, 32, 1, 8192, 128)    # 256: quad
    assert ws(1, 32, 8, 1, 256, 128, BF16) == 0                                    # one split: finished in quad
    assert ws(1, 32, 8, 1, 257, 128, BF16) == split_bytes(1, 32, 1, 257, 128)
    assert ws(8, 32, 8, 1, 8192, 256, BF16) == split_bytes(8, 32, 1, 8192, 256)    # wide split
    # Lq >= 384 (prefill) needs none, at every 16-bit head dim
    assert ws(1, 32, 8, 384, 32768, 128, BF16) == 0
    assert ws(1, 32, 8, 384, 4096, 256, BF16) == 0
    assert ws(1, 32, 8, 384, 4096, 256, F32) == split_bytes(1, 32, 384, 4096, 256)
    # partials above 256 MiB: the call runs in query-row chunks and the query reports one chunk's need
    cap = 256 * 2 ** 20
    assert split_bytes(1, 32, 383, 32768, 128) > cap
    lc = cap // (split_bytes(1, 32, 1, 32768, 128) + 256)
    assert ws(1, 32, 8, 383, 32768, 128, F32) == split_bytes(1, 32, lc, 32768, 128) <= cap
    # 16-bit D <= 128 with at least 64 query rows per KV head takes the prefill kernel below 384 rows too
    assert ws(1, 32, 8, 383, 32768, 128, BF16) == 0
    assert ws(32, 16, 4, 16, 1024, 128, BF16) == 0                                 # 4 x 16 = 64 rows
    # ... on a prefill grid of more than 64 workgroups; smaller grids keep the split kernel
    assert ws(1, 8, 8, 384, 8192, 128, BF16) == split_bytes(1, 8, 384, 8192, 128)  # 6 x 8 = 48
    assert ws(16, 16, 4, 15, 2048, 128, BF16) == split_bytes(16, 16, 15, 2048, 128)  # 60 rows: split
    assert ws(1, 32, 8, 8192, 8192, 128, F32) <= cap
    assert ws(1, 1, 1, 1, 0, 128, BF16) == 0
    assert ws(1, 1, 1, 1, 10, 128, 7) == 0
    assert ws(1, 32, 0, 1, 10, 128, BF16) == 0
    assert ws(1, 32, 5, 1, 10, 128, BF16) == 0


def test_variant_policy_and_validation(lib):
    assert [lib.bi_variant_splits(m) for m in (1, 16, 17, 64, 65, 128, 129, 4096)] == [8, 8, 4, 4, 2, 2, 1, 1]
    assert lib.bi_variant_workspace_bytes(4, 32, 8) == 8 * 4 * 32 * 4
    assert lib.bi_variant_workspace_bytes(4, 32, 1) == 0
    assert lib.bi_variant_linear(P16, 64, P16b, 64, None, P16, 32, 4, 32, 64, BF16, BF16, 0, None, 0,
                                 None) == INVALID
    assert lib.bi_variant_linear(P16, 64, P16b, 64, None, P16, 32, 4, 32, 64, BF16, BF16, 4, None, 0,
                                 None) == WORKSPACE


def test_python_binding_rejects_cpu_tensors_and_dtypes():
    import torch
    import invariant_deterministic_gemm_amd as bi
    x = torch.zeros(2, 8)
    with pytest.raises(ValueError):
        bi.bi_linear(x, x)
    with pytest.raises(ValueError):
        bi.scaled_dot_product_attention(torch.zeros(1, 1, 1, 64), torch.zeros(1, 1, 1, 64),
                                        torch.zeros(1, 1, 1, 64), mask="sliding")


def test_kernel_name_queries(lib):
    name = lambda *a: lib.bi_sdpa_kernel_name(*a).decode()
    assert name(1, 32, 8, 1, 1024, 128, BF16) == "sdpa_quad16+combine"
    assert name(1, 32, 8, 1, 256, 128, BF16) == "sdpa_quad16"
    assert name(8, 32, 8, 1, 1024, 128, BF16) == "sdpa_quad16+combine"        # 256 workgroups
    assert name(9, 32, 8, 1, 1024, 128, BF16) == "sdpa_fused16"
    assert name(1, 32, 8, 1, 8192, 128, BF16) == "sdpa_quad16+combine"
    assert name(1, 32, 8, 1, 8193, 128, BF16) == "sdpa_split16+combine"
    assert name(1, 32, 8, 384, 1025, 128, F16) == "sdpa_prefill16"
    assert name(1, 32, 8, 384, 1024, 128, BF16) == "sdpa_prefill16"
    # below 384 rows: prefill once a KV head has 64 query rows and the quad kernel does not apply
    assert name(4, 32, 8, 64, 1025, 128, F16) == "sdpa_prefill16"                # 4 x 4 x 8 = 128 workgroups
    assert name(1, 32, 8, 64, 1025, 128, F16) == "sdpa_split16+combine"          # 32: the split kernel
    assert name(1, 32, 8, 383, 1024, 128, BF16) == "sdpa_prefill16"
    assert name(1, 8, 8, 384, 8192, 128, BF16) == "sdpa_split16+combine"         # 48 workgroups
    assert name(16, 32, 8, 16, 1025, 128, F16) == "sdpa_prefill16"               # 4 x 16 = 64 rows
    assert name(16, 32, 8, 15, 1025, 128, F16) == "sdpa_split16+combine"         # 60 rows
    assert name(8, 32, 8, 15, 1024, 128, BF16) == "sdpa_fused16"
    assert name(4, 32, 8, 15, 1024, 128, BF16) == "sdpa_quad16+combine"          # 4 x 2 x 4 x 8 = 256"
    assert name(1, 32, 8, 1, 300, 128, F32) == "sdpa_split+combine"
    assert name(1, 32, 8, 1, 300, 64, BF16) == "sdpa_quad16+combine"           # D <= 128: padded
    assert name(64, 32, 8, 1, 300, 64, BF16) == "sdpa_fused16"
    assert name(1, 32, 8, 1, 3000, 96, BF16) == "sdpa_quad16+combine"
    assert name(8, 32, 8, 1, 3000, 96, BF16) == "sdpa_split+combine"
    assert name(8, 32, 8, 1, 8192, 64, BF16) == "sdpa_split16+combine"         # 128-byte key rows
    assert name(8, 32, 8, 1, 8192, 64, F32) == "sdpa_split+combine"
    assert name(1, 32, 8, 1, 300, 160, BF16) == "sdpa_split+combine"
    assert name(8, 32, 8, 1, 8192, 256, BF16) == "sdpa_split16w+combine"       # 16 x 1 x 8 x 8 = 1024
    assert name(9, 32, 8, 1, 8192, 256, BF16) == "sdpa_split+combine"
    assert name(8, 32, 8, 1, 8192, 192, BF16) == "sdpa_split+combine"
    assert name(1, 32, 8, 384, 2048, 160, BF16) == "sdpa_prefill16w"          # D > 128: two column halves
    assert name(1, 32, 8, 384, 2048, 256, F16) == "sdpa_prefill16w"
    assert name(1, 32, 8, 383, 2048, 256, F16) == "sdpa_prefill16w"            # >= 64 rows, >= 192 in the batch
    assert name(4, 32, 8, 64, 2048, 256, F16) == "sdpa_prefill16w"
    assert name(1, 32, 8, 128, 2048, 256, F16) == "sdpa_split16w+combine"
    assert name(4, 32, 8, 32, 2048, 192, BF16) == "sdpa_split+combine"
    assert name(1, 32, 8, 384, 2048, 256, F32) == "sdpa_split+combine"
    assert name(1, 32, 8, 1, 300, 64, F32) == "sdpa_split+combine"
    for bad in ((0, 32, 8, 1, 10, 128, BF16), (1, 32, 8, 1, 0, 128, BF16), (1, 32, 8, 1, 10, 80, BF16),
                (1, 32, 8, 1, 10, 288, BF16), (1, 32, 8, 1, 10, 128, 7), (1, 32, 0, 1, 10, 128, BF16),
                (1, 32, 5, 1, 10, 128, BF16)):
        assert name(*bad) == "none"
    assert lib.bi_gemm_kernel_name(1, 4096, 4096, BF16, 0).decode().startswith("gemm16_strip_nk/")
    assert lib.bi_gemm_kernel_name(4096, 4096, 4096, BF16, 0).decode().startswith("gemm16_ring_nk/")
    # the largest tile with at least 160 tiles: 176 tiles of 256x256 rather than 352 of 256x128
    assert lib.bi_gemm_kernel_name(2048, 5632, 2048, BF16, 0).decode() == "gemm16_ring_nk/256x256"
    assert lib.bi_gemm_kernel_name(1280, 8192, 4096, BF16, 0).decode() == "gemm16_ring_nk/256x256"   # 160
    assert lib.bi_gemm_kernel_name(1024, 8192, 4096, BF16, 0).decode() == "gemm16_ring_nk/256x128"   # 128 / 256
    assert lib.bi_gemm_kernel_name(512, 14336, 4096, BF16, 0).decode() == "gemm16_ring_nk/256x128"   # 112 / 224
    assert lib.bi_gemm_kernel_name(0, 4096, 4096, BF16, 0).decode() == "none"


def test_rowsum_validation(lib):
    assert lib.bi_rowsum(P16, 64, P16b, 4, 64, 0, 9, None) == INVALID           # dtype
    assert lib.bi_rowsum(P16, 64, P16b, -1, 64, 0, BF16, None) == INVALID
    assert lib.bi_rowsum(P16, 32, P16b, 4, 64, 0, BF16, None) == INVALID         # ldx < N
    assert lib.bi_rowsum(None, 64, P16b, 4, 64, 1, F32, None) == INVALID         # null input
    assert lib.bi_rowsum(P16, 64, None, 4, 64, 1, F32, None) == INVALID          # null output
    assert lib.bi_rowsum(None, 0, None, 0, 64, 0, F32, None) == OK               # nothing to do


def qlinear(lib, M=4, N=32, K=128, bits=4, gs=64, dt=BF16, x=P16, wq=P16b, sc=P16, sb=P16b, ldx=None, ldwq=None,
            ldsb=None, ldy=None, bias=None, y=P16, ws=None, ws_bytes=0):
    return lib.bi_quantized_linear(x, K if ldx is None else ldx, wq, K * bits // 32 if ldwq is None else ldwq,
                                   sc, sb, K // gs if ldsb is None else ldsb, bits, gs, bias, y,
                                   N if ldy is None else ldy, M, N, K, dt, ws, ws_bytes, None)


def test_quantized_linear_validation(lib):
    for bits in (1, 3, 5, 6, 16):
        assert qlinear(lib, bits=bits) == UNSUPPORTED, bits
    assert "not supported" in lib.bi_last_error().decode()
    for gs in (16, 48, 256):
        assert qlinear(lib, gs=gs, K=768) == UNSUPPORTED, gs
    assert qlinear(lib, dt=F32) == UNSUPPORTED
    assert qlinear(lib, dt=9) == INVALID
    assert qlinear(lib, K=96, gs=64) == INVALID                  # K not a multiple of the group size
    assert qlinear(lib, M=-1) == INVALID
    assert qlinear(lib, x=None) == INVALID
    assert qlinear(lib, wq=None) == INVALID
    assert qlinear(lib, sc=None) == INVALID
    assert qlinear(lib, y=None) == INVALID
    assert qlinear(lib, ldx=64) == INVALID                       # ldx < K
    assert qlinear(lib, ldwq=8) == INVALID                       # < K * bits / 32 = 16
    assert qlinear(lib, ldsb=1) == INVALID                       # < K / gs = 2
    assert qlinear(lib, ldy=16) == INVALID                       # ldy < N
    assert qlinear(lib, x=P_MIS) == UNSUPPORTED                  # x not 16-byte aligned
    assert qlinear(lib, ldx=132) == UNSUPPORTED                  # ldx not a multiple of 8
    assert qlinear(lib, bits=8, ldwq=33) == UNSUPPORTED          # 8-bit rows: a pitch of 4k words
    assert qlinear(lib, bits=4, ldwq=18) == UNSUPPORTED          # 4-bit rows: a pitch of 4k words
    assert qlinear(lib, bits=4, wq=ctypes.c_void_p(0x7f0000000008)) == UNSUPPORTED   # 16-byte alignment
    # 2-bit rows need 4 bytes only (stopped by the missing workspace, after the alignment checks)
    assert qlinear(lib, M=65, K=192, bits=2, ldwq=13, wq=ctypes.c_void_p(0x7f0000000004)) == WORKSPACE
    assert qlinear(lib, ldx=1 << 24) == UNSUPPORTED              # 32-bit offsets inside the kernel
    assert qlinear(lib, ldwq=1 << 25) == UNSUPPORTED
    assert qlinear(lib, ldsb=1 << 26) == UNSUPPORTED
    assert qlinear(lib, M=0) == OK and qlinear(lib, N=0) == OK   # nothing to do
    # more than 64 rows with K a multiple of 128 dequantise inside the tile kernel (no workspace); other K
    # need the dequantisation workspace: min(N, 8192) * K * 2 bytes
    assert lib.bi_quantized_linear_workspace_bytes(64, 32, 192, BF16) == 0
    assert lib.bi_quantized_linear_workspace_bytes(65, 32, 128, BF16) == 0
    assert lib.bi_quantized_linear_workspace_bytes(1000, 20000, 4096, F16) == 0
    assert lib.bi_quantized_linear_workspace_bytes(65, 32, 192, BF16) == 32 * 192 * 2
    assert lib.bi_quantized_linear_workspace_bytes(1000, 20000, 4032, F16) == 8192 * 4032 * 2
    assert lib.bi_quantized_linear_workspace_bytes(65, 32, 192, F32) == 0
    assert qlinear(lib, M=65, K=192) == WORKSPACE
    assert qlinear(lib, M=65, K=192, ws=P16, ws_bytes=32 * 192 * 2 - 1) == WORKSPACE
    assert qlinear(lib, M=65, K=192, ws=P_MIS, ws_bytes=1 << 20) == WORKSPACE     # not 256-byte aligned


def test_quantize_helper_round_trip():
    """The offline quantiser's packing and groups, read back by the oracle: every weight within half a
    step of its group's grid, and the extreme values of each group exact up to the 16-bit scale."""
    import numpy as np
    import torch
    import oracle
    import invariant_deterministic_gemm_amd as bi
    g = torch.Generator().manual_seed(5)
    w = (torch.randn(24, 256, generator=g) * 0.02).to(torch.bfloat16)
    for bits, gs in ((2, 32), (4, 64), (8, 128)):
        wq, sc, sb = bi.quantize(w, bits, gs)
        assert wq.shape == (24, 256 * bits // 32) and wq.dtype == torch.int32
        assert sc.shape == (24, 256 // gs) and sc.dtype == torch.bfloat16
        deq = oracle.dequantize(wq, sc, sb, bits, gs)
        step = np.repeat(sc.double().numpy(), gs, axis=1)
        err = np.abs(deq - w.double().numpy())
        assert (err <= 0.5 * step + 2e-3 * np.abs(w.double().numpy()) + 1e-6).all(), (bits, gs, err.max())
