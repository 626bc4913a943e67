// libbi host side: argument validation, kernel selection and error reporting
// behind the C ABI declared in include/bi.h.
//
// Selection rules (mlx-batch-invariant README, section "Why MLX is not
// invariant": the variance there comes entirely from WHICH kernel a shape
// picks).  Here every configuration a call can pick runs the same
// per-element arithmetic, so selection may look at M for occupancy without
// affecting bits; nothing looks at the stream, the device state or the
// environment.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <mutex>
#include <string>

#include "bi.h"
#include "device.h"
#include "gemm.h"
#include "rowsum.h"
#include "qgemm.h"
#include "sdpa.h"

namespace {

// Major 2: the attention path queries take Hkv (the kernel choice depends on the grid size).
constexpr int kAbiMajor = 2;
// Bump when a compile-time constant that shapes arithmetic changes
// (k-step order, MFMA shapes, KV_SPLIT / KV_BLOCK, combine order).
// 3: 16-bit GEMM chain on v_mfma_f32_16x16x32 again (2 used 32x32x16).
// 4: fp16 results (GEMM outputs, dequantised fp16 weights) rounded from the fp32 fmaf result in every
//    kernel (some had fused the fmaf with the conversion and rounded once).
constexpr int kBitsVersion = 4;

thread_local std::string g_last_error;

bi_status fail(bi_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bi_status ok() {
    g_last_error.clear();
    return BI_OK;
}

int esize(bi_dtype d) { return d == BI_F32 ? 4 : 2; }

bool dtype_known(int d) { return d == BI_F32 || d == BI_F16 || d == BI_BF16; }

bool pair_supported(bi_dtype in, bi_dtype out) {
    if (in == BI_F32) return out == BI_F32;
    if (in == BI_BF16) return out == BI_BF16 || out == BI_F32;
    if (in == BI_F16) return out == BI_F16 || out == BI_F32;
    return false;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, int a) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0; }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

bi_status device_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(BI_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// Shared checks of the GEMM family.  `b_kn` selects the (K, N) layout of B.
bi_status check_gemm(const char *fn, const void *a, int64_t lda, const void *b, int64_t ldb, bool b_kn,
                     const void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, bi_dtype in_dt,
                     bi_dtype out_dt) {
    if (!dtype_known(in_dt) || !dtype_known(out_dt))
        return fail(BI_ERR_INVALID, "%s: unknown dtype code (in %d, out %d)", fn, (int)in_dt, (int)out_dt);
    if (!pair_supported(in_dt, out_dt))
        return fail(BI_ERR_UNSUPPORTED, "%s: dtype pair in=%d out=%d is not supported", fn, (int)in_dt,
                    (int)out_dt);
    if (M < 0 || N < 0 || K < 0) return fail(BI_ERR_INVALID, "%s: negative size M=%lld N=%lld K=%lld", fn,
                                             (long long)M, (long long)N, (long long)K);
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(BI_ERR_UNSUPPORTED, "%s: sizes must be below 2^31", fn);
    if (M == 0 || N == 0) return ok();
    if (y == nullptr) return fail(BI_ERR_INVALID, "%s: output pointer is null", fn);
    if (K > 0 && (a == nullptr || b == nullptr)) return fail(BI_ERR_INVALID, "%s: input pointer is null", fn);
    if (lda < K) return fail(BI_ERR_INVALID, "%s: lda=%lld < K=%lld", fn, (long long)lda, (long long)K);
    if (b_kn ? (ldb < N) : (ldb < K))
        return fail(BI_ERR_INVALID, "%s: ldb=%lld too small", fn, (long long)ldb);
    if (ldy < N) return fail(BI_ERR_INVALID, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
    const int epc = 16 / esize(in_dt);
    if (K % epc != 0)
        return fail(BI_ERR_UNSUPPORTED, "%s: K=%lld must be a multiple of %d for this dtype", fn, (long long)K, epc);
    if (K > 0) {
        if (!aligned16(a) || !aligned16(b))
            return fail(BI_ERR_UNSUPPORTED, "%s: input pointers must be 16-byte aligned", fn);
        if (lda % epc != 0 || ldb % epc != 0)
            return fail(BI_ERR_UNSUPPORTED, "%s: lda / ldb must be multiples of %d elements", fn, epc);
        if (b_kn && N % epc != 0)
            return fail(BI_ERR_UNSUPPORTED, "%s: N=%lld must be a multiple of %d for a (K, N) operand", fn,
                        (long long)N, epc);
    }
    if (!aligned_to(y, esize(out_dt))) return fail(BI_ERR_UNSUPPORTED, "%s: output pointer misaligned", fn);
    return ok();
}

// Resolve the (K, N) operand of bi_matmul / bi_addmm given by two strides into
// one of the two kernel layouts.
bi_status resolve_b(const char *fn, int64_t sk, int64_t sn, int64_t K, int64_t N, bool &b_kn, int64_t &ldb) {
    if (sk == 1 && (N <= 1 || sn != 1)) {          // column-major: the (N, K) layout
        b_kn = false;
        ldb = N <= 1 ? (K > 0 ? K : 1) : sn;
        if (N > 1 && sn < K)
            return fail(BI_ERR_INVALID, "%s: b column stride %lld < K=%lld", fn, (long long)sn, (long long)K);
        return BI_OK;
    }
    if (sn == 1) {                                   // row-major (K, N)
        b_kn = true;
        ldb = K <= 1 ? (N > 0 ? N : 1) : sk;
        if (K > 1 && sk < N)
            return fail(BI_ERR_INVALID, "%s: b row stride %lld < N=%lld", fn, (long long)sk, (long long)N);
        return BI_OK;
    }
    return fail(BI_ERR_UNSUPPORTED, "%s: b needs a unit stride along k or n (got %lld, %lld)", fn,
                (long long)sk, (long long)sn);
}

bi::GemmParams make_params(const void *a, int64_t lda, const void *b, int64_t ldb, const void *c, int64_t ldc,
                           void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, float alpha, float beta) {
    bi::GemmParams p{};
    p.A = a;
    p.lda = lda;
    p.B = b;
    p.ldb = ldb;
    p.C = c;
    p.ldc = ldc;
    p.Y = y;
    p.ldy = ldy;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.alpha = alpha;
    p.beta = beta;
    p.splits = 1;
    p.partial = nullptr;
    return p;
}

}  // namespace

extern "C" {

bi_status bi_linear(const void *x, int64_t ldx, const void *w, int64_t ldw, const void *bias, void *y,
                    int64_t ldy, int64_t M, int64_t N, int64_t K, bi_dtype in_dt, bi_dtype out_dt,
                    void *stream) {
    bi_status s = check_gemm("bi_linear", x, ldx, w, ldw, false, y, ldy, M, N, K, in_dt, out_dt);
    if (s != BI_OK || M == 0 || N == 0) return s;
    if (bias != nullptr && !aligned_to(bias, esize(out_dt)))
        return fail(BI_ERR_UNSUPPORTED, "bi_linear: bias pointer misaligned");
    bi::GemmParams p = make_params(x, ldx, w, ldw, bias, 0, y, ldy, M, N, K, 1.0f, 1.0f);
    return device_status(bi::launch_gemm(p, in_dt, out_dt, false, (hipStream_t)stream), "bi_linear");
}

bi_status bi_matmul(const void *a, int64_t lda, const void *b, int64_t b_stride_k, int64_t b_stride_n, void *c,
                    int64_t ldc, int64_t M, int64_t N, int64_t K, bi_dtype in_dt, bi_dtype out_dt, void *stream) {
    bool b_kn = true;
    int64_t ldb = 0;
    if (M > 0 && N > 0) {
        bi_status r = resolve_b("bi_matmul", b_stride_k, b_stride_n, K, N, b_kn, ldb);
        if (r != BI_OK) return r;
    }
    bi_status s = check_gemm("bi_matmul", a, lda, b, ldb, b_kn, c, ldc, M, N, K, in_dt, out_dt);
    if (s != BI_OK || M == 0 || N == 0) return s;
    bi::GemmParams p = make_params(a, lda, b, ldb, nullptr, 0, c, ldc, M, N, K, 1.0f, 0.0f);
    return device_status(bi::launch_gemm(p, in_dt, out_dt, b_kn, (hipStream_t)stream), "bi_matmul");
}

bi_status bi_addmm(const void *cin, int64_t ldcin, const void *a, int64_t lda, const void *b, int64_t b_stride_k,
                   int64_t b_stride_n, void *out, int64_t ldo, int64_t M, int64_t N, int64_t K, float alpha,
                   float beta, bi_dtype in_dt, bi_dtype out_dt, void *stream) {
    bool b_kn = true;
    int64_t ldb = 0;
    if (M > 0 && N > 0) {
        bi_status r = resolve_b("bi_addmm", b_stride_k, b_stride_n, K, N, b_kn, ldb);
        if (r != BI_OK) return r;
    }
    bi_status s = check_gemm("bi_addmm", a, lda, b, ldb, b_kn, out, ldo, M, N, K, in_dt, out_dt);
    if (s != BI_OK || M == 0 || N == 0) return s;
    if (!std::isfinite(alpha) || !std::isfinite(beta))
        return fail(BI_ERR_INVALID, "bi_addmm: alpha and beta must be finite");
    const void *c = nullptr;
    if (beta != 0.0f) {
        if (cin == nullptr) return fail(BI_ERR_INVALID, "bi_addmm: cin is null while beta != 0");
        if (ldcin != 0 && ldcin < N)
            return fail(BI_ERR_INVALID, "bi_addmm: ldcin=%lld must be 0 or >= N", (long long)ldcin);
        if (ldcin < 0) return fail(BI_ERR_INVALID, "bi_addmm: negative ldcin");
        if (!aligned_to(cin, esize(out_dt))) return fail(BI_ERR_UNSUPPORTED, "bi_addmm: cin misaligned");
        if (cin == out && ldcin != ldo)
            return fail(BI_ERR_INVALID, "bi_addmm: out may alias cin only with ldo == ldcin");
        c = cin;
    }
    bi::GemmParams p = make_params(a, lda, b, ldb, c, ldcin, out, ldo, M, N, K, alpha, beta);
    return device_status(bi::launch_gemm(p, in_dt, out_dt, b_kn, (hipStream_t)stream), "bi_addmm");
}

bi_status bi_matmul_batched(const void *a, int64_t lda, int64_t stride_a, const void *b, int64_t b_stride_k,
                            int64_t b_stride_n, int64_t stride_b, void *c, int64_t ldc, int64_t stride_c,
                            int64_t batch, int64_t M, int64_t N, int64_t K, bi_dtype in_dt, bi_dtype out_dt,
                            void *stream) {
    const char *fn = "bi_matmul_batched";
    if (batch < 0) return fail(BI_ERR_INVALID, "%s: negative batch %lld", fn, (long long)batch);
    if (batch > kMaxDim) return fail(BI_ERR_UNSUPPORTED, "%s: batch must be below 2^31", fn);
    bool b_kn = true;
    int64_t ldb = 0;
    if (M > 0 && N > 0) {
        bi_status r = resolve_b(fn, b_stride_k, b_stride_n, K, N, b_kn, ldb);
        if (r != BI_OK) return r;
    }
    bi_status s = check_gemm(fn, a, lda, b, ldb, b_kn, c, ldc, M, N, K, in_dt, out_dt);
    if (s != BI_OK || M == 0 || N == 0 || batch == 0) return s;
    if (stride_a < 0 || stride_b < 0 || stride_c < 0)
        return fail(BI_ERR_INVALID, "%s: negative batch stride", fn);
    if (batch > 1 && stride_c < (M - 1) * ldc + N)
        return fail(BI_ERR_INVALID, "%s: stride_c=%lld lets output elements overlap", fn, (long long)stride_c);
    const int epc = 16 / esize(in_dt);
    if (K > 0 && (stride_a % epc != 0 || stride_b % epc != 0))
        return fail(BI_ERR_UNSUPPORTED, "%s: stride_a / stride_b must be multiples of %d elements", fn, epc);
    bi::GemmParams p = make_params(a, lda, b, ldb, nullptr, 0, c, ldc, M, N, K, 1.0f, 0.0f);
    p.sa = stride_a;
    p.sb = stride_b;
    p.sy = stride_c;
    // one launch per 65535 elements (the grid's third dimension)
    for (int64_t z0 = 0; z0 < batch; z0 += 65535) {
        bi::GemmParams q = p;
        q.batch = (int)std::min<int64_t>(65535, batch - z0);
        q.A = static_cast<const char *>(a) + z0 * stride_a * esize(in_dt);
        q.B = static_cast<const char *>(b) + z0 * stride_b * esize(in_dt);
        q.Y = static_cast<char *>(c) + z0 * stride_c * esize(out_dt);
        bi_status st = device_status(bi::launch_gemm(q, in_dt, out_dt, b_kn, (hipStream_t)stream), fn);
        if (st != BI_OK) return st;
    }
    return BI_OK;
}

size_t bi_sdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, bi_dtype dt) {
    if (!dtype_known(dt)) return 0;
    return bi::sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D, (int)dt);
}

static bi_status sdpa_impl(const char *fn, const void *q, const int64_t q_str[4], const void *k,
                           const int64_t k_str[4], const void *v, const int64_t v_str[4], void *o,
                           const int64_t o_str[4], int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S,
                           int64_t D, float scale, int causal, int mask_kind, const void *mask,
                           const int64_t mask_str[4], const float *sinks, bi_dtype dt, void *ws, size_t ws_bytes,
                           void *stream, bool variant = false) {
    if (!dtype_known(dt)) return fail(BI_ERR_INVALID, "%s: unknown dtype code %d", fn, (int)dt);
    if (mask_kind != BI_MASK_NONE && mask_kind != BI_MASK_BOOL && mask_kind != BI_MASK_ADD)
        return fail(BI_ERR_INVALID, "%s: unknown mask kind %d", fn, mask_kind);
    if (mask_kind == BI_MASK_NONE) mask = nullptr;
    if (mask_kind != BI_MASK_NONE && mask == nullptr)
        return fail(BI_ERR_INVALID, "%s: mask kind %d with a null mask", fn, mask_kind);
    if (B < 0 || Hq < 0 || Hkv <= 0 || Lq < 0 || S < 0 || D <= 0)
        return fail(BI_ERR_INVALID, "%s: bad sizes B=%lld Hq=%lld Hkv=%lld Lq=%lld S=%lld D=%lld", fn,
                    (long long)B, (long long)Hq, (long long)Hkv, (long long)Lq, (long long)S, (long long)D);
    if (Hq % Hkv != 0) return fail(BI_ERR_INVALID, "%s: Hq=%lld is not a multiple of Hkv=%lld", fn,
                                   (long long)Hq, (long long)Hkv);
    if (causal && Lq > S)
        return fail(BI_ERR_INVALID, "%s: causal attention needs Lq <= S (Lq=%lld, S=%lld)", fn, (long long)Lq,
                    (long long)S);
    if (D % 32 != 0 || D > 256)
        return fail(BI_ERR_UNSUPPORTED, "%s: head dim %lld not supported (a multiple of 32 up to 256)", fn,
                    (long long)D);
    if (!std::isfinite(scale)) return fail(BI_ERR_INVALID, "%s: scale must be finite", fn);
    if (B == 0 || Hq == 0 || Lq == 0) return ok();
    if (!q_str || !k_str || !v_str || !o_str) return fail(BI_ERR_INVALID, "%s: stride array is null", fn);
    if (q == nullptr || o == nullptr || (S > 0 && (k == nullptr || v == nullptr)))
        return fail(BI_ERR_INVALID, "%s: tensor pointer is null", fn);
    const int epc = 16 / esize(dt);
    const int64_t *strs[4] = {q_str, k_str, v_str, o_str};
    const void *ptrs[4] = {q, k, v, o};
    const char *names[4] = {"q", "k", "v", "o"};
    for (int t = 0; t < 4; ++t) {
        if (strs[t][3] != 1) return fail(BI_ERR_UNSUPPORTED, "%s: %s must be contiguous in its last dim", fn, names[t]);
        for (int d = 0; d < 3; ++d)
            if (strs[t][d] < 0 || strs[t][d] % epc != 0)
                return fail(BI_ERR_UNSUPPORTED, "%s: %s stride[%d]=%lld must be a non-negative multiple of %d",
                            fn, names[t], d, (long long)strs[t][d], epc);
        if ((t != 1 && t != 2) || S > 0)
            if (!aligned16(ptrs[t])) return fail(BI_ERR_UNSUPPORTED, "%s: %s must be 16-byte aligned", fn, names[t]);
    }
    const int64_t G = Hq / Hkv;
    const int64_t R = G * Lq;
    if ((R + 15) / 16 > 65535 || B * Hkv > 65535 || B * Hq * Lq > kMaxDim || S > kMaxDim - 2 * bi::KV_SPLIT)
        return fail(BI_ERR_UNSUPPORTED, "%s: problem too large for one launch", fn);
    if (mask != nullptr) {
        if (!mask_str) return fail(BI_ERR_INVALID, "%s: mask strides are null", fn);
        for (int d = 0; d < 4; ++d)
            if (mask_str[d] < 0) return fail(BI_ERR_INVALID, "%s: negative mask stride", fn);
        if (mask_kind == BI_MASK_ADD && !aligned_to(mask, esize(dt)))
            return fail(BI_ERR_UNSUPPORTED, "%s: additive mask misaligned for its dtype", fn);
    }
    if (sinks != nullptr && !aligned_to(sinks, 4)) return fail(BI_ERR_UNSUPPORTED, "%s: sinks misaligned", fn);
    const size_t need = variant ? bi::sdpa_variant_workspace_bytes(B, Hq, Hkv, Lq, S, D)
                                : bi::sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D, (int)dt);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(BI_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    if (need > 0 && !aligned_to(ws, 256)) return fail(BI_ERR_UNSUPPORTED, "%s: workspace must be 256-byte aligned", fn);

    bi::SdpaParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    for (int d = 0; d < 3; ++d) {
        p.qs[d] = q_str[d];
        p.ks[d] = k_str[d];
        p.vs[d] = v_str[d];
        p.os[d] = o_str[d];
    }
    p.mask = mask;
    p.mask_add = mask_kind == BI_MASK_ADD ? 1 : 0;
    if (mask != nullptr) {
        // four consecutive keys per load: unit key stride, S a multiple of 4, every mask row 4-key aligned
        const int eb = p.mask_add ? (int)esize(dt) : 1;
        p.mask_vec = mask_str[3] == 1 && S % 4 == 0 && aligned_to(mask, 4 * eb) && mask_str[0] % 4 == 0 &&
                     mask_str[1] % 4 == 0 && mask_str[2] % 4 == 0;
    }
    for (int d = 0; d < 4; ++d) p.ms[d] = mask ? mask_str[d] : 0;
    p.sinks = sinks;
    p.B = (int)B;
    p.Hq = (int)Hq;
    p.Hkv = (int)Hkv;
    p.Lq = (int)Lq;
    p.S = (int)S;
    p.G = (int)G;
    p.causal = causal ? 1 : 0;
    p.dr = (int)D;
    p.c = (float)((double)scale * 1.4426950408889634);   // log2(e), rounded once to fp32
    p.split_len = variant ? (int)bi::sdpa_variant_split_len(G, Lq, S) : bi::KV_SPLIT;
    p.nsplit = (int)((S + p.split_len - 1) / p.split_len);
    if (variant) {
        if (need > 0) bi::sdpa_bind_workspace(p, ws);
        return device_status(bi::launch_sdpa_variant(p, dt, (int)D, (hipStream_t)stream), fn);
    }
    const int64_t Lc = bi::sdpa_chunk_rows(B, Hq, Hkv, Lq, S, D, (int)dt);
    if (Lc >= Lq) {
        if (need > 0) bi::sdpa_bind_workspace(p, ws);
        return device_status(bi::launch_sdpa(p, dt, (int)D, (hipStream_t)stream), fn);
    }
    // query rows c0 .. c0 + Lc - 1 as calls of their own: q, o and the mask start at row c0, and a causal
    // chunk sees the keys up to its last row (bottom-right alignment keeps every row's position)
    const int64_t eb = esize(dt);
    for (int64_t c0 = 0; c0 < Lq; c0 += Lc) {
        bi::SdpaParams pc = p;
        const int64_t lc = std::min(Lc, Lq - c0);
        pc.q = static_cast<const char *>(q) + c0 * q_str[2] * eb;
        pc.o = static_cast<char *>(o) + c0 * o_str[2] * eb;
        if (mask != nullptr) pc.mask = static_cast<const char *>(mask) + c0 * mask_str[2] * (pc.mask_add ? eb : 1);
        pc.Lq = (int)lc;
        pc.S = causal ? (int)(S - Lq + c0 + lc) : (int)S;
        pc.nsplit = (pc.S + bi::KV_SPLIT - 1) / bi::KV_SPLIT;
        pc.mask_vec = p.mask_vec && pc.S % 4 == 0;    // 4-key mask groups need S % 4 == 0
        if (bi::sdpa_workspace_bytes(B, Hq, Hkv, lc, pc.S, D, (int)dt) > 0) bi::sdpa_bind_workspace(pc, ws);
        const bi_status st = device_status(bi::launch_sdpa(pc, dt, (int)D, (hipStream_t)stream), fn);
        if (st != BI_OK) return st;
    }
    return ok();
}

bi_status bi_sdpa(const void *q, const int64_t q_str[4], const void *k, const int64_t k_str[4], const void *v,
                  const int64_t v_str[4], void *o, const int64_t o_str[4], int64_t B, int64_t Hq, int64_t Hkv,
                  int64_t Lq, int64_t S, int64_t D, float scale, int causal, const uint8_t *mask,
                  const int64_t mask_str[4], bi_dtype dt, void *ws, size_t ws_bytes, void *stream) {
    return sdpa_impl("bi_sdpa", q, q_str, k, k_str, v, v_str, o, o_str, B, Hq, Hkv, Lq, S, D, scale, causal,
                     mask ? BI_MASK_BOOL : BI_MASK_NONE, mask, mask_str, nullptr, dt, ws, ws_bytes, stream);
}

bi_status bi_sdpa_ex(const void *q, const int64_t q_str[4], const void *k, const int64_t k_str[4], const void *v,
                     const int64_t v_str[4], void *o, const int64_t o_str[4], int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Lq, int64_t S, int64_t D, float scale, int causal, int mask_kind, const void *mask,
                     const int64_t mask_str[4], const float *sinks, bi_dtype dt, void *ws, size_t ws_bytes,
                     void *stream) {
    return sdpa_impl("bi_sdpa_ex", q, q_str, k, k_str, v, v_str, o, o_str, B, Hq, Hkv, Lq, S, D, scale, causal,
                     mask_kind, mask, mask_str, sinks, dt, ws, ws_bytes, stream);
}

int bi_variant_splits(int64_t M) {
    if (M <= 16) return 8;
    if (M <= 64) return 4;
    if (M <= 128) return 2;
    return 1;
}

size_t bi_variant_workspace_bytes(int64_t M, int64_t N, int splits) {
    if (splits <= 1 || M <= 0 || N <= 0) return 0;
    return (size_t)splits * (size_t)M * (size_t)N * 4;
}

bi_status bi_variant_sdpa(const void *q, const int64_t q_str[4], const void *k, const int64_t k_str[4],
                          const void *v, const int64_t v_str[4], void *o, const int64_t o_str[4], int64_t B,
                          int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, float scale, int causal,
                          const uint8_t *mask, const int64_t mask_str[4], bi_dtype dt, void *ws, size_t ws_bytes,
                          void *stream) {
    return sdpa_impl("bi_variant_sdpa", q, q_str, k, k_str, v, v_str, o, o_str, B, Hq, Hkv, Lq, S, D, scale,
                     causal, mask ? BI_MASK_BOOL : BI_MASK_NONE, mask, mask_str, nullptr, dt, ws, ws_bytes, stream,
                     true);
}

size_t bi_variant_sdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D) {
    return bi::sdpa_variant_workspace_bytes(B, Hq, Hkv, Lq, S, D);
}

int64_t bi_variant_sdpa_split_len(int64_t G, int64_t Lq, int64_t S) { return bi::sdpa_variant_split_len(G, Lq, S); }

// ---------------------------------------------------------------- attention without a caller workspace
// For callers that cannot allocate device memory (code under graph capture, serving loops, harnesses that
// forbid it): the split partials go to one file-scope device array per GPU, set up once per device the
// first time the entry point needs it, with that device current.  Host code uses the address
// hipGetSymbolAddress returns for the current device, never the array's name (a host-side stand-in).
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kScratchDevices];

static bi_status scratch_for_current_device(const char *fn, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, fn);
    if (dev < 0 || dev >= kScratchDevices)
        return fail(BI_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library keeps scratch for", fn, dev,
                    kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return device_status(e, fn);
        if (ptr == nullptr) return fail(BI_ERR_DEVICE, "%s: no device address for the scratch array", fn);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return BI_OK;
}

size_t bi_sdpa_scratch_limit(void) { return kScratchBytes; }

bi_status bi_sdpa_ex_noalloc(const void *q, const int64_t q_str[4], const void *k, const int64_t k_str[4],
                             const void *v, const int64_t v_str[4], void *o, const int64_t o_str[4], int64_t B,
                             int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, float scale, int causal,
                             int mask_kind, const void *mask, const int64_t mask_str[4], const float *sinks,
                             bi_dtype dt, void *stream) {
    const char *fn = "bi_sdpa_ex_noalloc";
    const size_t need = dtype_known(dt) ? bi::sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D, (int)dt) : 0;
    if (need > kScratchBytes)
        return fail(BI_ERR_UNSUPPORTED, "%s: these sizes need %zu bytes of partials, above the %zu-byte scratch "
                    "limit of this entry point (use bi_sdpa_ex with a workspace)", fn, need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        const bi_status st = scratch_for_current_device(fn, &ws);
        if (st != BI_OK) return st;
    }
    return sdpa_impl(fn, q, q_str, k, k_str, v, v_str, o, o_str, B, Hq, Hkv, Lq, S, D, scale, causal, mask_kind,
                     mask, mask_str, sinks, dt, ws, ws ? kScratchBytes : 0, stream);
}

bi_status bi_variant_linear(const void *x, int64_t ldx, const void *w, int64_t ldw, const void *bias, void *y,
                            int64_t ldy, int64_t M, int64_t N, int64_t K, bi_dtype in_dt, bi_dtype out_dt,
                            int splits, void *ws, size_t ws_bytes, void *stream) {
    bi_status s = check_gemm("bi_variant_linear", x, ldx, w, ldw, false, y, ldy, M, N, K, in_dt, out_dt);
    if (s != BI_OK || M == 0 || N == 0) return s;
    if (splits < 1 || splits > 16) return fail(BI_ERR_INVALID, "bi_variant_linear: splits must be in 1..16");
    const size_t need = bi_variant_workspace_bytes(M, N, splits);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(BI_ERR_WORKSPACE, "bi_variant_linear: workspace of %zu bytes needed", need);
    if (need > 0 && !aligned16(ws)) return fail(BI_ERR_UNSUPPORTED, "bi_variant_linear: workspace misaligned");
    bi::GemmParams p = make_params(x, ldx, w, ldw, bias, 0, y, ldy, M, N, K, 1.0f, 1.0f);
    return device_status(bi::launch_gemm_splitk(p, in_dt, out_dt, splits, (float *)ws, (hipStream_t)stream),
                         "bi_variant_linear");
}

bi_status bi_rowsum(const void *x, int64_t ldx, void *y, int64_t M, int64_t N, int mean, bi_dtype dt,
                    void *stream) {
    const char *fn = "bi_rowsum";
    if (!dtype_known(dt)) return fail(BI_ERR_INVALID, "%s: unknown dtype code %d", fn, (int)dt);
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim)
        return fail(BI_ERR_INVALID, "%s: bad sizes M=%lld N=%lld", fn, (long long)M, (long long)N);
    if (M == 0) return ok();
    if (y == nullptr || (N > 0 && x == nullptr)) return fail(BI_ERR_INVALID, "%s: tensor pointer is null", fn);
    if (M > 1 && ldx < N) return fail(BI_ERR_INVALID, "%s: ldx=%lld < N=%lld", fn, (long long)ldx, (long long)N);
    return device_status(bi::launch_rowsum(x, M > 1 ? ldx : N, y, M, N, mean ? 1 : 0, (int)dt, (hipStream_t)stream),
                         fn);
}

bi_status bi_quantized_linear(const void *x, int64_t ldx, const uint32_t *wq, int64_t ldwq, const void *scales,
                              const void *biases, int64_t ldsb, int bits, int64_t group_size, const void *bias,
                              void *y, int64_t ldy, int64_t M, int64_t N, int64_t K, bi_dtype dt, void *ws,
                              size_t ws_bytes, void *stream) {
    const char *fn = "bi_quantized_linear";
    if (!dtype_known(dt)) return fail(BI_ERR_INVALID, "%s: unknown dtype code %d", fn, (int)dt);
    if (dt != BI_BF16 && dt != BI_F16) return fail(BI_ERR_UNSUPPORTED, "%s: dtype must be bf16 or fp16", fn);
    if (bits != 2 && bits != 4 && bits != 8)
        return fail(BI_ERR_UNSUPPORTED, "%s: %d-bit weights are not supported (2, 4 or 8)", fn, bits);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(BI_ERR_UNSUPPORTED, "%s: group_size %lld is not supported (32, 64 or 128)", fn,
                    (long long)group_size);
    if (M < 0 || N < 0 || K < 0) return fail(BI_ERR_INVALID, "%s: negative size", fn);
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(BI_ERR_UNSUPPORTED, "%s: sizes must be below 2^31", fn);
    if (K % group_size != 0)
        return fail(BI_ERR_INVALID, "%s: K=%lld is not a multiple of group_size %lld", fn, (long long)K,
                    (long long)group_size);
    if (M == 0 || N == 0) return ok();
    if (y == nullptr) return fail(BI_ERR_INVALID, "%s: output pointer is null", fn);
    if (K > 0 && (x == nullptr || wq == nullptr || scales == nullptr || biases == nullptr))
        return fail(BI_ERR_INVALID, "%s: input pointer is null", fn);
    if (ldy < N) return fail(BI_ERR_INVALID, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
    if (K > 0) {
        if (ldx < K) return fail(BI_ERR_INVALID, "%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
        if (ldwq < K * bits / 32)
            return fail(BI_ERR_INVALID, "%s: ldwq=%lld < K*bits/32=%lld", fn, (long long)ldwq, (long long)(K * bits / 32));
        if (ldsb < K / group_size)
            return fail(BI_ERR_INVALID, "%s: ldsb=%lld < K/group_size=%lld", fn, (long long)ldsb,
                        (long long)(K / group_size));
        if (!aligned16(x) || ldx % 8 != 0)
            return fail(BI_ERR_UNSUPPORTED, "%s: x must be 16-byte aligned with ldx a multiple of 8", fn);
        if (bits == 2 ? !aligned_to(wq, 4) : (!aligned16(wq) || ldwq % 4 != 0))
            return fail(BI_ERR_UNSUPPORTED,
                        "%s: wq must be 4-byte aligned (4 and 8 bits: 16-byte aligned, ldwq a multiple of 4)", fn);
        // the fused kernel addresses 64 rows of x and 16 rows of wq / scales with 32-bit byte offsets
        if (ldx >= (int64_t(1) << 24) || ldwq >= (int64_t(1) << 25) || ldsb >= (int64_t(1) << 26))
            return fail(BI_ERR_UNSUPPORTED, "%s: row pitches must be below 2^24 (x), 2^25 (wq), 2^26 (scales)", fn);
        if (!aligned_to(scales, 2) || !aligned_to(biases, 2))
            return fail(BI_ERR_UNSUPPORTED, "%s: scales / biases misaligned", fn);
    }
    if (bias != nullptr && !aligned_to(bias, 2)) return fail(BI_ERR_UNSUPPORTED, "%s: bias pointer misaligned", fn);
    if (!aligned_to(y, 2)) return fail(BI_ERR_UNSUPPORTED, "%s: output pointer misaligned", fn);
    const size_t need = bi::qgemm_workspace_bytes(M, N, K);
    if (need > 0) {
        if (ws == nullptr || ws_bytes < need)
            return fail(BI_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu%s)", fn, need, ws_bytes,
                        ws == nullptr ? ", null" : "");
        if (!aligned_to(ws, 256)) return fail(BI_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    }
    bi::QGemmParams q{};
    q.g = make_params(x, ldx, nullptr, 0, bias, 0, y, ldy, M, N, K, 1.0f, 1.0f);
    q.wq = wq;
    q.ldwq = ldwq;
    q.scales = scales;
    q.biases = biases;
    q.ldsb = ldsb;
    q.bits = bits;
    q.group_size = (int)group_size;
    return device_status(bi::launch_qgemm(q, (int)dt, need > 0 ? ws : nullptr, (hipStream_t)stream), fn);
}

size_t bi_quantized_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, bi_dtype dt) {
    if (dt != BI_BF16 && dt != BI_F16) return 0;
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
    return bi::qgemm_workspace_bytes(M, N, K);
}

const char *bi_gemm_kernel_name(int64_t M, int64_t N, int64_t K, bi_dtype in_dt, int b_kn) {
    if (M <= 0 || N <= 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || !dtype_known(in_dt))
        return "none";
    return bi::gemm_kernel_name((int)M, (int)N, (int)K, (int)in_dt, b_kn != 0);
}

const char *bi_sdpa_kernel_name(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, bi_dtype dt) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Lq <= 0 || S <= 0 || B > kMaxDim || Hq > kMaxDim ||
        Lq > kMaxDim || S > kMaxDim || (D <= 0 || D % 32 != 0 || D > 256) || !dtype_known(dt))
        return "none";
    return bi::sdpa_kernel_name(B, Hq, Hkv, Lq, S, D, (int)dt);
}

const char *bi_status_name(bi_status s) {
    switch (s) {
        case BI_OK: return "BI_OK";
        case BI_ERR_INVALID: return "BI_ERR_INVALID";
        case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED";
        case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE";
        case BI_ERR_DEVICE: return "BI_ERR_DEVICE";
    }
    return "BI_UNKNOWN_STATUS";
}

const char *bi_last_error(void) { return g_last_error.c_str(); }

int bi_abi_version(void) { return (kAbiMajor << 16) | kBitsVersion; }

}  // extern "C"
