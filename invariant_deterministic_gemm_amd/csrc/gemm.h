// Host-visible launch interface of the GEMM kernels (internal to libbi).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

struct GemmParams {
    const void *A;   // (M, K) rows of lda elements
    int64_t lda;
    const void *B;   // (N, K) rows of ldb elements when !b_kn, else (K, N) rows of ldb elements
    int64_t ldb;
    const void *C;   // output dtype; nullptr => no C term
    int64_t ldc;     // 0 => one row broadcast over m
    void *Y;         // (M, N) rows of ldy elements, output dtype
    int64_t ldy;
    int M, N, K;
    float alpha, beta;
    int total_steps; // k steps of the whole chain (set by the launcher)
    // Split-K comparator only (splits > 1): split s covers k steps
    // [total_steps*s/splits, total_steps*(s+1)/splits) and writes its raw fp32
    // sums to partial[(s * M + m) * N + n] instead of running the epilogue.
    int splits;
    float *partial;
    // Batched calls (bi_matmul_batched): `batch` independent products, element z at A + z sa, B + z sb,
    // Y + z sy (strides in elements; grid dimension z).  0 or 1: one product.
    int batch;
    int64_t sa, sb, sy;
};
// Grid depth of a launch: the batch (at least 1).
inline unsigned gemm_batch(const GemmParams &p) { return p.batch > 1 ? (unsigned)p.batch : 1u; }

// The invariant path: picks a tile configuration from (M, N, K, layout) --
// all configurations run the same per-element MFMA chain -- and enqueues it.
hipError_t launch_gemm(const GemmParams &p, int in_dt, int out_dt, bool b_kn, hipStream_t stream);

// Batch-variant comparator: split-K into `splits` ranges + ordered reduce.
hipError_t launch_gemm_splitk(const GemmParams &p, int in_dt, int out_dt, int splits, float *ws,
                              hipStream_t stream);

// Name of the kernel configuration launch_gemm picks ("gemm_skinny_nk/fm1", ...).
const char *gemm_kernel_name(int M, int N, int K, int in_dt, bool b_kn);

// Number of k steps (one 16-byte chunk per lane each) a K of this dtype needs.
int gemm_k_steps(int K, int in_dt);

}  // namespace bi
