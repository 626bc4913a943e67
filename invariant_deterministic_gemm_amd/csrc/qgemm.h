// Host-visible launch interface of the quantized linear kernel (internal to libbi).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace bi {

struct QGemmParams {
    GemmParams g;           // A = x (M, K), C = bias row (ldc 0) or null, Y = y; alpha = beta = 1
    const uint32_t *wq;     // (N, K * bits / 32) packed words, rows of ldwq words
    int64_t ldwq;
    const void *scales;     // (N, K / group_size) in the input dtype, rows of ldsb elements
    const void *biases;     // same layout as scales
    int64_t ldsb;
    int bits;               // 2, 4 or 8
    int group_size;         // 32, 64 or 128
    int group_shift;        // log2(group_size), set by the launcher
};

// Rows up to this many run the strip kernel (up to 32 when N > 4096); more rows run the tile kernel,
// which dequantises the weight tiles on their way into LDS, when K is a multiple of QGEMM_TILE_K, else
// (above 64 rows) dequantise chunks of at most QGEMM_CHUNK_N columns into a workspace and run the tile
// GEMM kernels on them.
constexpr int64_t QGEMM_FUSED_MAX_M = 64;
constexpr int64_t QGEMM_TILE_K = 128;
constexpr int64_t QGEMM_CHUNK_N = 8192;
// Above this many 16-column strips a workgroup of the fused kernel takes two strips (x read half as often).
constexpr int64_t QGEMM_WIDE_STRIPS = 256;
bool qgemm_uses_workspace(int64_t M, int64_t K);
size_t qgemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

// ws: qgemm_workspace_bytes(M, N, K) bytes of device memory (unused, may be null, when that is 0).
hipError_t launch_qgemm(const QGemmParams &p, int dt, void *ws, hipStream_t stream);

// Rows of x one workgroup takes (16, 32 or 64): an arithmetic-identical tile choice.
int qgemm_tile_rows(int M);

}  // namespace bi
