// Batch-invariant GEMM kernels for 16-bit inputs (bf16 / fp16) on gfx950:
// the cooperative strip kernel (small M) and the tile kernels (larger M), for
// B in the (N, K) layout and (strip, 128x128 pipelined tile) row-major (K, N).
//
// Chain for 16-bit inputs (fixed; these kernels and the generic ones of
// gemm.hip all run exactly this): one v_mfma_f32_16x16x32_{bf16,f16} per k
// step of 32, steps walking k upwards from 0; in step s, lane group
// g = lane / 16 holds the 16-byte chunk k in [32 s + 8 g, 32 s + 8 g + 8) of
// its A row (lane % 16) and of its B column (lane % 16); the accumulator
// starts at +0; chunks past K are zero; no step past ceil(K / 32) runs.
// The 16x16 result: lane l, register i holds row 4 (l / 16) + i, column
// l % 16.  Fragment element (i, j) depends only on A row i, B column j and
// accumulator (i, j), so no tile choice can change an element's bits.
#pragma once

#include "device.h"
#include "gemm.h"

namespace bi {

// Whether one of these kernels serves the call (else the generic kernels of gemm.hip do).
bool gemm16_applies(int M, int N, int K, bool b_kn, int splits);
hipError_t launch_gemm16(const GemmParams &p, int in_dt, int out_dt, bool b_kn, hipStream_t st);
const char *gemm16_kernel_name(int M, int N, int K, bool b_kn);

}  // namespace bi
