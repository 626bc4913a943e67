// Batch-invariant GEMM kernels for 16-bit inputs (bf16 / fp16) on gfx950.
//
// Chain for 16-bit inputs (fixed; every kernel below runs exactly this):
//   one v_mfma_f32_32x32x16_{bf16,f16} per k step of 16, steps walking k
//   upwards from 0; in step s, lane half h = lane / 32 holds the 16-byte chunk
//   k in [16 s + 8 h, 16 s + 8 h + 8) of its A row (lane % 32) and of its B
//   column (lane % 32); the accumulator starts at +0; chunks past K are zero.
//   Result element (row, col) of the 32x32 fragment sits in lane col + 32 h,
//   register 8 (r / 4) + ... (see frag_row below).
// The 32x32x16 shape is the one that reaches the matrix cores' full rate on
// gfx950 (the 16x16x32 shape runs at half of it), so it is used for every M:
// decode-sized problems waste rows of the fragment but are bound by the weight
// stream anyway.  Tile choice cannot change bits because fragment element
// (i, j) depends only on A row i, B column j and accumulator (i, j).
#pragma once

#include "device.h"
#include "gemm.h"

namespace bi {

template <int dt> struct Mfma32;
template <> struct Mfma32<DT_BF16> {
    static __device__ __forceinline__ f32x16 step(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <> struct Mfma32<DT_F16> {
    static __device__ __forceinline__ f32x16 step(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    }
};

// Row of the 32x32 fragment held by lane half h in accumulator register r.
__device__ __forceinline__ int frag_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

hipError_t launch_gemm32(const GemmParams &p, int in_dt, int out_dt, bool b_kn, hipStream_t st);
const char *gemm32_kernel_name(int M, int N, int K, bool b_kn, int splits);

}  // namespace bi
