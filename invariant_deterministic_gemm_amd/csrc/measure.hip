// Measured ceilings of the GPU the library runs on, for the benchmark's
// achievable-fraction columns (include/bi_measure.h).  Nothing on the compute
// path calls these kernels.
//
//  * measure_stream_read: every 16-byte chunk of a buffer read exactly once
//    (grid-stride over 1 KiB wavefront blocks), XOR-folded in registers; a
//    lane stores its fold only if it equals a fixed constant, so the loads
//    cannot be removed and the store traffic is nil in practice.
//  * measure_mfma: W independent v_mfma_f32_16x16x32_bf16 chains per
//    wavefront on register operands, no memory traffic inside the loop:
//    the matrix cores' issue rate with nothing else competing.
#include <hip/hip_runtime.h>

#include "bi_measure.h"
#include "device.h"

namespace bi {

constexpr uint32_t kNeverFold = 0x9e3779b9u;

__global__ __launch_bounds__(256) void measure_stream_read(const u32x4 *__restrict__ src, int64_t n16,
                                                           uint32_t *sink) {
    u32x4 acc = zero_u4();
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) acc ^= src[i];
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == kNeverFold) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

constexpr int kMfmaChains = 8;   // a dependent step waits ~52 cycles and issues every 16: 8 chains cover it

__global__ __launch_bounds__(256) void measure_mfma(uint32_t *sink, int iters) {
    const int lane = threadIdx.x & 63;
    // small finite operands so the accumulators stay finite over any iteration count
    const uint32_t h = 0x3c00u + (uint32_t)(lane & 7);      // bf16 values near 2^-7
    const u32x4 a = u32x4{h | (h << 16), h | (h << 16), h | (h << 16), h | (h << 16)};
    const u32x4 b = u32x4{h ^ 0x8000u, h, h, h ^ 0x80000000u};
    f32x4 acc[kMfmaChains];
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) acc[j] = zero4();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kMfmaChains; ++j) acc[j] = Mfma<DT_BF16>::step(a, b, acc[j]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) s = s + acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (__float_as_uint(s) == kNeverFold) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = 1u;
}

}  // namespace bi

extern "C" {

int bi_measure_stream_read(const void *src, size_t bytes, void *sink, int workgroups, void *stream) {
    if (src == nullptr || sink == nullptr || workgroups <= 0 || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
        return 1;
    hipLaunchKernelGGL(bi::measure_stream_read, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const bi::u32x4 *>(src), (int64_t)(bytes / 16), static_cast<uint32_t *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

double bi_measure_mfma(void *sink, int workgroups, int iters, void *stream) {
    if (sink == nullptr || workgroups <= 0 || iters <= 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
        return -1.0;
    hipLaunchKernelGGL(bi::measure_mfma, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t *>(sink), iters);
    if (hipGetLastError() != hipSuccess) return -1.0;
    // per wavefront and iteration: kMfmaChains instructions of 2 * 16 * 16 * 32 flops
    return (double)workgroups * 4.0 * iters * bi::kMfmaChains * 2.0 * 16 * 16 * 32;
}

}  // extern "C"
