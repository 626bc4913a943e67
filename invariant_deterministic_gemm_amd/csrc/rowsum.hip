// Batch-invariant row sum / row mean over the last dimension for gfx950.
//
// The mlx-batch-invariant README (section "Why MLX is not invariant", the
// paragraph after the attention bullets) lists sum and mean among the ops a
// batch-invariant stack relies on and keeps a regression test that they stay
// invariant.  On MI355X that test fails for PyTorch's fp32 sum / mean over the
// last dimension: with few rows the reduction is spread over more threads, so
// the summation order of a row depends on how many rows there are.  This
// kernel fixes the order from the row length alone:
//   thread t of the row's 256 adds elements t, t + 256, t + 512, ... in
//   ascending order in fp32 (starting from +0); the 64 partials of a
//   wavefront are combined by a butterfly over lane distances 32, 16, 8, 4,
//   2, 1; the four wavefront sums are combined as (w0 + w1) + (w2 + w3);
//   the mean divides that sum by N once (IEEE division); one rounding to the
//   output dtype.
// One workgroup per row, so no other row can influence the order.
#include "device.h"
#include "rowsum.h"

namespace bi {

template <int dt>
__global__ __launch_bounds__(256) void rowsum_kernel(const void *x, int64_t ldx, void *y, int64_t N, int mean) {
    __shared__ float part[4];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const char *xr = static_cast<const char *>(x) + row * ldx * Elem<dt>::bytes;
    float acc = 0.0f;
    for (int64_t j = t; j < N; j += 256) acc = acc + load_as_f32<dt>(xr, j);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d);
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (t == 0) {
        float s = (part[0] + part[1]) + (part[2] + part[3]);
        if (mean) s = s / (float)N;
        store_from_f32<dt>(y, row, s);
    }
}

hipError_t launch_rowsum(const void *x, int64_t ldx, void *y, int64_t M, int64_t N, int mean, int dt,
                         hipStream_t st) {
    if (M <= 0) return hipSuccess;
    if (M > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)M), block(256);
    if (dt == DT_F32) hipLaunchKernelGGL((rowsum_kernel<DT_F32>), grid, block, 0, st, x, ldx, y, N, mean);
    else if (dt == DT_BF16) hipLaunchKernelGGL((rowsum_kernel<DT_BF16>), grid, block, 0, st, x, ldx, y, N, mean);
    else if (dt == DT_F16) hipLaunchKernelGGL((rowsum_kernel<DT_F16>), grid, block, 0, st, x, ldx, y, N, mean);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace bi
