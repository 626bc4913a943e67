// Host-visible launch interface of the row reduction kernel (internal to libbi).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

// y[m] = sum (or mean) over n < N of x[m * ldx + n], fixed order per row (see rowsum.hip).
hipError_t launch_rowsum(const void *x, int64_t ldx, void *y, int64_t M, int64_t N, int mean, int dt,
                         hipStream_t stream);

}  // namespace bi
