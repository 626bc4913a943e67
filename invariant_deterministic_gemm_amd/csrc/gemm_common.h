// Device helpers shared by the GEMM kernels: chunk geometry, the epilogue,
// split ranges for the comparator and the XCD-aware tile order.
#pragma once

#include "device.h"
#include "gemm.h"

namespace bi {

template <int dt> struct Chunk {
    static constexpr int EB = Elem<dt>::bytes;
    static constexpr int EPC = 16 / EB;     // elements per 16-byte chunk
    static constexpr int CK = 4 * EPC;      // k per step (four lane groups)
};

// One step of the chain for one 16x16 output fragment.
template <int dt>
__device__ __forceinline__ f32x4 mfma_chunk(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (dt == DT_F32) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            c = Mfma<DT_F32>::step(__uint_as_float(a[u]), __uint_as_float(b[u]), c);
        return c;
    } else {
        return Mfma<dt>::step(a, b, c);
    }
}

// Epilogue for one element: one fp32 fma with the C / bias term, one rounding.
template <int odt>
__device__ __forceinline__ void epilogue(const GemmParams &p, int m, int n, float acc) {
    float t = 0.0f;
    if (p.C != nullptr) {
        const float c = load_as_f32<odt>(p.C, (int64_t)m * p.ldc + n);
        t = p.beta * c;
    }
    store_from_f32<odt>(p.Y, (int64_t)m * p.ldy + n, __builtin_fmaf(p.alpha, acc, t));
}

template <int odt>
__device__ __forceinline__ void finish(const GemmParams &p, int split, int m, int n, float acc) {
    if (p.splits > 1) {
        p.partial[((int64_t)split * p.M + m) * p.N + n] = acc;
    } else {
        epilogue<odt>(p, m, n, acc);
    }
}

// k steps covered by one split (the whole chain when splits == 1).
__device__ __forceinline__ void split_range(const GemmParams &p, int split, int &sb, int &se) {
    sb = (int)((int64_t)p.total_steps * split / p.splits);
    se = (int)((int64_t)p.total_steps * (split + 1) / p.splits);
}

// Stages [s0, s1) of nst covered by this workgroup's split (blockIdx.y of splits; all of them when
// splits == 1).  Comparator only: the invariant path always runs one split.
__device__ __forceinline__ void split_stages(const GemmParams &p, int nst, int &s0, int &s1) {
    const int s = (int)blockIdx.y;
    s0 = (int)((int64_t)nst * s / p.splits);
    s1 = (int)((int64_t)nst * (s + 1) / p.splits);
}

__device__ __forceinline__ void tile_coords(int b, int ntm, int ntn, int gm, int &tm, int &tn) {
    const int T = ntm * ntn;
    int L = b;
    if ((T & 7) == 0) L = (b & 7) * (T >> 3) + (b >> 3);    // consecutive tiles on one XCD
    const int per_group = gm * ntn;
    const int group = L / per_group;
    const int first_m = group * gm;
    const int gsize = min(gm, ntm - first_m);
    const int r = L - group * per_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

// Moves the operands to element z of a batched call (no C term there).
template <int idt, int odt>
__device__ __forceinline__ void batch_shift(GemmParams &p, int z) {
    if (z == 0) return;
    p.A = static_cast<const char *>(p.A) + (int64_t)z * p.sa * Elem<idt>::bytes;
    p.B = static_cast<const char *>(p.B) + (int64_t)z * p.sb * Elem<idt>::bytes;
    p.Y = static_cast<char *>(p.Y) + (int64_t)z * p.sy * Elem<odt>::bytes;
}

}  // namespace bi
