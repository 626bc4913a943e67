// LDS-staged epilogue shared by the 16x16-fragment tile kernels.
#pragma once

#include "device.h"
#include "gemm.h"

namespace bi {

// ============================================================ LDS-staged epilogue
// The BM x BN tile goes through LDS (rows of BN output elements, 16-byte
// chunk index XOR ((row / 4) mod 4) * 2, so the four rows one fragment store
// touches land on distinct banks) and is written with 16-byte coalesced
// stores.  Same arithmetic as `epilogue`: one fmaf with the C / bias term, one
// rounding; the bias of a column is read once.
template <int odt, int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void store_tile16(const GemmParams &p, const f32x4 (&acc)[BM / WGM / 16][BN / WGN / 16],
                                             int m0, int n0, char *lds) {
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int EO = Elem<odt>::bytes;
    constexpr int ROW = BN * EO;
    constexpr int NT = 64 * WGM * WGN;
    static_assert(ROW % 128 == 0, "rows must hold whole groups of 8 chunks");
    auto pos = [](int row, int byte) {
        return row * ROW + ((((byte >> 4) ^ (((row >> 2) & 3) << 1)) << 4) | (byte & 15));
    };
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r16 = lane & 15, g = lane >> 4;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int nl = wn * WN + 16 * j + r16;
        const int n = min(n0 + nl, p.N - 1);
        float tb = 0.0f;
        if (p.C != nullptr && p.ldc == 0) tb = p.beta * load_as_f32<odt>(p.C, n);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ml = wm * WM + 16 * i + 4 * g + e;
                float t = tb;
                if (p.C != nullptr && p.ldc != 0) {
                    const int m = min(m0 + ml, p.M - 1);
                    t = p.beta * load_as_f32<odt>(p.C, (int64_t)m * p.ldc + n);
                }
                const float y = __builtin_fmaf(p.alpha, acc[i][j][e], t);
                char *dst = lds + pos(ml, nl * EO);
                if constexpr (EO == 2) *reinterpret_cast<uint16_t *>(dst) =
                    (uint16_t)(odt == DT_BF16 ? f32_to_bf16(y) : f32_to_f16(y));
                else *reinterpret_cast<float *>(dst) = y;
            }
    }
    __syncthreads();
    constexpr int CPR = BN * EO / 16;                  // 16-byte chunks per tile row
    constexpr int EPC = 16 / EO;
    for (int id = tid; id < BM * CPR; id += NT) {
        const int ml = id / CPR, c = id % CPR;
        const int m = m0 + ml, n = n0 + c * EPC;
        if (m >= p.M || n >= p.N) continue;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + pos(ml, c * 16));
        char *gdst = static_cast<char *>(p.Y) + ((int64_t)m * p.ldy + n) * EO;
        if (n + EPC <= p.N && ((reinterpret_cast<uintptr_t>(gdst) & 15) == 0)) {
            *reinterpret_cast<u32x4 *>(gdst) = v;
        } else {
            const int cnt = min(EPC, p.N - n);
            for (int e = 0; e < cnt; ++e) {
                if constexpr (EO == 2) reinterpret_cast<uint16_t *>(gdst)[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                else reinterpret_cast<uint32_t *>(gdst)[e] = v[e];
            }
        }
    }
}

}  // namespace bi
