// Generic batch-invariant GEMM kernels for gfx950 (every dtype, any layout,
// any K, split ranges for the comparator), the split-K comparator's reduce,
// and the host dispatch.  16-bit calls with (N, K) weights go to the faster
// strip / ring kernels of gemm16.hip when they apply; both files run the
// same per-element chain.
//
// Method (mlx-batch-invariant README, section "How the kernels work", GEMM
// paragraph): one workgroup owns the entire reduction over K, the trip count
// depends on K alone, there is no split-K and no atomics, accumulators are
// fp32, and the bias is added into the fp32 accumulator and rounded once.
//
// CDNA4 realisation.  Every output element (m, n) is produced by ONE chain
// of MFMA instructions over k, identical in every kernel configuration:
//
//   k "steps" of CK elements walk upwards from k = 0 (CK = 32 for bf16/fp16,
//   16 for fp32).  In a step, lane group g = lane / 16 holds the 16-byte
//   chunk k in [s*CK + g*EPC, s*CK + (g+1)*EPC) of its row of A and of its
//   column of B (EPC = elements per 16 bytes: 8, or 4 for fp32).
//     bf16/fp16: one v_mfma_f32_16x16x32 per step, k slots in that order;
//     fp32:      four v_mfma_f32_16x16x4_f32 per step, u = 0..3, where the
//                instruction u takes element u of every lane group's chunk.
//   The accumulator starts at +0; chunks past K are zero; no step past the
//   last one (ceil(K / CK)) runs.
//
// MFMA output element (i, j) depends only on A row i, B column j and the
// incoming accumulator (i, j), so the tile shape, the grid and the position
// of a row inside a tile do not change any element's bits.  That is what lets
// the host pick a kernel by M without changing results: every kernel runs
// exactly the chain above, followed by the same epilogue
//      y = round_out( fmaf(alpha, acc, beta * c) ).

#include <cstdio>

#include "device.h"
#include "gemm.h"
#include "gemm_common.h"
#include "gemm16.h"

namespace bi {

// ============================================================ skinny kernels
// One wavefront per 16-column strip of the output, all M <= 16 * FM rows.
// The strip of B is streamed once, with PD steps of loads in flight held in
// registers.  Rows of A past M are clamped to row M - 1 (their results are
// computed and discarded), columns past N to column N - 1.

// B in the (N, K) layout: a lane's B chunk is 16 contiguous bytes of row n.
template <int idt, int odt, int FM, int PD>
__global__ __launch_bounds__(64) void gemm_skinny_nk(GemmParams p) {
    batch_shift<idt, odt>(p, blockIdx.z);
    using C = Chunk<idt>;
    const int lane = threadIdx.x;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int nrow = min(n0 + r16, p.N - 1);

    const char *bptr = static_cast<const char *>(p.B) + (int64_t)nrow * p.ldb * C::EB + g * 16;
    const char *aptr[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
        const int m = min(16 * f + r16, p.M - 1);
        aptr[f] = static_cast<const char *>(p.A) + (int64_t)m * p.lda * C::EB + g * 16;
    }
    const int split = blockIdx.y;
    int s_begin, s_end;
    split_range(p, split, s_begin, s_end);
    const int nsteps = s_end - s_begin;

    f32x4 acc[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) acc[f] = zero4();

    u32x4 bq[PD];
    u32x4 aq[PD][FM];
    auto load = [&](int s, int slot) {
        const int k = (s_begin + s) * C::CK + g * C::EPC;
        const int64_t off = (int64_t)(s_begin + s) * C::CK * C::EB;
        if (k < p.K) {
            bq[slot] = ldg16(bptr + off);
#pragma unroll
            for (int f = 0; f < FM; ++f) aq[slot][f] = ldg16(aptr[f] + off);
        } else {
            bq[slot] = zero_u4();
#pragma unroll
            for (int f = 0; f < FM; ++f) aq[slot][f] = zero_u4();
        }
    };
#pragma unroll
    for (int j = 0; j < PD; ++j)
        if (j < nsteps) load(j, j);
    for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            const int s = s0 + j;
            if (s < nsteps) {
#pragma unroll
                for (int f = 0; f < FM; ++f) acc[f] = mfma_chunk<idt>(aq[j][f], bq[j], acc[f]);
                if (s + PD < nsteps) load(s + PD, j);
            }
        }
    }

    const int n = n0 + r16;
    if (n < p.N) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * f + 4 * g + i;
                if (m < p.M) finish<odt>(p, split, m, n, acc[f][i]);
            }
    }
}

// B in the (K, N) layout: each step the wave loads the CK x 16 block of B
// with coalesced 16-byte row pieces and transposes it through LDS so that a
// lane again holds EPC consecutive k of one column.
template <int idt, int odt, int FM, int PD>
__global__ __launch_bounds__(64) void gemm_skinny_kn(GemmParams p) {
    batch_shift<idt, odt>(p, blockIdx.z);
    using C = Chunk<idt>;
    constexpr int CPR = C::EB;               // chunks per 16-column row piece (32 or 64 bytes)
    constexpr int TROW = C::CK * C::EB + 16; // LDS bytes per column (padded)
    __shared__ __attribute__((aligned(16))) char tbuf[2][16 * TROW];

    const int lane = threadIdx.x;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    // load-side coordinates: lane L fetches row kr = L / CPR, columns h*EPC.. of the strip
    const int kr = lane / CPR;
    const int h = lane % CPR;
    const bool col_ok = n0 + h * C::EPC < p.N;
    const char *bptr = static_cast<const char *>(p.B) + ((int64_t)n0 + h * C::EPC) * C::EB;

    const char *aptr[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
        const int m = min(16 * f + r16, p.M - 1);
        aptr[f] = static_cast<const char *>(p.A) + (int64_t)m * p.lda * C::EB + g * 16;
    }
    const int split = blockIdx.y;
    int s_begin, s_end;
    split_range(p, split, s_begin, s_end);
    const int nsteps = s_end - s_begin;

    f32x4 acc[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) acc[f] = zero4();

    u32x4 bq[PD];
    u32x4 aq[PD][FM];
    auto load = [&](int s, int slot) {
        const int sk = (s_begin + s) * C::CK;
        const int kb = sk + kr;                  // B row this lane fetches
        bq[slot] = (kb < p.K && col_ok) ? ldg16(bptr + (int64_t)kb * p.ldb * C::EB) : zero_u4();
        const int ka = sk + g * C::EPC;          // A chunk this lane needs
        const int64_t off = (int64_t)sk * C::EB;
#pragma unroll
        for (int f = 0; f < FM; ++f) aq[slot][f] = (ka < p.K) ? ldg16(aptr[f] + off) : zero_u4();
    };
#pragma unroll
    for (int j = 0; j < PD; ++j)
        if (j < nsteps) load(j, j);
    int buf = 0;
    for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            const int s = s0 + j;
            if (s < nsteps) {
                // transpose: element e of this lane's piece is B[k = kr][col = h*EPC + e]
                char *t = tbuf[buf];
                if constexpr (C::EB == 2) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t word = bq[j][e >> 1];
                        const uint16_t val = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
                        *reinterpret_cast<uint16_t *>(t + (h * 8 + e) * TROW + kr * 2) = val;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<uint32_t *>(t + (h * 4 + e) * TROW + kr * 4) = bq[j][e];
                }
                __syncthreads();
                const u32x4 bfrag = *reinterpret_cast<const u32x4 *>(t + r16 * TROW + g * 16);
#pragma unroll
                for (int f = 0; f < FM; ++f) acc[f] = mfma_chunk<idt>(aq[j][f], bfrag, acc[f]);
                if (s + PD < nsteps) load(s + PD, j);
                buf ^= 1;
            }
        }
    }

    const int n = n0 + r16;
    if (n < p.N) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * f + 4 * g + i;
                if (m < p.M) finish<odt>(p, split, m, n, acc[f][i]);
            }
    }
}

// ============================================================ tiled kernel
// BM x BN output tile per 256-thread workgroup (2 x 2 wavefronts), K walked
// in tiles of 128 bytes per row (two steps) staged through double-buffered
// LDS.  LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by
// (row & 7), which keeps both the cooperative 16-byte stores and the
// fragment reads free of bank conflicts.
template <int idt, int odt, bool KN, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_tiled(GemmParams p) {
    batch_shift<idt, odt>(p, (int)blockIdx.z / p.splits);       // z = batch element x splits + split
    using C = Chunk<idt>;
    constexpr int FM = BM / 32, FN = BN / 32;
    constexpr int ROWB = 128;                        // bytes of k per LDS row per tile
    constexpr int KT = ROWB / C::EB;                 // k per tile
    constexpr int A_CHUNKS = BM * 8 / 256;           // 16-byte chunks per thread
    constexpr int B_CHUNKS = BN * 8 / 256;
    static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");
    __shared__ __attribute__((aligned(16))) char As[2][BM * ROWB];
    __shared__ __attribute__((aligned(16))) char Bs[2][BN * ROWB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r16 = lane & 15, g = lane >> 4;

    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;

    const char *Ab = static_cast<const char *>(p.A);
    const char *Bb = static_cast<const char *>(p.B);

    // global -> register staging
    u32x4 ra[A_CHUNKS], rb[B_CHUNKS];
    const int split = (int)blockIdx.z % p.splits;
    int s_begin, s_end;
    split_range(p, split, s_begin, s_end);
    const int nsteps = s_end - s_begin;
    const int ntiles = (nsteps + 1) / 2;

    auto gload = [&](int tile) {
        const int kbase = s_begin * C::CK + tile * KT;   // first k of this tile
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int id = tid + 256 * i;
            const int row = id >> 3, c = id & 7;
            const int k = kbase + c * C::EPC;
            const int m = min(m0 + row, p.M - 1);
            const bool ok = k < p.K && (k - s_begin * C::CK) < nsteps * C::CK;
            ra[i] = ok ? ldg16(Ab + ((int64_t)m * p.lda + k) * C::EB) : zero_u4();
        }
        if constexpr (!KN) {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int id = tid + 256 * i;
                const int row = id >> 3, c = id & 7;
                const int k = kbase + c * C::EPC;
                const int n = min(n0 + row, p.N - 1);
                const bool ok = k < p.K && (k - s_begin * C::CK) < nsteps * C::CK;
                rb[i] = ok ? ldg16(Bb + ((int64_t)n * p.ldb + k) * C::EB) : zero_u4();
            }
        } else {
            constexpr int CPRK = BN / C::EPC;            // chunks per k row of the tile
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int id = tid + 256 * i;
                const int kr = id / CPRK, cn = id % CPRK;
                const int k = kbase + kr;
                const int n = n0 + cn * C::EPC;
                const bool ok = k < p.K && (k - s_begin * C::CK) < nsteps * C::CK && n < p.N;
                rb[i] = ok ? ldg16(Bb + ((int64_t)k * p.ldb + n) * C::EB) : zero_u4();
            }
        }
    };
    auto swz = [](int row, int c) { return row * ROWB + ((c ^ (row & 7)) << 4); };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int id = tid + 256 * i;
            *reinterpret_cast<u32x4 *>(As[buf] + swz(id >> 3, id & 7)) = ra[i];
        }
        if constexpr (!KN) {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int id = tid + 256 * i;
                *reinterpret_cast<u32x4 *>(Bs[buf] + swz(id >> 3, id & 7)) = rb[i];
            }
        } else {
            constexpr int CPRK = BN / C::EPC;
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int id = tid + 256 * i;
                const int kr = id / CPRK, cn = id % CPRK;
                const int kb = kr * C::EB;                   // byte offset of k in the LDS row
#pragma unroll
                for (int e = 0; e < C::EPC; ++e) {
                    const int n = cn * C::EPC + e;
                    char *dst = Bs[buf] + n * ROWB + (((kb >> 4) ^ (n & 7)) << 4) + (kb & 15);
                    if constexpr (C::EB == 2) {
                        const uint32_t word = rb[i][e >> 1];
                        *reinterpret_cast<uint16_t *>(dst) = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
                    } else {
                        *reinterpret_cast<uint32_t *>(dst) = rb[i][e];
                    }
                }
            }
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = zero4();

    if (ntiles > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
    }
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ntiles) gload(t + 1);
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            if (2 * t + ss < nsteps) {
                u32x4 af[FM], bfr[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int row = wm * (BM / 2) + 16 * i + r16;
                    af[i] = *reinterpret_cast<const u32x4 *>(As[cur] + swz(row, 4 * ss + g));
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int row = wn * (BN / 2) + 16 * j + r16;
                    bfr[j] = *reinterpret_cast<const u32x4 *>(Bs[cur] + swz(row, 4 * ss + g));
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = mfma_chunk<idt>(af[i], bfr[j], acc[i][j]);
            }
        }
        if (t + 1 < ntiles) sstore(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * (BN / 2) + 16 * j + r16;
            if (n >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * (BM / 2) + 16 * i + 4 * g + e;
                if (m < p.M) finish<odt>(p, split, m, n, acc[i][j][e]);
            }
        }
}

// ============================================================ split-K reduce
// Comparator only: y = epilogue( sum over splits in ascending order ).
template <int odt>
__global__ __launch_bounds__(256) void gemm_splitk_reduce(GemmParams p, const float *part, int splits) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.M * p.N;
    if (idx >= total) return;
    const int m = (int)(idx / p.N), n = (int)(idx % p.N);
    float s = part[idx];
    for (int i = 1; i < splits; ++i) s = s + part[(int64_t)i * total + idx];
    epilogue<odt>(p, m, n, s);
}

// ============================================================ host dispatch
int gemm_k_steps(int K, int in_dt) {
    // one 16-byte chunk per lane group per step: 32 k for 16-bit inputs, 16 k for fp32
    return in_dt == DT_F32 ? (K + 15) / 16 : (K + 31) / 32;
}

// fp32 inputs: 16x16x4 chain (skinny kernel for M <= 64, LDS-tiled above).
// Every configuration runs the same per-element chain; M only picks occupancy.
struct GemmPlan16 {
    int kind;          // 0 = skinny (one wave per 16 columns), 1 = LDS-tiled
    int fm;            // skinny: 16-row fragments per wave
    int bm;            // tiled: square tile
};

static GemmPlan16 plan16(int M, int N) {
    if (M <= 64) return GemmPlan16{0, (M + 15) / 16 > 0 ? (M + 15) / 16 : 1, 0};
    const long tiles128 = (long)((M + 127) / 128) * ((N + 127) / 128);
    return GemmPlan16{1, 0, tiles128 >= 256 ? 128 : 64};
}

// The generic kernels (any layout, any K, split ranges): skinny for M <= 64,
// LDS-tiled above.  Every configuration runs the same per-element chain; M
// only picks occupancy.
template <int idt, int odt>
static hipError_t launch_generic(const GemmParams &p, bool b_kn, hipStream_t st) {
    const GemmPlan16 pl = plan16(p.M, p.N);
    const unsigned sp = (unsigned)p.splits;
    if (pl.kind == 0) {
        const dim3 grid((p.N + 15) / 16, sp, gemm_batch(p)), block(64);
#define SKINNY(FMV, PDV)                                                                             \
    do {                                                                                             \
        if (b_kn) hipLaunchKernelGGL((gemm_skinny_kn<idt, odt, FMV, PDV>), grid, block, 0, st, p); \
        else hipLaunchKernelGGL((gemm_skinny_nk<idt, odt, FMV, PDV>), grid, block, 0, st, p);      \
    } while (0)
        switch (pl.fm) {
            case 1: SKINNY(1, 16); break;
            case 2: SKINNY(2, 12); break;
            case 3: SKINNY(3, 8); break;
            default: SKINNY(4, 8); break;
        }
#undef SKINNY
        return hipGetLastError();
    }
    if (pl.bm == 128) {
        const dim3 grid((p.N + 127) / 128, (p.M + 127) / 128, sp * gemm_batch(p)), block(256);
        if (b_kn) hipLaunchKernelGGL((gemm_tiled<idt, odt, true, 128, 128>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((gemm_tiled<idt, odt, false, 128, 128>), grid, block, 0, st, p);
    } else {
        const dim3 grid((p.N + 63) / 64, (p.M + 63) / 64, sp * gemm_batch(p)), block(256);
        if (b_kn) hipLaunchKernelGGL((gemm_tiled<idt, odt, true, 64, 64>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((gemm_tiled<idt, odt, false, 64, 64>), grid, block, 0, st, p);
    }
    return hipGetLastError();
}

static hipError_t launch_generic_dt(const GemmParams &p, int in_dt, int out_dt, bool b_kn, hipStream_t st) {
    if (in_dt == DT_F32 && out_dt == DT_F32) return launch_generic<DT_F32, DT_F32>(p, b_kn, st);
    if (in_dt == DT_BF16 && out_dt == DT_BF16) return launch_generic<DT_BF16, DT_BF16>(p, b_kn, st);
    if (in_dt == DT_F16 && out_dt == DT_F16) return launch_generic<DT_F16, DT_F16>(p, b_kn, st);
    if (in_dt == DT_BF16 && out_dt == DT_F32) return launch_generic<DT_BF16, DT_F32>(p, b_kn, st);
    if (in_dt == DT_F16 && out_dt == DT_F32) return launch_generic<DT_F16, DT_F32>(p, b_kn, st);
    return hipErrorInvalidValue;
}

const char *gemm_kernel_name(int M, int N, int K, int in_dt, bool b_kn) {
    if (in_dt != DT_F32 && gemm16_applies(M, N, K, b_kn, 1)) return gemm16_kernel_name(M, N, K, b_kn);
    const GemmPlan16 pl = plan16(M, N);
    static thread_local char buf[64];
    if (pl.kind == 0) snprintf(buf, sizeof buf, "gemm_skinny_%s/fm%d", b_kn ? "kn" : "nk", pl.fm);
    else snprintf(buf, sizeof buf, "gemm_tiled_%s/%dx%d", b_kn ? "kn" : "nk", pl.bm, pl.bm);
    return buf;
}

static hipError_t dispatch_dt(const GemmParams &p0, int in_dt, int out_dt, bool b_kn, int splits, float *ws,
                              hipStream_t st) {
    GemmParams p = p0;
    p.total_steps = gemm_k_steps(p.K, in_dt);
    p.splits = splits;
    p.partial = splits > 1 ? ws : nullptr;
    hipError_t e;
    if (in_dt != DT_F32 && gemm16_applies(p.M, p.N, p.K, b_kn, splits)) e = launch_gemm16(p, in_dt, out_dt, b_kn, st);
    else e = launch_generic_dt(p, in_dt, out_dt, b_kn, st);
    if (e != hipSuccess || splits <= 1) return e;
    const int64_t total = (int64_t)p.M * p.N;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (out_dt == DT_F32) hipLaunchKernelGGL((gemm_splitk_reduce<DT_F32>), grid, dim3(256), 0, st, p, (const float *)ws, splits);
    else if (out_dt == DT_BF16) hipLaunchKernelGGL((gemm_splitk_reduce<DT_BF16>), grid, dim3(256), 0, st, p, (const float *)ws, splits);
    else hipLaunchKernelGGL((gemm_splitk_reduce<DT_F16>), grid, dim3(256), 0, st, p, (const float *)ws, splits);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams &p, int in_dt, int out_dt, bool b_kn, hipStream_t st) {
    return dispatch_dt(p, in_dt, out_dt, b_kn, 1, nullptr, st);
}

hipError_t launch_gemm_splitk(const GemmParams &p, int in_dt, int out_dt, int splits, float *ws,
                              hipStream_t st) {
    return dispatch_dt(p, in_dt, out_dt, false, splits, ws, st);
}

}  // namespace bi
