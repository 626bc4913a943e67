// Batch-invariant GEMM kernels for 16-bit inputs on gfx950 (v_mfma_f32_16x16x32).
//
// Method (mlx-batch-invariant README, section "How the kernels work", GEMM
// paragraph): the whole K reduction of an output element stays in one place
// with a trip count that depends on K alone; no split-K, no atomics, fp32
// accumulation, bias added in fp32 and rounded once.  The chain itself is
// described in gemm16.h.  Two kernels here run it for B in the (N, K) layout:
//   gemm16_strip  M <= 32, and M <= 64 unless N is wide: loader wavefronts
//                 stream a 16- or 32-column strip of the weights (and the
//                 rows of A) into LDS for one consumer wavefront that runs
//                 the chains of all M rows;
//   gemm16_ring   M in the thousands (256-row tiles), K a multiple of 64:
//                 LDS tiles fed through a ring of stages by direct-to-LDS loads;
//   gemm16_pipe   M above the strip range up to the thousands: the same
//                 loads with fragments read several steps ahead and one
//                 barrier per stage.
// The strip kernel (M <= 64) and the 128x128 pipelined kernel (K a multiple of
// 64) also take row-major (K, N) weights; other K with that layout, and fp32,
// run the generic kernels of gemm.hip, which implement the same chain.  The batch-variant
// split-K comparator runs these same kernels with the stage loop cut into
// ranges (grid dimension y) whose raw sums go to a workspace; with one split
// (the invariant path) every workgroup runs the whole chain.
#include <cstdio>

#include "gemm16.h"
#include "gemm16_store.h"
#include "gemm_common.h"

namespace bi {

// ============================================================ cooperative strip kernel
// One workgroup per strip of 16 NB output columns.  NL loader wavefronts
// stream the strip's weight rows and AR rows of A into an LDS ring with direct-to-LDS
// loads, so many more bytes are in flight per strip than one wavefront could
// keep outstanding.  The consumer wavefront issues no global loads (so memory
// back-pressure never stalls the chains) and runs the FM x NB independent
// 16x16 fragment chains out of LDS, reading stage t + 1 (into a second register
// set) while the MFMAs of stage t run.
// A stage covers 128 k: 16 NB B rows then AR A rows, 256 bytes each, chunk c of
// row r at slot c ^ (r & 15) (the 16 rows one ds_read_b128 pass serves hit 16
// distinct bank groups).  Load instruction q moves rows 4q .. 4q+3 of the
// stage (1 KiB); loader l issues instructions l, l + NL, ... (loaders below
// Q mod NL issue one more, and wait with their own vmcnt thresholds).  Chunks
// past K are fetched from a clamped in-bounds address and replaced by zeros
// when read, and steps past the end of the chain are not run.
// KN (B row-major (K, N), 16-column strips): the stage's B part is its 128 k-rows of the strip, 32 bytes
// each, row r at byte 32 r with bit 7 of the offset flipped by bit 8 (the four lane groups of a transposed
// read then cover both halves of the banks); load instruction q moves k-rows 32 q .. 32 q + 31, each lane
// the 16-byte piece that belongs at its slot.  The consumer reads column fragments with transposing LDS
// reads (two per 32-k chunk: k-rows 8 g .. 8 g + 3 and 8 g + 4 .. 8 g + 7 of column r16), which hold the
// same k as the (N, K) path's 16-byte chunks, in the same order.  The strips are dealt so that each
// XCD (workgroup b runs on XCD b mod 8) gets a contiguous range: neighbouring strips read the same
// 128-byte lines of a k-row and share them in that XCD's L2.
__device__ __forceinline__ u32x2 lds_tr16(const char *lds_ptr) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(size_t)(uint32_t)(uintptr_t)BI_LDS_PTR(lds_ptr));
    return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ int kn_swz(int off) { return off ^ (((off >> 8) & 1) << 7); }

template <int idt, int odt, int NB, int FM, int AR, int NS, int NL, bool KN = false>
__global__ __launch_bounds__(64 * (1 + NL)) void gemm16_strip(GemmParams p) {
    batch_shift<idt, odt>(p, blockIdx.z);
    constexpr int ROWB = 256;
    constexpr int SW = 16 * NB;                  // strip width: NB 16-column fragments
    constexpr int QB = SW / 4, QA = AR / 4, Q = QB + QA;
    constexpr int QHI = (Q + NL - 1) / NL, QLO = Q / NL, NHI = Q % NL;
    constexpr int STAGE = Q * 1024;
    static_assert(AR % 4 == 0 && AR >= 4 && AR <= 16 * FM, "A rows per stage");
    static_assert(NS >= 2 && QHI * (NS - 1) <= 63, "vmcnt range");
    static_assert(!KN || NB == 1, "(K, N) weights take 16-column strips");
    __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int strip = blockIdx.x;
    if constexpr (KN) {
        const int nstrip = (p.N + SW - 1) / SW, per = (nstrip + 7) / 8;
        strip = (blockIdx.x % 8) * per + blockIdx.x / 8;
        if (strip >= nstrip) return;                 // the whole workgroup, before any barrier
    }
    const int n0 = strip * SW;
    const int nchunk = p.K >> 3;                 // 16-byte chunks per row
    int sbase, send;                             // this split's stages (all of them without split-K)
    split_stages(p, (p.K + 127) >> 7, sbase, send);
    const int nstages = send - sbase;
    const int total_steps = p.total_steps;
    const bool consumer = wave == 0;
    const int lw = consumer ? 0 : wave - 1;      // loader index
    const int myq = consumer ? 0 : (lw < NHI ? QHI : QLO);

    // load side: lane L of instruction q covers stage row 4 q + L / 16, slot L mod 16
    const char *src[QHI];
    int cl[QHI];
#pragma unroll
    for (int j = 0; j < QHI; ++j) {
        const int q = min(lw + NL * j, Q - 1);
        const int row = 4 * q + (lane >> 4);
        cl[j] = (lane & 15) ^ (row & 15);
        if (KN && q < QB) {
            // the piece stored at this lane's slot: k-row 32 q + o / 32, columns n0 + 8 ((o / 16) mod 2) ..
            const int o = kn_swz(16 * lane);
            cl[j] = 32 * q + (o >> 5);
            src[j] = static_cast<const char *>(p.B) + (int64_t)min(n0 + 8 * ((o >> 4) & 1), p.N - 8) * 2;
        } else if (row < SW) {
            src[j] = static_cast<const char *>(p.B) + (int64_t)min(n0 + row, p.N - 1) * p.ldb * 2;
        } else {
            src[j] = static_cast<const char *>(p.A) + (int64_t)min(row - SW, p.M - 1) * p.lda * 2;
        }
    }
    auto issue = [&](int stage) {
        char *buf = lds + (stage % NS) * STAGE;
#pragma unroll
        for (int j = 0; j < QHI; ++j) {
            if (j < myq) {
                const int q = lw + NL * j;
                const char *from;
                if (KN && q < QB) {
                    const int kr = min((sbase + stage) * 128 + cl[j], p.K - 1);
                    from = src[j] + (int64_t)kr * p.ldb * 2;
                } else {
                    const int gc = min((sbase + stage) * 16 + cl[j], nchunk - 1);
                    from = src[j] + (int64_t)gc * 16;
                }
                __builtin_amdgcn_global_load_lds(static_cast<const void *>(from), BI_LDS_PTR(buf + q * 1024), 16,
                                                 0, 0);
            }
        }
    };
    // loaders: wait until at most `keep` (NS - 1, NS - 2 or 0) of their stages are in flight
    auto wait_keep = [&](int keep) {
        if (consumer) return;
        if (lw < NHI) {
            if (keep == NS - 1) BI_WAIT_VMCNT(QHI * (NS - 1));
            else if (keep == NS - 2) BI_WAIT_VMCNT(QHI * (NS - 2));
            else BI_WAIT_VMCNT(0);
        } else {
            if (keep == NS - 1) BI_WAIT_VMCNT(QLO * (NS - 1));
            else if (keep == NS - 2) BI_WAIT_VMCNT(QLO * (NS - 2));
            else BI_WAIT_VMCNT(0);
        }
    };

    // consume side
    const int r16 = lane & 15, g = lane >> 4;
    int aoff[FM], aswz[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
        const int arow = SW + min(16 * f + r16, AR - 1);
        aoff[f] = arow * ROWB;
        aswz[f] = arow & 15;
    }
    f32x4 acc[NB][FM];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int f = 0; f < FM; ++f) acc[j][f] = zero4();
    // two register sets: the fragments of stage t and those of stage t + 1
    u32x4 xa[4][FM], xb[4][NB], ya[4][FM], yb[4][NB];
    auto read_stage = [&](int stage, u32x4 (&a)[4][FM], u32x4 (&b)[4][NB]) {
        const char *buf = lds + (stage % NS) * STAGE;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = 4 * u + g;
            if constexpr (KN) {
                const int kr = 32 * u + 8 * g + (r16 >> 2);
                const u32x2 lo = lds_tr16(buf + kn_swz(32 * kr + 8 * (r16 & 3)));
                const u32x2 hi = lds_tr16(buf + kn_swz(32 * (kr + 4) + 8 * (r16 & 3)));
                b[u][0] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            } else {
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    b[u][j] = *reinterpret_cast<const u32x4 *>(buf + (16 * j + r16) * ROWB + ((c ^ r16) << 4));
            }
#pragma unroll
            for (int f = 0; f < FM; ++f)
                a[u][f] = *reinterpret_cast<const u32x4 *>(buf + aoff[f] + ((c ^ aswz[f]) << 4));
        }
    };
    auto mma_stage = [&](const u32x4 (&a)[4][FM], const u32x4 (&b)[4][NB]) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int f = 0; f < FM; ++f) acc[j][f] = Mfma<idt>::step(a[u][f], b[u][j], acc[j][f]);
    };
    // the last stage: only steps of the chain, chunks past K read as zero
    auto mma_last = [&](int stage, const u32x4 (&a)[4][FM], const u32x4 (&b)[4][NB]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if ((sbase + stage) * 4 + u < total_steps) {
                const bool past = (sbase + stage) * 16 + 4 * u + g >= nchunk;
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                    for (int f = 0; f < FM; ++f)
                        acc[j][f] = Mfma<idt>::step(past ? zero_u4() : a[u][f], past ? zero_u4() : b[u][j], acc[j][f]);
            }
        }
    };
    // stage t's fragments are in registers: read stage t + 1 into the other
    // set, then run stage t's MFMAs (the reads complete under the chain)
    auto consume_xy = [&](int stage) { read_stage(stage + 1, ya, yb); mma_stage(xa, xb); };
    auto consume_yx = [&](int stage) { read_stage(stage + 1, xa, xb); mma_stage(ya, yb); };
    auto sync_steady = [&]() {
        wait_keep(NS - 2);
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    };
    auto sync_drain = [&]() {
        BI_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();
    };

    // prologue: all NS buffers in flight, stage 0 landed everywhere and read
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < nstages) issue(s);
    if (nstages > 0) {
        wait_keep(nstages >= NS ? NS - 1 : 0);
        __builtin_amdgcn_s_barrier();
        if (consumer) read_stage(0, xa, xb);
    }
    // iteration t: stage t + 1 has landed (at most NS - 2 stages still in
    // flight) and the consumer's reads of stage t are done, so loaders refill
    // the buffer of stage t with stage t + NS while the consumer reads stage
    // t + 1 and runs the MFMAs of stage t.  Only the last stage can be partial.
    // The loop is unrolled twice so that the two register sets alternate.
    int t = 0;
    const int steady = nstages - NS;
    for (; t + 2 <= steady; t += 2) {
        sync_steady();
        if (consumer) consume_xy(t);
        else issue(t + NS);
        sync_steady();
        if (consumer) consume_yx(t + 1);
        else issue(t + 1 + NS);
    }
    bool in_y = false;                               // the set holding stage t's fragments
    if (t < steady) {
        sync_steady();
        if (consumer) consume_xy(t);
        else issue(t + NS);
        ++t;
        in_y = true;
    }
    for (; t < nstages - 1; ++t) {
        sync_drain();
        if (consumer) {
            if (in_y) consume_yx(t);
            else consume_xy(t);
        }
        in_y = !in_y;
    }
    if (nstages > 0 && consumer) {
        if (in_y) mma_last(nstages - 1, ya, yb);
        else mma_last(nstages - 1, xa, xb);
    }
    if (!consumer) return;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int n = n0 + 16 * j + r16;
        if (n >= p.N) continue;
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * f + 4 * g + i;
                if (m < p.M) finish<odt>(p, blockIdx.y, m, n, acc[j][f][i]);
            }
    }
}

// ============================================================ deep-ring tile kernel
// BM x BN tile, WGM x WGN wavefronts, K a multiple of 64.  NS LDS stages of 64
// k (two chain steps; 128-byte LDS rows of 8 chunks, chunk c of row r at slot
// c ^ ((r / 2) mod 8), so the 16 rows one ds_read_b128 pass serves hit 16
// distinct bank groups).  All NS stages are in flight with manual vmcnt waits
// and raw barriers, and the fragment reads of one step overlap the MFMAs of
// the other:
//   iteration t (step-0 fragments of stage t already in registers):
//     read step 1 of stage t; MFMAs of step 0;
//     wait for this wave's loads of stage t + 1; barrier (now every wave has
//     finished reading stage t and stage t + 1 has landed everywhere);
//     issue stage t + NS into the buffer stage t used; read step 0 of stage
//     t + 1; MFMAs of step 1.
// Every wave issues exactly QW loads per stage, so the vmcnt thresholds are exact.
template <int idt, int odt, int BM, int BN, int WGM, int WGN, int NS>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm16_ring(GemmParams p) {
    batch_shift<idt, odt>(p, blockIdx.z);
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int ROWB = 128, CPR = 8, RPW = 2, RPI = 8;
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int QA = BM / RPI, QB = BN / RPI;
    constexpr int QW = (QA + QB) / NW;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");
    static_assert((QA + QB) % NW == 0, "every wave must issue the same number of loads per stage");
    static_assert(NS >= 2 && QW * (NS - 1) <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r16 = lane & 15, g = lane >> 4;

    const int ntm = (p.M + BM - 1) / BM, ntn = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, ntm, ntn, 8, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    int sbase, send;                                 // this split's stages (all of them without split-K)
    split_stages(p, p.K / 64, sbase, send);
    const int nstages = send - sbase;

    const char *src[QW];
#pragma unroll
    for (int j = 0; j < QW; ++j) {
        const int q = wave + NW * j;
        const int rloc = (q < QA ? q : q - QA) * RPI + lane / CPR;
        const int c = (lane % CPR) ^ ((rloc / RPW) % CPR);
        if (q < QA)
            src[j] = static_cast<const char *>(p.A) + (int64_t)min(m0 + rloc, p.M - 1) * p.lda * 2 + c * 16;
        else
            src[j] = static_cast<const char *>(p.B) + (int64_t)min(n0 + rloc, p.N - 1) * p.ldb * 2 + c * 16;
    }
    auto issue = [&](int stage) {
        const int64_t koff = (int64_t)(sbase + stage) * ROWB;
        char *buf = lds + (stage % NS) * STAGE;
#pragma unroll
        for (int j = 0; j < QW; ++j) {
            const int q = wave + NW * j;
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(src[j] + koff), BI_LDS_PTR(buf + q * 1024), 16,
                                             0, 0);
        }
    };
    auto read_step = [&](int stage, int u, u32x4 (&af)[FM], u32x4 (&bfr)[FN]) {
        const char *As = lds + (stage % NS) * STAGE;
        const char *Bs = As + BM * ROWB;
        const int c = 4 * u + g;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WM + 16 * i + r16;
            af[i] = *reinterpret_cast<const u32x4 *>(As + row * ROWB + ((c ^ ((row / RPW) % CPR)) << 4));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * WN + 16 * j + r16;
            bfr[j] = *reinterpret_cast<const u32x4 *>(Bs + row * ROWB + ((c ^ ((row / RPW) % CPR)) << 4));
        }
    };
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = zero4();
    auto mma = [&](const u32x4 (&af)[FM], const u32x4 (&bfr)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = Mfma<idt>::step(af[i], bfr[j], acc[i][j]);
    };

    // prologue: stages 0 .. NS-1 in flight; stage 0 landed everywhere; its step 0 read
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < nstages) issue(s);
    u32x4 a0[FM], b0[FN], a1[FM], b1[FN];
    if (nstages > 0) {
        if (nstages >= NS) BI_WAIT_VMCNT(QW * (NS - 1));
        else BI_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        read_step(0, 0, a0, b0);
    }
    // steady state: every iteration issues stage t + NS and may leave NS - 2 stages in flight
    const int steady = nstages - NS;
    int t = 0;
    for (; t < steady; ++t) {
        read_step(t, 1, a1, b1);
        mma(a0, b0);
        BI_WAIT_VMCNT(QW * (NS - 2));
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this wave's LDS reads of stage t are done
        __builtin_amdgcn_s_barrier();
        issue(t + NS);
        read_step(t + 1, 0, a0, b0);
        mma(a1, b1);
    }
    // tail: nothing left to issue; drain
    for (; t < nstages; ++t) {
        read_step(t, 1, a1, b1);
        mma(a0, b0);
        BI_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();
        if (t + 1 < nstages) read_step(t + 1, 0, a0, b0);
        mma(a1, b1);
    }
    if constexpr (BM * BN * Elem<odt>::bytes <= NS * STAGE) {
        if (p.splits == 1) {
            store_tile16<odt, BM, BN, WGM, WGN>(p, acc, m0, n0, lds);     // the ring's LDS holds the whole tile
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WN + 16 * j + r16;
            if (n >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * WM + 16 * i + 4 * g + e;
                if (m < p.M) finish<odt>(p, blockIdx.y, m, n, acc[i][j][e]);
            }
        }
}

// ============================================================ pipelined ring kernel
// BM x BN tile, WGM x WGN wavefronts, KS-wide k stages (K a multiple of KS),
// NS LDS stages (at least 3).  Rows are KS * 2 bytes; chunk c of row r sits
// at slot c ^ (r mod 16) for 256-byte rows and c ^ ((r / 2) mod 8) for
// 128-byte rows (the 16 rows one ds_read_b128 pass serves hit distinct bank
// groups).  Two things keep the MFMAs fed:
//   * fragments are read DR chain steps ahead into a ring of DR + 1 register
//     sets, so each step's LDS latency hides under the MFMAs of the steps
//     before it;
//   * a stage's buffer is refilled one stage late: the barrier taken DR steps
//     before the end of stage t (once stage t + 1 has landed) hands the
//     buffer of stage t - 1, which every wavefront has finished reading, to
//     the loads of stage t + NS - 1.  No wavefront waits for its own LDS
//     reads before a barrier, and one barrier per stage is the only
//     synchronisation.
// The chain itself (step order, k-slot mapping, instruction) is the one
// described in gemm16.h.
template <int KS> __device__ __forceinline__ int pipe_swz(int row) {
    if constexpr (KS == 128) return row & 15;
    else return (row >> 1) & 7;
}

// KN (B row-major (K, N); 128-column tiles, 64-k stages): the stage's B part is its 64 k-rows of the
// tile's 128 columns, 256 bytes each, 16-byte chunk c of k-row r at slot c ^ kn_pipe_swz(r); load
// instruction q moves four k-rows.  B fragments are read with transposing LDS reads as in the strip
// kernel's (K, N) form (k-rows 8 g .. 8 g + 3 and 8 g + 4 .. 8 g + 7 of each 32-k step), the same k in
// the same order as the (N, K) chunks.  The swizzle puts the four k-rows one read pass takes at distinct
// 32-byte bank ranges, and the two lane groups served together (k-rows 8 apart) on different halves.
__device__ __forceinline__ int kn_pipe_swz(int r) { return 2 * (r & 3) ^ 8 * ((r >> 3) & 1); }

template <int idt, int odt, int BM, int BN, int WGM, int WGN, int NS, int KS, int DR, bool KN = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm16_pipe(GemmParams p) {
    batch_shift<idt, odt>(p, blockIdx.z);
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int ROWB = 2 * KS, CPR = KS / 8, RPI = 64 / CPR;
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int Q = (BM + BN) / RPI, QW = Q / NW;
    constexpr int SPS = KS / 32;                     // chain steps per stage
    constexpr int NSET = DR + 1;
    constexpr int U = (NSET % SPS == 0) ? NSET : (SPS % NSET == 0 ? SPS : NSET * SPS);
    static_assert(KS == 64 || KS == 128, "stage width");
    static_assert(WM % 16 == 0 && WN % 16 == 0 && BM % 16 == 0, "wave tile");
    static_assert(Q % NW == 0, "every wave issues the same number of loads per stage");
    static_assert(NS >= 3 && QW * (NS - 2) <= 63, "vmcnt range");
    static_assert(DR >= 1 && DR <= SPS, "read-ahead");
    static_assert(!KN || (BN == 128 && KS == 64 && BM % RPI == 0), "(K, N) form: 128-column tiles, 64-k stages");
    constexpr int QA = BM / RPI;                     // load instructions of the A rows
    __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r16 = lane & 15, g = lane >> 4;

    const int ntm = (p.M + BM - 1) / BM, ntn = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, ntm, ntn, 8, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    int sbase, send;                                 // this split's stages (all of them without split-K)
    split_stages(p, p.K / KS, sbase, send);
    const int nstages = send - sbase;
    const int nsteps = nstages * SPS;

    // load side: instruction q covers stage rows RPI q .. RPI q + RPI - 1; lane L row RPI q + L / CPR,
    // slot L mod CPR, which receives chunk slot ^ swz(row)
    const char *src[QW];
#pragma unroll
    for (int j = 0; j < QW; ++j) {
        const int q = wave + NW * j;
        const int rloc = q * RPI + lane / CPR;
        const int c = (lane % CPR) ^ pipe_swz<KS>(rloc);
        if (KN && q >= QA) {
            // k-row 4 (q - QA) + L / 16 of the stage, the chunk that belongs at slot L mod 16
            const int kr = 4 * (q - QA) + (lane >> 4);
            const int cb = (lane & 15) ^ kn_pipe_swz(kr);
            src[j] = static_cast<const char *>(p.B) + (int64_t)kr * p.ldb * 2 + (int64_t)min(n0 + 8 * cb, p.N - 8) * 2;
        } else if (rloc < BM) {
            src[j] = static_cast<const char *>(p.A) + (int64_t)min(m0 + rloc, p.M - 1) * p.lda * 2 + c * 16;
        } else {
            src[j] = static_cast<const char *>(p.B) + (int64_t)min(n0 + rloc - BM, p.N - 1) * p.ldb * 2 + c * 16;
        }
    }
    auto issue = [&](int stage) {
        const int64_t koff = (int64_t)(sbase + stage) * ROWB;
        const int64_t kroff = (int64_t)(sbase + stage) * KS * p.ldb * 2;
        char *buf = lds + (stage % NS) * STAGE;
#pragma unroll
        for (int j = 0; j < QW; ++j) {
            const int q = wave + NW * j;
            const int64_t off = (KN && q >= QA) ? kroff : koff;
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(src[j] + off), BI_LDS_PTR(buf + q * 1024), 16,
                                             0, 0);
        }
    };
    int aoff[FM], boff[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) aoff[i] = (wm * WM + 16 * i + r16) * ROWB;
#pragma unroll
    for (int j = 0; j < FN; ++j) boff[j] = (BM + wn * WN + 16 * j + r16) * ROWB;
    const int swz = pipe_swz<KS>(r16);             // rows of a fragment start at multiples of 16
    u32x4 fa[NSET][FM], fb[NSET][FN];
    auto read_step = [&](int step, u32x4 (&a)[FM], u32x4 (&b)[FN]) {
        const char *buf = lds + ((step / SPS) % NS) * STAGE;
        const int c = 4 * (step % SPS) + g;
        const int off = (c ^ swz) << 4;
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const u32x4 *>(buf + aoff[i] + off);
        if constexpr (KN) {
            const char *bb = buf + BM * ROWB;
            const int kr = 32 * (step % SPS) + 8 * g + (r16 >> 2);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int ch = (wn * WN + 16 * j) / 8 + ((r16 & 3) >> 1);   // chunk of this lane's 4 columns
                const u32x2 lo = lds_tr16(bb + kr * 256 + ((ch ^ kn_pipe_swz(kr)) << 4) + 8 * (r16 & 1));
                const u32x2 hi = lds_tr16(bb + (kr + 4) * 256 + ((ch ^ kn_pipe_swz(kr + 4)) << 4) + 8 * (r16 & 1));
                b[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const u32x4 *>(buf + boff[j] + off);
        }
    };
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = zero4();

    // prologue: stages 0 .. NS - 2 in flight, stage 0 landed everywhere, steps 0 .. DR - 1 read
    const int pro = min(NS - 1, nstages);
    for (int s = 0; s < pro; ++s) issue(s);
    if (nstages > 0) {
        if (pro == NS - 1) BI_WAIT_VMCNT(QW * (NS - 2));
        else BI_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int d = 0; d < DR; ++d)
            if (d < nsteps) read_step(d, fa[d], fb[d]);
    }
    // step s: read step s + DR (crossing into stage t + 1 first waits for it and refills the buffer of
    // stage t - 1 with stage t + NS - 1), then run the MFMAs of step s
    for (int s0 = 0; s0 < nsteps; s0 += U) {
#pragma unroll
        for (int d = 0; d < U; ++d) {
            const int s = s0 + d;
            if (s < nsteps) {
                const int sr = s + DR;
                if (sr < nsteps) {
                    if ((d + DR) % SPS == 0) {
                        const int tr = sr / SPS;           // the stage being entered (>= 1)
                        if (tr + NS - 3 <= nstages - 1) BI_WAIT_VMCNT(QW * (NS - 3));
                        else BI_WAIT_VMCNT(0);
                        __builtin_amdgcn_s_barrier();
                        if (tr + NS - 2 < nstages) issue(tr + NS - 2);
                    }
                    read_step(sr, fa[(d + DR) % NSET], fb[(d + DR) % NSET]);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = Mfma<idt>::step(fa[d % NSET][i], fb[d % NSET][j], acc[i][j]);
            }
        }
    }
    if constexpr (BM * BN * Elem<odt>::bytes <= NS * STAGE) {
        if (p.splits == 1) {
            store_tile16<odt, BM, BN, WGM, WGN>(p, acc, m0, n0, lds);
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WN + 16 * j + r16;
            if (n >= p.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * WM + 16 * i + 4 * g + e;
                if (m < p.M) finish<odt>(p, blockIdx.y, m, n, acc[i][j][e]);
            }
        }
}

// ============================================================ plan + launch
// Strip instantiations by M (fragments, A rows per stage, stages, loader
// waves) and ring tiles, largest first.  The ring plan takes the largest tile
// that still yields about one tile per CU (160 of 256), else the smallest.
// Used only to pick a kernel, never changes bits.
struct StripCfg { int nb, fm, ar, ns, nl; };
// More than one 16-column strip per CU: A re-reads from L2 start to cost.
static bool wide_n(int N) { return (N + 15) / 16 > 256; }
static StripCfg strip_cfg(int M, int N) {
    // 32-column strips halve the re-reads of A once N is wide
    // A rows staged per stage follow M, and 16 of them take a 4-deep ring: the LDS per workgroup then
    // lets every 16-column strip of N = 14336 be resident at once (M = 8: 27.1 -> 25.2 us there)
    if (M <= 4) return StripCfg{1, 1, 4, 6, 3};
    if (M <= 8) return StripCfg{1, 1, 8, 6, 3};
    if (M <= 16) return StripCfg{1, 1, 16, 4, 3};
    if (M <= 32) return wide_n(N) ? StripCfg{2, 2, 32, 4, 3} : StripCfg{1, 2, 32, 4, 3};
    return wide_n(N) ? StripCfg{2, 4, 64, 3, 3} : StripCfg{1, 4, 64, 4, 3};
}
// Strip for M <= 32; for M <= 64 too unless N is wide and the ring applies
// (at M > 32 the ring's tiles re-read far less of A than 32-column strips).
static bool use_strip(int M, int N, int K) {
    if (M <= 32) return true;
    if (M <= 64) return !(wide_n(N) && K % 64 == 0);
    return false;
}
// Tiles for M above the strip range, largest first.  Up to 256 rows (where the
// weight stream bounds the call) the plan takes the
// largest tile that yields about one tile per CU (160 of 256), skipping tiles at
// least twice as tall as M (their rows would be mostly clamped copies), else the
// smallest one allowed.  The 256-row tiles run the two-stage ring; the others
// the pipelined kernel, except that the 128x64 tile runs the ring when it spans
// more than one row of tiles (measured faster there), and the 32x64 and 64x64
// tiles, which use 128-k stages, fall back to the ring's 64x64 tile when K is
// not a multiple of 128.
enum TileKind { RING256x256, RING256x128, PIPE128x128, PIPE128x64, PIPE64x64, PIPE32x64, RING128x64, RING64x64 };
struct TileCfg { int bm, bn; TileKind kind; };
static const TileCfg kTiles[] = {{256, 256, RING256x256}, {256, 128, RING256x128}, {128, 128, PIPE128x128},
                                 {128, 64, PIPE128x64},   {64, 64, PIPE64x64},     {32, 64, PIPE32x64}};
// 160 rather than a full round of 256: a larger tile that leaves some CUs idle beats a smaller one that
// needs a second round (measured M = 2048, N = 5632, K = 2048: 176 tiles of 256x256 861 TFLOP/s against
// 352 of 256x128 687; every shape with 192 or more tiles of some size keeps its tile).
constexpr long kMinTiles = 160;

// Above 256 rows the plan weighs wave quantisation instead: a tile kind costs ceil(tiles / 256) rounds of
// its tile area at its measured full-chip rate (K = 4096 / 14336, TFLOP/s), and a smaller tile replaces a
// larger one only when that cost is at least 5% lower.  Measured against every tile kernel on M in {384,
// 768, 2048, 8192} x (N, K) in {(6144, 4096), (28672, 4096), (4096, 14336), (1024, 4096), (128256, 4096)}
// and the large-M cells, this picks the fastest tile or one within 2% of it (M = 768, N = 6144: 256x128,
// 668 TFLOP/s against 501 for the 128x128 tile the tile-count rule took; M = 384: 128x128, 478 against
// 398; M = 768, N = 28672: 256x128, 943 against 884; M = 2048, N = 512: the 64x64 ring, 344 against 312).
struct TileRate { int bm, bn; TileKind kind; int tflops; };
static const TileRate kRates[] = {{256, 256, RING256x256, 1290}, {256, 128, RING256x128, 1060},
                                  {128, 128, PIPE128x128, 860},  {128, 64, RING128x64, 690},
                                  {64, 64, RING64x64, 650},      {32, 64, PIPE32x64, 270}};

static TileCfg tile_cfg(int M, int N, int K) {
    if (M > 256) {
        TileCfg pick = {kRates[0].bm, kRates[0].bn, kRates[0].kind};
        double best = 0.0;
        for (const TileRate &c : kRates) {
            if (c.kind == PIPE32x64 && K % 128 != 0) continue;
            const long tiles = (long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
            const double cost = (double)((tiles + 255) / 256) * c.bm * c.bn / c.tflops;
            if (best == 0.0 || cost < 0.95 * best) {
                best = cost;
                pick = TileCfg{c.bm, c.bn, c.kind};
            }
        }
        return pick;
    }
    TileCfg pick = kTiles[0];
    for (const TileCfg &c : kTiles) {
        if (c.bm >= 2 * M && c.bm > 32) continue;
        pick = c;
        const long tiles = (long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        if (tiles >= kMinTiles) break;
    }
    if ((pick.kind == PIPE64x64 || pick.kind == PIPE32x64) && K % 128 != 0) pick = TileCfg{64, 64, RING64x64};
    if (pick.kind == PIPE128x64 && M > 128) pick.kind = RING128x64;
    return pick;
}

bool gemm16_applies(int M, int N, int K, bool b_kn, int splits) {
    (void)N;
    (void)splits;                                // split-K ranges run on the same kernels
    if (b_kn) return M <= 64 || K % 64 == 0;     // the strip and 128x128 pipelined kernels' (K, N) forms
    return M <= 64 || K % 64 == 0;
}

// (K, N) weights: 16-column strips (the strip configurations above with one fragment column)
static StripCfg strip_cfg_kn(int M) {
    if (M <= 4) return StripCfg{1, 1, 4, 6, 3};
    if (M <= 8) return StripCfg{1, 1, 8, 6, 3};
    if (M <= 16) return StripCfg{1, 1, 16, 4, 3};
    if (M <= 32) return StripCfg{1, 2, 32, 4, 3};
    return StripCfg{1, 4, 64, 4, 3};
}

template <int idt, int odt>
static hipError_t launch16_typed(const GemmParams &p, bool b_kn, hipStream_t st) {
    if (b_kn && p.M > 64) {
        const dim3 tiles((unsigned)(((p.M + 127) / 128) * ((p.N + 127) / 128)), p.splits, gemm_batch(p));
        hipLaunchKernelGGL((gemm16_pipe<idt, odt, 128, 128, 2, 4, 4, 64, 2, true>), tiles, dim3(512), 0, st, p);
        return hipGetLastError();
    }
    if (b_kn) {
        const StripCfg c = strip_cfg_kn(p.M);
        const int per = ((p.N + 15) / 16 + 7) / 8;   // strips per XCD
        const dim3 grid(8 * per, p.splits, gemm_batch(p)), block(64 * (1 + c.nl));
        if (c.ar == 4) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 1, 4, 6, 3, true>), grid, block, 0, st, p);
        else if (c.ar == 8) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 1, 8, 6, 3, true>), grid, block, 0, st, p);
        else if (c.ar == 16) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 1, 16, 4, 3, true>), grid, block, 0, st, p);
        else if (c.ar == 32) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 2, 32, 4, 3, true>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 4, 64, 4, 3, true>), grid, block, 0, st, p);
        return hipGetLastError();
    }
    if (use_strip(p.M, p.N, p.K)) {
        const StripCfg c = strip_cfg(p.M, p.N);
        const dim3 grid((p.N + 16 * c.nb - 1) / (16 * c.nb), p.splits, gemm_batch(p)), block(64 * (1 + c.nl));
        if (c.ar == 4) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 1, 4, 6, 3>), grid, block, 0, st, p);
        else if (c.ar == 8) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 1, 8, 6, 3>), grid, block, 0, st, p);
        else if (c.ar == 16) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 1, 16, 4, 3>), grid, block, 0, st, p);
        else if (c.ar == 32 && c.nb == 1) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 2, 32, 4, 3>), grid, block, 0, st, p);
        else if (c.ar == 32) hipLaunchKernelGGL((gemm16_strip<idt, odt, 2, 2, 32, 4, 3>), grid, block, 0, st, p);
        else if (c.nb == 1) hipLaunchKernelGGL((gemm16_strip<idt, odt, 1, 4, 64, 4, 3>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((gemm16_strip<idt, odt, 2, 4, 64, 3, 3>), grid, block, 0, st, p);
        return hipGetLastError();
    }
    const TileCfg c = tile_cfg(p.M, p.N, p.K);
    const dim3 tiles((unsigned)(((p.M + c.bm - 1) / c.bm) * ((p.N + c.bn - 1) / c.bn)), p.splits, gemm_batch(p));
    switch (c.kind) {
        case RING256x256:
            hipLaunchKernelGGL((gemm16_ring<idt, odt, 256, 256, 2, 4, 2>), tiles, dim3(512), 0, st, p);
            break;
        case RING256x128:
            hipLaunchKernelGGL((gemm16_ring<idt, odt, 256, 128, 4, 2, 3>), tiles, dim3(512), 0, st, p);
            break;
        case PIPE128x128:
            hipLaunchKernelGGL((gemm16_pipe<idt, odt, 128, 128, 2, 4, 4, 64, 2>), tiles, dim3(512), 0, st, p);
            break;
        case PIPE128x64:
            hipLaunchKernelGGL((gemm16_pipe<idt, odt, 128, 64, 4, 2, 6, 64, 2>), tiles, dim3(512), 0, st, p);
            break;
        case PIPE64x64:
            hipLaunchKernelGGL((gemm16_pipe<idt, odt, 64, 64, 2, 4, 4, 128, 2>), tiles, dim3(512), 0, st, p);
            break;
        case PIPE32x64:
            hipLaunchKernelGGL((gemm16_pipe<idt, odt, 32, 64, 2, 4, 5, 128, 2>), tiles, dim3(512), 0, st, p);
            break;
        case RING128x64:
            hipLaunchKernelGGL((gemm16_ring<idt, odt, 128, 64, 2, 2, 4>), tiles, dim3(256), 0, st, p);
            break;
        case RING64x64:
            hipLaunchKernelGGL((gemm16_ring<idt, odt, 64, 64, 2, 2, 4>), tiles, dim3(256), 0, st, p);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm16(const GemmParams &p, int in_dt, int out_dt, bool b_kn, hipStream_t st) {
    if (in_dt == DT_BF16 && out_dt == DT_BF16) return launch16_typed<DT_BF16, DT_BF16>(p, b_kn, st);
    if (in_dt == DT_F16 && out_dt == DT_F16) return launch16_typed<DT_F16, DT_F16>(p, b_kn, st);
    if (in_dt == DT_BF16 && out_dt == DT_F32) return launch16_typed<DT_BF16, DT_F32>(p, b_kn, st);
    if (in_dt == DT_F16 && out_dt == DT_F32) return launch16_typed<DT_F16, DT_F32>(p, b_kn, st);
    return hipErrorInvalidValue;
}

const char *gemm16_kernel_name(int M, int N, int K, bool b_kn) {
    static thread_local char buf[64];
    if (b_kn) {
        if (M > 64) snprintf(buf, sizeof buf, "gemm16_pipe_kn/128x128");
        else snprintf(buf, sizeof buf, "gemm16_strip_kn/w16_a%d", strip_cfg_kn(M).ar);
        return buf;
    }
    if (use_strip(M, N, K)) {
        const StripCfg c = strip_cfg(M, N);
        snprintf(buf, sizeof buf, "gemm16_strip_nk/w%d_a%d", 16 * c.nb, c.ar);
    }
    else {
        const TileCfg c = tile_cfg(M, N, K);
        const bool ring = c.kind == RING256x256 || c.kind == RING256x128 || c.kind == RING128x64 || c.kind == RING64x64;
        snprintf(buf, sizeof buf, "gemm16_%s_nk/%dx%d", ring ? "ring" : "pipe", c.bm, c.bn);
    }
    return buf;
}

}  // namespace bi
