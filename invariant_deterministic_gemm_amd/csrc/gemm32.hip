// Batch-invariant GEMM kernels for 16-bit inputs on gfx950 (v_mfma_f32_32x32x16).
//
// Method (mlx-batch-invariant README, section "How the kernels work", GEMM
// paragraph): the whole K reduction of an output element stays in one place
// with a trip count that depends on K alone; no split-K, no atomics, fp32
// accumulation, bias added in fp32 and rounded once.  The chain itself is
// described in gemm32.h.  Four kernels run it:
//   gemm32_strip           M <= 64, (N, K) layout: loader wavefronts per strip
//                          of 16 or 32 columns feeding one chain per fragment;
//   gemm32_skinny_{nk,kn}  one wavefront per 32-column strip, M <= 64 (the
//                          (K, N) layout and the split-K comparator);
//   gemm32_tile            LDS-tiled, register-staged loads (any layout, any K,
//                          and the split-K comparator);
//   gemm32_ring            LDS-tiled with direct-to-LDS loads through a ring of
//                          stages, (N, K) layout, K a multiple of 32: the
//                          large-M path.
#include <cstdio>

#include "gemm32.h"
#include "gemm_common.h"

namespace bi {

// 16-byte global chunk offset (bytes) of lane half h in step s.
__device__ __forceinline__ int64_t step_off(int s, int h) { return (int64_t)s * 32 + h * 16; }

// LDS rows of 128 bytes hold 8 chunks of 16 bytes.  Chunk c of row r sits at
// slot c ^ ((r >> 1) & 7): a ds_read_b128 is served 16 lanes at a time over
// 64 four-byte banks (256 bytes), and 16 consecutive rows then land on 16
// distinct (row parity, slot) bank groups.
__device__ __forceinline__ int swz_slot(int row, int c) { return c ^ ((row >> 1) & 7); }

// ============================================================ skinny kernels
// B in the (N, K) layout: a lane's B chunk is 16 contiguous bytes of row n.
template <int idt, int odt, int FM, int PD>
__global__ __launch_bounds__(64) void gemm32_skinny_nk(GemmParams p) {
    const int lane = threadIdx.x;
    const int r32 = lane & 31, h = lane >> 5;
    const int n0 = blockIdx.x * 32;
    const char *bptr = static_cast<const char *>(p.B) + (int64_t)min(n0 + r32, p.N - 1) * p.ldb * 2;
    const char *aptr[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f)
        aptr[f] = static_cast<const char *>(p.A) + (int64_t)min(32 * f + r32, p.M - 1) * p.lda * 2;
    const int split = blockIdx.y;
    int s_begin, s_end;
    split_range(p, split, s_begin, s_end);
    const int nsteps = s_end - s_begin;

    f32x16 acc[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) acc[f] = zero16();
    u32x4 bq[PD];
    u32x4 aq[PD][FM];
    auto load = [&](int s, int slot) {
        const int st = s_begin + s;
        const int64_t off = step_off(st, h);
        if (st * 16 + 8 * h < p.K) {
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
                for (int f = 0; f < FM; ++f) acc[f] = Mfma32<idt>::step(aq[j][f], bq[j], acc[f]);
                if (s + PD < nsteps) load(s + PD, j);
            }
        }
    }
    const int n = n0 + r32;
    if (n < p.N) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * f + frag_row(r, h);
                if (m < p.M) finish<odt>(p, split, m, n, acc[f][r]);
            }
    }
}

// B in the row-major (K, N) layout.  Each step the wave loads the 16 x 32
// block of B as 16 rows of 64 contiguous bytes into LDS (lane L's 16 bytes at
// L * 16), then gathers its fragment with two gfx950 transpose reads
// (ds_read_b64_tr_b16): within each 16-lane group, result lane i element v is
// element (i mod 4) of source lane (i / 4 + 4 v), so source lane j points at
// k row 8 h + 4 jj + j / 4, columns 16 (group mod 2) + 4 (j mod 4).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ds_read_tr16(const char *lds_addr) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)((__attribute__((address_space(3))) char *)lds_addr));
    return __builtin_bit_cast(u32x2, v);
}

template <int idt, int odt, int FM, int PD>
__global__ __launch_bounds__(64) void gemm32_skinny_kn(GemmParams p) {
    __shared__ __attribute__((aligned(16))) char tbuf[2][1024];
    const int lane = threadIdx.x;
    const int r32 = lane & 31, h = lane >> 5;
    const int n0 = blockIdx.x * 32;
    // load side: lane L fetches k row L / 4, bytes 16 (L mod 4) of the strip's 64-byte row piece
    const int kr = lane >> 2, cq = lane & 3;
    const bool col_ok = n0 + cq * 8 < p.N;
    const char *bptr = static_cast<const char *>(p.B) + ((int64_t)n0 + cq * 8) * 2;
    // transpose-read side
    const int grp = lane >> 4, j16 = lane & 15;
    const int tr_off = (8 * h + (j16 >> 2)) * 64 + 32 * (grp & 1) + 8 * (j16 & 3);

    const char *aptr[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f)
        aptr[f] = static_cast<const char *>(p.A) + (int64_t)min(32 * f + r32, p.M - 1) * p.lda * 2;
    const int split = blockIdx.y;
    int s_begin, s_end;
    split_range(p, split, s_begin, s_end);
    const int nsteps = s_end - s_begin;

    f32x16 acc[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) acc[f] = zero16();
    u32x4 bq[PD];
    u32x4 aq[PD][FM];
    auto load = [&](int s, int slot) {
        const int st = s_begin + s;
        const int kb = st * 16 + kr;
        bq[slot] = (kb < p.K && col_ok) ? ldg16(bptr + (int64_t)kb * p.ldb * 2) : zero_u4();
        const bool aok = st * 16 + 8 * h < p.K;
        const int64_t off = step_off(st, h);
#pragma unroll
        for (int f = 0; f < FM; ++f) aq[slot][f] = aok ? ldg16(aptr[f] + off) : zero_u4();
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
                char *t = tbuf[buf];
                *reinterpret_cast<u32x4 *>(t + lane * 16) = bq[j];
                __syncthreads();
                const u32x2 lo = ds_read_tr16(t + tr_off);
                const u32x2 hi = ds_read_tr16(t + tr_off + 4 * 64);
                const u32x4 bfrag = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int f = 0; f < FM; ++f) acc[f] = Mfma32<idt>::step(aq[j][f], bfrag, acc[f]);
                if (s + PD < nsteps) load(s + PD, j);
                buf ^= 1;
            }
        }
    }
    const int n = n0 + r32;
    if (n < p.N) {
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * f + frag_row(r, h);
                if (m < p.M) finish<odt>(p, split, m, n, acc[f][r]);
            }
    }
}

// ============================================================ cooperative strip kernel
// Small M with B in the (N, K) layout.  One workgroup per strip of SW output
// columns (SW = 32, or 16 with fragment columns 16..31 repeating 0..15, which
// doubles the number of workgroups for narrow N and leaves every column's
// chain unchanged).  NL loader wavefronts stream the strip's weight rows and AR
// rows of A into an LDS ring with direct-to-LDS loads, so many more bytes are
// in flight per strip than one wavefront can keep outstanding; FM consumer
// wavefronts, one per 32-row fragment, issue no global loads (so memory
// back-pressure never stalls a chain) and run the chain out of LDS, reading
// stage t + 1 while the MFMAs of stage t run.
// A stage covers 128 k: SW B rows then AR A rows, 256 bytes each, chunk c of
// row r at slot c ^ (r & 15) (16 consecutive rows of one chunk hit 16 distinct
// bank groups).  Load instruction q moves rows 4q .. 4q+3 of the stage (1 KiB);
// loader l issues instructions l, l + NL, ... (loaders below Q mod NL issue
// one more, and wait with their own vmcnt thresholds).  Chunks past K are
// fetched from a clamped in-bounds address and replaced by zeros when read,
// and steps past the end of the chain are not run (an extra zero step could
// turn -0 into +0).
template <int idt, int odt, int SW, int FM, int AR, int NS, int NL>
__global__ __launch_bounds__(64 * (FM + NL)) void gemm32_strip(GemmParams p) {
    constexpr int ROWB = 256;
    constexpr int QB = SW / 4, QA = AR / 4, Q = QB + QA;
    constexpr int QHI = (Q + NL - 1) / NL, QLO = Q / NL, NHI = Q % NL;
    constexpr int STAGE = Q * 1024;
    static_assert(SW == 16 || SW == 32, "strip width");
    static_assert(AR % 4 == 0 && AR >= 4 && AR <= 32 * FM, "A rows per stage");
    static_assert(NS >= 2 && QHI * (NS - 1) <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * SW;
    const int nchunk = p.K >> 3;                 // 16-byte chunks per row
    const int nstages = (p.K + 127) >> 7;
    const int total_steps = p.total_steps;
    const bool consumer = wave < FM;
    const int lw = consumer ? 0 : wave - FM;     // loader index
    const int myq = consumer ? 0 : (lw < NHI ? QHI : QLO);

    // load side: lane L of instruction q covers stage row 4 q + L / 16, slot L mod 16
    const char *src[QHI];
    int cl[QHI];
#pragma unroll
    for (int j = 0; j < QHI; ++j) {
        const int q = min(lw + NL * j, Q - 1);
        const int row = 4 * q + (lane >> 4);
        cl[j] = (lane & 15) ^ (row & 15);
        if (row < SW)
            src[j] = static_cast<const char *>(p.B) + (int64_t)min(n0 + row, p.N - 1) * p.ldb * 2;
        else
            src[j] = static_cast<const char *>(p.A) + (int64_t)min(row - SW, p.M - 1) * p.lda * 2;
    }
    auto issue = [&](int stage) {
        char *buf = lds + (stage % NS) * STAGE;
#pragma unroll
        for (int j = 0; j < QHI; ++j) {
            if (j < myq) {
                const int q = lw + NL * j;
                const int g = min(stage * 16 + cl[j], nchunk - 1);
                __builtin_amdgcn_global_load_lds(static_cast<const void *>(src[j] + (int64_t)g * 16),
                                                 BI_LDS_PTR(buf + q * 1024), 16, 0, 0);
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
    const int r32 = lane & 31, h = lane >> 5;
    const int arow = SW + min(32 * wave + r32, AR - 1);
    const int brow = r32 & (SW - 1);
    const int aoff = arow * ROWB, boff = brow * ROWB;
    const int aswz = arow & 15, bswz = brow & 15;
    f32x16 acc = zero16();
    u32x4 fa[8], fb[8];
    auto frag = [&](int stage, int u, u32x4 &a, u32x4 &b) {
        const char *buf = lds + (stage % NS) * STAGE;
        const int c = 2 * u + h;
        a = *reinterpret_cast<const u32x4 *>(buf + aoff + ((c ^ aswz) << 4));
        b = *reinterpret_cast<const u32x4 *>(buf + boff + ((c ^ bswz) << 4));
    };
    // the eight steps of a full stage, each followed by the read of the same
    // step of the next stage into the registers it just consumed
    auto mma_then_read = [&](int stage) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc = Mfma32<idt>::step(fa[u], fb[u], acc);
            frag(stage + 1, u, fa[u], fb[u]);
        }
    };
    // the last stage: only steps of the chain, chunks past K read as zero
    auto mma_last = [&](int stage) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (stage * 8 + u < total_steps) {
                const bool past = stage * 16 + 2 * u + h >= nchunk;
                acc = Mfma32<idt>::step(past ? zero_u4() : fa[u], past ? zero_u4() : fb[u], acc);
            }
        }
    };

    // prologue: all NS buffers in flight, stage 0 landed everywhere and read
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < nstages) issue(s);
    if (nstages > 0) {
        wait_keep(nstages >= NS ? NS - 1 : 0);
        __builtin_amdgcn_s_barrier();
        if (consumer) {
#pragma unroll
            for (int u = 0; u < 8; ++u) frag(0, u, fa[u], fb[u]);
        }
    }
    // iteration t: stage t + 1 has landed (at most NS - 2 stages still in
    // flight) and every consumer's reads of stage t are done, so loaders
    // refill the buffer of stage t with stage t + NS while consumers run the
    // MFMAs of stage t and read stage t + 1.  Only the last stage can be partial.
    int t = 0;
    for (; t < nstages - NS; ++t) {
        wait_keep(NS - 2);
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (consumer) mma_then_read(t);
        else issue(t + NS);
    }
    for (; t < nstages - 1; ++t) {
        BI_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();
        if (consumer) mma_then_read(t);
    }
    if (nstages > 0 && consumer) mma_last(nstages - 1);
    if (!consumer) return;
    const int n = n0 + r32;
    if (r32 < SW && n < p.N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * wave + frag_row(r, h);
            if (m < p.M) epilogue<odt>(p, m, n, acc[r]);
        }
    }
}

// ============================================================ LDS-tiled, register-staged
// BM x BN tile, WGM x WGN wavefronts, K walked in tiles of 64 (128 bytes per
// LDS row, four steps) through double-buffered LDS with the 16-byte chunk
// index XOR-swizzled (swz_slot).  A row-major (K, N) B is transposed into
// n-major LDS rows on the way in.  Handles K tails and split-K ranges.
template <int idt, int odt, bool KN, int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm32_tile(GemmParams p) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int ROWB = 128;
    constexpr int A_CHUNKS = BM * 8 / NT;
    constexpr int B_CHUNKS = BN * 8 / NT;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile");
    __shared__ __attribute__((aligned(16))) char As[2][BM * ROWB];
    __shared__ __attribute__((aligned(16))) char Bs[2][BN * ROWB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r32 = lane & 31, h = lane >> 5;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const char *Ab = static_cast<const char *>(p.A);
    const char *Bb = static_cast<const char *>(p.B);
    const int split = blockIdx.z;
    int s_begin, s_end;
    split_range(p, split, s_begin, s_end);
    const int nsteps = s_end - s_begin;
    const int ntiles = (nsteps + 3) / 4;
    const int kend = min(p.K, s_end * 16);

    u32x4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto gload = [&](int tile) {
        const int kbase = (s_begin + 4 * tile) * 16;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int id = tid + NT * i;
            const int row = id >> 3, c = id & 7;
            const int k = kbase + c * 8;
            const int m = min(m0 + row, p.M - 1);
            ra[i] = k < kend ? ldg16(Ab + ((int64_t)m * p.lda + k) * 2) : zero_u4();
        }
        if constexpr (!KN) {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int id = tid + NT * i;
                const int row = id >> 3, c = id & 7;
                const int k = kbase + c * 8;
                const int n = min(n0 + row, p.N - 1);
                rb[i] = k < kend ? ldg16(Bb + ((int64_t)n * p.ldb + k) * 2) : zero_u4();
            }
        } else {
            constexpr int CPRK = BN / 8;
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int id = tid + NT * i;
                const int kr = id / CPRK, cn = id % CPRK;
                const int k = kbase + kr;
                const int n = n0 + cn * 8;
                rb[i] = (k < kend && n < p.N) ? ldg16(Bb + ((int64_t)k * p.ldb + n) * 2) : zero_u4();
            }
        }
    };
    auto swz = [](int row, int c) { return row * ROWB + (swz_slot(row, c) << 4); };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int id = tid + NT * i;
            *reinterpret_cast<u32x4 *>(As[buf] + swz(id >> 3, id & 7)) = ra[i];
        }
        if constexpr (!KN) {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int id = tid + NT * i;
                *reinterpret_cast<u32x4 *>(Bs[buf] + swz(id >> 3, id & 7)) = rb[i];
            }
        } else {
            constexpr int CPRK = BN / 8;
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int id = tid + NT * i;
                const int kr = id / CPRK, cn = id % CPRK;
                const int kb = kr * 2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int n = cn * 8 + e;
                    const uint32_t word = rb[i][e >> 1];
                    *reinterpret_cast<uint16_t *>(Bs[buf] + n * ROWB + (swz_slot(n, kb >> 4) << 4) + (kb & 15)) =
                        (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
                }
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = zero16();
    if (ntiles > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
    }
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ntiles) gload(t + 1);
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
            if (4 * t + ss < nsteps) {
                u32x4 af[FM], bfr[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[i] = *reinterpret_cast<const u32x4 *>(As[cur] + swz(wm * WM + 32 * i + r32, 2 * ss + h));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bfr[j] = *reinterpret_cast<const u32x4 *>(Bs[cur] + swz(wn * WN + 32 * j + r32, 2 * ss + h));
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = Mfma32<idt>::step(af[i], bfr[j], acc[i][j]);
            }
        }
        if (t + 1 < ntiles) sstore(cur ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WN + 32 * j + r32;
            if (n >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WM + 32 * i + frag_row(r, h);
                if (m < p.M) finish<odt>(p, split, m, n, acc[i][j][r]);
            }
        }
}

// ============================================================ LDS-staged epilogue
// Runs the epilogue of every element (same fmaf and single rounding as
// epilogue()) in the fragment layout, parks the rounded tile in LDS as
// row-major rows (16-byte chunk c of row r at chunk c ^ (4 * ((r >> 2) & 1)),
// so the two lane halves, which write rows 4 apart, hit different banks), then
// writes it out with 16-byte stores covering whole row pieces.  A bias row
// (ldc == 0) is read once per column.  Called by every thread of the
// workgroup after the main loop; `lds` must hold BM * BN * sizeof(out) bytes.
template <int odt, int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void store_tile_staged(const GemmParams &p, const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                                  int m0, int n0, char *lds) {
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int EO = Elem<odt>::bytes;
    constexpr int ROW = BN * EO;
    constexpr int NT = 64 * WGM * WGN;
    static_assert(ROW % 128 == 0, "rows must hold whole groups of 8 chunks");
    auto pos = [](int row, int byte) { return row * ROW + ((((byte >> 4) ^ (((row >> 2) & 1) << 2)) << 4) | (byte & 15)); };
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r32 = lane & 31, h = lane >> 5;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int nl = wn * WN + 32 * j + r32;
        const int n = min(n0 + nl, p.N - 1);
        float tb = 0.0f;
        if (p.C != nullptr && p.ldc == 0) tb = p.beta * load_as_f32<odt>(p.C, n);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = wm * WM + 32 * i + frag_row(r, h);
                float t = tb;
                if (p.C != nullptr && p.ldc != 0) {
                    const int m = min(m0 + ml, p.M - 1);
                    t = p.beta * load_as_f32<odt>(p.C, (int64_t)m * p.ldc + n);
                }
                const float y = __builtin_fmaf(p.alpha, acc[i][j][r], t);
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

// ============================================================ deep-ring kernel
// (N, K) layout, K a multiple of KS, no split.  NS LDS stages of KS k each
// (KS = 32: 64-byte LDS rows; KS = 64: 128-byte rows).  Within a 256-byte bank
// window of RPW = 256 / row-bytes rows, chunk c of row r sits at slot
// c ^ ((r / RPW) mod chunks-per-row), so the 16 rows one ds_read_b128 pass
// serves hit 16 distinct bank groups.  All NS stages are in flight with manual
// vmcnt waits and raw barriers, and the fragment reads of each step overlap
// the MFMAs of the one before:
//   iteration t (step-0 fragments of stage t already in registers):
//     for each step u but the last: read step u + 1 of stage t; MFMAs of u;
//     wait for this wave's loads of stage t + 1; barrier (now every wave has
//     finished reading stage t and stage t + 1 has landed everywhere);
//     issue stage t + NS into the buffer stage t used; read step 0 of stage
//     t + 1; MFMAs of the last step.
// Every wave issues exactly QW loads per stage, so the vmcnt thresholds are exact.
template <int idt, int odt, int BM, int BN, int WGM, int WGN, int NS, int KS = 32>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm32_ring(GemmParams p) {
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int ROWB = KS * 2;
    constexpr int CPR = ROWB / 16;                   // chunks per row
    constexpr int RPW = 256 / ROWB;                  // rows per 256-byte bank window
    constexpr int RPI = 1024 / ROWB;                 // rows per 1 KiB load instruction
    constexpr int SPS = KS / 16;                     // chain steps per stage
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int QA = BM / RPI, QB = BN / RPI;
    constexpr int QW = (QA + QB) / NW;
    static_assert(KS == 32 || KS == 64, "stage width");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
    static_assert(BM % RPI == 0 && BN % RPI == 0, "whole load instructions");
    static_assert((QA + QB) % NW == 0, "every wave must issue the same number of loads per stage");
    static_assert(NS >= 2 && QW * (NS - 1) <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r32 = lane & 31, h = lane >> 5;

    const int ntm = (p.M + BM - 1) / BM, ntn = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, ntm, ntn, 8, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nstages = p.total_steps / SPS;

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
        const int64_t koff = (int64_t)stage * ROWB;
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
        const int c = 2 * u + h;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WM + 32 * i + r32;
            af[i] = *reinterpret_cast<const u32x4 *>(As + row * ROWB + ((c ^ ((row / RPW) % CPR)) << 4));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * WN + 32 * j + r32;
            bfr[j] = *reinterpret_cast<const u32x4 *>(Bs + row * ROWB + ((c ^ ((row / RPW) % CPR)) << 4));
        }
    };
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = zero16();
    auto mma = [&](const u32x4 (&af)[FM], const u32x4 (&bfr)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = Mfma32<idt>::step(af[i], bfr[j], acc[i][j]);
    };

    // prologue: stages 0 .. NS-1 in flight; stage 0 landed everywhere; its step 0 read
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < nstages) issue(s);
    u32x4 fa[2][FM], fb[2][FN];
    if (nstages > 0) {
        if (nstages >= NS) BI_WAIT_VMCNT(QW * (NS - 1));
        else BI_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        read_step(0, 0, fa[0], fb[0]);
    }
    // steady state: every iteration issues stage t + NS and may leave NS - 2 stages in flight
    const int steady = nstages - NS;
    int t = 0;
    for (; t < steady; ++t) {
#pragma unroll
        for (int u = 0; u < SPS - 1; ++u) {
            read_step(t, u + 1, fa[(u + 1) & 1], fb[(u + 1) & 1]);
            mma(fa[u & 1], fb[u & 1]);
        }
        BI_WAIT_VMCNT(QW * (NS - 2));
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this wave's LDS reads of stage t are done
        __builtin_amdgcn_s_barrier();
        issue(t + NS);
        read_step(t + 1, 0, fa[SPS & 1], fb[SPS & 1]);
        mma(fa[(SPS - 1) & 1], fb[(SPS - 1) & 1]);
    }
    // tail: nothing left to issue; drain
    for (; t < nstages; ++t) {
#pragma unroll
        for (int u = 0; u < SPS - 1; ++u) {
            read_step(t, u + 1, fa[(u + 1) & 1], fb[(u + 1) & 1]);
            mma(fa[u & 1], fb[u & 1]);
        }
        BI_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();
        if (t + 1 < nstages) read_step(t + 1, 0, fa[SPS & 1], fb[SPS & 1]);
        mma(fa[(SPS - 1) & 1], fb[(SPS - 1) & 1]);
    }
    if constexpr (BM * BN * Elem<odt>::bytes <= NS * STAGE) {
        store_tile_staged<odt, BM, BN, WGM, WGN>(p, acc, m0, n0, lds);
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WN + 32 * j + r32;
                if (n >= p.N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * WM + 32 * i + frag_row(r, h);
                    if (m < p.M) epilogue<odt>(p, m, n, acc[i][j][r]);
                }
            }
    }
}

// ============================================================ plan + launch
struct Plan32 {
    int kind;                 // 0 skinny, 1 register-staged tile, 2 deep-ring tile, 3 cooperative strip
    int fm;                   // skinny / strip fragments
    int bm, bn;               // tile
};

// Deep-ring tiles, largest first.  The plan takes the largest tile that still
// yields about one tile per CU (192 of 256), else the smallest: below that the
// chip is short of waves, above it bigger tiles move fewer bytes per flop.
// Used only to pick a kernel, never changes bits.
struct Cfg32 { int bm, bn; };
static const Cfg32 kRing32[] = {{256, 256}, {256, 128}, {128, 128}, {128, 64}, {64, 64}};
constexpr long kRingMinTiles = 192;

// Strip instantiations (width, fragments, A rows per stage, stages, loader
// waves); used only to pick a kernel, never changes bits.  Narrow strips
// double the workgroups when 32-wide strips would leave CUs idle, and always
// for M <= 4; wider strips re-read A from L2 half as often.
struct StripCfg { int sw, fm, ar, ns, nl; };
static StripCfg strip_cfg(int M, int N) {
    const bool narrow = M <= 4 || (N + 15) / 16 <= 256;
    if (M <= 4) return StripCfg{16, 1, 4, 4, 3};
    if (M <= 16) return narrow ? StripCfg{16, 1, 16, 6, 3} : StripCfg{32, 1, 16, 6, 3};
    if (M <= 32) return narrow ? StripCfg{16, 1, 32, 4, 3} : StripCfg{32, 1, 32, 4, 3};
    return narrow ? StripCfg{16, 2, 64, 4, 2} : StripCfg{32, 2, 64, 3, 2};
}

static Plan32 plan32(int M, int N, int K, bool b_kn, int splits) {
    if (M <= 64) {
        if (!b_kn && splits == 1) return Plan32{3, M <= 32 ? 1 : 2, 0, 0};
        return Plan32{0, M <= 32 ? 1 : 2, 0, 0};
    }
    if (!b_kn && splits == 1 && K % 64 == 0) {
        for (const Cfg32 &c : kRing32) {
            const long tiles = (long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
            if (tiles >= kRingMinTiles) return Plan32{2, 0, c.bm, c.bn};
        }
        return Plan32{2, 0, 64, 64};
    }
    const long tiles128 = (long)((M + 127) / 128) * ((N + 127) / 128);
    if (tiles128 >= 256) return Plan32{1, 0, 128, 128};
    return Plan32{1, 0, 64, 64};
}

template <int idt, int odt>
static hipError_t launch32_typed(const GemmParams &p, bool b_kn, hipStream_t st) {
    const Plan32 pl = plan32(p.M, p.N, p.K, b_kn, p.splits);
    const unsigned sp = (unsigned)p.splits;
    if (pl.kind == 0) {
        const dim3 grid((p.N + 31) / 32, sp), block(64);
        if (pl.fm == 1) {
            if (b_kn) hipLaunchKernelGGL((gemm32_skinny_kn<idt, odt, 1, 16>), grid, block, 0, st, p);
            else hipLaunchKernelGGL((gemm32_skinny_nk<idt, odt, 1, 16>), grid, block, 0, st, p);
        } else {
            if (b_kn) hipLaunchKernelGGL((gemm32_skinny_kn<idt, odt, 2, 12>), grid, block, 0, st, p);
            else hipLaunchKernelGGL((gemm32_skinny_nk<idt, odt, 2, 12>), grid, block, 0, st, p);
        }
        return hipGetLastError();
    }
    if (pl.kind == 3) {
        const StripCfg c = strip_cfg(p.M, p.N);
        const dim3 grid((p.N + c.sw - 1) / c.sw), block(64 * (c.fm + c.nl));
        if (c.ar == 4) hipLaunchKernelGGL((gemm32_strip<idt, odt, 16, 1, 4, 4, 3>), grid, block, 0, st, p);
        else if (c.ar == 16 && c.sw == 16) hipLaunchKernelGGL((gemm32_strip<idt, odt, 16, 1, 16, 6, 3>), grid, block, 0, st, p);
        else if (c.ar == 16) hipLaunchKernelGGL((gemm32_strip<idt, odt, 32, 1, 16, 6, 3>), grid, block, 0, st, p);
        else if (c.ar == 32 && c.sw == 16) hipLaunchKernelGGL((gemm32_strip<idt, odt, 16, 1, 32, 4, 3>), grid, block, 0, st, p);
        else if (c.ar == 32) hipLaunchKernelGGL((gemm32_strip<idt, odt, 32, 1, 32, 4, 3>), grid, block, 0, st, p);
        else if (c.sw == 16) hipLaunchKernelGGL((gemm32_strip<idt, odt, 16, 2, 64, 4, 2>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((gemm32_strip<idt, odt, 32, 2, 64, 3, 2>), grid, block, 0, st, p);
        return hipGetLastError();
    }
    if (pl.kind == 2) {
        const unsigned tiles = (unsigned)(((p.M + pl.bm - 1) / pl.bm) * ((p.N + pl.bn - 1) / pl.bn));
        if (pl.bm == 256 && pl.bn == 256)
            hipLaunchKernelGGL((gemm32_ring<idt, odt, 256, 256, 2, 4, 5, 32>), dim3(tiles), dim3(512), 0, st, p);
        else if (pl.bm == 256)
            hipLaunchKernelGGL((gemm32_ring<idt, odt, 256, 128, 4, 2, 3, 64>), dim3(tiles), dim3(512), 0, st, p);
        else if (pl.bn == 128)
            hipLaunchKernelGGL((gemm32_ring<idt, odt, 128, 128, 2, 2, 3, 64>), dim3(tiles), dim3(256), 0, st, p);
        else if (pl.bm == 128)
            hipLaunchKernelGGL((gemm32_ring<idt, odt, 128, 64, 2, 2, 4, 64>), dim3(tiles), dim3(256), 0, st, p);
        else
            hipLaunchKernelGGL((gemm32_ring<idt, odt, 64, 64, 2, 2, 4, 64>), dim3(tiles), dim3(256), 0, st, p);
        return hipGetLastError();
    }
    if (pl.bm == 128) {
        const dim3 grid((p.N + 127) / 128, (p.M + 127) / 128, sp), block(256);
        if (b_kn) hipLaunchKernelGGL((gemm32_tile<idt, odt, true, 128, 128, 2, 2>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((gemm32_tile<idt, odt, false, 128, 128, 2, 2>), grid, block, 0, st, p);
    } else {
        const dim3 grid((p.N + 63) / 64, (p.M + 63) / 64, sp), block(256);
        if (b_kn) hipLaunchKernelGGL((gemm32_tile<idt, odt, true, 64, 64, 2, 2>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((gemm32_tile<idt, odt, false, 64, 64, 2, 2>), grid, block, 0, st, p);
    }
    return hipGetLastError();
}

hipError_t launch_gemm32(const GemmParams &p, int in_dt, int out_dt, bool b_kn, hipStream_t st) {
    if (in_dt == DT_BF16 && out_dt == DT_BF16) return launch32_typed<DT_BF16, DT_BF16>(p, b_kn, st);
    if (in_dt == DT_F16 && out_dt == DT_F16) return launch32_typed<DT_F16, DT_F16>(p, b_kn, st);
    if (in_dt == DT_BF16 && out_dt == DT_F32) return launch32_typed<DT_BF16, DT_F32>(p, b_kn, st);
    if (in_dt == DT_F16 && out_dt == DT_F32) return launch32_typed<DT_F16, DT_F32>(p, b_kn, st);
    return hipErrorInvalidValue;
}

const char *gemm32_kernel_name(int M, int N, int K, bool b_kn, int splits) {
    const Plan32 pl = plan32(M, N, K, b_kn, splits);
    static thread_local char buf[64];
    if (pl.kind == 0) snprintf(buf, sizeof buf, "gemm32_skinny_%s/fm%d", b_kn ? "kn" : "nk", pl.fm);
    else if (pl.kind == 3) {
        const StripCfg c = strip_cfg(M, N);
        snprintf(buf, sizeof buf, "gemm32_strip_nk/w%d_a%d", c.sw, c.ar);
    }
    else if (pl.kind == 1) snprintf(buf, sizeof buf, "gemm32_tile_%s/%dx%d", b_kn ? "kn" : "nk", pl.bm, pl.bn);
    else snprintf(buf, sizeof buf, "gemm32_ring_nk/%dx%d", pl.bm, pl.bn);
    return buf;
}

}  // namespace bi
