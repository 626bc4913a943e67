// Batch-invariant quantized linear for gfx950: y = x . dequant(Wq)^T + bias.
//
// Weights are 2, 4 or 8-bit group-wise affine (mlx-batch-invariant README,
// section "Quantized models": the weight is unpacked inside the K loop of an
// invariant kernel).  Each weight is dequantised as one fp32 fma of its
// group's scale and bias, rounded once to the input dtype:
//   w[n, k] = round_dt(fmaf(scale[n, k / gs], q[n, k], bias[n, k / gs])),
// q[n, k] being field k mod (32 / bits) of word k / (32 / bits) of row n,
// lowest bits first.  The MFMA chain and the epilogue are exactly those of
// bi_linear (16x16x32 steps in ascending k, fp32 accumulation, one fmaf with
// the bias, one rounding), so the result equals bi_linear on the dequantised
// weight bit for bit, and like it does not depend on M.
//
// Up to 64 rows: one workgroup of five wavefronts per (strip of 16 output
// columns, tile of 16 FM rows of x).  Wavefronts 1-4 unpack: a stage of 256 k
// (128 k for four row fragments) is 256 units, each thread loading its unit's
// packed words, scale and bias with one buffer load each and unpacking it into
// a double-buffered LDS stage (256 or 512-byte rows; the slot of a 16-byte
// chunk is swizzled by row and by chunk so both the strided unpacking writes
// and the consumer's 16-row reads are free of bank conflicts), several stages
// ahead through a register ring.  Wavefront 0 only consumes: it requests a
// stage's fragments together and runs every row fragment's chain.  x goes
// through the LDS stages as well, except for a single row, which the consumer
// loads itself.  Buffer resources end at the last byte of each operand's rows,
// so rows past N or M, k past K and stages past the end read as zeros with no
// clamping arithmetic.  Only ordinary loads are in flight and no branch
// surrounds them, so the compiler's waits are exact.  More rows: chunks of
// columns are dequantised into a workspace with the same arithmetic and the
// tile GEMM kernels of bi_linear run on them (the same chain, so the same
// bits; the choice of path depends on M only as a tile choice does).
#include "device.h"
#include "gemm_common.h"
#include "gemm16_store.h"
#include "qgemm.h"

#include <type_traits>

namespace bi {

namespace {

template <int BITS> struct Packed;
template <> struct Packed<2> { using T = uint32_t; };   // 8 values = half a word
template <> struct Packed<4> { using T = uint32_t; };   // 8 values = one word
template <> struct Packed<8> { using T = u32x2; };      // 8 values = two words

// two fp32 values rounded to nearest even in the input dtype, packed low | high << 16
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int dt> __device__ __forceinline__ uint32_t round_pack(float lo, float hi) {
    if constexpr (dt == DT_BF16) return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
    else return f32_to_f16(lo) | f32_to_f16(hi) << 16;        // each rounded from its fp32 value
}
template <int dt> __device__ __forceinline__ float half_to_f32(uint32_t h) {
    if constexpr (dt == DT_BF16) return bf16_to_f32(h);
    else return f16_to_f32(h);
}

// LDS writes of this wavefront done, then the workgroup barrier; loads still in flight stay in flight
// (__syncthreads would also wait for every outstanding global load, emptying the prefetch ring)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
}

}  // namespace

// Byte b of x as an fp32 value (v_cvt_f32_ubyte<b>).
template <int B> __device__ __forceinline__ float byte_f32(uint32_t x) { return (float)((x >> (8 * B)) & 0xFFu); }
// Hides x's known bits from the optimiser, so that masked fields are converted with the byte-select
// converts above instead of being re-extracted one at a time.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm("" : "+v"(x));
    return x;
}

// Stage geometry of the fused kernel: k per stage, values each producer thread unpacks per stage (one
// load of VPT * BITS / 8 bytes, one scale and one bias: VPT never exceeds a group), packed words per
// unit, weight stages in flight per thread; x rows staged in LDS per stage (16 FM, or XS < 16 when the
// call has at most XS rows).
template <int FM, int BITS, int NB, int XS, int KS_> struct QStrip {
    static constexpr int KS = KS_;
    static constexpr int VPT = NB * KS / 16;                     // 16 NB rows x KS values over 256 threads
    static constexpr int TPR = 16 / NB;                          // producer threads per weight row
    static constexpr int WPU = VPT * BITS >= 32 ? VPT * BITS / 32 : 1;
    static constexpr bool HALF = VPT * BITS < 32;              // 2 bits, 8 values: half a word
    static constexpr int DEPTH = WPU >= 4 ? 4 : 8;
    // x goes through LDS, XS rows of KS values: XU 16-byte chunks per producer thread per stage (the last
    // threads may have none), XD stages ahead
    static constexpr int XCH = XS * KS / 8;
    static constexpr int XU = (XCH + 255) / 256;
    static constexpr int XD = FM == 1 ? 4 : 1;
};

// LDS slot of weight chunk c (16 bytes) in strip row r: the row bits keep the consumer's 16-row reads
// conflict-free, the chunk-index bits (c / CPT, CPT chunks per producer thread) do the same for the
// producers' strided writes; a bijection on the chunks of a row.
template <int CPT> __device__ __forceinline__ int wslot(int c, int r) {
    if constexpr (CPT == 1) return c ^ (r & 15);
    else return c ^ (r & 15) ^ ((c / CPT) & 7);
}

struct u32x8 {
    u32x4 lo, hi;
};
template <int N> struct Words;
template <> struct Words<1> { using T = uint32_t; };
template <> struct Words<2> { using T = u32x2; };
template <> struct Words<4> { using T = u32x4; };
template <> struct Words<8> { using T = u32x8; };

__device__ __forceinline__ int sat_off(uint32_t lane_off, uint32_t st_off) {
    return (int)__builtin_elementwise_add_sat(lane_off, st_off);
}
// packed words of one unit at lane_off + st_off (saturating: an offset marked out of range stays so)
template <int WPU>
__device__ __forceinline__ typename Words<WPU>::T load_words(__amdgpu_buffer_rsrc_t r, uint32_t lane_off,
                                                             uint32_t st_off) {
    if constexpr (WPU == 1) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, sat_off(lane_off, st_off), 0, 0);
    } else if constexpr (WPU == 2) {
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, sat_off(lane_off, st_off), 0, 0));
    } else if constexpr (WPU == 4) {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, sat_off(lane_off, st_off), 0, 0));
    } else {
        u32x8 w;
        w.lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, sat_off(lane_off, st_off), 0, 0));
        w.hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, sat_off(lane_off + 16u, st_off), 0, 0));
        return w;
    }
}
template <int WPU> __device__ __forceinline__ uint32_t word_at(const typename Words<WPU>::T &w, int i) {
    if constexpr (WPU == 1) return w;
    else if constexpr (WPU == 8) return i < 4 ? w.lo[i] : w.hi[i - 4];
    else return w[i];
}

// Fields 8 h .. 8 h + 7 of a unit as fp32 values in k order (fields lowest bits first).  hshift
// selects the half word of a 2-bit unit of 8 values.
template <int BITS, int WPU>
__device__ __forceinline__ void unpack8(const typename Words<WPU>::T &w, int h, uint32_t hshift, float (&f)[8]) {
    if constexpr (BITS == 8) {
        const uint32_t x0 = word_at<WPU>(w, 2 * h), x1 = word_at<WPU>(w, 2 * h + 1);
        f[0] = byte_f32<0>(x0);
        f[1] = byte_f32<1>(x0);
        f[2] = byte_f32<2>(x0);
        f[3] = byte_f32<3>(x0);
        f[4] = byte_f32<0>(x1);
        f[5] = byte_f32<1>(x1);
        f[6] = byte_f32<2>(x1);
        f[7] = byte_f32<3>(x1);
    } else if constexpr (BITS == 4) {
        const uint32_t x = word_at<WPU>(w, h);
        const uint32_t lo = opaque(x & 0x0F0F0F0Fu), hi = opaque((x >> 4) & 0x0F0F0F0Fu);
        f[0] = byte_f32<0>(lo);
        f[1] = byte_f32<0>(hi);
        f[2] = byte_f32<1>(lo);
        f[3] = byte_f32<1>(hi);
        f[4] = byte_f32<2>(lo);
        f[5] = byte_f32<2>(hi);
        f[6] = byte_f32<3>(lo);
        f[7] = byte_f32<3>(hi);
    } else {
        const uint32_t x = word_at<WPU>(w, h / 2) >> (hshift + 16u * (uint32_t)(h & 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t t = opaque((x >> (2 * j)) & 0x03030303u);   // byte b: field 4 b + j
            f[j] = byte_f32<0>(t);
            f[4 + j] = byte_f32<1>(t);
        }
    }
}

template <int dt, int FM, int BITS, int NB, int XS, int KS_>
__global__ __launch_bounds__(64 * (NB + 4)) void qgemm16_strip(QGemmParams q) {
    using G = QStrip<FM, BITS, NB, XS, KS_>;
    constexpr int KS = G::KS, VPT = G::VPT, WPU = G::WPU, QD = G::DEPTH, XU = G::XU, XD = G::XD;
    constexpr int XCH = G::XCH;
    static_assert(XS <= 16 * FM, "x rows staged");
    constexpr int ROWB = KS * 2;                 // bytes of one LDS row (KS values of 16 bits)
    constexpr int CH = ROWB / 16;                // 16-byte chunks per LDS row
    constexpr int AR = 16 * FM;                  // x rows per workgroup
    constexpr int WROWS = 16 * NB;               // weight rows (output columns) per workgroup
    constexpr int STAGE = (WROWS + XS) * ROWB;
    constexpr int SPS = KS / 32;                 // chain steps per stage
    constexpr int HS = FM == 1 ? (SPS < 8 ? SPS : 8) : (SPS < 4 ? SPS : 4);   // steps read together
    constexpr uint32_t OOB = 0x80000000u;        // offset past every resource: the load returns zeros
    using W = typename Words<WPU>::T;
    static_assert(QD % XD == 0 && QD % 2 == 0, "ring geometry");
    __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];

    const GemmParams &p = q.g;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int nstrip = (p.N + WROWS - 1) / WROWS;
    const int n0 = (blockIdx.x % nstrip) * WROWS;
    const int m0 = (blockIdx.x / nstrip) * AR;
    const int nst = (p.K + KS - 1) / KS;
    const int nround = (nst + QD - 1) / QD * QD;     // stages the loops run (whole rounds of QD)
    const int rows = min(WROWS, p.N - n0), xrows = min(AR, p.M - m0);

    // Buffer resources of this workgroup's rows, each ending at the last byte of its last row's K
    // values (none at all when K = 0, where the tensors may be empty).  Offsets are 32-bit and
    // combined with saturating adds, so an offset marked out of range stays out of range; anything
    // past a resource (rows past N or M, k past K, stages past the end) reads as zero.  The host keeps
    // each resource below 2^31 bytes.
    const uint32_t kb = p.K > 0 ? 1u : 0u;
    const uint32_t xrow_b = (uint32_t)p.lda * 2u;
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(p.A) + (int64_t)m0 * p.lda * 2), 0,
        (int)(kb * ((uint32_t)(xrows - 1) * xrow_b + (uint32_t)p.K * 2u)), 0x00020000);
    auto stage_off = [&](int s, uint32_t per) { return s < nst ? (uint32_t)s * per : OOB; };

    if (wave < NB) {
        // consumer of 16-column strip cb: FM row fragments against its columns; every fragment of a
        // stage is requested before its first step, so the steps wait on LDS once per stage; k past K
        // is never read
        const int cb = wave;
        const int r16 = lane & 15, g = lane >> 4;
        f32x4 acc[FM];
#pragma unroll
        for (int f = 0; f < FM; ++f) acc[f] = zero4();
        lds_barrier();                                   // stage 0 unpacked
        constexpr int CU = 2;                            // consumer unroll: buffer parity constant
        for (int s0 = 0; s0 < nround; s0 += CU) {
#pragma unroll
            for (int j = 0; j < CU; ++j) {
                const int s = s0 + j;
                const char *buf = lds + (j & 1) * STAGE;
#pragma unroll
                for (int h = 0; h < SPS / HS; ++h) {          // HS steps at a time
                    u32x4 b[HS], a[HS][FM];
#pragma unroll
                    for (int v = 0; v < HS; ++v) {
                        const int u = h * HS + v, c = 4 * u + g;
                        b[v] = *reinterpret_cast<const u32x4 *>(buf + (16 * cb + r16) * ROWB +
                                                                 (wslot<VPT / 8>(c, r16) << 4));
#pragma unroll
                        for (int f = 0; f < FM; ++f) {
                            // rows past XS (never stored: the call has at most XS rows) read row XS - 1
                            const int row = WROWS + min(16 * f + r16, XS - 1);
                            a[v][f] = *reinterpret_cast<const u32x4 *>(buf + row * ROWB + ((c ^ (row & 15)) << 4));
                        }
                    }
                    const int u0 = s * SPS + h * HS;
                    if (u0 + HS <= p.total_steps) {           // uniform: whole steps of the chain
#pragma unroll
                        for (int v = 0; v < HS; ++v)
#pragma unroll
                            for (int f = 0; f < FM; ++f) acc[f] = Mfma<dt>::step(a[v][f], b[v], acc[f]);
                    } else {                                  // the end of K: its steps before K only
#pragma unroll
                        for (int v = 0; v < HS; ++v)
                            if (u0 + v < p.total_steps)
#pragma unroll
                                for (int f = 0; f < FM; ++f) acc[f] = Mfma<dt>::step(a[v][f], b[v], acc[f]);
                    }
                }
                lds_barrier();                           // stage s read; stage s + 1 unpacked
            }
        }
        const int n = n0 + 16 * cb + r16;
        if (n >= p.N) return;
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 16 * f + 4 * g + i;
                if (m < p.M) epilogue<dt>(p, m, n, acc[f][i]);
            }
        return;
    }

    // producers (the four wavefronts after the consumers): unpack the weights (and copy x, several
    // fragments) into the LDS stages
    if (nst == 0) {                                      // K = 0: nothing to load
        lds_barrier();
        return;
    }
    const int tid = threadIdx.x - 64 * NB;
    const uint32_t wrow_b = (uint32_t)q.ldwq * 4u, srow_b = (uint32_t)q.ldsb * 2u;
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(q.wq + (int64_t)n0 * q.ldwq), 0,
        (int)((uint32_t)(rows - 1) * wrow_b + (uint32_t)p.K / 8u * (uint32_t)BITS), 0x00020000);
    const uint32_t sb_records = (uint32_t)(rows - 1) * srow_b + ((uint32_t)p.K >> q.group_shift) * 2u;
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(q.scales) + (int64_t)n0 * q.ldsb * 2), 0, (int)sb_records,
        0x00020000);
    const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(q.biases) + (int64_t)n0 * q.ldsb * 2), 0, (int)sb_records,
        0x00020000);

    // this thread's weight unit: row wr of the workgroup's rows, VPT values at k = KS s + VPT wc of stage s
    const int wr = tid / G::TPR, wc = tid % G::TPR;
    const uint32_t w_lane = wr < rows ? (uint32_t)wr * wrow_b + (uint32_t)(VPT * wc * BITS / 8) / 4u * 4u : OOB;
    const uint32_t s_lane = wr < rows ? (uint32_t)wr * srow_b + (uint32_t)((VPT * wc) >> q.group_shift) * 2u : OOB;
    const uint32_t hshift = G::HALF ? 16u * (uint32_t)(wc & 1) : 0u;
    constexpr uint32_t W_STAGE = KS * BITS / 8;                        // packed bytes of a row per stage
    const uint32_t S_STAGE = (uint32_t)(KS >> q.group_shift) * 2u;     // scale bytes of a row per stage

    W raw[QD];
    uint32_t rsc[QD], rbi[QD];
    auto loadW = [&](int s, W &r, uint32_t &sc, uint32_t &bi) {
        r = load_words<WPU>(wres, w_lane, stage_off(s, W_STAGE));
        const int so = sat_off(s_lane, stage_off(s, S_STAGE));
        sc = __builtin_amdgcn_raw_buffer_load_b16(sres, so, 0, 0);
        bi = __builtin_amdgcn_raw_buffer_load_b16(bres, so, 0, 0);
    };
    // unpack into LDS: chunk c of strip row r at slot wslot(c, r)
    auto storeW = [&](const W &r, uint32_t scr, uint32_t bir, char *buf) {
        const float sc = half_to_f32<dt>(scr), bi = half_to_f32<dt>(bir);
#pragma unroll
        for (int h = 0; h < VPT / 8; ++h) {
            float w[8];
            unpack8<BITS, WPU>(r, h, hshift, w);
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = __builtin_fmaf(sc, w[j], bi);
            const int c = (VPT / 8) * wc + h;
            *reinterpret_cast<u32x4 *>(buf + wr * ROWB + (wslot<VPT / 8>(c, wr) << 4)) =
                u32x4{round_pack<dt>(w[0], w[1]), round_pack<dt>(w[2], w[3]), round_pack<dt>(w[4], w[5]),
                      round_pack<dt>(w[6], w[7])};
        }
    };
    // several x fragments: XU chunks of 16 bytes per thread per stage, in a ring of XD stages
    constexpr int XUA = XU > 0 ? XU : 1;
    uint32_t x_lane[XUA];
#pragma unroll
    for (int f = 0; f < XUA; ++f) {
        const int u = tid + 256 * f, r = u / CH, c = u % CH;
        x_lane[f] = (XCH % 256 == 0 || u < XCH) && r < xrows ? (uint32_t)r * xrow_b + (uint32_t)c * 16u : OOB;
    }
    u32x4 araw[XD][XUA];
    auto loadA = [&](int s, u32x4 (&a)[XUA]) {
        const uint32_t so = stage_off(s, (uint32_t)ROWB);
#pragma unroll
        for (int f = 0; f < XU; ++f)
            a[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, sat_off(x_lane[f], so), 0, 0));
    };
    auto storeA = [&](const u32x4 (&a)[XUA], char *buf) {
#pragma unroll
        for (int f = 0; f < XU; ++f) {
            const int u = tid + 256 * f, r = u / CH, c = u % CH;
            const int row = WROWS + r;
            if (XCH % 256 == 0 || u < XCH) *reinterpret_cast<u32x4 *>(buf + row * ROWB + ((c ^ (row & 15)) << 4)) = a[f];
        }
    };

    // prologue: rings filled with stages 0 .. depth-1, stage 0 unpacked, the freed slots refilled
#pragma unroll
    for (int j = 0; j < XD; ++j) loadA(j, araw[j]);
#pragma unroll
    for (int j = 0; j < QD; ++j) loadW(j, raw[j], rsc[j], rbi[j]);
    storeA(araw[0], lds);
    loadA(XD, araw[0]);
    storeW(raw[0], rsc[0], rbi[0], lds);
    loadW(QD, raw[0], rsc[0], rbi[0]);
    lds_barrier();
    // while the consumer reads stage s: store x of stage s + 1 and refill its ring slot with stage
    // s + 1 + XD; unpack the weights of stage s + 1 into the other buffer and refill that slot with
    // stage s + 1 + QD.  No branch around loads (stages past the end read as zeros and are never
    // consumed), so the compiler counts each wait exactly.
    for (int s0 = 0; s0 < nround; s0 += QD) {
#pragma unroll
        for (int j = 0; j < QD; ++j) {
            const int s = s0 + j;
            const int jn = (j + 1) % QD;                  // constants once the loop is unrolled
            const int xn = (j + 1) % XD;
            char *nxt = lds + ((j + 1) & 1) * STAGE;     // s0 is a multiple of QD (even)
            storeA(araw[xn], nxt);
            loadA(s + 1 + XD, araw[xn]);
            storeW(raw[jn], rsc[jn], rbi[jn], nxt);
            loadW(s + 1 + QD, raw[jn], rsc[jn], rbi[jn]);
            lds_barrier();
        }
    }
}

// More rows (M > 64, K a multiple of 128): the tile scheme of bi_linear's mid-M kernel (LDS stages of KS
// k with 2 KS-byte rows, chunk c of row r at slot c ^ swz(r), fragments read DR chain steps ahead, one
// barrier per stage whose buffer refill lags a stage behind) with the weight rows dequantised on their way
// into LDS.  x arrives by direct-to-LDS loads as in the 16-bit kernel.  For its share of a stage's weight
// rows, each thread owns one 16-byte chunk (8 values) per piece: direct-to-LDS loads bring the chunk's
// packed words, scale and bias into a small staging area of its own, R stages ahead; when the stage's
// buffer is handed over the thread reads them back, unpacks them with the arithmetic of the kernels above
// and writes the chunk where the 16-bit kernel's direct-to-LDS load would have put it.  No load returns a
// register and the loads are issued as asm, so every wait is one of the kernel's own counted waits.  The MFMA side is the 16-bit kernel's:
// every element is bi_linear's chain on the dequantised weight.  No workspace.
// Direct-to-LDS loads written as asm (M0 = the wave-uniform LDS address; lane L's 16 bytes at M0 + 16 L,
// its 4 or 2 bytes at M0 + 4 L):
// the compiler then neither reorders them nor adds waits of its own for them (it would wait for every
// such load in flight before the next LDS read).  The kernel counts them itself; they write no register.
__device__ __forceinline__ void qdma16(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void qdma4(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void qdma2(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_ushort %1, off" ::"s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)BI_LDS_PTR(p); }

template <int KS> __device__ __forceinline__ int qtile_swz(int row) {
    if constexpr (KS == 128) return row & 15;
    else return (row >> 1) & 7;
}
constexpr int qtile_gcd(int a, int b) { return b == 0 ? a : qtile_gcd(b, a % b); }

template <int dt, int BITS, int BM, int BN, int WGM, int WGN, int NS, int KS, int DR>
__global__ __launch_bounds__(64 * WGM * WGN) void qgemm16_tile(QGemmParams q) {
    const GemmParams &p = q.g;
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int ROWB = 2 * KS, CPR = KS / 8, RPI = 64 / CPR;
    constexpr int STAGE = (BM + BN) * ROWB;
    constexpr int QA = BM / RPI, QB = BN / RPI;          // 1 KiB pieces of a stage: x rows, weight rows
    constexpr int QAW = QA / NW, QBW = QB / NW;          // per wavefront
    constexpr int SPS = KS / 32;                         // chain steps per stage
    constexpr int NSET = DR + 1;
    constexpr int R = NS - 2;                            // stages of packed weights staged ahead
    constexpr int U = NSET * R * SPS / qtile_gcd(NSET, R * SPS);   // steps per unrolled iteration
    constexpr int WPC = BITS == 8 ? 2 : 1;               // packed words per 8-value chunk
    constexpr int L = QAW + QBW * (WPC + 2);             // loads a wavefront issues per stage
    constexpr int PIECE = 64 * 4 * (WPC + 2);            // staging bytes of one piece: words, scales, biases
    constexpr int SSTAGE = NW * QBW * PIECE;             // staging bytes of one stage
    static_assert(KS == 64 || KS == 128, "stage width");
    static_assert(WM % 16 == 0 && WN % 16 == 0 && QA % NW == 0 && QB % NW == 0, "tile geometry");
    static_assert(NS >= 3 && L * (NS - 2) <= 63, "vmcnt range");
    static_assert(DR >= 1 && DR <= SPS, "read-ahead");
    __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];
    __shared__ __attribute__((aligned(256))) char stg[R * SSTAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int r16 = lane & 15, g = lane >> 4;

    const int ntm = (p.M + BM - 1) / BM, ntn = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, ntm, ntn, 8, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nstages = p.K / KS;
    const int nsteps = nstages * SPS;

    // x: piece j of this wavefront covers stage rows RPI (wave + NW j) .. + RPI - 1 (as the 16-bit kernel)
    const char *asrc[QAW];
#pragma unroll
    for (int j = 0; j < QAW; ++j) {
        const int rloc = (wave + NW * j) * RPI + lane / CPR;
        const int c = (lane % CPR) ^ qtile_swz<KS>(rloc);
        asrc[j] = static_cast<const char *>(p.A) + (int64_t)min(m0 + rloc, p.M - 1) * p.lda * 2 + c * 16;
    }
    // weights: piece j covers stage rows BM + RPI (wave + NW j) ..; this lane's chunk c of weight row n
    const char *wsrc[QBW];
    const char *ssrc[QBW], *bsrc[QBW];
    int bchunk[QBW];
#pragma unroll
    for (int j = 0; j < QBW; ++j) {
        const int qb = wave + NW * j;
        const int rloc = BM + qb * RPI + lane / CPR;
        const int c = (lane % CPR) ^ qtile_swz<KS>(rloc);
        const int n = min(n0 + qb * RPI + lane / CPR, p.N - 1);
        bchunk[j] = c;
        wsrc[j] = reinterpret_cast<const char *>(q.wq + (int64_t)n * q.ldwq) + (8 * c * BITS) / 32 * 4;
        ssrc[j] = static_cast<const char *>(q.scales) + (int64_t)n * q.ldsb * 2;
        bsrc[j] = static_cast<const char *>(q.biases) + (int64_t)n * q.ldsb * 2;
    }
    // staging of stage st (slot st mod R): piece j of this wavefront at wave, j: words [WPC][64], then
    // scales [64], biases [64], each lane's in 4 bytes (a 2-byte direct-to-LDS load fills lane L's value
    // into bytes 4 L, 4 L + 1 and zeroes the other two)
    auto piece_at = [&](int slot, int j) { return stg + slot * SSTAGE + (wave * QBW + j) * PIECE; };
    auto stage_packed = [&](int st, int slot) {
        const int sc = min(st, nstages - 1);           // past the end: the last stage again, never read
#pragma unroll
        for (int j = 0; j < QBW; ++j) {
            char *pc = piece_at(slot, j);
            const int grp = (sc * KS + 8 * bchunk[j]) >> q.group_shift;
            const char *w = wsrc[j] + (int64_t)sc * (KS * BITS / 8);
#pragma unroll
            for (int u = 0; u < WPC; ++u) qdma4(w + 4 * u, lds_addr(pc + 256 * u));
            qdma2(ssrc[j] + 2 * grp, lds_addr(pc + 256 * WPC));
            qdma2(bsrc[j] + 2 * grp, lds_addr(pc + 256 * WPC + 256));
        }
    };
    // stage st: its weight chunks from the staging slot into its LDS buffer, then the packed loads of stage
    // st + R into the slot just read, then its x pieces.  L loads per stage in every case (stages past the
    // end load the last stage again into places nobody reads), so every count of loads in flight is exact.
    auto fill = [&](int st, int slot) {
        char *buf = lds + (st % NS) * STAGE;
#pragma unroll
        for (int j = 0; j < QBW; ++j) {
            const char *pc = piece_at(slot, j);
            const float sc = half_to_f32<dt>(*reinterpret_cast<const uint16_t *>(pc + 256 * WPC + 4 * lane));
            const float bi = half_to_f32<dt>(*reinterpret_cast<const uint16_t *>(pc + 256 * WPC + 256 + 4 * lane));
            float f[8];
            if constexpr (BITS == 8) {
                const u32x2 w = u32x2{*reinterpret_cast<const uint32_t *>(pc + 4 * lane),
                                      *reinterpret_cast<const uint32_t *>(pc + 256 + 4 * lane)};
                unpack8<8, 2>(w, 0, 0u, f);
            } else {
                const uint32_t w = *reinterpret_cast<const uint32_t *>(pc + 4 * lane);
                if constexpr (BITS == 4) unpack8<4, 1>(w, 0, 0u, f);
                else unpack8<2, 1>(w, 0, 16u * (uint32_t)(bchunk[j] & 1), f);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = __builtin_fmaf(sc, f[e], bi);
            *reinterpret_cast<u32x4 *>(buf + (QA + wave + NW * j) * 1024 + lane * 16) =
                u32x4{round_pack<dt>(f[0], f[1]), round_pack<dt>(f[2], f[3]), round_pack<dt>(f[4], f[5]),
                      round_pack<dt>(f[6], f[7])};
        }
        stage_packed(st + R, slot);
        const int64_t koff = (int64_t)min(st, nstages - 1) * ROWB;
#pragma unroll
        for (int j = 0; j < QAW; ++j) qdma16(asrc[j] + koff, lds_addr(buf + (wave + NW * j) * 1024));
    };

    int aoff[FM], boff[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) aoff[i] = (wm * WM + 16 * i + r16) * ROWB;
#pragma unroll
    for (int j = 0; j < FN; ++j) boff[j] = (BM + wn * WN + 16 * j + r16) * ROWB;
    const int swz = qtile_swz<KS>(r16);
    u32x4 fa[NSET][FM], fb[NSET][FN];
    auto read_step = [&](int step, u32x4 (&a)[FM], u32x4 (&b)[FN]) {
        const char *buf = lds + ((step / SPS) % NS) * STAGE;
        const int c = 4 * (step % SPS) + g;
        const int off = (c ^ swz) << 4;
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const u32x4 *>(buf + aoff[i] + off);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const u32x4 *>(buf + boff[j] + off);
    };
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = zero4();

    // prologue: packed stages 0 .. R - 1 staged; stages 0 .. NS - 2 filled (the fill of stage st first
    // waits for its own staged data, issued before the x pieces of stage st - R); stage 0 landed
    // everywhere; steps 0 .. DR - 1 read
    if (nstages > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) stage_packed(r, r);
        BI_WAIT_VMCNT(0);
#pragma unroll
        for (int st = 0; st < NS - 1; ++st) {
            if (st >= R) BI_WAIT_VMCNT(QAW + L * (R - 1));    // stage st's staged data (fill st - R) landed
            fill(st, st % R);
        }
        BI_WAIT_VMCNT(L * (NS - 2));                  // this wavefront's x pieces of stage 0 landed
        __builtin_amdgcn_s_waitcnt(0xc07f);           // and its chunk writes done
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int d = 0; d < DR; ++d)
            if (d < nsteps) read_step(d, fa[d], fb[d]);
    }
    // step s: read step s + DR (entering stage tr first waits for it, which also covers the staged data of
    // stage tr + NS - 2 = tr + R, issued in the fill of stage tr before its x pieces, and fills that stage
    // into the buffer of stage tr - 2), then the MFMAs of step s.  s0 is a multiple of U (a multiple of R
    // stages), so the staging slot of a stage is a constant in the unrolled body.  Whole iterations run
    // without a condition; the rest runs with the checks.
    auto step = [&](int s0, int d, auto checked) {
        constexpr bool CHECK = decltype(checked)::value;
        const int s = s0 + d;
        if (CHECK && s >= nsteps) return;
        const int sr_ = s + DR;
        if (!CHECK || sr_ < nsteps) {
            if ((d + DR) % SPS == 0) {
                const int tr = sr_ / SPS;              // the stage being entered (>= 1)
                BI_WAIT_VMCNT(L * (NS - 3));
                __builtin_amdgcn_s_waitcnt(0xc07f);
                __builtin_amdgcn_s_barrier();
                fill(tr + NS - 2, ((d + DR) / SPS + NS - 2) % R);   // slot: a constant once unrolled
            }
            read_step(sr_, fa[(d + DR) % NSET], fb[(d + DR) % NSET]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = Mfma<dt>::step(fa[d % NSET][i], fb[d % NSET][j], acc[i][j]);
    };
    const int nfull = nsteps > DR ? (nsteps - DR) / U : 0;
    for (int it = 0; it < nfull; ++it) {
#pragma unroll
        for (int d = 0; d < U; ++d) step(it * U, d, std::false_type{});
    }
    for (int s0 = nfull * U; s0 < nsteps; s0 += U) {
#pragma unroll
        for (int d = 0; d < U; ++d) step(s0, d, std::true_type{});
    }
    BI_WAIT_VMCNT(0);                                  // no load of this wavefront outlives the kernel's LDS
    if constexpr (BM * BN * 2 <= NS * STAGE) {
        store_tile16<dt, BM, BN, WGM, WGN>(p, acc, m0, n0, lds);
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WN + 16 * j + r16;
                if (n >= p.N) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + wm * WM + 16 * i + 4 * g + e;
                    if (m < p.M) epilogue<dt>(p, m, n, acc[i][j][e]);
                }
            }
    }
}

// Large batches: the weights of columns [n0, n0 + nc) dequantised into an (nc, K) buffer of the input
// dtype with exactly the arithmetic of storeW above (one fmaf, one rounding), for the tile GEMM kernels.
// One thread per 8 values.
template <int dt, int BITS>
__global__ __launch_bounds__(256) void qdequant16(QGemmParams q, int n0, int nc, void *out) {
    constexpr int PER = 32 / BITS;
    constexpr uint32_t FIELD = (1u << BITS) - 1u;
    using P = typename Packed<BITS>::T;
    const int64_t units = (int64_t)nc * (q.g.K / 8);
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= units) return;
    const int r = (int)(id / (q.g.K / 8)), k = (int)(id % (q.g.K / 8)) * 8;
    const int n = n0 + r;
    const uint32_t *wrow = q.wq + (int64_t)n * q.ldwq;
    P raw;
    if constexpr (BITS == 8) raw = *reinterpret_cast<const u32x2 *>(wrow + k / PER);
    else raw = wrow[k / PER];
    const int grp = k >> q.group_shift;
    const float sc = half_to_f32<dt>(static_cast<const uint16_t *>(q.scales)[(int64_t)n * q.ldsb + grp]);
    const float bi = half_to_f32<dt>(static_cast<const uint16_t *>(q.biases)[(int64_t)n * q.ldsb + grp]);
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t f;
        if constexpr (BITS == 8) f = (raw[j >> 2] >> (8 * (j & 3))) & FIELD;
        else if constexpr (BITS == 4) f = (raw >> (4 * j)) & FIELD;
        else f = (raw >> (16 * ((k >> 3) & 1) + 2 * j)) & FIELD;
        w[j] = __builtin_fmaf(sc, (float)f, bi);
    }
    *reinterpret_cast<u32x4 *>(static_cast<char *>(out) + ((int64_t)r * q.g.K + k) * 2) =
        u32x4{round_pack<dt>(w[0], w[1]), round_pack<dt>(w[2], w[3]), round_pack<dt>(w[4], w[5]),
              round_pack<dt>(w[6], w[7])};
}

int qgemm_tile_rows(int M) { return M <= 16 ? 16 : (M <= 32 ? 32 : 64); }

bool qgemm_uses_workspace(int64_t M, int64_t K) { return M > QGEMM_FUSED_MAX_M && K % QGEMM_TILE_K != 0; }

size_t qgemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!qgemm_uses_workspace(M, K) || N <= 0 || K <= 0) return 0;
    const int64_t nc = N < QGEMM_CHUNK_N ? N : QGEMM_CHUNK_N;
    return (size_t)(nc * K * 2);
}

template <int dt, int FM, int NB, int XS, int KS>
static hipError_t launch_fm(const QGemmParams &q, hipStream_t st) {
    const int64_t nstrip = (q.g.N + 16 * NB - 1) / (16 * NB), ntile = (q.g.M + 16 * FM - 1) / (16 * FM);
    const int64_t nwg = nstrip * ntile;
    if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nwg), block(64 * (NB + 4));
    if (q.bits == 2) hipLaunchKernelGGL((qgemm16_strip<dt, FM, 2, NB, XS, KS>), grid, block, 0, st, q);
    else if (q.bits == 4) hipLaunchKernelGGL((qgemm16_strip<dt, FM, 4, NB, XS, KS>), grid, block, 0, st, q);
    else if (q.bits == 8) hipLaunchKernelGGL((qgemm16_strip<dt, FM, 8, NB, XS, KS>), grid, block, 0, st, q);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int dt>
static hipError_t launch_dt(const QGemmParams &q, hipStream_t st) {
    const int rows = qgemm_tile_rows(q.g.M);
    // two 16-column strips per workgroup once N is wide: x is then read half as often
    const bool wide = (q.g.N + 15) / 16 > QGEMM_WIDE_STRIPS;
    // one 16-row fragment: 512-k stages for one strip per workgroup (8.1 -> 7.8 us at N = 4096, M = 1),
    // 256 for two (512 was slower there); calls of at most four rows stage four x rows (more workgroups
    // per CU: M = 1 7.9 -> 7.0 us at N = 4096, 15.0 -> 13.8 at N = 14336)
    if (rows == 16 && q.g.M <= 4) return wide ? launch_fm<dt, 1, 2, 4, 256>(q, st) : launch_fm<dt, 1, 1, 4, 512>(q, st);
    if (rows == 16) return wide ? launch_fm<dt, 1, 2, 16, 256>(q, st) : launch_fm<dt, 1, 1, 16, 512>(q, st);
    if (rows == 32) return wide ? launch_fm<dt, 2, 2, 32, 256>(q, st) : launch_fm<dt, 2, 1, 32, 256>(q, st);
    return wide ? launch_fm<dt, 4, 2, 64, 128>(q, st) : launch_fm<dt, 4, 1, 64, 128>(q, st);
}

// More rows: 128 x 128 tiles when they give about one tile per CU, else 64 x 64 (the 16-bit plan's
// thresholds); either way the chain of every element is bi_linear's.
template <int dt, int BITS>
static hipError_t launch_tile_bits(const QGemmParams &q, hipStream_t st) {
    const int64_t t128 = ((q.g.M + 127) / 128) * ((q.g.N + 127) / 128);
    if (t128 >= 192) {
        const dim3 grid((unsigned)t128);
        hipLaunchKernelGGL((qgemm16_tile<dt, BITS, 128, 128, 2, 4, 4, 64, 2>), grid, dim3(512), 0, st, q);
    } else {
        const int64_t t64 = ((q.g.M + 63) / 64) * ((q.g.N + 63) / 64);
        if (t64 > INT32_MAX) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((qgemm16_tile<dt, BITS, 64, 64, 2, 4, 4, 128, 2>), dim3((unsigned)t64), dim3(512), 0, st, q);
    }
    return hipGetLastError();
}

template <int dt>
static hipError_t launch_tile(const QGemmParams &q, hipStream_t st) {
    if (q.bits == 2) return launch_tile_bits<dt, 2>(q, st);
    if (q.bits == 4) return launch_tile_bits<dt, 4>(q, st);
    if (q.bits == 8) return launch_tile_bits<dt, 8>(q, st);
    return hipErrorInvalidValue;
}

template <int dt>
static hipError_t launch_chunks(const QGemmParams &q, void *ws, hipStream_t st) {
    // columns in chunks of at most QGEMM_CHUNK_N: dequantise into ws, then the invariant GEMM on them
    for (int n0 = 0; n0 < q.g.N; n0 += (int)QGEMM_CHUNK_N) {
        const int nc = q.g.N - n0 < QGEMM_CHUNK_N ? q.g.N - n0 : (int)QGEMM_CHUNK_N;
        const int64_t units = (int64_t)nc * (q.g.K / 8);
        const int64_t nblk = (units + 255) / 256;
        if (nblk > INT32_MAX) return hipErrorInvalidConfiguration;
        if (q.bits == 2) hipLaunchKernelGGL((qdequant16<dt, 2>), dim3((unsigned)nblk), dim3(256), 0, st, q, n0, nc, ws);
        else if (q.bits == 4) hipLaunchKernelGGL((qdequant16<dt, 4>), dim3((unsigned)nblk), dim3(256), 0, st, q, n0, nc, ws);
        else hipLaunchKernelGGL((qdequant16<dt, 8>), dim3((unsigned)nblk), dim3(256), 0, st, q, n0, nc, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        GemmParams g = q.g;
        g.B = ws;
        g.ldb = q.g.K;
        g.N = nc;
        g.Y = static_cast<char *>(q.g.Y) + (int64_t)n0 * 2;
        if (g.C != nullptr) g.C = static_cast<const char *>(q.g.C) + (int64_t)n0 * 2;
        e = launch_gemm(g, dt, dt, false, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_qgemm(const QGemmParams &qin, int dt, void *ws, hipStream_t st) {
    if (qin.g.M <= 0 || qin.g.N <= 0) return hipSuccess;
    QGemmParams q = qin;
    q.g.total_steps = q.g.K / 32;
    q.group_shift = q.group_size == 32 ? 5 : (q.group_size == 64 ? 6 : 7);
    if ((1 << q.group_shift) != q.group_size) return hipErrorInvalidValue;
    // the tile kernel above 64 rows, and from 33 rows when N is wide (measured at M = 64, K = 4096, 4-bit:
    // 27.8 against 33.8 us at N = 14336; 26.8 against 15.1 at N = 4096, where it has 64 tiles only)
    const bool tile = q.g.K > 0 && q.g.K % QGEMM_TILE_K == 0 &&
                      (q.g.M > QGEMM_FUSED_MAX_M || (q.g.M > 32 && q.g.N > 4096));
    if (tile) {
        if (dt == DT_BF16) return launch_tile<DT_BF16>(q, st);
        if (dt == DT_F16) return launch_tile<DT_F16>(q, st);
        return hipErrorInvalidValue;
    }
    if (qgemm_uses_workspace(q.g.M, q.g.K) && q.g.K > 0) {
        if (ws == nullptr) return hipErrorInvalidValue;
        if (dt == DT_BF16) return launch_chunks<DT_BF16>(q, ws, st);
        if (dt == DT_F16) return launch_chunks<DT_F16>(q, ws, st);
        return hipErrorInvalidValue;
    }
    if (dt == DT_BF16) return launch_dt<DT_BF16>(q, st);
    if (dt == DT_F16) return launch_dt<DT_F16>(q, st);
    return hipErrorInvalidValue;
}

}  // namespace bi
