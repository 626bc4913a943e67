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
// Up to 64 rows: one workgroup of four wavefronts per (strip of 16 output
// columns, tile of 16 FM rows of x).  A 128-k stage is 256 units of 8 weights: each thread
// unpacks one unit (its packed word(s), the group's scale and bias) into the
// LDS stage in the strip kernel's layout (256-byte rows, chunk c of row r at
// slot c ^ (r mod 16)) together with its share of the x rows; wavefront 0
// then runs every row's chain for the stage.  Packed weights and x are
// prefetched several stages ahead through register rings; the LDS stage is
// double-buffered with one barrier per stage.  Only ordinary loads
// are in flight, so the compiler's waits are exact.  More rows: chunks of
// columns are dequantised into a workspace with the same arithmetic and the
// tile GEMM kernels of bi_linear run on them (the same chain, so the same
// bits; the choice of path depends on M only as a tile choice does).
#include "device.h"
#include "gemm_common.h"
#include "qgemm.h"

namespace bi {

namespace {

constexpr int QDEPTH = 8;                // packed-weight stages in flight per thread
// x stages in flight per thread (divides QDEPTH): deep for one row fragment, where x latency paces the
// stage loop; one stage ahead for more rows, where the registers cost occupancy
template <int FM> struct XDepth { static constexpr int value = FM == 1 ? 4 : 1; };
constexpr int QSTAGE_K = 128;

template <int BITS> struct Packed;
template <> struct Packed<2> { using T = uint32_t; };   // 8 values = half a word
template <> struct Packed<4> { using T = uint32_t; };   // 8 values = one word
template <> struct Packed<8> { using T = u32x2; };      // 8 values = two words

// two fp32 values rounded to nearest even in the input dtype, packed low | high << 16
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int dt> __device__ __forceinline__ uint32_t round_pack(float lo, float hi) {
    if constexpr (dt == DT_BF16) return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
    else return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
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

template <int dt, int FM, int BITS>
__global__ __launch_bounds__(256) void qgemm16_strip(QGemmParams q) {
    constexpr int ROWB = 256;                    // 128 k of 16-bit values
    constexpr int AR = 16 * FM;                  // x rows per workgroup
    constexpr int STAGE = (16 + AR) * ROWB;
    constexpr int PER = 32 / BITS;               // values per packed word
    constexpr uint32_t FIELD = (1u << BITS) - 1u;
    using P = typename Packed<BITS>::T;
    constexpr int XD = XDepth<FM>::value;
    __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];

    const GemmParams &p = q.g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nstrip = (p.N + 15) / 16;
    const int n0 = (blockIdx.x % nstrip) * 16;
    const int m0 = (blockIdx.x / nstrip) * AR;
    const int nst = (p.K + QSTAGE_K - 1) / QSTAGE_K;

    // this thread's weight unit: row wr of the strip, 8 values at chunk wc of each stage
    const int wr = tid >> 4, wc = tid & 15;
    const int wn = min(n0 + wr, p.N - 1);
    const uint32_t *wrow = q.wq + (int64_t)wn * q.ldwq;
    const void *srow = static_cast<const char *>(q.scales) + (int64_t)wn * q.ldsb * 2;
    const void *brow = static_cast<const char *>(q.biases) + (int64_t)wn * q.ldsb * 2;
    const int wslot = ((wc ^ (wr & 15)) << 4);

    // register ring: packed values, raw 16-bit scale and bias of the unit for DEPTH stages (converted
    // only when unpacked, so nothing waits for a load before its stage comes up)
    P raw[QDEPTH];
    uint32_t rsc[QDEPTH], rbi[QDEPTH];
    const uint16_t *sp16 = static_cast<const uint16_t *>(srow);
    const uint16_t *bp16 = static_cast<const uint16_t *>(brow);
    auto loadW = [&](int s, P &r, uint32_t &sc, uint32_t &bi) {
        const int k = min(s * QSTAGE_K + 8 * wc, p.K - 8);        // k < K: clamped, unused past K
        if constexpr (BITS == 8) r = *reinterpret_cast<const u32x2 *>(wrow + k / PER);
        else r = wrow[k / PER];
        const int grp = k >> q.group_shift;
        sc = sp16[grp];
        bi = bp16[grp];
    };
    auto storeW = [&](int s, const P &r, uint32_t scr, uint32_t bir, char *buf) {
        const int k = s * QSTAGE_K + 8 * wc;
        const float sc = half_to_f32<dt>(scr), bi = half_to_f32<dt>(bir);
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t f;
            if constexpr (BITS == 8) f = (r[j >> 2] >> (8 * (j & 3))) & FIELD;
            else if constexpr (BITS == 4) f = (r >> (4 * j)) & FIELD;
            else f = (r >> (16 * ((k >> 3) & 1) + 2 * j)) & FIELD;
            w[j] = __builtin_fmaf(sc, (float)f, bi);
        }
        u32x4 v = u32x4{round_pack<dt>(w[0], w[1]), round_pack<dt>(w[2], w[3]), round_pack<dt>(w[4], w[5]),
                        round_pack<dt>(w[6], w[7])};
        if (k >= p.K) v = zero_u4();
        *reinterpret_cast<u32x4 *>(buf + wr * ROWB + wslot) = v;
    };
    // x rows: FM units of 16 bytes per thread per stage, in a ring of XD stages
    u32x4 araw[XD][FM];
    auto loadA = [&](int s, u32x4 (&a)[FM]) {    // clamped to k < K; chunks past K are zeroed when stored
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            const int u = tid + 256 * f, r = u >> 4, c = u & 15;
            const int k = min(s * QSTAGE_K + 8 * c, p.K - 8);
            const int m = min(m0 + r, p.M - 1);
            a[f] = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.A) + ((int64_t)m * p.lda + k) * 2);
        }
    };
    auto storeA = [&](int s, const u32x4 (&a)[FM], char *buf) {
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            const int u = tid + 256 * f, r = u >> 4, c = u & 15;
            const int row = 16 + r;
            const u32x4 v = s * QSTAGE_K + 8 * c < p.K ? a[f] : zero_u4();
            *reinterpret_cast<u32x4 *>(buf + row * ROWB + ((c ^ (row & 15)) << 4)) = v;
        }
    };

    // consumer (wavefront 0): FM row fragments against the strip's 16 columns
    const int r16 = lane & 15, g = lane >> 4;
    f32x4 acc[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) acc[f] = zero4();
    auto consume = [&](int s, const char *buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (s * 4 + u < p.total_steps) {             // uniform: the chain's steps, none past K
                const int c = 4 * u + g;
                const u32x4 b = *reinterpret_cast<const u32x4 *>(buf + r16 * ROWB + ((c ^ r16) << 4));
#pragma unroll
                for (int f = 0; f < FM; ++f) {
                    const int row = 16 + 16 * f + r16;
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(buf + row * ROWB + ((c ^ (row & 15)) << 4));
                    acc[f] = Mfma<dt>::step(a, b, acc[f]);
                }
            }
        }
    };

    // prologue: rings filled with stages 0 .. DEPTH-1, stage 0 unpacked, stage DEPTH requested
    if (nst > 0) {
#pragma unroll
        for (int j = 0; j < XD; ++j) loadA(j, araw[j]);
#pragma unroll
        for (int j = 0; j < QDEPTH; ++j) loadW(j, raw[j], rsc[j], rbi[j]);
        storeA(0, araw[0], lds);
        loadA(XD, araw[0]);
        storeW(0, raw[0], rsc[0], rbi[0], lds);
        loadW(QDEPTH, raw[0], rsc[0], rbi[0]);
        lds_barrier();
    }
    // stage s: consume it; store x of stage s + 1 (x ring slot (s + 1) mod XD) and refill that slot
    // with stage s + 1 + XD; unpack stage s + 1 (weight ring slot (s + 1) mod DEPTH) into the other
    // buffer and refill that slot with stage s + 1 + DEPTH.  The body has no branch
    // around loads (stages past the end load clamped addresses and store zeros; the stage count is
    // rounded up to whole rounds of DEPTH), so the compiler counts each wait exactly.
    for (int s0 = 0; s0 < nst; s0 += QDEPTH) {
#pragma unroll
        for (int j = 0; j < QDEPTH; ++j) {
            const int s = s0 + j;
            const int jn = (j + 1) % QDEPTH;               // constants once the loop is unrolled
            const int xn = (j + 1) % XD;
            char *cur = lds + (s & 1) * STAGE;
            char *nxt = lds + ((s + 1) & 1) * STAGE;
            if (wave == 0) consume(s, cur);
            storeA(s + 1, araw[xn], nxt);
            loadA(s + 1 + XD, araw[xn]);
            storeW(s + 1, raw[jn], rsc[jn], rbi[jn], nxt);
            loadW(s + 1 + QDEPTH, raw[jn], rsc[jn], rbi[jn]);
            lds_barrier();
        }
    }

    if (wave != 0) return;
    const int n = n0 + r16;
    if (n >= p.N) return;
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + 16 * f + 4 * g + i;
            if (m < p.M) epilogue<dt>(p, m, n, acc[f][i]);
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

bool qgemm_uses_workspace(int64_t M) { return M > QGEMM_FUSED_MAX_M; }

size_t qgemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!qgemm_uses_workspace(M) || N <= 0 || K <= 0) return 0;
    const int64_t nc = N < QGEMM_CHUNK_N ? N : QGEMM_CHUNK_N;
    return (size_t)(nc * K * 2);
}

template <int dt, int FM>
static hipError_t launch_fm(const QGemmParams &q, hipStream_t st) {
    const int64_t nstrip = (q.g.N + 15) / 16, ntile = (q.g.M + 16 * FM - 1) / (16 * FM);
    const int64_t nwg = nstrip * ntile;
    if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nwg), block(256);
    if (q.bits == 2) hipLaunchKernelGGL((qgemm16_strip<dt, FM, 2>), grid, block, 0, st, q);
    else if (q.bits == 4) hipLaunchKernelGGL((qgemm16_strip<dt, FM, 4>), grid, block, 0, st, q);
    else if (q.bits == 8) hipLaunchKernelGGL((qgemm16_strip<dt, FM, 8>), grid, block, 0, st, q);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int dt>
static hipError_t launch_dt(const QGemmParams &q, hipStream_t st) {
    const int rows = qgemm_tile_rows(q.g.M);
    if (rows == 16) return launch_fm<dt, 1>(q, st);
    if (rows == 32) return launch_fm<dt, 2>(q, st);
    return launch_fm<dt, 4>(q, st);
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
    if (qgemm_uses_workspace(q.g.M) && q.g.K > 0) {
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
