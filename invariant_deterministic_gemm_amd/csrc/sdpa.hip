// Batch-invariant scaled dot-product attention for gfx950.
//
// Method (mlx-batch-invariant README, section "How the kernels work",
// attention paragraph): online softmax in fp32 and a FIXED reduction
// structure that no query length, batch size or context length can change.
// The README's section "Why MLX is not invariant" lists what must not move
// the bits: the query count picking another kernel, the split-KV count
// depending on the GQA factor times the query count, and a one-pass /
// two-pass switch as the KV cache grows.
//
// CDNA4 realisation.  One kernel body serves decode and prefill:
//   * keys are cut at ABSOLUTE positions into splits of KV_SPLIT = 256 keys
//     and each split into blocks of KV_BLOCK = 64 keys;
//   * one wavefront handles a tile of 16 query rows (the G query heads that
//     share a KV head times consecutive query positions, packed row =
//     query_index * G + head_in_group) against one split, so K and V are
//     read once per KV head;
//   * per block, in ascending order, and per row:
//        S^T = K . Q^T on the MFMA (contracting over d in fixed chunks),
//        s  = fp32(S * c) with c = scale * log2(e) computed once on the host,
//        invisible keys (causal, mask, or past S) -> s = -inf,
//        m_blk = max s;  a block with m_blk = -inf leaves (m, l, O) untouched,
//        m' = max(m, m_blk), alpha = exp2(m - m'), p = exp2(s - m'),
//        l = fmaf(l, alpha, sum p)  (sum in a fixed lane / register order),
//        O = O * alpha, then O += P . V on the MFMA (P rounded to the input
//        dtype for bf16 / fp16, kept fp32 for fp32);
//   * split partials (m, l, O) go to a workspace, and a second kernel folds
//     them left to right in ascending split order, divides by l, turns -0
//     into +0 and rounds once.
// A row's result therefore depends only on its own query, the keys it may
// see, and the fixed split / block boundaries: a token decoded alone (keys
// after it absent) and the same token inside a prefill chunk (keys after it
// masked) run the same operations on the same operands, and appending masked
// keys to the cache only appends identity steps.

#include <algorithm>
#include <type_traits>

#include "device.h"
#include "sdpa.h"

namespace bi {

template <int dt, int D> struct AttnShape {
    static constexpr int EB = Elem<dt>::bytes;
    static constexpr int EPC = 16 / EB;
    static constexpr int NCH = D * EB / 64;          // 16-byte chunks of d per lane (contraction over d)
    static constexpr int ND = D / 16;                // 16-wide d tiles of the output
    static constexpr int VROW = D * EB + (EB == 2 ? 8 : 16);   // padded LDS row of V (bytes)
    static constexpr int VCH = D * EB / 16;          // 16-byte chunks per V row
    // element offset of this lane group's chunk c of a row, for the q.k contraction
    static __device__ __forceinline__ int d_of(int c, int g) {
        if constexpr (EB == 2) return 32 * c + 8 * g;     // one MFMA per chunk: k slots 8g..8g+7
        else return g * (D / 4) + 4 * c;                  // four MFMAs per chunk, one d each
    }
};

template <int dt>
__device__ __forceinline__ f32x4 attn_mfma_chunk(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (dt == DT_F32) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            c = Mfma<DT_F32>::step(__uint_as_float(a[u]), __uint_as_float(b[u]), c);
        return c;
    } else {
        return Mfma<dt>::step(a, b, c);
    }
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(e) rounded to fp32: additive mask values and sink logits move to the exp2 domain with it
constexpr float LOG2E_F = 1.44269504088896340736f;

// 16-bit head dims below 128 run the D = 128 kernels on zero-padded rows: the loads of 16-byte chunks at
// d >= D read this zero page instead of memory, so the padding costs no HBM traffic; its zero products
// add exact zeros to the q.k chain and its output columns are never stored.
__device__ __attribute__((aligned(256))) uint32_t g_zero_page[64];

// The mask row of query row (b, h, iq): byte pointer to its element for key 0, or null.
__device__ __forceinline__ const char *mask_row(const SdpaParams &p, int b, int h, int iq, int eb) {
    if (p.mask == nullptr) return nullptr;
    const int64_t e = (int64_t)b * p.ms[0] + (int64_t)h * p.ms[1] + (int64_t)iq * p.ms[2];
    return static_cast<const char *>(p.mask) + e * (p.mask_add ? eb : 1);
}
// Score of one key in the exp2 domain: s = S * c, or fmaf(a, log2 e, S * c) with the additive mask
// value a of the key (-inf removes it); ok: the key passes causality, the end of the cache and a
// boolean mask.  Invisible keys score -inf.
template <int dt>
__device__ __forceinline__ float masked_score(const SdpaParams &p, const char *mrow, int key, bool ok, float sdot) {
    const float sv = sdot * p.c;
    if (mrow == nullptr) return ok ? sv : -__builtin_huge_valf();
    if (p.mask_add) {
        const float a = load_as_f32<dt>(mrow, (int64_t)key * p.ms[3]);
        return ok ? __builtin_fmaf(a, LOG2E_F, sv) : -__builtin_huge_valf();
    }
    return ok && reinterpret_cast<const uint8_t *>(mrow)[(int64_t)key * p.ms[3]] != 0 ? sv : -__builtin_huge_valf();
}
// Scores of a lane's 16 keys kb + 16 kt + 4 g + i of one block (exp2 domain, -inf when invisible), from
// the block's raw scores st: key past S, causality (pos) and the mask.  With mask_vec the lane reads its
// mask values as four 4-key vectors, all requested before the first is used (one wait for the four;
// S % 4 == 0, so a 4-key group is entirely before S or entirely past it and is then read clamped).
template <int dt>
__device__ __forceinline__ void block_scores(const SdpaParams &p, const char *mrow, int kb, int g, bool row_ok,
                                             int pos, const f32x4 (&st)[4], float (&s)[4][4]) {
    constexpr int EB = Elem<dt>::bytes;
    constexpr float NEG_INF = -__builtin_huge_valf();
    if (mrow != nullptr && p.mask_vec) {
        // the four loads of a mask kind are issued together, with no branch between them
        auto vis = [&](int kt, int i) {
            const int key = kb + 16 * kt + 4 * g + i;
            bool ok = row_ok && key < p.S;
            if (p.causal) ok = ok && key <= pos;
            return ok;
        };
        if (!p.mask_add) {
            uint32_t raw[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                raw[kt] = *reinterpret_cast<const uint32_t *>(mrow + min(kb + 16 * kt + 4 * g, p.S - 4));
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = vis(kt, i) && ((raw[kt] >> (8 * i)) & 0xffu) != 0;
                    s[kt][i] = ok ? st[kt][i] * p.c : NEG_INF;
                }
        } else if constexpr (EB == 2) {
            u32x2 raw[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                raw[kt] = *reinterpret_cast<const u32x2 *>(mrow + (int64_t)min(kb + 16 * kt + 4 * g, p.S - 4) * 2);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t h16 = (raw[kt][i >> 1] >> (16 * (i & 1))) & 0xffffu;
                    const float a = dt == DT_BF16 ? bf16_to_f32(h16) : f16_to_f32(h16);
                    s[kt][i] = vis(kt, i) ? __builtin_fmaf(a, LOG2E_F, st[kt][i] * p.c) : NEG_INF;
                }
        } else {
            u32x4 raw[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                raw[kt] = *reinterpret_cast<const u32x4 *>(mrow + (int64_t)min(kb + 16 * kt + 4 * g, p.S - 4) * 4);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s[kt][i] = vis(kt, i) ? __builtin_fmaf(__uint_as_float(raw[kt][i]), LOG2E_F, st[kt][i] * p.c) : NEG_INF;
        }
        return;
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kb + 16 * kt + 4 * g + i;
            bool ok = row_ok && key < p.S;
            if (p.causal) ok = ok && key <= pos;
            s[kt][i] = masked_score<dt>(p, mrow, min(key, p.S - 1), ok, st[kt][i]);
        }
}

// The sink of query head h in the exp2 domain, as the first partial of every fold: (m, l, O) =
// (sink * log2 e, 1, 0).
__device__ __forceinline__ float sink2(const SdpaParams &p, int h) { return p.sinks[h] * LOG2E_F; }

// x op x[lane ^ 16] and x op x[lane ^ 32] for a commutative op, through the VALU lane swaps (no
// LDS round trip): a swap of x with itself leaves one lane of each pair holding both values, the
// other lane the same two in the other order, which a commutative op does not see.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work item of a one-dimensional grid of `ntile` query-row tiles times
// `ngroup` (split, batch, KV head) groups.  Workgroups are dealt to the eight
// XCDs in turn, so when the grid size is a multiple of 8 the ids are permuted
// to give each XCD one contiguous run of groups: the tiles that read the same
// K / V block then share one L2.  Picks work only, never arithmetic.
__device__ __forceinline__ void attn_work(int ntile, int ngroup, int &tile, int &group) {
    const int total = ntile * ngroup;
    int L = blockIdx.x;
    if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
    tile = L % ntile;
    group = L / ntile;
}

template <int dt, int D>
__global__ __launch_bounds__(64) void sdpa_split(SdpaParams p) {
    using A = AttnShape<dt, D>;
    constexpr float NEG_INF = -__builtin_huge_valf();
    constexpr bool SLIM = A::EB == 4 && D > 128;
    __shared__ __attribute__((aligned(16))) char vs[KV_BLOCK * A::VROW];

    const int lane = threadIdx.x;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int R = p.G * p.Lq;
    int tile, grp;
    attn_work((R + 15) / 16, p.nsplit * p.B * p.Hkv, tile, grp);
    const int sp = grp % p.nsplit;
    const int b = grp / p.nsplit / p.Hkv;
    const int gk = grp / p.nsplit % p.Hkv;

    // the score row this lane carries (column r16 of S^T)
    const int rg = tile * 16 + r16;
    const bool row_ok = rg < R;
    const int rgc = min(rg, R - 1);
    const int iq = rgc / p.G;
    const int h = gk * p.G + rgc % p.G;
    const int pos = p.S - p.Lq + iq;

    const int kbeg = sp * p.split_len;          // KV_SPLIT except in the comparator
    const int kend = min(kbeg + p.split_len, p.S);
    int nblk = (kend - kbeg + KV_BLOCK - 1) / KV_BLOCK;
    if (p.causal) {
        // rows are ordered by query index, so the tile's last row sees the most keys
        const int rlast = min(tile * 16 + 15, R - 1);
        const int pos_last = p.S - p.Lq + rlast / p.G;
        nblk = pos_last < kbeg ? 0 : min(nblk, (pos_last - kbeg) / KV_BLOCK + 1);
    }

    const char *qrow = static_cast<const char *>(p.q) +
                       ((int64_t)b * p.qs[0] + (int64_t)h * p.qs[1] + (int64_t)iq * p.qs[2]) * A::EB;
    const char *kbase = static_cast<const char *>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)gk * p.ks[1]) * A::EB;
    const char *vbase = static_cast<const char *>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)gk * p.vs[1]) * A::EB;
    const char *mrow = mask_row(p, b, h, iq, A::EB);

    u32x4 qf[A::NCH];
#pragma unroll
    for (int c = 0; c < A::NCH; ++c) qf[c] = ldg16(qrow + A::d_of(c, g) * A::EB);

    float m_run = NEG_INF, l_run = 0.0f;
    f32x4 o[A::ND];
#pragma unroll
    for (int t = 0; t < A::ND; ++t) o[t] = zero4();

    for (int blk = 0; blk < nblk; ++blk) {
        const int kb = kbeg + blk * KV_BLOCK;
        f32x4 st[4];
        if constexpr (SLIM) {
            // fp32 rows above 128: V staged in four pieces, K one key tile at a time (the whole block's
            // fragments would need 512 registers per lane); same loads, same chains
            constexpr int NV = KV_BLOCK * A::VCH / 64, VP = NV / 4;
            static_assert(NV % 4 == 0, "four V pieces");
            __syncthreads();                             // the previous block's V reads are done
#pragma unroll
            for (int piece = 0; piece < 4; ++piece) {
                u32x4 vr[VP];
#pragma unroll
                for (int i = 0; i < VP; ++i) {
                    const int id = lane + 64 * (piece * VP + i);
                    const int key = id / A::VCH, c = id % A::VCH;
                    vr[i] = (kb + key < p.S) ? ldg16(vbase + ((int64_t)(kb + key) * p.vs[2] + c * A::EPC) * A::EB)
                                             : zero_u4();
                }
#pragma unroll
                for (int i = 0; i < VP; ++i) {
                    const int id = lane + 64 * (piece * VP + i);
                    const int key = id / A::VCH, c = id % A::VCH;
                    *reinterpret_cast<u32x4 *>(vs + key * A::VROW + c * 16) = vr[i];
                }
            }
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int key = kb + 16 * kt + r16;
                const char *krow = kbase + (int64_t)key * p.ks[2] * A::EB;
                u32x4 kf[A::NCH];
#pragma unroll
                for (int c = 0; c < A::NCH; ++c) kf[c] = key < p.S ? ldg16(krow + A::d_of(c, g) * A::EB) : zero_u4();
                st[kt] = zero4();
#pragma unroll
                for (int c = 0; c < A::NCH; ++c) st[kt] = attn_mfma_chunk<dt>(kf[c], qf[c], st[kt]);
            }
        } else {
            // ---- K fragments straight from HBM (A operand of S^T = K Q^T)
            u32x4 kf[4][A::NCH];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int key = kb + 16 * kt + r16;
                const char *krow = kbase + (int64_t)key * p.ks[2] * A::EB;
#pragma unroll
                for (int c = 0; c < A::NCH; ++c)
                    kf[kt][c] = key < p.S ? ldg16(krow + A::d_of(c, g) * A::EB) : zero_u4();
            }
            // ---- V block -> LDS, row-major with padded rows; absent keys are zero
            u32x4 vr[KV_BLOCK * A::VCH / 64];
#pragma unroll
            for (int i = 0; i < KV_BLOCK * A::VCH / 64; ++i) {
                const int id = lane + 64 * i;
                const int key = id / A::VCH, c = id % A::VCH;
                vr[i] = (kb + key < p.S) ? ldg16(vbase + ((int64_t)(kb + key) * p.vs[2] + c * A::EPC) * A::EB)
                                         : zero_u4();
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < KV_BLOCK * A::VCH / 64; ++i) {
                const int id = lane + 64 * i;
                const int key = id / A::VCH, c = id % A::VCH;
                char *dst = vs + key * A::VROW + c * 16;
                if constexpr (A::EB == 2) {
                    reinterpret_cast<u32x2 *>(dst)[0] = u32x2{vr[i][0], vr[i][1]};
                    reinterpret_cast<u32x2 *>(dst)[1] = u32x2{vr[i][2], vr[i][3]};
                } else {
                    *reinterpret_cast<u32x4 *>(dst) = vr[i];
                }
            }
            // ---- scores: lane holds S^T[key 16 kt + 4 g + i][row r16]
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                st[kt] = zero4();
#pragma unroll
                for (int c = 0; c < A::NCH; ++c) st[kt] = attn_mfma_chunk<dt>(kf[kt][c], qf[c], st[kt]);
            }
        }
        float s[4][4];
        float mb = NEG_INF;
        block_scores<dt>(p, mrow, kb, g, row_ok, pos, st, s);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mb = fmaxf(mb, s[kt][i]);
        mb = max_xor32(max_xor16(mb));
        const bool empty = mb == NEG_INF;
        const float m_new = empty ? m_run : fmaxf(m_run, mb);
        const float alpha = empty ? 1.0f : exp2_hw(m_run - m_new);
        float pr[4][4];
        float rs = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[kt][i] = s[kt][i] == NEG_INF ? 0.0f : exp2_hw(s[kt][i] - m_new);
                rs = rs + pr[kt][i];
            }
        rs = add_xor32(add_xor16(rs));
        l_run = __builtin_fmaf(l_run, alpha, rs);
        m_run = m_new;
        // ---- rescale O: lane holds O rows 4 g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
            for (int t = 0; t < A::ND; ++t) o[t][i] = o[t][i] * ai;
        }
        __syncthreads();   // V block visible in LDS
        // ---- O += P . V
        if constexpr (A::EB == 2) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // k slot 8 g + j <-> key 32 c + 4 g + j (j < 4), 32 c + 16 + 4 g + (j - 4) (j >= 4)
                const u32x4 pf = u32x4{pack2<dt>(pr[2 * c][0], pr[2 * c][1]), pack2<dt>(pr[2 * c][2], pr[2 * c][3]),
                                       pack2<dt>(pr[2 * c + 1][0], pr[2 * c + 1][1]),
                                       pack2<dt>(pr[2 * c + 1][2], pr[2 * c + 1][3])};
                const int key0 = 32 * c + 4 * g;
#pragma unroll
                for (int t = 0; t < A::ND; ++t) {
                    const char *col = vs + (16 * t + r16) * 2;
                    uint32_t w[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int ka = key0 + (jj < 2 ? 2 * jj : 16 + 2 * (jj - 2));
                        const uint32_t lo = *reinterpret_cast<const uint16_t *>(col + ka * A::VROW);
                        const uint32_t hi = *reinterpret_cast<const uint16_t *>(col + (ka + 1) * A::VROW);
                        w[jj] = lo | (hi << 16);
                    }
                    o[t] = Mfma<dt>::step(pf, u32x4{w[0], w[1], w[2], w[3]}, o[t]);
                }
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * kt + 4 * g + i;
#pragma unroll
                    for (int t = 0; t < A::ND; ++t) {
                        const float vv = *reinterpret_cast<const float *>(vs + key * A::VROW + (16 * t + r16) * 4);
                        o[t] = Mfma<DT_F32>::step(pr[kt][i], vv, o[t]);
                    }
                }
        }
        __syncthreads();   // everyone done with this V block
    }

    // ---- partials
    if (g == 0 && row_ok) {
        const int64_t rowid = ((int64_t)b * p.Hq + h) * p.Lq + iq;
        float *ml = p.ws_ml + (rowid * p.nsplit + sp) * 2;
        ml[0] = m_run;
        ml[1] = l_run;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ro = tile * 16 + 4 * g + i;
        if (ro < R) {
            const int iq_o = ro / p.G;
            const int h_o = gk * p.G + ro % p.G;
            const int64_t rowid = ((int64_t)b * p.Hq + h_o) * p.Lq + iq_o;
            float *dst = p.ws_o + (rowid * p.nsplit + sp) * D;
#pragma unroll
            for (int t = 0; t < A::ND; ++t) dst[16 * t + r16] = o[t][i];
        }
    }
}

// 16-bit inputs, D = 128: the same arithmetic as sdpa_split (bit for bit), with
// the K and V blocks loaded into LDS by direct-to-LDS loads and no registers
// held for them: the next block's K is requested as soon as this block's
// scores have read K, its V as soon as P.V has read V, so each transfer
// overlaps the other half of the block's work (32 KiB of LDS per wavefront,
// five wavefronts per CU).  LDS rows are the 256-byte key rows; K chunk c of
// row r sits at slot c ^ (r mod 16) (the 16 key rows one fragment read serves
// hit 16 distinct bank groups), V chunk c at slot c ^ 2 (r mod 8) (the four
// 32-byte row pieces one transpose read serves hit distinct banks).  The P.V
// operand is gathered with ds_read_b64_tr_b16: within each 16-lane group,
// output lane i element v is element i mod 4 of source lane i / 4 + 4 v, so
// source lane j points at key row base + j / 4, columns 16 t + 4 (j mod 4).
// Keys past S are loaded from a clamped row and their V rows are zeroed in
// LDS before use (their scores are -inf anyway).
// P rounded to the input dtype, two values per dword (low = a).  P is finite
// and in [0, 1]; bf16 uses the gfx950 round-to-nearest-even pack instruction.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int dt> __device__ __forceinline__ uint32_t pack_p(float a, float b) {
    if constexpr (dt == DT_BF16) return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
    else return pack2<dt>(a, b);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const char *lds_addr) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)((__attribute__((address_space(3))) char *)lds_addr));
    return __builtin_bit_cast(u32x2, v);
}

// The 16 query rows of one row tile as one wavefront sees them: lane r16
// carries score row r16 (column r16 of S^T); lanes hold O rows 4 g + i.
// NC = 4 for rows of 128 (or zero-padded to 128), 8 for rows of 256.
template <int NC>
struct Rows16T {
    bool row_ok;            // score row r16 is a real row (rows past R are computed and never stored)
    int pos;                // its key position (bottom-right alignment)
    int pos_first;          // key position of the tile's first row, the smallest in the tile
    const char *mrow;       // its mask row, or null
    u32x4 qf[NC];           // its q fragments (d chunks 32 c + 8 g .. + 7)
};
using Rows16 = Rows16T<4>;

template <int dt, int NC>
__device__ __forceinline__ void rows16_load(const SdpaParams &p, int tile, int b, int gk, Rows16T<NC> &r) {
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int R = p.G * p.Lq;
    const int rg = tile * 16 + r16;
    r.row_ok = rg < R;
    const int rgc = min(rg, R - 1);
    const int iq = rgc / p.G;
    const int h = gk * p.G + rgc % p.G;
    r.pos = p.S - p.Lq + iq;
    r.pos_first = p.S - p.Lq + (tile * 16) / p.G;
    r.mrow = mask_row(p, b, h, iq, 2);
    const char *qrow = static_cast<const char *>(p.q) +
                       ((int64_t)b * p.qs[0] + (int64_t)h * p.qs[1] + (int64_t)iq * p.qs[2]) * 2;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        r.qf[c] = zero_u4();
        if (32 * c < p.dr) r.qf[c] = ldg16(qrow + (32 * c + 8 * g) * 2);
    }
}

// Scores of one 64-key block for a wavefront's 16 rows (K block in LDS, 64 NC-byte key rows, chunk c
// of key r at slot c ^ (r mod 16)): lane holds S^T[key 16 kt + 4 g + i][row r16].  The K fragments of
// four d chunks are read first; the four chains (one per kt) each accumulate d chunks c = 0 .. NC - 1
// in order.  The K reads may still be in flight on return.
// Rows of 64 values (D = 64) are 128 bytes: chunk c of key r at slot c ^ ((r / 2) mod 8) instead, which keeps
// the 16 rows of one read pass on distinct bank groups.
template <int dt, int NC>
__device__ __forceinline__ void attn_scores16(const Rows16T<NC> &r, const char *Ks, f32x4 (&st)[4]) {
    constexpr int ROWB = 64 * NC;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) st[kt] = zero4();
    if constexpr (NC == 2) {
        u32x4 kf[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                kf[kt][c] = *reinterpret_cast<const u32x4 *>(Ks + (16 * kt + r16) * ROWB +
                                                             (((4 * c + g) ^ ((r16 >> 1) & 7)) << 4));
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) st[kt] = Mfma<dt>::step(kf[kt][c], r.qf[c], st[kt]);
    }
#pragma unroll
    for (int h = 0; h < NC / 4; ++h) {
        u32x4 kf[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                kf[kt][c] = *reinterpret_cast<const u32x4 *>(Ks + (16 * kt + r16) * ROWB +
                                                             (((4 * (4 * h + c) + g) ^ r16) << 4));
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) st[kt] = Mfma<dt>::step(kf[kt][c], r.qf[4 * h + c], st[kt]);
    }
}

// The online-softmax half of one block [kb, kb + 64) given its scores: visibility, the update of (m, l)
// and the rescale of O, leaving P rounded to the input dtype as the A fragments of the two 32-key
// halves of P . V (k slot 8 g + j <-> key 32 c + 4 g + j (j < 4), 32 c + 16 + 4 g + (j - 4) (j >= 4)).
// VISIBLE: the caller knows every key of the block is visible to every row (no mask, inside S, before
// the tile's first causal position), which is the case the visibility test would pick.  RESCALE_ALWAYS:
// O is multiplied by alpha even when no row's maximum moved (alpha = 1 then, and O * 1 = O), so the
// update has no branch.  Neither changes any result.  OT: the caller accumulates O transposed (lane
// holds O[row r16][16 t + 4 g + i], see sdpa_prefill16p), so each lane rescales by its own row's alpha.
template <int dt, int NC, int NT, bool VISIBLE = false, bool RESCALE_ALWAYS = false, bool OT = false>
__device__ __forceinline__ void attn_softmax16(const SdpaParams &p, const Rows16T<NC> &r, const f32x4 (&st)[4],
                                               int kb, float &m_run, float &l_run, f32x4 (&o)[NT],
                                               u32x4 (&pf)[2]) {
    constexpr float NEG_INF = -__builtin_huge_valf();
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    float s[4][4];
    // block maximum of the row (exact in any order): a tree over the lane's 16 scores, then the lane
    // groups; taken in each branch next to the products it reads, which the compiler then knows to be
    // canonical (no quieting step before each maximum)
    auto lane_max = [&]() {
        float mk[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mk[kt] = fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3]));
        return fmaxf(NEG_INF, fmaxf(fmaxf(mk[0], mk[1]), fmaxf(mk[2], mk[3])));   // all-NaN -> -inf
    };
    float mb;
    const bool visible =
        VISIBLE || (p.mask == nullptr && kb + KV_BLOCK <= p.S && (!p.causal || kb + KV_BLOCK - 1 <= r.pos_first));
    if (visible) {
        // rows past R get real scores too: they are per-row, never stored, and touch no other row
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[kt][i] = st[kt][i] * p.c;
        mb = lane_max();
    } else {
        block_scores<dt>(p, r.mrow, kb, g, r.row_ok, r.pos, st, s);
        mb = lane_max();
    }
    mb = max_xor32(max_xor16(mb));
    const bool empty = mb == NEG_INF;
    const float m_new = empty ? m_run : fmaxf(m_run, mb);
    const float alpha = empty ? 1.0f : exp2_hw(m_run - m_new);
    // p = exp2(s - m_new), and 0 for an invisible key: exp2(-inf) is exactly +0, so only a block with no
    // visible key (m_new possibly -inf, where -inf - -inf would be NaN) needs a different reference
    const float mref = empty ? 0.0f : m_new;
    float pr[4][4];
    float rs = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[kt][i] = exp2_hw(s[kt][i] - mref);
            rs = rs + pr[kt][i];
        }
    rs = add_xor32(add_xor16(rs));
    l_run = __builtin_fmaf(l_run, alpha, rs);
    m_run = m_new;
    // O * 1 = O: the rescale is skipped when no row's maximum moved
    if (RESCALE_ALWAYS || __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = OT ? alpha : __shfl(alpha, 4 * g + i);
#pragma unroll
            for (int t = 0; t < NT; ++t) o[t][i] = o[t][i] * ai;
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
        pf[c] = u32x4{pack_p<dt>(pr[2 * c][0], pr[2 * c][1]), pack_p<dt>(pr[2 * c][2], pr[2 * c][3]),
                      pack_p<dt>(pr[2 * c + 1][0], pr[2 * c + 1][1]), pack_p<dt>(pr[2 * c + 1][2], pr[2 * c + 1][3])};
}

// V fragments of 32-key half c for the NT 16-column tiles (V block in LDS, 32 NT-byte rows, chunk c of key
// r at slot c ^ 2 (r mod 8)): B operand of P . V, k slot j as in attn_softmax16.
// Rows of 64 values (NT = 4) are 128 bytes: chunk c of key r at slot c ^ 2 ((r / 2) mod 4).
template <int NT>
__device__ __forceinline__ int vswz16(int row) {
    if constexpr (NT == 4) return ((row >> 1) & 3) << 1;
    else return (row & 7) << 1;
}
template <int NT>
__device__ __forceinline__ void attn_vfrags16(const char *Vs, int c, u32x4 (&vf)[NT]) {
    constexpr int ROWB = 32 * NT;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int row0 = 32 * c + 4 * g + (r16 >> 2);
    const int row1 = row0 + 16;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int ch = 2 * t + ((r16 & 3) >> 1);
        const int off = 8 * (r16 & 1);
        const u32x2 lo = lds_read_tr16(Vs + row0 * ROWB + ((ch ^ vswz16<NT>(row0)) << 4) + off);
        const u32x2 hi = lds_read_tr16(Vs + row1 * ROWB + ((ch ^ vswz16<NT>(row1)) << 4) + off);
        vf[t] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
}

// The rest of one block [kb, kb + 64) given its scores: attn_softmax16, then O += P . V from the V block
// in LDS (rows of keys past S must read as zero by the time v_ready() returns, which is before the first
// V read).  The V fragments of a half (c) are read before its NT MFMAs; o[t] takes c = 0 then c = 1.
// OT: O is accumulated transposed, O^T += V^T . P^T (the V fragments as the A operand, P as the B
// operand): every element gets the products and k order of P . V, and lane (r16, g) holds
// O[row r16][16 t + 4 g + i] instead of O[row 4 g + i][16 t + r16].
template <int dt, class VReady, int NC, int NT, bool OT = false>
__device__ __forceinline__ void attn_update16(const SdpaParams &p, const Rows16T<NC> &r, const f32x4 (&st)[4],
                                              const char *Vs, int kb, float &m_run, float &l_run, f32x4 (&o)[NT],
                                              VReady v_ready) {
    u32x4 pf[2];
    attn_softmax16<dt, NC, NT, false, false, OT>(p, r, st, kb, m_run, l_run, o, pf);
    v_ready();
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        u32x4 vf[NT];
        attn_vfrags16<NT>(Vs, c, vf);
#pragma unroll
        for (int t = 0; t < NT; ++t) o[t] = OT ? Mfma<dt>::step(vf[t], pf[c], o[t]) : Mfma<dt>::step(pf[c], vf[t], o[t]);
    }
}


// One 64-key block [kb, kb + 64) of the online softmax for a wavefront's 16
// rows, K and V blocks in LDS as attn_scores16 and attn_update16 take them.
// k_done() runs once every K read of the block is complete, v_ready() before
// the first V read.
template <int dt, bool OT = false, class KDone, class VReady, int NC, int NT>
__device__ __forceinline__ void attn_block16(const SdpaParams &p, const Rows16T<NC> &r, const char *Ks, const char *Vs,
                                             int kb, float &m_run, float &l_run, f32x4 (&o)[NT], KDone k_done,
                                             VReady v_ready) {
    f32x4 st[4];
    attn_scores16<dt>(r, Ks, st);
    __builtin_amdgcn_s_waitcnt(0xc07f);               // every K read of this block done
    k_done();
    attn_update16<dt, VReady, NC, NT, OT>(p, r, st, Vs, kb, m_run, l_run, o, v_ready);
}

// One wavefront's share: split `sp` of row tile `tile` of (b, gk), its K / V
// blocks staged in `lds` (2 * KV_BLOCK * 64 NC bytes: rows of 32 NC elements,
// NC = 4 for D <= 128 and 8 for D = 160 ... 256, zero-padded); leaves the
// split's (m, l) of row r16 and its O fragment (rows 4 g + i, columns 16 t + r16;
// with OT, row r16, columns 16 t + 4 g + i: see attn_update16).
template <int dt, int NC = 4, bool OT = false>
__device__ __forceinline__ void split16_body(const SdpaParams &p, int sp, int tile, int b, int gk, char *lds,
                                             float &m_out, float &l_out, f32x4 (&o)[2 * NC]) {
    constexpr int D = 32 * NC;
    constexpr int ROWB = D * 2;                       // bytes per key row
    constexpr int KBYTES = KV_BLOCK * ROWB;           // one K (or V) block
    constexpr int QB = KBYTES / 1024;                 // 1 KiB load instructions per block half
    constexpr int RPQ = 1024 / ROWB;                  // key rows per load instruction
    constexpr int SPR = ROWB / 16;                    // 16-byte slots per key row
    constexpr int KP = 16 / RPQ, VP = 8 / RPQ;        // periods (in q) of the K and V chunk patterns
    static_assert(QB == 16 * NC / 4 && QB <= 63, "load count per block half");
    static_assert(NC == 2 || NC >= 4, "rows of 64 values or of at least 128");
    constexpr float NEG_INF = -__builtin_huge_valf();
    const int lane = threadIdx.x & 63;
    const int R = p.G * p.Lq;

    const int kbeg = sp * KV_SPLIT;
    const int kend = min(kbeg + KV_SPLIT, p.S);
    int nblk = (kend - kbeg + KV_BLOCK - 1) / KV_BLOCK;
    if (p.causal) {
        // rows are ordered by query index, so the tile's last row sees the most keys
        const int rlast = min(tile * 16 + 15, R - 1);
        const int pos_last = p.S - p.Lq + rlast / p.G;
        nblk = pos_last < kbeg ? 0 : min(nblk, (pos_last - kbeg) / KV_BLOCK + 1);
    }

    const char *kbase = static_cast<const char *>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)gk * p.ks[1]) * 2;
    const char *vbase = static_cast<const char *>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)gk * p.vs[1]) * 2;

    // load side: instruction q covers key rows RPQ q .. RPQ q + RPQ - 1 of the block; lane L row
    // RPQ q + L / SPR, slot L mod SPR.  The swizzled chunk depends on q only through q mod KP (K) and
    // q mod VP (V), so the per-lane parts are computed once and a block's addresses are one base plus
    // multiples of the stride.
    const int lrow = lane / SPR, lslot = lane % SPR;
    const int64_t kstr = p.ks[2] * 2, vstr = p.vs[2] * 2;      // bytes between key rows
    const char *klane = kbase + lrow * kstr;
    const char *vlane = vbase + lrow * vstr;
    int kch[KP], vch[VP];
    bool kz[KP], vz[VP];                              // chunk at d >= D: read the zero page
#pragma unroll
    for (int r = 0; r < KP; ++r) {
        const int row = RPQ * r + lrow;
        const int c = lslot ^ (NC == 2 ? (row >> 1) & 7 : row & 15);
        kch[r] = c << 4;
        kz[r] = 8 * c >= p.dr;
    }
#pragma unroll
    for (int r = 0; r < VP; ++r) {
        const int c = lslot ^ vswz16<2 * NC>(RPQ * r + lrow);
        vch[r] = c << 4;
        vz[r] = 8 * c >= p.dr;
    }
    const char *zp = reinterpret_cast<const char *>(g_zero_page);
    // instructions q0 .. q1 - 1 of a block half
    auto issueK = [&](int blk, int q0, int q1) {
        const int kb = kbeg + blk * KV_BLOCK;
        if (kb + KV_BLOCK <= p.S) {
            const char *bp = klane + (int64_t)kb * kstr + (int64_t)q0 * RPQ * kstr;
#pragma unroll
            for (int q = q0; q < q1; ++q) {
                __builtin_amdgcn_global_load_lds(static_cast<const void *>(kz[q % KP] ? zp : bp + kch[q % KP]),
                                                 BI_LDS_PTR(lds + q * 1024), 16, 0, 0);
                bp += RPQ * kstr;
            }
        } else {                                       // the block crosses S: rows past it read row S - 1
#pragma unroll
            for (int q = q0; q < q1; ++q) {
                const int key = min(kb + RPQ * q + lrow, p.S - 1);
                __builtin_amdgcn_global_load_lds(
                    static_cast<const void *>(kz[q % KP] ? zp : kbase + key * kstr + kch[q % KP]),
                    BI_LDS_PTR(lds + q * 1024), 16, 0, 0);
            }
        }
    };
    auto issueV = [&](int blk, int q0, int q1) {
        const int kb = kbeg + blk * KV_BLOCK;
        if (kb + KV_BLOCK <= p.S) {
            const char *bp = vlane + (int64_t)kb * vstr + (int64_t)q0 * RPQ * vstr;
#pragma unroll
            for (int q = q0; q < q1; ++q) {
                __builtin_amdgcn_global_load_lds(static_cast<const void *>(vz[q % VP] ? zp : bp + vch[q % VP]),
                                                 BI_LDS_PTR(lds + KBYTES + q * 1024), 16, 0, 0);
                bp += RPQ * vstr;
            }
        } else {
#pragma unroll
            for (int q = q0; q < q1; ++q) {
                const int key = min(kb + RPQ * q + lrow, p.S - 1);
                __builtin_amdgcn_global_load_lds(
                    static_cast<const void *>(vz[q % VP] ? zp : vbase + key * vstr + vch[q % VP]),
                    BI_LDS_PTR(lds + KBYTES + q * 1024), 16, 0, 0);
            }
        }
    };

    Rows16T<NC> r;
    rows16_load<dt>(p, tile, b, gk, r);
    float m_run = NEG_INF, l_run = 0.0f;
#pragma unroll
    for (int t = 0; t < 2 * NC; ++t) o[t] = zero4();

    if constexpr (NC <= 4) {
        // at most one K block and one V block (32 loads) in flight
        if (nblk > 0) {
            issueK(0, 0, QB);
            issueV(0, 0, QB);
        }
        for (int blk = 0; blk < nblk; ++blk) {
            const int kb = kbeg + blk * KV_BLOCK;
            char *Vs = lds + KBYTES;
            BI_WAIT_VMCNT(QB);                        // K of this block landed (its V may be in flight)
            attn_block16<dt, OT>(
                p, r, lds, Vs, kb, m_run, l_run, o,
                [&]() {
                    if (blk + 1 < nblk) issueK(blk + 1, 0, QB);
                },
                [&]() {
                    if (blk + 1 < nblk) BI_WAIT_VMCNT(QB);     // V of this block landed (next K may be in flight)
                    else BI_WAIT_VMCNT(0);
                    if (kb + KV_BLOCK > p.S) {
                        for (int row = max(p.S - kb, 0) + lrow; row < KV_BLOCK; row += RPQ)
                            *reinterpret_cast<u32x4 *>(Vs + row * ROWB + lslot * 16) = zero_u4();
                        __builtin_amdgcn_s_waitcnt(0xc07f);
                    }
                });
            __builtin_amdgcn_s_waitcnt(0xc07f);       // every V read of this block done
            if (blk + 1 < nblk) issueV(blk + 1, 0, QB);
        }
    } else {
        // 32 loads per block half: each half goes out in two pieces of H = 16 so that at most 48 loads
        // are in flight (the vector-memory counter holds 63).  Sequence per block: K landed -> second
        // piece of V; scores -> first piece of the next K; V landed -> its second piece; P . V -> first
        // piece of the next V.
        constexpr int H = QB / 2;
        static_assert(H == 16, "two pieces of 16 loads");
        if (nblk > 0) {
            issueK(0, 0, QB);
            issueV(0, 0, H);
        }
        for (int blk = 0; blk < nblk; ++blk) {
            const int kb = kbeg + blk * KV_BLOCK;
            char *Vs = lds + KBYTES;
            BI_WAIT_VMCNT(H);                         // K of this block landed (first piece of V in flight)
            issueV(blk, H, QB);
            attn_block16<dt, OT>(
                p, r, lds, Vs, kb, m_run, l_run, o,
                [&]() {
                    if (blk + 1 < nblk) issueK(blk + 1, 0, H);
                },
                [&]() {
                    if (blk + 1 < nblk) {
                        BI_WAIT_VMCNT(H);             // V of this block landed (a piece of the next K in flight)
                        issueK(blk + 1, H, QB);
                    } else {
                        BI_WAIT_VMCNT(0);
                    }
                    if (kb + KV_BLOCK > p.S) {
                        for (int row = max(p.S - kb, 0) + lrow; row < KV_BLOCK; row += RPQ)
                            *reinterpret_cast<u32x4 *>(Vs + row * ROWB + lslot * 16) = zero_u4();
                        __builtin_amdgcn_s_waitcnt(0xc07f);
                    }
                });
            __builtin_amdgcn_s_waitcnt(0xc07f);       // every V read of this block done
            if (blk + 1 < nblk) issueV(blk + 1, 0, H);
        }
    }

    m_out = m_run;
    l_out = l_run;
}

// W wavefronts per workgroup take W consecutive splits of one (batch, KV
// head, row tile): neighbouring wavefronts stream neighbouring K / V ranges.
// Each wavefront writes its own split's partial; the work split never changes
// the arithmetic.  NC = 8 serves rows of 256 (D = 256).
template <int dt, int W, int NC = 4>
__global__ __launch_bounds__(64 * W) void sdpa_split16(SdpaParams p) {
    constexpr int PER_WAVE = 2 * KV_BLOCK * 64 * NC;
    __shared__ __attribute__((aligned(1024))) char lds[W * PER_WAVE];   // per wave: K block, V block
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int R = p.G * p.Lq;
    const int nsg = (p.nsplit + W - 1) / W;          // split groups per (batch, KV head)
    int tile, grp;
    attn_work((R + 15) / 16, nsg * p.B * p.Hkv, tile, grp);
    const int sp = (grp % nsg) * W + wave;
    const int b = grp / nsg / p.Hkv, gk = grp / nsg % p.Hkv;
    if (sp >= p.nsplit) return;
    float m_run, l_run;
    f32x4 o[2 * NC];
    split16_body<dt, NC, true>(p, sp, tile, b, gk, lds + wave * PER_WAVE, m_run, l_run, o);
    // O accumulated transposed: lane (r16, g) holds row r16, columns 16 t + 4 g .. + 3 (one 16-byte store)
    const int rg = tile * 16 + r16;
    if (rg < R) {
        const int64_t rowid = ((int64_t)b * p.Hq + gk * p.G + rg % p.G) * p.Lq + rg / p.G;
        if (g == 0) {
            float *ml = p.ws_ml + (rowid * p.nsplit + sp) * 2;
            ml[0] = m_run;
            ml[1] = l_run;
        }
        float *dst = p.ws_o + (rowid * p.nsplit + sp) * p.dr;
#pragma unroll
        for (int t = 0; t < 2 * NC; ++t)
            if (16 * t < p.dr) *reinterpret_cast<f32x4 *>(dst + 16 * t + 4 * g) = o[t];
    }
}

// Short KV (at most MAXW splits): one workgroup per row tile with one
// wavefront per split, the split partials exchanged through LDS and folded
// in the workgroup with exactly sdpa_combine's arithmetic (ascending split
// order, same operations), so the result is bit-identical to the two-kernel
// path and needs no workspace round trip or second launch.  The launch gives
// each workgroup FUSED_LDS_PER_WAVE bytes of LDS per wavefront (a K and a V
// block), so that workgroups of one or two splits share a CU.
constexpr int FUSED_MAXW = 4;
constexpr int FUSED_LDS_PER_WAVE = 2 * KV_BLOCK * 256;
template <int dt>
__global__ __launch_bounds__(64 * FUSED_MAXW) void sdpa_fused16(SdpaParams p) {
    constexpr float NEG_INF = -__builtin_huge_valf();
    constexpr int D = 128;
    constexpr int PER_WAVE = FUSED_LDS_PER_WAVE;
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = blockDim.x >> 6;                  // == nsplit
    const int r16 = lane & 15, g = lane >> 4;
    const int R = p.G * p.Lq;
    int tile, grp;
    attn_work((R + 15) / 16, p.B * p.Hkv, tile, grp);
    const int b = grp / p.Hkv, gk = grp % p.Hkv;
    float m_run, l_run;
    f32x4 o[8];
    split16_body<dt, 4, true>(p, wave, tile, b, gk, lds + wave * PER_WAVE, m_run, l_run, o);
    __syncthreads();                                 // every wavefront is done with its K / V blocks
    // the partials reuse the K / V space: nw * (16 * 2 + 16 * D) floats + padding <= nw * PER_WAVE bytes
    float *pml = reinterpret_cast<float *>(lds);                     // [split][16 rows][2]
    float *po = pml + FUSED_MAXW * 16 * 2;                           // [split][16 rows][D]
    if (g == 0) {
        pml[(wave * 16 + r16) * 2] = m_run;
        pml[(wave * 16 + r16) * 2 + 1] = l_run;
    }
    // O transposed: lane (r16, g) holds row r16, columns 16 t + 4 g .. + 3
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4 *>(po + (wave * 16 + r16) * D + 16 * t + 4 * g) = o[t];
    __syncthreads();
    for (int e = tid; e < 16 * p.dr; e += 64 * nw) {
        const int row = e / p.dr, d = e % p.dr;
        const int ro = tile * 16 + row;
        if (ro >= R) continue;
        const int iq = ro / p.G, h = gk * p.G + ro % p.G;
        bool have = false;
        float m = 0.0f, l = 0.0f, acc = 0.0f;
        if (p.sinks) {                               // the sink is the fold's first partial
            m = sink2(p, h);
            l = 1.0f;
            have = true;
        }
        for (int sp = 0; sp < nw; ++sp) {
            const float ms = pml[(sp * 16 + row) * 2], ls = pml[(sp * 16 + row) * 2 + 1];
            if (ms == NEG_INF) continue;
            const float os = po[(sp * 16 + row) * D + d];
            if (!have) {
                m = ms;
                l = ls;
                acc = os;
                have = true;
                continue;
            }
            const float m2 = fmaxf(m, ms);
            const float a = exp2_hw(m - m2);
            const float bs = exp2_hw(ms - m2);
            l = __builtin_fmaf(l, a, ls * bs);
            acc = __builtin_fmaf(acc, a, os * bs);
            m = m2;
        }
        float r = have ? acc / l : 0.0f;
        r = r + 0.0f;                                // -0 -> +0
        char *orow = static_cast<char *>(p.o) +
                     ((int64_t)b * p.os[0] + (int64_t)h * p.os[1] + (int64_t)iq * p.os[2]) * Elem<dt>::bytes;
        store_from_f32<dt>(orow, d, r);
    }
}

// Few query rows: one workgroup per (T row tiles, split, batch, KV head) with
// one wavefront per (64-key block of the split, row tile), so the whole split
// (K and V, 128 KiB) is requested at once instead of one block at a time, and
// with T = 2 two row tiles share it.  The online-softmax recurrence of
// split16_body is then evaluated in stages that keep every operation and
// operand of it, per row tile:
//   1. wavefront (j, t) computes block j's scores for tile t and their row
//      maximum;
//   2. each rebuilds the running maximum before its block from the earlier
//      blocks' maxima (the same select / fmaxf sequence), then its alpha, P
//      (rounded as in split16_body) and row sum;
//   3. l = fmaf(l, alpha, sum) runs over the blocks in order, and
//      O = O * alpha, O += P . V over the blocks in order, each wavefront for
//      two of the eight 16-wide column tiles (columns are independent chains),
//      accumulated transposed as in attn_update16.
// A tile only visits the blocks split16_body visits for it (its own causal
// limit), so its bits never depend on the other tile.  The split's (m, l, O)
// goes to the workspace like sdpa_split16's, and the combine kernel folds the
// splits, so the bits are those of the split path.
template <int dt, int T>
__global__ __launch_bounds__(64 * 4 * T) void sdpa_quad16(SdpaParams p) {
    constexpr int ROWB = 256;
    constexpr int KBYTES = KV_BLOCK * ROWB;           // one K (or V) block
    constexpr int QB = KBYTES / 1024;                 // 1 KiB load instructions per block half
    constexpr int BPS = KV_SPLIT / KV_BLOCK;          // blocks per split
    constexpr int QT = QB / T;                        // load instructions per wavefront per block half
    constexpr float NEG_INF = -__builtin_huge_valf();
    static_assert(BPS == 4 && QB == 16 && QB % T == 0, "four blocks, four key rows per load instruction");
    __shared__ __attribute__((aligned(1024))) char lds[BPS * 2 * KBYTES];   // [block][K block | V block]
    __shared__ u32x4 pbuf[T][BPS][2][64];              // P fragments: tile, block, half c, lane
    __shared__ float xm[T][BPS][16], xa[T][BPS][16], xr[T][BPS][16];   // per block and row: max, alpha, sum

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int w = wave % BPS, wt = wave / BPS;        // block of the split, tile of the workgroup
    const int r16 = lane & 15, g = lane >> 4;
    const int R = p.G * p.Lq;
    const int ntile = (R + 15) / 16;
    int tg, grp;
    attn_work((ntile + T - 1) / T, p.nsplit * p.B * p.Hkv, tg, grp);
    const int sp = grp % p.nsplit;
    const int b = grp / p.nsplit / p.Hkv, gk = grp / p.nsplit % p.Hkv;
    const int tile = tg * T + wt;                     // tiles past the last compute clamped rows, store nothing

    const int kbeg = sp * KV_SPLIT;
    const int kend = min(kbeg + KV_SPLIT, p.S);
    const int nfull = (kend - kbeg + KV_BLOCK - 1) / KV_BLOCK;
    // blocks split16_body visits for a tile (rows are ordered by query index, so its last row sees the most)
    auto tile_blocks = [&](int t) {
        if (!p.causal) return nfull;
        const int rlast = min(t * 16 + 15, R - 1);
        const int pos_last = p.S - p.Lq + rlast / p.G;
        return pos_last < kbeg ? 0 : min(nfull, (pos_last - kbeg) / KV_BLOCK + 1);
    };
    const int nblk = tile_blocks(tile);                               // this wavefront's tile
    const int nload = tile_blocks(min(tg * T + T - 1, ntile - 1));    // the workgroup's (its last tile's)
    const int kb = kbeg + w * KV_BLOCK;               // this wavefront's block
    char *Ks = lds + w * 2 * KBYTES;
    char *Vs = Ks + KBYTES;

    // ---- stage 1: q, then this wavefront's share of its block's K and V (direct to LDS, layout as
    // split16_body: instruction q covers key rows 4 q .. 4 q + 3), then scores
    const int lrow = lane >> 4, lslot = lane & 15;
    const bool loads = w < nload;
    Rows16 r;
    rows16_load<dt>(p, tile, b, gk, r);
    if (loads) {
        const char *kbase = static_cast<const char *>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)gk * p.ks[1]) * 2;
        const char *vbase = static_cast<const char *>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)gk * p.vs[1]) * 2;
        const int64_t kstr = p.ks[2] * 2, vstr = p.vs[2] * 2;
        const char *zp = reinterpret_cast<const char *>(g_zero_page);
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            const int q = wt * QT + j;
            const int row = 4 * q + lrow;
            const int c = lslot ^ (row & 15);
            const int64_t key = min(kb + row, p.S - 1);          // rows past S read row S - 1
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(8 * c >= p.dr ? zp : kbase + key * kstr + (c << 4)),
                                             BI_LDS_PTR(Ks + q * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            const int q = wt * QT + j;
            const int row = 4 * q + lrow;
            const int c = lslot ^ ((row & 7) << 1);
            const int64_t key = min(kb + row, p.S - 1);
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(8 * c >= p.dr ? zp : vbase + key * vstr + (c << 4)),
                                             BI_LDS_PTR(Vs + q * 1024), 16, 0, 0);
        }
        BI_WAIT_VMCNT(QT);                            // q and this wavefront's part of K landed
    } else {
        BI_WAIT_VMCNT(0);                             // q landed
    }
    if constexpr (T > 1) __syncthreads();             // every part of every K block landed
    const bool active = w < nblk;
    float mb = NEG_INF;
    float s[4][4];
    if (active) {
        f32x4 st[4];
        attn_scores16<dt>(r, Ks, st);
        const bool visible = p.mask == nullptr && kb + KV_BLOCK <= p.S && (!p.causal || kb + KV_BLOCK - 1 <= r.pos_first);
        if (visible) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[kt][i] = st[kt][i] * p.c;
        } else {
            block_scores<dt>(p, r.mrow, kb, g, r.row_ok, r.pos, st, s);
        }
        float mk[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mk[kt] = fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3]));
        mb = fmaxf(NEG_INF, fmaxf(fmaxf(mk[0], mk[1]), fmaxf(mk[2], mk[3])));   // all-NaN -> -inf
        mb = max_xor32(max_xor16(mb));
        if (g == 0) xm[wt][w][r16] = mb;
    }
    __syncthreads();

    // ---- stage 2: the running maximum before this block, alpha, P and the row sum
    if (active) {
        float m_run = NEG_INF;
        for (int u = 0; u < w; ++u) {
            const float mu = xm[wt][u][r16];
            m_run = mu == NEG_INF ? m_run : fmaxf(m_run, mu);
        }
        const bool empty = mb == NEG_INF;
        const float m_new = empty ? m_run : fmaxf(m_run, mb);
        const float alpha = empty ? 1.0f : exp2_hw(m_run - m_new);
        const float mref = empty ? 0.0f : m_new;
        float pr[4][4];
        float rs = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[kt][i] = exp2_hw(s[kt][i] - mref);
                rs = rs + pr[kt][i];
            }
        rs = add_xor32(add_xor16(rs));
        if (g == 0) {
            xa[wt][w][r16] = alpha;
            xr[wt][w][r16] = rs;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
            pbuf[wt][w][c][lane] = u32x4{pack_p<dt>(pr[2 * c][0], pr[2 * c][1]), pack_p<dt>(pr[2 * c][2], pr[2 * c][3]),
                                         pack_p<dt>(pr[2 * c + 1][0], pr[2 * c + 1][1]),
                                         pack_p<dt>(pr[2 * c + 1][2], pr[2 * c + 1][3])};
    }
    if (loads) {
        BI_WAIT_VMCNT(0);                             // this wavefront's part of the V block landed
        if (kb + KV_BLOCK > p.S) {                    // V rows past S read as zero (the rows it loaded)
#pragma unroll
            for (int j = 0; j < QT; ++j) {
                const int row = 4 * (wt * QT + j) + lrow;
                if (kb + row >= p.S) *reinterpret_cast<u32x4 *>(Vs + row * ROWB + lslot * 16) = zero_u4();
            }
        }
    }
    __syncthreads();

    // ---- stage 3: l and m over the tile's blocks in order; O for column tiles 2 w, 2 w + 1
    float l_run = 0.0f, m_run = NEG_INF;
    f32x4 o[2] = {zero4(), zero4()};
    for (int u = 0; u < nblk; ++u) {
        const float alpha = xa[wt][u][r16];
        const float mu = xm[wt][u][r16];
        m_run = mu == NEG_INF ? m_run : fmaxf(m_run, mu);
        l_run = __builtin_fmaf(l_run, alpha, xr[wt][u][r16]);
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {      // O transposed: row r16 in every lane
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[0][i] = o[0][i] * alpha;
                o[1][i] = o[1][i] * alpha;
            }
        }
        const char *Vu = lds + u * 2 * KBYTES + KBYTES;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const u32x4 pf = pbuf[wt][u][c][lane];
            const int row0 = 32 * c + 4 * g + (r16 >> 2);
            const int row1 = row0 + 16;
            u32x4 vf[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ch = 2 * (2 * w + j) + ((r16 & 3) >> 1);
                const int off = 8 * (r16 & 1);
                const u32x2 lo = lds_read_tr16(Vu + row0 * ROWB + ((ch ^ ((row0 & 7) << 1)) << 4) + off);
                const u32x2 hi = lds_read_tr16(Vu + row1 * ROWB + ((ch ^ ((row1 & 7) << 1)) << 4) + off);
                vf[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) o[j] = Mfma<dt>::step(vf[j], pf, o[j]);    // O^T += V^T . P^T
        }
    }

    if (p.nsplit == 1) {
        // one split: sdpa_combine's fold of a single partial (after the sink, if any), done here; lane
        // (r16, g) holds row r16, columns 16 t + 4 g + i
        const int ro = tile * 16 + r16;
        if (ro >= R) return;
        const float ms = m_run, ls = l_run;
        const int iq = ro / p.G, h = gk * p.G + ro % p.G;
        {
            bool have = false;
            float m = 0.0f, l = 0.0f;
            if (p.sinks) {
                m = sink2(p, h);
                l = 1.0f;
                have = true;
            }
            float a = 0.0f, bs = 0.0f;
            bool first = false;
            const bool skip = ms == NEG_INF;
            if (!skip) {
                if (!have) {
                    first = true;
                    l = ls;
                } else {
                    const float m2 = fmaxf(m, ms);
                    a = exp2_hw(m - m2);
                    bs = exp2_hw(ms - m2);
                    l = __builtin_fmaf(l, a, ls * bs);
                }
                have = true;
            }
            char *orow = static_cast<char *>(p.o) +
                         ((int64_t)b * p.os[0] + (int64_t)h * p.os[1] + (int64_t)iq * p.os[2]) * Elem<dt>::bytes;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int t = 2 * w + j;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float acc = skip ? 0.0f : first ? o[j][i] : __builtin_fmaf(0.0f, a, o[j][i] * bs);
                    float v = have ? acc / l : 0.0f;
                    v = v + 0.0f;                    // -0 -> +0
                    if (16 * t < p.dr) store_from_f32<dt>(orow, 16 * t + 4 * g + i, v);
                }
            }
        }
        return;
    }

    // ---- the split's partial, as sdpa_split16 stores it (row r16, columns 16 t + 4 g .. + 3 per lane)
    const int rg = tile * 16 + r16;
    if (rg < R) {
        const int64_t rowid = ((int64_t)b * p.Hq + gk * p.G + rg % p.G) * p.Lq + rg / p.G;
        if (w == 0 && g == 0) {
            float *ml = p.ws_ml + (rowid * p.nsplit + sp) * 2;
            ml[0] = m_run;
            ml[1] = l_run;
        }
        float *dst = p.ws_o + (rowid * p.nsplit + sp) * p.dr;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = 2 * w + j;
            if (16 * t < p.dr) *reinterpret_cast<f32x4 *>(dst + 16 * t + 4 * g) = o[j];
        }
    }
}

// sdpa_combine's step for one split's partial (m_run, l_run, o) of the rows of a wavefront's 16-row tile,
// folded into the running state (have, mt, lt, ot): per score row (lane r16), skip an empty partial, copy
// the first non-empty one, otherwise rescale both sides to the larger maximum; O rows 4 g + i take the
// factors of their score rows.  The split state then restarts empty.  When no row of the tile skips or
// copies (the common case), the selects between the three outcomes are left out: they would all pick
// the rescaled sum.
template <int NT, bool OT = false>
__device__ __forceinline__ void fold_split16(float &m_run, float &l_run, f32x4 (&o)[NT], bool &have, float &mt,
                                             float &lt, f32x4 (&ot)[NT]) {
    constexpr float NEG_INF = -__builtin_huge_valf();
    const int g = (threadIdx.x & 63) >> 4;
    const bool skip = m_run == NEG_INF;
    const bool first = !skip && !have;
    const float m2 = fmaxf(mt, m_run);
    const float a = exp2_hw(mt - m2);
    const float bs = exp2_hw(m_run - m2);
    if (first) {
        mt = m_run;
        lt = l_run;
    } else if (!skip) {
        lt = __builtin_fmaf(lt, a, l_run * bs);
        mt = m2;
    }
    if (__builtin_amdgcn_ballot_w64(skip || first) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int src = 4 * g + i;
            const float a_i = OT ? a : __shfl(a, src), b_i = OT ? bs : __shfl(bs, src);
#pragma unroll
            for (int t = 0; t < NT; ++t) ot[t][i] = __builtin_fmaf(ot[t][i], a_i, o[t][i] * b_i);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int src = 4 * g + i;
            const bool skip_i = OT ? skip : __shfl((int)skip, src) != 0;
            const bool first_i = OT ? first : __shfl((int)first, src) != 0;
            const float a_i = OT ? a : __shfl(a, src), b_i = OT ? bs : __shfl(bs, src);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float f = __builtin_fmaf(ot[t][i], a_i, o[t][i] * b_i);
                ot[t][i] = first_i ? o[t][i] : skip_i ? ot[t][i] : f;
            }
        }
    }
    have = have || !skip;
    m_run = NEG_INF;
    l_run = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] = zero4();
}

// sdpa_combine's step when every row's split partial is non-empty (m_run finite): the rescaled sum, with no
// branch.  A running state that is still empty (mt = -inf, lt = 0, ot = 0) takes the partial itself, as
// the combine's copy does: a = exp2(-inf) = 0 and bs = 1 give lt = l_run and ot = o, except that a zero of
// o may come out with the other sign, which no later fold, the division or the final -0 -> +0 step can turn
// into a different output bit.
template <int NT, bool OT = false>
__device__ __forceinline__ void fold_split16_full(float &m_run, float &l_run, f32x4 (&o)[NT], bool &have,
                                                  float &mt, float &lt, f32x4 (&ot)[NT]) {
    constexpr float NEG_INF = -__builtin_huge_valf();
    const int g = (threadIdx.x & 63) >> 4;
    const float m2 = fmaxf(mt, m_run);
    const float a = exp2_hw(mt - m2);
    const float bs = exp2_hw(m_run - m2);
    lt = __builtin_fmaf(lt, a, l_run * bs);
    mt = m2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int src = 4 * g + i;
        const float a_i = OT ? a : __shfl(a, src), b_i = OT ? bs : __shfl(bs, src);
#pragma unroll
        for (int t = 0; t < NT; ++t) ot[t][i] = __builtin_fmaf(ot[t][i], a_i, o[t][i] * b_i);
    }
    have = true;
    m_run = NEG_INF;
    l_run = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] = zero4();
}

// Direct-to-LDS loads written as asm, so that the compiler does not know about them: it would otherwise
// wait for every such load in flight before any transposed LDS read (it cannot tell which buffer a
// transposed read touches).  The kernel that issues them waits for them itself (asm_wait_vmcnt0, then a
// barrier) before any wavefront reads the bytes; they write no register.  saddr form: a uniform 64-bit
// base plus this lane's 32-bit offset; vaddr form: this lane's 64-bit address.
__device__ __forceinline__ void dma16_saddr(const char *base, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff), "s"(base)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma16_vaddr(const char *src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void asm_wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The V fragments of one 32-key half as attn_vfrags16 reads them, for output column tiles t < NT: va[t] is
// the LDS address of tile t's first row-0 read of half 0 in the buffer, HOFF the byte offset of the half
// (+ 16 key rows for the second read of a tile).
__device__ __forceinline__ u32x2 lds_tr16_at(uint32_t addr) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(size_t)addr);
    return __builtin_bit_cast(u32x2, v);
}
template <int HOFF, int NT, int ROWB = 256>
__device__ __forceinline__ void vfrags_tr(const uint32_t (&va)[NT], u32x4 (&vf)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const u32x2 lo = lds_tr16_at(va[t] + HOFF), hi = lds_tr16_at(va[t] + HOFF + 16 * ROWB);
        vf[t] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
}

// Long prefill for 16-bit head dims D = 32, 64, 96, 128, software-pipelined over key blocks.  W row
// tiles of one (batch, KV head), one per wavefront, share each K and V block through LDS; K runs two
// blocks ahead and V one: while block j's softmax runs, block j + 1's scores are formed from its K block
// on the matrix cores, and the loads of K(j + 2) and V(j + 1) are in flight.  Per tile the arithmetic is
// the split path's: the same score chains (d chunks in order), attn_softmax16, P . V over the two 32-key
// halves in order, a fresh (m, l, O) at every 256-key split and the combine's fold into the running
// state, so every row gets the bits of the split + combine path.  Splits whose blocks every row of the
// workgroup sees completely (no mask, inside S, before the first row's causal position) run a
// branch-free body: visibility known, rescale by alpha always (O * 1 = O), the fold without its
// empty-partial cases.  O is accumulated transposed (V^T . P^T on the matrix cores: each lane then holds
// output columns of its own score row, so the rescale and the split fold need no lane exchange; the
// products and their k order are those of P . V).  Causal workgroups start longest first.  Below D = 128 the kernel takes only the
// head dim's D / 32 score chunks and D / 16 output column tiles (the LDS rows keep the 256-byte layout;
// chunks at d >= D are neither loaded nor read), which are the split kernel's chains for that D.
template <int dt, int W, int D>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
void sdpa_prefill16p(SdpaParams p) {
    constexpr int NC = D / 32;                         // d chunks of the score chains
    constexpr int NT = D / 16;                         // output column tiles
    static_assert(D % 32 == 0 && D <= 128, "head dims 32, 64, 96, 128");
    // key rows of 256 bytes (chunks at d >= D neither loaded nor read), or of 128 for D = 64, which halves
    // the LDS per workgroup so that its ~150 registers per lane can run three wavefronts per SIMD
    constexpr bool C128 = D == 64;
    constexpr int ROWB = C128 ? 128 : 256;
    constexpr int RPL = 1024 / ROWB;                   // key rows per 1 KiB load
    constexpr int KBYTES = KV_BLOCK * ROWB;            // one K or V block
    constexpr int QW = KBYTES / 1024 / W;              // 1 KiB loads per wavefront per K (or V) block
    constexpr int BPS = KV_SPLIT / KV_BLOCK;           // blocks per split
    constexpr float NEG_INF = -__builtin_huge_valf();
    static_assert((KBYTES / 1024) % W == 0, "every wavefront issues the same loads");
    // LDS: K block buffers and V block buffers, two of each
    __shared__ __attribute__((aligned(1024))) char kbuf0[KBYTES];
    __shared__ __attribute__((aligned(1024))) char kbuf1[KBYTES];
    __shared__ __attribute__((aligned(1024))) char vbufs[2 * KBYTES];
    char *const vbuf0 = vbufs, *const vbuf1 = vbufs + KBYTES;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int R = p.G * p.Lq;
    const int ntile = (R + 15) / 16;
    const int nwt = (ntile + W - 1) / W;
    int wt, grp;
    attn_work(nwt, p.B * p.Hkv, wt, grp);
    if (p.causal) wt = nwt - 1 - wt;                   // the workgroups with the most keys start first
    const int b = grp / p.Hkv, gk = grp % p.Hkv;
    const int tile = wt * W + wave;                    // tiles past the last compute clamped rows, store nothing

    const int rlast = min((wt + 1) * W * 16 - 1, R - 1);
    const int nkeys = p.causal ? min(p.S - p.Lq + rlast / p.G + 1, p.S) : p.S;
    const int nblk = (nkeys + KV_BLOCK - 1) / KV_BLOCK;
    // splits every row of the workgroup sees completely; the last block always runs the general body
    const int pos_wg = p.S - p.Lq + (wt * W * 16) / p.G;           // first row's causal position
    int nfast = p.mask != nullptr ? 0 : (p.causal ? min(pos_wg + 1, p.S) : p.S) / KV_SPLIT;
    nfast = max(0, min(nfast, (nblk - 1) / BPS));

    const char *kbase = static_cast<const char *>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)gk * p.ks[1]) * 2;
    const char *vbase = static_cast<const char *>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)gk * p.vs[1]) * 2;
    const int64_t kstr = p.ks[2] * 2, vstr = p.vs[2] * 2;
    // load j of a K (or V) block covers key rows RPL q .. RPL q + RPL - 1, q = wave + W j: lane L row
    // RPL q + L / SPR, slot L mod SPR (K chunk slot ^ (row mod 16), V chunk slot ^ 2 (row mod 8); for
    // 128-byte rows K slot ^ ((row / 2) mod 8), V slot ^ 2 ((row / 2) mod 4)).  A block
    // inside S is a uniform base plus these 32-bit lane offsets; the block crossing S (and every block when
    // a key row stride is too large for 32-bit offsets) clamps rows to S - 1 in 64-bit arithmetic.
    constexpr int SPR = ROWB / 16;                     // slots per key row
    const int lrow = lane / SPR, lslot = lane % SPR;
    const bool off32 = (uint64_t)max(kstr, vstr) * KV_BLOCK + ROWB <= 0xffffffffull;
    // the chunk slots do not depend on j (RPL W j is a multiple of 16), so load j is load 0 plus RPL W j rows
    static_assert((RPL * W) % 16 == 0, "row period of the chunk swizzles");
    const int row0 = RPL * wave + lrow;
    const int ck = lslot ^ (C128 ? (row0 >> 1) & 7 : row0 & 15);
    const int cv = lslot ^ (C128 ? ((row0 >> 1) & 3) << 1 : (row0 & 7) << 1);
    const bool kin = 8 * ck < D, vin = 8 * cv < D;     // this lane's chunk lies inside the head dim
    const uint32_t koff = (uint32_t)(row0 * kstr) + (ck << 4), voff = (uint32_t)(row0 * vstr) + (cv << 4);
    auto issue = [&](int blk, char *buf, bool isv) {
        const int kb = blk * KV_BLOCK;
        const char *base = isv ? vbase : kbase;
        const int64_t str = isv ? vstr : kstr;
        const uint32_t lbase = (uint32_t)(uintptr_t)BI_LDS_PTR(buf) + wave * 1024;
        if (D == 128 || (isv ? vin : kin)) {
            if (off32 && kb + KV_BLOCK <= p.S) {
#pragma unroll
                for (int j = 0; j < QW; ++j)
                    dma16_saddr(base + (int64_t)(kb + RPL * W * j) * str, isv ? voff : koff, lbase + W * j * 1024);
            } else {
#pragma unroll
                for (int j = 0; j < QW; ++j) {
                    const int row = row0 + RPL * W * j;
                    const int64_t key = min(kb + row, p.S - 1);
                    dma16_vaddr(base + key * str + ((isv ? cv : ck) << 4), lbase + W * j * 1024);
                }
            }
        }
    };

    Rows16T<NC> r;
    rows16_load<dt>(p, tile, b, gk, r);
    // running fold over splits (per score row in lane r16; empty: mt = -inf, lt = 0) and the current
    // split's state; the sink, if any, is the fold's first partial
    bool have = false;
    float mt = NEG_INF, lt = 0.0f;
    if (p.sinks) {
        const int rgc = min(tile * 16 + r16, R - 1);
        mt = sink2(p, gk * p.G + rgc % p.G);
        lt = 1.0f;
        have = true;
    }
    float m_run = NEG_INF, l_run = 0.0f;
    f32x4 o[NT], ot[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        o[t] = zero4();
        ot[t] = zero4();
    }
    // per-lane LDS addresses of the V reads (attn_vfrags16's row-0 address of tile t, half 0) in buffer 0;
    // buffer 1 is KBYTES further
    uint32_t va[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int row0 = 4 * g + (r16 >> 2);
        const int ch = 2 * t + ((r16 & 3) >> 1);
        const int sw = C128 ? ((row0 >> 1) & 3) << 1 : (row0 & 7) << 1;      // same for row0 + 16, + 32
        const uint32_t off = (uint32_t)(row0 * ROWB + ((ch ^ sw) << 4) + 8 * (r16 & 1));
        va[t] = (uint32_t)(uintptr_t)BI_LDS_PTR(vbufs) + off;
    }
    // scores of a block from its K block: each key tile's chain takes d chunks 0 .. NC - 1 in order
    auto scores = [&](const char *Ks, f32x4 (&st)[4]) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            u32x4 kf[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c)
                kf[c] = *reinterpret_cast<const u32x4 *>(Ks + (16 * kt + r16) * ROWB +
                                                         (((4 * c + g) ^ (C128 ? (r16 >> 1) & 7 : r16)) << 4));
            st[kt] = zero4();
#pragma unroll
            for (int c = 0; c < NC; ++c) st[kt] = Mfma<dt>::step(kf[c], r.qf[c], st[kt]);
        }
    };
    // the V fragments of V buffer VB (both 32-key halves), and O += P . V from them
    auto vread = [&](auto vb, u32x4 (&vf)[2][NT]) {
        constexpr int VB = decltype(vb)::value;
        vfrags_tr<VB * KBYTES, NT, ROWB>(va, vf[0]);
        vfrags_tr<VB * KBYTES + 32 * ROWB, NT, ROWB>(va, vf[1]);
    };
    // O^T += V^T . P^T: the V fragments as the A operand and P as the B operand give each element the
    // products and k order of O += P . V, with rows and columns of the tile swapped
    auto pv = [&](const u32x4 (&pf)[2], const u32x4 (&vf)[2][NT]) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t = 0; t < NT; ++t) o[t] = Mfma<dt>::step(vf[c][t], pf[c], o[t]);
    };

    using VB0 = std::integral_constant<int, 0>;
    using VB1 = std::integral_constant<int, 1>;
    f32x4 st_cur[4], st_nxt[4];
    // block j: its V block (and K of block j + 1) landed, published by the barrier; then K(j + 2) goes into
    // the K buffer block j's scores were read from (in block j - 1) and V(j + 1) into the V buffer block
    // j - 1 read; block j + 1's scores, block j's softmax and P . V
    auto top = [&](int j, char *kfree, char *vnext, char *vcur) {
        const int kb = j * KV_BLOCK;
        asm_wait_vmcnt0();                               // this wavefront's loads of K(j + 1) and V(j) landed
        if (kb + KV_BLOCK > p.S) {
            // V rows past S read as zero; each wavefront clears the rows its own loads filled
#pragma unroll
            for (int jj = 0; jj < QW; ++jj) {
                const int row = RPL * (wave + W * jj) + lrow;
                if (kb + row >= p.S) *reinterpret_cast<u32x4 *>(vcur + row * ROWB + lslot * 16) = zero_u4();
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
        }
        __syncthreads();
        if (j + 2 < nblk) issue(j + 2, kfree, false);
        if (j + 1 < nblk) issue(j + 1, vnext, true);
    };
    auto fast_block = [&](int j, char *kfree, const char *knext, char *vnext, char *vcur, auto vb) {
        top(j, kfree, vnext, vcur);
        scores(knext, st_nxt);
        u32x4 pf[2];
        attn_softmax16<dt, NC, NT, true, true, true>(p, r, st_cur, j * KV_BLOCK, m_run, l_run, o, pf);
        u32x4 vf[2][NT];
        vread(vb, vf);
        pv(pf, vf);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) st_cur[kt] = st_nxt[kt];
    };
    auto general_block = [&](int j, char *kfree, const char *knext, char *vnext, char *vcur, auto vb) {
        top(j, kfree, vnext, vcur);
        if (j + 1 < nblk) scores(knext, st_nxt);
        u32x4 pf[2];
        attn_softmax16<dt, NC, NT, false, false, true>(p, r, st_cur, j * KV_BLOCK, m_run, l_run, o, pf);
        u32x4 vf[2][NT];
        vread(vb, vf);
        pv(pf, vf);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) st_cur[kt] = st_nxt[kt];
        if ((j + 1) % BPS == 0 || j + 1 == nblk) fold_split16<NT, true>(m_run, l_run, o, have, mt, lt, ot);
    };

    if (nblk > 0) {
        issue(0, kbuf0, false);
        issue(0, vbuf0, true);
        if (nblk > 1) issue(1, kbuf1, false);
        asm_wait_vmcnt0();
        __syncthreads();
        scores(kbuf0, st_cur);
    }
    // block j reads K(j + 1) from kbuf[(j + 1) % 2] and V(j) from vbuf[j % 2]
    for (int sp = 0; sp < nfast; ++sp) {
        const int j = sp * BPS;
        fast_block(j, kbuf0, kbuf1, vbuf1, vbuf0, VB0{});
        fast_block(j + 1, kbuf1, kbuf0, vbuf0, vbuf1, VB1{});
        fast_block(j + 2, kbuf0, kbuf1, vbuf1, vbuf0, VB0{});
        fast_block(j + 3, kbuf1, kbuf0, vbuf0, vbuf1, VB1{});
        fold_split16_full<NT, true>(m_run, l_run, o, have, mt, lt, ot);
    }
    for (int j = nfast * BPS; j < nblk; j += 2) {
        general_block(j, kbuf0, kbuf1, vbuf1, vbuf0, VB0{});
        if (j + 1 < nblk) general_block(j + 1, kbuf1, kbuf0, vbuf0, vbuf1, VB1{});
    }

    // normalise, canonicalise -0, round once: O row r16, columns 16 t + 4 g + i
    const int ro = tile * 16 + r16;
    if (ro < R) {
        const int iq = ro / p.G, h = gk * p.G + ro % p.G;
        char *orow = static_cast<char *>(p.o) +
                     ((int64_t)b * p.os[0] + (int64_t)h * p.os[1] + (int64_t)iq * p.os[2]) * Elem<dt>::bytes;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = have ? ot[t][i] / lt : 0.0f;
                v = v + 0.0f;                            // -0 -> +0
                store_from_f32<dt>(orow, 16 * t + 4 * g + i, v);
            }
    }
}

// Long prefill for 16-bit head dims 160 ... 256: rows zero-padded to 256 (chunks at d >= D read the zero
// page).  A workgroup produces NT 16-wide output column tiles: all 16 (NT = 16, the launched form), or
// one half (NT = 8: two workgroups per row tile group, each computing the full scores and P and
// applying P to its 128 columns of V; measured 1.3-1.5x slower, as the scores are computed twice).
// Every output column is the same chain as in the split kernel (scores over all d chunks in order, P
// rounded once, P . V over each block's keys).  Otherwise as the D = 128 prefill: W row tiles of one (batch,
// KV head) walk the key blocks in ascending order with NB LDS buffers, restart (m, l, O) at every
// 256-key split and fold the split partials in registers with the combine's operations.  A buffer holds
// the K block with 512-byte rows (load q covers key rows 2 q and 2 q + 1, lane L row 2 q + L / 32, slot
// L mod 32, chunk slot ^ (row mod 16)) and the workgroup's V columns with 32 NT-byte rows (chunk c of
// key r at slot c ^ 2 (r mod 8)).
template <int dt, int W, int NB, int NT = 8>
__global__ __launch_bounds__(64 * W) void sdpa_prefill16w(SdpaParams p) {
    constexpr int NC = 8;                              // 32-wide d chunks of a padded row
    constexpr int NH = 16 / NT;                        // workgroups per row tile group (column halves)
    constexpr int KROWB = 512, VROWB = 32 * NT;
    constexpr int RPV = 1024 / VROWB, SPV = VROWB / 16;   // V rows per load instruction, slots per V row
    constexpr int KBYTES = KV_BLOCK * KROWB;           // one K block
    constexpr int VBYTES = KV_BLOCK * VROWB;           // the V block's columns of this workgroup
    constexpr int BUF = KBYTES + VBYTES;
    constexpr int QKB = KBYTES / 1024, QVB = VBYTES / 1024;
    constexpr int QBLK = QKB + QVB;                    // 1 KiB loads per block
    constexpr int QW = QBLK / W;                       // loads per wavefront per block
    constexpr int QKW = QKB / W;                       // of which K loads (j < QKW)
    constexpr int BPS = KV_SPLIT / KV_BLOCK;
    constexpr float NEG_INF = -__builtin_huge_valf();
    static_assert(QBLK % W == 0 && QKB % W == 0, "every wavefront issues the same loads");
    static_assert(NB >= 2 && QW * (NB - 2) <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char lds[NB * BUF];   // [buffer][K block | V columns]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int R = p.G * p.Lq;
    const int ntile = (R + 15) / 16;
    int wt, grp;
    attn_work((ntile + W - 1) / W, p.B * p.Hkv * NH, wt, grp);
    const int half = grp % NH;                         // output columns 16 NT half .. + 16 NT - 1
    const int b = (grp / NH) / p.Hkv, gk = (grp / NH) % p.Hkv;
    const int tile = wt * W + wave;

    const int rlast = min(wt * W * 16 + W * 16 - 1, R - 1);
    const int nkeys = p.causal ? min(p.S - p.Lq + rlast / p.G + 1, p.S) : p.S;
    const int nblk = (nkeys + KV_BLOCK - 1) / KV_BLOCK;

    const char *kbase = static_cast<const char *>(p.k) + ((int64_t)b * p.ks[0] + (int64_t)gk * p.ks[1]) * 2;
    const char *vbase = static_cast<const char *>(p.v) + ((int64_t)b * p.vs[0] + (int64_t)gk * p.vs[1]) * 2 +
                        VROWB * half;
    const int64_t kstr = p.ks[2] * 2, vstr = p.vs[2] * 2;
    // per load j of this wavefront: its key row in the block, LDS byte offset, source chunk byte offset
    int lrowj[QW], ldst[QW], lcb[QW];
    bool lz[QW];
#pragma unroll
    for (int j = 0; j < QW; ++j) {
        const int q = wave + W * j;
        if (j < QKW) {
            const int row = 2 * q + (lane >> 5), slot = lane & 31;
            const int c = slot ^ (row & 15);
            lrowj[j] = row;
            ldst[j] = q * 1024;
            lcb[j] = c << 4;
            lz[j] = 8 * c >= p.dr;
        } else {
            const int qv = q - QKB;
            const int row = RPV * qv + lane / SPV, slot = lane % SPV;
            const int c = slot ^ ((row & 7) << 1);
            lrowj[j] = row;
            ldst[j] = KBYTES + qv * 1024;
            lcb[j] = c << 4;
            lz[j] = 16 * NT * half + 8 * c >= p.dr;
        }
    }
    const char *zp = reinterpret_cast<const char *>(g_zero_page);
    auto issue = [&](int blk) {
        const int kb = blk * KV_BLOCK;
        char *buf = lds + (blk % NB) * BUF;
#pragma unroll
        for (int j = 0; j < QW; ++j) {
            const int64_t key = min(kb + lrowj[j], p.S - 1);   // rows past S read row S - 1
            const char *src = lz[j] ? zp : (j < QKW ? kbase + key * kstr : vbase + key * vstr) + lcb[j];
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(src), BI_LDS_PTR(buf + ldst[j]), 16, 0, 0);
        }
    };

    Rows16T<NC> r;
    rows16_load<dt>(p, tile, b, gk, r);
    bool have = false;
    float mt = 0.0f, lt = 0.0f;
    if (p.sinks) {
        const int rgc = min(tile * 16 + r16, R - 1);
        mt = sink2(p, gk * p.G + rgc % p.G);
        lt = 1.0f;
        have = true;
    }
    f32x4 ot[NT];
    float m_run = NEG_INF, l_run = 0.0f;
    f32x4 o[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        ot[t] = zero4();
        o[t] = zero4();
    }
    auto fold_split = [&]() { fold_split16(m_run, l_run, o, have, mt, lt, ot); };

    for (int j = 0; j < NB - 1 && j < nblk; ++j) issue(j);
    for (int blk = 0; blk < nblk; ++blk) {
        const int kb = blk * KV_BLOCK;
        char *Ks = lds + (blk % NB) * BUF;
        char *Vs = Ks + KBYTES;
        if (blk + NB - 2 < nblk) BI_WAIT_VMCNT(QW * (NB - 2));   // this wavefront's loads of block blk landed
        else BI_WAIT_VMCNT(0);
        if (kb + KV_BLOCK > p.S) {
            // V rows past S read as zero; each wavefront clears the rows its own loads filled
#pragma unroll
            for (int j = QKW; j < QW; ++j) {
                const int row = lrowj[j];
                if (kb + row >= p.S) *reinterpret_cast<u32x4 *>(Vs + row * VROWB + (lane % SPV) * 16) = zero_u4();
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
        }
        __syncthreads();                                 // block blk visible to all; block blk - 1 no longer read
        if (blk + NB - 1 < nblk) issue(blk + NB - 1);
        attn_block16<dt>(p, r, Ks, Vs, kb, m_run, l_run, o, []() {}, []() {});
        if ((blk + 1) % BPS == 0 || blk + 1 == nblk) fold_split();
    }

    const float lrow_l = lt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ro = tile * 16 + 4 * g + i;
        const bool have_i = __shfl((int)have, 4 * g + i) != 0;
        const float l_i = __shfl(lrow_l, 4 * g + i);
        if (ro >= R) continue;
        const int iq = ro / p.G, h = gk * p.G + ro % p.G;
        char *orow = static_cast<char *>(p.o) +
                     ((int64_t)b * p.os[0] + (int64_t)h * p.os[1] + (int64_t)iq * p.os[2]) * Elem<dt>::bytes;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float v = have_i ? ot[t][i] / l_i : 0.0f;
            v = v + 0.0f;                                // -0 -> +0
            const int col = 16 * NT * half + 16 * t + r16;
            if (col < p.dr) store_from_f32<dt>(orow, col, v);
        }
    }
}

// Fold the split partials of one query row left to right, normalise, round.
// One thread per output column; the partials of CH splits are loaded together
// (independent loads in flight at once), then folded one split at a time in
// ascending order.
template <int dt, int D, int CH = 16>
__global__ __launch_bounds__(D) void sdpa_combine(SdpaParams p) {
    constexpr float NEG_INF = -__builtin_huge_valf();
    const int64_t rowid = blockIdx.x;
    const int d = threadIdx.x;
    const int iq = (int)(rowid % p.Lq);
    const int h = (int)((rowid / p.Lq) % p.Hq);
    const int b = (int)(rowid / ((int64_t)p.Lq * p.Hq));
    const float *ml = p.ws_ml + rowid * p.nsplit * 2;
    const float *po = p.ws_o + rowid * p.nsplit * D;

    bool have = false;
    float m = 0.0f, l = 0.0f, o = 0.0f;
    if (p.sinks) {                                 // the sink is the fold's first partial
        m = sink2(p, h);
        l = 1.0f;
        have = true;
    }
    for (int s0 = 0; s0 < p.nsplit; s0 += CH) {
        float ms[CH], ls[CH], os[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int sp = min(s0 + u, p.nsplit - 1);
            ms[u] = ml[2 * sp];
            ls[u] = ml[2 * sp + 1];
            os[u] = po[sp * D + d];
        }
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            if (s0 + u >= p.nsplit || ms[u] == NEG_INF) continue;   // past the end / split saw no key of this row
            if (!have) {
                m = ms[u];
                l = ls[u];
                o = os[u];
                have = true;
                continue;
            }
            const float m2 = fmaxf(m, ms[u]);
            const float a = exp2_hw(m - m2);
            const float bs = exp2_hw(ms[u] - m2);
            l = __builtin_fmaf(l, a, ls[u] * bs);
            o = __builtin_fmaf(o, a, os[u] * bs);
            m = m2;
        }
    }
    char *orow = static_cast<char *>(p.o) +
                 ((int64_t)b * p.os[0] + (int64_t)h * p.os[1] + (int64_t)iq * p.os[2]) * Elem<dt>::bytes;
    float r = have ? o / l : 0.0f;
    r = r + 0.0f;                                  // -0 -> +0
    store_from_f32<dt>(orow, d, r);
}

// The same fold for rows with many splits: one workgroup of 256 threads per query row stages the partials
// of up to CHUNK splits in LDS, every load requested before any is used, and its first D threads fold them
// in ascending split order while the next chunk's loads are in flight.  The fold is sdpa_combine's written
// without branches: the empty state is m = -inf, l = o = 0, so a first partial enters through the ordinary
// step (a = exp2(-inf) = 0, bs = exp2(0) = 1, hence l = ls and o = os, exactly) and an empty split's step is
// computed and then discarded by a select.  The two forms give the same bits up to the sign of a zero o,
// which the final o / l + 0 removes.  Without branches the eight steps of a group share one basic block, so
// their exponentials overlap and only the max / fma chains are serial.
template <int dt, int D, int CHUNK>
__global__ __launch_bounds__(256) void sdpa_combine_lds(SdpaParams p) {
    constexpr float NEG_INF = -__builtin_huge_valf();
    constexpr int PER = CHUNK * D / 4 / 256;           // 16-byte loads of O partials per thread per chunk
    static_assert(CHUNK * D % 1024 == 0 && 2 * CHUNK <= 256 && CHUNK % 8 == 0, "chunk layout");
    __shared__ float sml[2 * CHUNK];
    __shared__ __attribute__((aligned(16))) float so[CHUNK * D];
    const int64_t rowid = blockIdx.x;
    const int tid = threadIdx.x, d = tid;
    const int iq = (int)(rowid % p.Lq);
    const int h = (int)((rowid / p.Lq) % p.Hq);
    const int b = (int)(rowid / ((int64_t)p.Lq * p.Hq));
    const float *ml = p.ws_ml + rowid * p.nsplit * 2;
    const float *po = p.ws_o + rowid * p.nsplit * D;

    f32x4 v[PER];
    float mlv;
    auto fetch = [&](int s0) {
        const int n = min(CHUNK, p.nsplit - s0);
        const f32x4 *src = reinterpret_cast<const f32x4 *>(po + (int64_t)s0 * D);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + 256 * k;
            v[k] = i < n * D / 4 ? src[i] : zero4();
        }
        mlv = tid < 2 * n ? ml[2 * s0 + tid] : NEG_INF;
    };

    // the sink is the fold's first partial
    float m = p.sinks ? sink2(p, h) : NEG_INF, l = p.sinks ? 1.0f : 0.0f, o = 0.0f;
    fetch(0);
    for (int s0 = 0; s0 < p.nsplit; s0 += CHUNK) {
        const int n = min(CHUNK, p.nsplit - s0);
#pragma unroll
        for (int k = 0; k < PER; ++k) reinterpret_cast<f32x4 *>(so)[tid + 256 * k] = v[k];
        if (tid < 2 * CHUNK) sml[tid] = mlv;
        __syncthreads();
        if (s0 + CHUNK < p.nsplit) fetch(s0 + CHUNK);
        if (d < D) {
            for (int u0 = 0; u0 < n; u0 += 8) {
                float ms[8], ls[8], os[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    ms[j] = sml[2 * (u0 + j)];             // -inf past the end: skipped like an empty split
                    ls[j] = sml[2 * (u0 + j) + 1];
                    os[j] = so[(u0 + j) * D + d];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bool skip = ms[j] == NEG_INF;     // split saw no key of this row
                    const float m2 = fmaxf(m, ms[j]);
                    const float a = exp2_hw(m - m2);
                    const float bs = exp2_hw(ms[j] - m2);
                    const float l2 = __builtin_fmaf(l, a, ls[j] * bs);
                    const float o2 = __builtin_fmaf(o, a, os[j] * bs);
                    l = skip ? l : l2;
                    o = skip ? o : o2;
                    m = m2;
                }
            }
        }
        __syncthreads();
    }
    if (d >= D) return;
    char *orow = static_cast<char *>(p.o) +
                 ((int64_t)b * p.os[0] + (int64_t)h * p.os[1] + (int64_t)iq * p.os[2]) * Elem<dt>::bytes;
    float r = m != NEG_INF ? o / l : 0.0f;
    r = r + 0.0f;                                  // -0 -> +0
    store_from_f32<dt>(orow, d, r);
}

// Query chunks of at least this many rows against caches longer than four
// splits take the workspace-free prefill kernel (measured: below ~300 rows the
// split kernel's extra parallelism wins, above it the shared K / V blocks do).
constexpr int64_t PREFILL_MIN_LQ = 384;
// Shorter chunks take it too when the quad kernel does not apply and a KV head has at least one full
// workgroup of rows (four 16-row tiles), measured at D = 128, causal (one-launch / split kernel against
// prefill): B = 8, 16 / 4 heads, 256 rows at 256 keys 51.3 -> 18.5 us, at 1024 keys 127.5 -> 35.0;
// B = 4, 32 / 8 heads, 128 rows at 2048 keys 98.3 -> 42.7; B = 2, 256 rows at 4096 keys 180.4 -> 73.8;
// B = 8, 64 rows at 1024 keys 70.2 -> 27.2; B = 16, 16 rows at 1024 keys 34.5 -> 27.8.  Decode rows
// (four per KV head) stay on the other kernels, which were as fast or faster there.
constexpr int64_t PREFILL_MIN_ROWS = 64;
// Either way (D <= 128) only when the prefill grid has more than this many workgroups: the split kernel
// also spreads a row tile's keys over workgroups, and on small grids with long caches that wins (B = 1,
// 32 / 32 heads, 64 rows at 2048 keys: 32 prefill workgroups 41.2 us, split 20.0; 384 rows of 8 / 8
// heads at 8192 keys: 48 workgroups 133 against 75; 16 / 16 heads, 256 rows at 8192 keys: 64, 136
// against 96), while from 96 workgroups on the prefill kernel was as fast or faster (16 / 16 heads, 384
// rows at 2048 keys: 39.7 against 43.7; 128 workgroups of 8 / 2 heads, 1024 rows at 8192 keys: 134
// against 179).
constexpr int64_t PREFILL_MIN_WG = 64;
static int64_t prefill_workgroups(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq) {
    return ((Hq / Hkv * Lq + 15) / 16 + 3) / 4 * B * Hkv;
}
// 16-bit head dims above 128 take the wide prefill kernel from 64 query rows on once the batch holds at
// least 192 of them (measured at D = 256 and 192 against the generic split kernel: B = 1, 2048 keys,
// 192 rows 132 -> 103 us; B = 4, 64 rows 173 -> 105 us; B = 1, 128 rows and B = 4, 32 rows stay
// faster on the split kernel).
constexpr int64_t WIDE_PREFILL_MIN_LQ = 64, WIDE_PREFILL_MIN_ROWS = 192;
// Calls whose quad grid (one workgroup per split and one or two row tiles)
// holds at most one workgroup per CU take the quad kernel, which requests a
// whole split at once (measured at 32 query heads, 8 KV heads, D = 128: one decode row at
// 1024 keys 14.5 -> 12.5 us, 16 rows 19.3 -> 14.1 us, one row at 8192 keys
// 21.2 -> 17.3 us; with 512 workgroups or more the one-launch and split
// kernels are faster).
constexpr int64_t QUAD_MAX_WG = 256;
// Row tiles per quad workgroup: one when that grid fits, else two (sharing the split's K / V; measured:
// 16 rows at 4096 keys 19.8 -> 16.7 us, 64 rows at 1024 keys 19.9 -> 17.0 us, while at grids that
// already fit two tiles per workgroup cost 0.1-0.3 us), else 0: the quad kernel does not apply.
static int64_t quad_tiles(int64_t B, int64_t Hkv, int64_t nsplit, int64_t ntile) {
    auto fits = [&](int64_t groups) {
        return B * Hkv <= QUAD_MAX_WG && groups <= QUAD_MAX_WG && nsplit <= QUAD_MAX_WG &&
               nsplit * groups * B * Hkv <= QUAD_MAX_WG;
    };
    if (fits(ntile)) return 1;
    if (ntile >= 2 && fits((ntile + 1) / 2)) return 2;
    return 0;
}
// 16-bit D = 256 decode takes the wide split kernel (two splits per workgroup) up to this many
// workgroups (measured at 32 query heads, 8 KV heads: B = 1 at 8192 keys 35.6 -> 29.9 us, B = 8
// 125.9 -> 117.5 us; at 4096 workgroups the generic kernel streams faster, and rows padded from 160
// or 192 are faster on the generic kernel at every size tried).
constexpr int64_t SPLIT16W_MAX_WG = 1024;

SdpaPath sdpa_path(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, int dt) {
    if (dt == DT_F32 || S <= 0) return SDPA_SPLIT;
    const bool prefill_grid = D > 128 || prefill_workgroups(B, Hq, Hkv, Lq) > PREFILL_MIN_WG;
    if (Lq >= PREFILL_MIN_LQ && prefill_grid) return SDPA_PREFILL16;
    if (D > 128 && Lq >= WIDE_PREFILL_MIN_LQ && B * Lq >= WIDE_PREFILL_MIN_ROWS) return SDPA_PREFILL16;
    if (D > 128) {
        const int64_t nsg = ((S + KV_SPLIT - 1) / KV_SPLIT + 1) / 2;
        const int64_t tiles = (Hq / Hkv * Lq + 15) / 16;
        const bool wide = D == 256 && B * Hkv <= SPLIT16W_MAX_WG && tiles <= SPLIT16W_MAX_WG &&
                          nsg <= SPLIT16W_MAX_WG && nsg * tiles * B * Hkv <= SPLIT16W_MAX_WG;
        return wide ? SDPA_SPLIT16W : SDPA_SPLIT;
    }
    const int64_t nsplit = (S + KV_SPLIT - 1) / KV_SPLIT;
    if (quad_tiles(B, Hkv, nsplit, (Hq / Hkv * Lq + 15) / 16) > 0) return SDPA_QUAD16;
    if (Hq / Hkv * Lq >= PREFILL_MIN_ROWS && prefill_grid) return SDPA_PREFILL16;
    if (nsplit <= FUSED_MAXW) return SDPA_FUSED16;
    return SDPA_SPLIT;
}

// Bytes of split partials for Lq query rows: the (m, l) pairs padded to 256 bytes, then the O rows.
static int64_t partial_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t S, int64_t D) {
    const int64_t rows = B * Hq * Lq;
    const int64_t nsplit = (S + KV_SPLIT - 1) / KV_SPLIT;
    const int64_t ml = (rows * nsplit * 2 * 4 + 255) / 256 * 256;
    return ml + rows * nsplit * D * 4;
}

int64_t sdpa_chunk_rows(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, int dt) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Lq <= 0 || S <= 0 || D <= 0) return Lq;
    const SdpaPath path = sdpa_path(B, Hq, Hkv, Lq, S, D, dt);
    if (path != SDPA_SPLIT && path != SDPA_QUAD16 && path != SDPA_SPLIT16W) return Lq;
    if (partial_bytes(B, Hq, Lq, S, D) <= SDPA_WS_CAP) return Lq;
    const int64_t per_row = partial_bytes(B, Hq, 1, S, D) + 256;
    return std::max<int64_t>(1, std::min<int64_t>(Lq, SDPA_WS_CAP / per_row));
}

size_t sdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, int dt) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Lq <= 0 || S <= 0 || D <= 0) return 0;
    const int64_t Lc = sdpa_chunk_rows(B, Hq, Hkv, Lq, S, D, dt);
    if (Lc < Lq) return (size_t)partial_bytes(B, Hq, Lc, S, D);  // bounds every chunk's path
    const SdpaPath path = sdpa_path(B, Hq, Hkv, Lq, S, D, dt);
    if (path != SDPA_SPLIT && path != SDPA_QUAD16 && path != SDPA_SPLIT16W) return 0;
    if (path == SDPA_QUAD16 && S <= KV_SPLIT) return 0;          // one split: the quad kernel finishes the rows
    return (size_t)partial_bytes(B, Hq, Lq, S, D);
}

void sdpa_bind_workspace(SdpaParams &p, void *ws) {
    const int64_t rows = (int64_t)p.B * p.Hq * p.Lq;
    const int64_t ml = (rows * p.nsplit * 2 * 4 + 255) / 256 * 256;
    p.ws_ml = static_cast<float *>(ws);
    p.ws_o = reinterpret_cast<float *>(static_cast<char *>(ws) + ml);
}

template <int dt, int D>
static hipError_t launch_typed(const SdpaParams &p, hipStream_t st) {
    const int R = p.G * p.Lq;
    const SdpaPath path = sdpa_path(p.B, p.Hq, p.Hkv, p.Lq, p.S, D, dt);
    if constexpr (dt != DT_F32 && D <= 128) {
        if (path == SDPA_PREFILL16) {
            constexpr int W = 4;                         // row tiles (one per wavefront) sharing each K / V block
            const int64_t nwg = (int64_t)(((R + 15) / 16 + W - 1) / W) * p.B * p.Hkv;
            if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((sdpa_prefill16p<dt, W, D>), dim3((unsigned)nwg), dim3(64 * W), 0, st, p);
            return hipGetLastError();
        }
        if (path == SDPA_FUSED16) {
            const int64_t nwg = (int64_t)((R + 15) / 16) * p.B * p.Hkv;
            if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((sdpa_fused16<dt>), dim3((unsigned)nwg), dim3(64 * p.nsplit),
                               (unsigned)(FUSED_LDS_PER_WAVE * p.nsplit), st, p);
            return hipGetLastError();
        }
    }
    if constexpr (dt != DT_F32 && D > 128) {
        if (path == SDPA_PREFILL16) {
            constexpr int W = 4;                         // row tiles per workgroup sharing each K / V block
            const int64_t nwg = (int64_t)(((R + 15) / 16 + W - 1) / W) * p.B * p.Hkv;
            if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((sdpa_prefill16w<dt, W, 2, 16>), dim3((unsigned)nwg), dim3(64 * W), 0, st, p);
            return hipGetLastError();
        }
    }
    if (p.nsplit > 0 && path == SDPA_QUAD16) {
        if constexpr (dt != DT_F32 && D <= 128) {
            const int64_t ntile = (R + 15) / 16;
            const int64_t T = quad_tiles(p.B, p.Hkv, p.nsplit, ntile);
            const int64_t nwg = (int64_t)p.nsplit * ((ntile + T - 1) / T) * p.B * p.Hkv;
            if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
            if (T == 2) hipLaunchKernelGGL((sdpa_quad16<dt, 2>), dim3((unsigned)nwg), dim3(64 * 4 * 2), 0, st, p);
            else hipLaunchKernelGGL((sdpa_quad16<dt, 1>), dim3((unsigned)nwg), dim3(64 * 4), 0, st, p);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess || p.nsplit == 1) return e;      // one split: no combine
        }
    } else if (p.nsplit > 0) {
        if constexpr (dt != DT_F32 && (D == 128 || D == 64)) {   // (D = 32, 96: the generic kernel)
            constexpr int W = 2;                         // splits per workgroup (measured best for long caches)
            const int64_t nwg = (int64_t)((p.nsplit + W - 1) / W) * ((R + 15) / 16) * p.B * p.Hkv;
            if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((sdpa_split16<dt, W, D / 32>), dim3((unsigned)nwg), dim3(64 * W), 0, st, p);
        } else if (dt != DT_F32 && D == 256 && path == SDPA_SPLIT16W) {
            if constexpr (dt != DT_F32 && D == 256) {
                constexpr int W = 2;
                const int64_t nwg = (int64_t)((p.nsplit + W - 1) / W) * ((R + 15) / 16) * p.B * p.Hkv;
                if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
                hipLaunchKernelGGL((sdpa_split16<dt, W, 8>), dim3((unsigned)nwg), dim3(64 * W), 0, st, p);
            }
        } else {
            const int64_t nwg = (int64_t)p.nsplit * ((R + 15) / 16) * p.B * p.Hkv;
            if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((sdpa_split<dt, D>), dim3((unsigned)nwg), dim3(64), 0, st, p);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 g2((unsigned)((int64_t)p.B * p.Hq * p.Lq));
    // the same fold with fewer loads in flight for short caches (measured 0.5-1.3 us less at four splits),
    // and through LDS for long ones, 32 partials per chunk: more workgroups per CU than with 128-partial
    // staging, and the next chunk's loads overlap the fold (B = 32, 8192 keys: 198.6 -> 193.5 us; 32768
    // keys: 742.6 -> 734.8)
    if (p.nsplit <= 4) hipLaunchKernelGGL((sdpa_combine<dt, D, 4>), g2, dim3(D), 0, st, p);
    else if (p.nsplit <= 8) hipLaunchKernelGGL((sdpa_combine<dt, D, 8>), g2, dim3(D), 0, st, p);
    else if (p.nsplit <= 16) hipLaunchKernelGGL((sdpa_combine<dt, D>), g2, dim3(D), 0, st, p);
    else hipLaunchKernelGGL((sdpa_combine_lds<dt, D, 32>), g2, dim3(256), 0, st, p);
    return hipGetLastError();
}

// The comparator's split length, following the page's account of the batch-variant library (README,
// "Why MLX is not invariant", attention): one pass over the whole cache up to 4096 keys, two passes
// above; the second pass's split count is 64 when G times the query count is at least 4, else 32.
int64_t sdpa_variant_split_len(int64_t G, int64_t Lq, int64_t S) {
    const int64_t s = S > 0 ? S : 1;
    if (s <= 4096) return (s + KV_BLOCK - 1) / KV_BLOCK * KV_BLOCK;
    const int64_t nsplit = G * Lq >= 4 ? 64 : 32;
    const int64_t len = (s + nsplit - 1) / nsplit;
    return (len + KV_BLOCK - 1) / KV_BLOCK * KV_BLOCK;
}

size_t sdpa_variant_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Lq <= 0 || S <= 0 || D <= 0) return 0;
    const int64_t len = sdpa_variant_split_len(Hq / Hkv, Lq, S);
    const int64_t rows = B * Hq * Lq;
    const int64_t nsplit = (S + len - 1) / len;
    const int64_t ml = (rows * nsplit * 2 * 4 + 255) / 256 * 256;
    return (size_t)(ml + rows * nsplit * D * 4);
}

template <int dt, int D>
static hipError_t launch_variant_typed(const SdpaParams &p, hipStream_t st) {
    const int R = p.G * p.Lq;
    const int64_t nwg = (int64_t)p.nsplit * ((R + 15) / 16) * p.B * p.Hkv;
    if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((sdpa_split<dt, D>), dim3((unsigned)nwg), dim3(64), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sdpa_combine<dt, D>), dim3((unsigned)((int64_t)p.B * p.Hq * p.Lq)), dim3(D), 0, st, p);
    return hipGetLastError();
}

template <int dt>
static hipError_t launch_variant_d(const SdpaParams &p, int D, hipStream_t st) {
    switch (D) {
        case 32: return launch_variant_typed<dt, 32>(p, st);
        case 64: return launch_variant_typed<dt, 64>(p, st);
        case 96: return launch_variant_typed<dt, 96>(p, st);
        case 128: return launch_variant_typed<dt, 128>(p, st);
        case 160: return launch_variant_typed<dt, 160>(p, st);
        case 192: return launch_variant_typed<dt, 192>(p, st);
        case 224: return launch_variant_typed<dt, 224>(p, st);
        case 256: return launch_variant_typed<dt, 256>(p, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sdpa_variant(const SdpaParams &p, int dt, int D, hipStream_t st) {
    if (p.nsplit <= 0) return hipSuccess;
    if (dt == DT_BF16) return launch_variant_d<DT_BF16>(p, D, st);
    if (dt == DT_F16) return launch_variant_d<DT_F16>(p, D, st);
    if (dt == DT_F32) return launch_variant_d<DT_F32>(p, D, st);
    return hipErrorInvalidValue;
}

const char *sdpa_kernel_name(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, int dt) {
    switch (sdpa_path(B, Hq, Hkv, Lq, S, D, dt)) {
        case SDPA_FUSED16: return "sdpa_fused16";
        case SDPA_PREFILL16: return D > 128 ? "sdpa_prefill16w" : "sdpa_prefill16";
        case SDPA_QUAD16: return S <= KV_SPLIT ? "sdpa_quad16" : "sdpa_quad16+combine";
        case SDPA_SPLIT16W: return "sdpa_split16w+combine";
        default: return dt != DT_F32 && (D == 128 || D == 64) ? "sdpa_split16+combine" : "sdpa_split+combine";
    }
}

template <int dt>
static hipError_t launch_d(const SdpaParams &p, int D, hipStream_t st) {
    switch (D) {
        case 32: return launch_typed<dt, 32>(p, st);
        case 64: return launch_typed<dt, 64>(p, st);
        case 96: return launch_typed<dt, 96>(p, st);
        case 128: return launch_typed<dt, 128>(p, st);
        case 160: return launch_typed<dt, 160>(p, st);
        case 192: return launch_typed<dt, 192>(p, st);
        case 224: return launch_typed<dt, 224>(p, st);
        case 256: return launch_typed<dt, 256>(p, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sdpa(const SdpaParams &p, int dt, int D, hipStream_t st) {
    if (dt == DT_BF16) return launch_d<DT_BF16>(p, D, st);
    if (dt == DT_F16) return launch_d<DT_F16>(p, D, st);
    if (dt == DT_F32) return launch_d<DT_F32>(p, D, st);
    return hipErrorInvalidValue;
}

}  // namespace bi
