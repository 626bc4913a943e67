/*
 * CPU oracle for the batch-invariant matrix-multiply and attention kernels.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark have an independent, obviously correct
 * answer to compare the GPU kernels against.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * Everything is evaluated in IEEE float64 straight from the mathematical
 * definition, with no blocking, fusion or reordering:
 *   - every bf16 / fp16 / fp32 input embeds exactly in a double, and the
 *     product of two such values is exact in a double (at most 24+24
 *     significant bits), so the only rounding in a GEMM element is the
 *     sequential double-precision sum over k;
 *   - attention uses libm exp() on the max-shifted scores.
 * Results are returned unrounded (float64); rounding to an output dtype is
 * the caller's business.
 *
 * Sources (mlx-batch-invariant README):
 *   - section "Use": linear(x, w, bias) with w in the (N, K) nn.Linear
 *     layout, matmul(a, b) with b in (K, N), addmm(c, a, b, alpha, beta),
 *     scaled_dot_product_attention(q, k, v, mask="causal");
 *   - section "Why MLX is not invariant", attention bullets: the query
 *     length is q.shape[2] and the grouped-query factor is H / Hkv;
 *   - section "Accuracy": the float64 reference that accuracy is judged
 *     against;
 *   - section "Quantized models": 2, 4 and 8-bit group-wise affine weights.
 * Readings where the page is silent (all documented with the library):
 *   causal alignment is bottom-right (query i sits at key position
 *   S - Lq + i); query head h reads KV head floor(h * Hkv / Hq); a boolean
 *   mask entry of 1 means "attend"; a row that sees no key returns 0;
 *   addmm with beta == 0 does not read C (BLAS convention).
 *
 * Parity status: every function here is pinned by CPU tests against exact
 * rational arithmetic, correctly rounded sums, closed forms and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

int oracle_threads(void) { return omp_get_max_threads(); }

void oracle_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}

/*
 * out[m, n] = alpha * sum_{k=0}^{K-1} A[m, k] * B[k, n] + beta * C[m, n]
 *
 * A      : element (m, k) at A[m * lda + k]
 * B      : b_is_nk == 0 -> element (k, n) at B[k * ldb + n]   (matmul layout)
 *          b_is_nk == 1 -> element (k, n) at B[n * ldb + k]   (nn.Linear W)
 * C      : may be NULL (treated as 0); ldc == 0 broadcasts row 0 to all m.
 *          Not read at all when beta == 0.
 * out    : element (m, n) at out[m * ldo + n]
 *
 * The sum over k is a plain ascending loop in double.  Several output
 * columns are carried side by side only to give the CPU independent
 * chains to overlap; no element's own summation order is touched.
 */
void oracle_gemm_f64(const double *A, int64_t lda,
                     const double *B, int64_t ldb, int b_is_nk,
                     const double *C, int64_t ldc,
                     double alpha, double beta,
                     double *out, int64_t ldo,
                     int64_t M, int64_t N, int64_t K)
{
    const int64_t NB = 4;
    const int64_t nblk = (N + NB - 1) / NB;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t jb = 0; jb < nblk; ++jb) {
            const int64_t n0 = jb * NB;
            const int64_t nn = (N - n0 < NB) ? (N - n0) : NB;
            double acc[4] = {0.0, 0.0, 0.0, 0.0};
            const double *arow = A + m * lda;
            for (int64_t k = 0; k < K; ++k) {
                const double a = arow[k];
                for (int64_t j = 0; j < nn; ++j) {
                    const int64_t n = n0 + j;
                    const double b = b_is_nk ? B[n * ldb + k] : B[k * ldb + n];
                    acc[j] = acc[j] + a * b;
                }
            }
            for (int64_t j = 0; j < nn; ++j) {
                const int64_t n = n0 + j;
                double r = alpha * acc[j];
                if (beta != 0.0 && C != NULL) {
                    const double c = C[(ldc == 0 ? 0 : m * ldc) + n];
                    r = r + beta * c;
                }
                out[m * ldo + n] = r;
            }
        }
    }
}

/*
 * Scaled dot-product attention with grouped-query heads, an optional
 * bottom-right causal mask, an optional boolean mask, an optional additive
 * mask and optional attention sinks (README, section "How the kernels work",
 * attention paragraph: the three mask forms; section "Limitations": sinks).
 *
 * q : (B, Hq,  Lq, D), element strides qs[0..3]
 * k : (B, Hkv, S,  D), element strides ks[0..3]
 * v : (B, Hkv, S,  D), element strides vs[0..3]
 * o : (B, Hq,  Lq, D), contiguous, written in float64
 * mask : NULL, or uint8 with element strides ms[0..3] over (B, Hq, Lq, S);
 *        a stride of 0 broadcasts that dimension; nonzero = may attend.
 * amask: NULL, or float64 with element strides as[0..3] over (B, Hq, Lq, S),
 *        added to the scaled scores; -inf removes the key.
 * sinks: NULL, or Hq float64 logits, one per query head: an extra softmax
 *        term on the scale of the scaled scores that carries no value.
 *
 * For query row (b, h, i):
 *   position   p   = S - Lq + i
 *   KV head    g   = floor(h * Hkv / Hq)
 *   added      a_j = amask[b,h,i,j] (0 without one)
 *   visible    j   : (causal == 0 or j <= p) and (mask == NULL or mask[b,h,i,j])
 *                    and a_j != -inf
 *   score      s_j = scale * sum_d q[b,h,i,d] * k[b,g,j,d] + a_j
 *   max        m   = max(max_visible s_j, sinks[h])
 *   weight     w_j = exp(s_j - m)
 *   output     o[b,h,i,:] = sum_visible w_j v[b,g,j,:]
 *                           / (sum_visible w_j + exp(sinks[h] - m))
 *   (the sink terms absent without sinks); a row with no visible key is 0.
 */
void oracle_sdpa_f64(const double *q, const int64_t *qs,
                     const double *k, const int64_t *ks,
                     const double *v, const int64_t *vs,
                     double *o,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                     int64_t S, int64_t D, double scale, int causal,
                     const uint8_t *mask, const int64_t *ms,
                     const double *amask, const int64_t *as, const double *sinks)
{
    const int64_t rows = B * Hq * Lq;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        unsigned char *vis = (unsigned char *)malloc((size_t)(S > 0 ? S : 1));
        double *num = (double *)malloc(sizeof(double) * (size_t)D);
        #pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t b = r / (Hq * Lq);
            const int64_t h = (r / Lq) % Hq;
            const int64_t i = r % Lq;
            const int64_t g = (h * Hkv) / Hq;
            const int64_t p = S - Lq + i;
            const double *qrow = q + b * qs[0] + h * qs[1] + i * qs[2];
            double *orow = o + ((b * Hq + h) * Lq + i) * D;

            int any = 0;
            double m = -INFINITY;
            for (int64_t j = 0; j < S; ++j) {
                int ok = 1;
                if (causal && j > p) ok = 0;
                if (ok && mask != NULL) {
                    ok = mask[b * ms[0] + h * ms[1] + i * ms[2] + j * ms[3]] != 0;
                }
                double add = 0.0;
                if (ok && amask != NULL) {
                    add = amask[b * as[0] + h * as[1] + i * as[2] + j * as[3]];
                    if (add == -INFINITY) ok = 0;
                }
                vis[j] = (unsigned char)ok;
                if (!ok) continue;
                const double *krow = k + b * ks[0] + g * ks[1] + j * ks[2];
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot = dot + qrow[d * qs[3]] * krow[d * ks[3]];
                s[j] = scale * dot + add;
                if (!any || s[j] > m) m = s[j];
                any = 1;
            }
            if (!any) {
                for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
                continue;
            }
            double den = 0.0;
            if (sinks != NULL) {
                const double sk = sinks[h];
                if (sk > m) m = sk;
                den = den + exp(sk - m);
            }
            for (int64_t d = 0; d < D; ++d) num[d] = 0.0;
            for (int64_t j = 0; j < S; ++j) {
                if (!vis[j]) continue;
                const double w = exp(s[j] - m);
                den = den + w;
                const double *vrow = v + b * vs[0] + g * vs[1] + j * vs[2];
                for (int64_t d = 0; d < D; ++d) num[d] = num[d] + w * vrow[d * vs[3]];
            }
            for (int64_t d = 0; d < D; ++d) orow[d] = num[d] / den;
        }
        free(s);
        free(vis);
        free(num);
    }
}

/*
 * Row reduction over the last dimension (README, section "Why MLX is not
 * invariant": sum and mean are among the ops a batch-invariant stack relies
 * on):  out[m] = sum_{n=0}^{N-1} x[m * ldx + n], or that sum divided by N
 * when mean != 0.  A plain ascending loop in double; N == 0 gives 0 (sum)
 * or NaN (mean, 0 / 0).
 */
void oracle_rowsum_f64(const double *x, int64_t ldx, int64_t M, int64_t N, int mean, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const double *row = x + m * ldx;
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) s = s + row[n];
        out[m] = mean ? s / (double)N : s;
    }
}

/*
 * Group-wise affine dequantisation (README, section "Quantized models": 2, 4
 * and 8-bit affine weights, one scale and one bias per group of k values).
 * The packing follows the layout the page's quantized checkpoints use: along
 * k, consecutive values share a 32-bit word, 32 / bits of them per word,
 * value j of a word in bits [j * bits, (j + 1) * bits).
 *
 *   q[n, k] = (wq[n * ldwq + k / per] >> ((k mod per) * bits)) & (2^bits - 1),
 *             per = 32 / bits
 *   w[n, k] = scales[n * ldsb + k / gs] * q[n, k] + biases[n * ldsb + k / gs]
 *
 * evaluated exactly in double (the scale and bias are bf16 / fp16 values and
 * q < 256, so the product and the sum are exact); out[n * K + k] = w[n, k].
 */
void oracle_dequant_f64(const uint32_t *wq, int64_t ldwq, const double *scales, const double *biases, int64_t ldsb,
                        int bits, int64_t gs, int64_t N, int64_t K, double *out) {
    const int64_t per = 32 / bits;
    const uint32_t fieldmask = (bits == 32) ? 0xffffffffu : ((1u << bits) - 1u);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; k++) {
            const uint32_t word = wq[n * ldwq + k / per];
            const uint32_t q = (word >> ((k % per) * bits)) & fieldmask;
            const int64_t grp = k / gs;
            out[n * K + k] = scales[n * ldsb + grp] * (double)q + biases[n * ldsb + grp];
        }
    }
}
