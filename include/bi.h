/*
 * bi.h -- batch-invariant matrix multiply and attention for AMD CDNA4 (gfx950).
 *
 * What "batch-invariant" means here (mlx-batch-invariant README, section
 * 'What "batch-invariant" means here'): the bits of every output row are the
 * same whatever the number of other rows in the call, whatever those rows
 * hold, however many query tokens were submitted together (decode or chunked
 * prefill), however long the KV cache is, and whether the call was made
 * eagerly or replayed from a captured HIP graph.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps a pointer after returning, never
 *    synchronises, and enqueues all its work on `stream` (a hipStream_t;
 *    NULL means the legacy default stream).  Calls are therefore safe to
 *    record into a HIP graph.
 *  - Element strides and leading dimensions are given in ELEMENTS.  The
 *    innermost dimension of every tensor must be contiguous (stride 1).
 *  - Every argument is validated on the host before anything is enqueued.
 *    A call that returns an error has written nothing.  No C++ exception
 *    crosses this interface.  bi_last_error() describes the last failure on
 *    the calling thread.
 *  - Nothing the library does depends on an environment variable or a
 *    global switch: the arithmetic of a call is a function of its
 *    arguments' values and of the compile-time tile and chunk constants,
 *    whose identity is reported by bi_abi_version().
 *  - Unsupported inputs are refused with BI_ERR_UNSUPPORTED; nothing falls
 *    back to a different (batch-variant) kernel.  (README, section "Use":
 *    anything that cannot be made invariant raises instead of silently
 *    falling back.)
 *
 * Where this interface differs from the plainest form of the four calls
 * -------------------------------------------------------------------
 *  - The GEMM calls take no workspace and have no workspace query: each
 *    output element's whole K reduction is one chain inside one kernel (no
 *    split-K and no fixed K-segment fold), so there is nothing to stage.
 *    Only the batch-variant comparator (bi_variant_linear) and the
 *    quantized linear above 64 rows with K not a multiple of 128 take one.
 *  - bi_sdpa_workspace_bytes takes Hkv and the dtype besides (B, Hq, Lq, S,
 *    D): which kernel runs, and whether the split partials go through a
 *    workspace at all, follows the grid size (B x Hkv x row tiles) and the
 *    dtype (fp32 always takes the split path).
 *  - bi_matmul / bi_addmm describe B by a row and a column stride instead of
 *    one leading dimension, so the transposed view of an (N, K) weight is
 *    passed without a copy and runs the bi_linear kernels.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BI_OK = 0,
    BI_ERR_INVALID = 1,     /* malformed arguments: bad shapes, null pointers, Hq % Hkv != 0 ... */
    BI_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported set (dtype pair, alignment, D) */
    BI_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than the *_workspace_bytes query */
    BI_ERR_DEVICE = 4       /* the HIP runtime reported an error (launch failure, no device) */
} bi_status;

typedef enum {
    BI_F32 = 0,   /* IEEE binary32 */
    BI_F16 = 1,   /* IEEE binary16 */
    BI_BF16 = 2   /* bfloat16 (upper half of a binary32) */
} bi_dtype;

/*
 * Matrix multiply family (README, section "Use": linear, matmul, addmm;
 * section "How the kernels work", GEMM paragraph).
 *
 * Arithmetic contract, identical for all three calls and every M:
 *   acc[m,n] = fp32 sum over k of A[m,k] * B[k,n], formed by one chain of
 *              gfx950 MFMA instructions walking k upwards from 0 in fixed
 *              steps: one v_mfma_f32_16x16x32_{bf16,f16} per 32 k for 16-bit
 *              inputs, four v_mfma_f32_16x16x4_f32 per 16 k for fp32 inputs;
 *              the accumulator starts at +0 and k past K contributes exact
 *              zeros.  The chain depends on K only;
 *              nothing splits K, and no tile choice changes the chain.
 *   t        = fp32(beta) * fp32(C[m,n])          (0 when there is no C / beta == 0)
 *   y[m,n]   = round_to_out_dtype( fmaf(alpha, acc, t) )
 *              i.e. the bias / C term is added to the fp32 accumulator and
 *              the sum is rounded ONCE to the output dtype (round to nearest
 *              even; NaN stays NaN).
 *
 * Supported dtype pairs (in_dt -> out_dt):
 *   F32 -> F32, BF16 -> BF16, F16 -> F16, BF16 -> F32, F16 -> F32.
 * The bias / C tensor, when present, has the OUTPUT dtype.
 * Shapes: M, N, K >= 0 and < 2^31.  M == 0 or N == 0 enqueues nothing.
 * Alignment (else BI_ERR_UNSUPPORTED): every base pointer 16-byte aligned;
 *   K a multiple of 8 (16-bit inputs) or 4 (fp32 inputs); lda, ldw and the
 *   non-unit stride of b multiples of 8 (16-bit) or 4 (fp32) elements; for a
 *   row-major (K, N) operand of bi_matmul / bi_addmm also N a multiple of 8
 *   (16-bit) or 4 (fp32).
 *
 * The (K, N) operand b of bi_matmul / bi_addmm is described by two element
 * strides, b_stride_k (between consecutive k) and b_stride_n (between
 * consecutive n); one of them must be 1:
 *   b_stride_n == 1 : row-major (K, N), row k at b + k * b_stride_k;
 *   b_stride_k == 1 : column-major (K, N), i.e. the (N, K) nn.Linear layout
 *                     (a transposed view such as w.t()), column n at
 *                     b + n * b_stride_n.
 * Both layouts give bit-identical results (same per-element chain).
 */

/* y (M,N) = x (M,K) . w^T + bias,  w in the (N,K) nn.Linear layout.
 * x: row m at x + m*ldx (ldx >= K).  w: row n at w + n*ldw (ldw >= K).
 * bias: NULL or N contiguous elements of out_dt.  y: row m at y + m*ldy (ldy >= N). */
bi_status bi_linear(const void *x, int64_t ldx,
                    const void *w, int64_t ldw,
                    const void *bias,
                    void *y, int64_t ldy,
                    int64_t M, int64_t N, int64_t K,
                    bi_dtype in_dt, bi_dtype out_dt,
                    void *stream);

/* c (M,N) = a (M,K) . b (K,N), b described by (b_stride_k, b_stride_n) as above. */
bi_status bi_matmul(const void *a, int64_t lda,
                    const void *b, int64_t b_stride_k, int64_t b_stride_n,
                    void *c, int64_t ldc,
                    int64_t M, int64_t N, int64_t K,
                    bi_dtype in_dt, bi_dtype out_dt,
                    void *stream);

/* Batched bi_matmul: for z in [0, batch), c_z = a_z . b_z with a_z = a + z*stride_a,
 * b_z = b + z*stride_b, c_z = c + z*stride_c (strides in elements, >= 0; a
 * stride of 0 reuses one operand for every element).  Each element computes
 * exactly bi_matmul's chain, so c_z has the bits bi_matmul(a_z, b_z) gives,
 * whatever the batch and the element's position (README, section "Why MLX
 * is not invariant", matmul paragraph: an output element's reduction must
 * not depend on the rest of the call); one launch per 65535 elements
 * instead of one per element.  batch == 0 does nothing.
 * Errors: as bi_matmul, plus BI_ERR_INVALID for a negative batch or stride
 * or a stride_c that lets two elements' outputs overlap, BI_ERR_UNSUPPORTED
 * for a batch of 2^31 or more and for 16-bit stride_a / stride_b not a
 * multiple of 8 elements (fp32: 4). */
bi_status bi_matmul_batched(const void *a, int64_t lda, int64_t stride_a,
                            const void *b, int64_t b_stride_k, int64_t b_stride_n, int64_t stride_b,
                            void *c, int64_t ldc, int64_t stride_c,
                            int64_t batch, int64_t M, int64_t N, int64_t K,
                            bi_dtype in_dt, bi_dtype out_dt,
                            void *stream);

/* out (M,N) = alpha * (a (M,K) . b (K,N)) + beta * cin, b as for bi_matmul.
 * cin: out_dt elements, row m at cin + m*ldcin; ldcin == 0 broadcasts one
 * row of N elements to every m (the bias form).  When beta == 0, cin is not
 * read and may be NULL (BLAS convention).  out may alias cin only if
 * ldo == ldcin and the pointers are equal (each element is read before its
 * own write and by no other thread). */
bi_status bi_addmm(const void *cin, int64_t ldcin,
                   const void *a, int64_t lda,
                   const void *b, int64_t b_stride_k, int64_t b_stride_n,
                   void *out, int64_t ldo,
                   int64_t M, int64_t N, int64_t K,
                   float alpha, float beta,
                   bi_dtype in_dt, bi_dtype out_dt,
                   void *stream);

/*
 * Scaled dot-product attention with grouped-query heads (README, section
 * "Use": scaled_dot_product_attention(q, k, v, mask="causal"); section "How
 * the kernels work", attention paragraph; section "Why MLX is not
 * invariant", attention bullets, for what must not change the bits).
 *
 * q (B, Hq, Lq, D), k and v (B, Hkv, S, D), o (B, Hq, Lq, D); all share
 * dtype dt (F32, F16 or BF16) and have element strides *_str[0..3] with
 * *_str[3] == 1.  Query head h reads KV head floor(h * Hkv / Hq).
 * Query i sits at key position S - Lq + i (bottom-right alignment); with
 * causal != 0 it sees keys j <= S - Lq + i.  mask: NULL, or uint8 over
 * (B, Hq, Lq, S) with element strides mask_str[0..3] (0 broadcasts that
 * dimension, any value for the key dimension), nonzero = may attend.
 * scale multiplies q.k; pass 1/sqrt(D) for the usual softmax scaling.
 * A query that sees no key produces a row of zeros.
 *
 * Arithmetic contract (fixed, independent of B, Lq, S and of the other rows):
 *   keys are cut at absolute positions into splits of 256, each split into
 *   blocks of 64.  Within a split, blocks are folded in ascending order with
 *   an online softmax in fp32 (exp2 with the scale pre-multiplied by
 *   log2(e)); a block with no visible key leaves the running state
 *   untouched.  Split partials (m, l, O) are then folded left to right in
 *   ascending split order, O is divided by l, -0 becomes +0, and the result
 *   is rounded once to dt.  For 16-bit dt the softmax weights are rounded
 *   to dt before the P.V product; fp32 keeps them in fp32.
 *
 * Supported: D a multiple of 32 up to 256 (README, section "Limitations":
 * head dimensions must be multiples of 32); Hq % Hkv == 0; Lq <= S when causal; every
 * base pointer 16-byte aligned and every stride except the last a multiple
 * of 8 (16-bit) or 4 (fp32) elements.
 * Workspace: ws must hold bi_sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D, dt)
 * bytes, 256-byte aligned, device memory owned by the caller; its contents on
 * entry do not matter and on return are unspecified.  Two calls that run at
 * the same time must not share a workspace.  The query stays at or below
 * 256 MiB (or the partials of one query row per head, if more): a call whose
 * partials would need more runs in chunks of query rows, one after the other
 * on `stream`, each with the keys up to its last row when causal; no row's
 * arithmetic changes.  The query returns 0 (ws may then
 * be NULL) for the shapes served without a workspace: 16-bit dt with either
 * Lq >= 384 (prefill: splits folded in registers; for D <= 128 only on a
 * prefill grid of more than 64 workgroups, for D > 128 also Lq >= 64 with
 * B Lq >= 192), or D <= 128 and S <= 256
 * on the quad kernel (one split, finished in the kernel), or D <= 128, more
 * than 256 quad workgroups and either (Hq / Hkv) Lq >= 64 on a prefill grid
 * of more than 64 workgroups (prefill) or S <= 1024 (one launch, splits
 * folded in LDS); see bi_sdpa_kernel_name.
 * Every path computes the same bits.
 */
bi_status bi_sdpa(const void *q, const int64_t q_str[4],
                  const void *k, const int64_t k_str[4],
                  const void *v, const int64_t v_str[4],
                  void *o, const int64_t o_str[4],
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D,
                  float scale, int causal,
                  const uint8_t *mask, const int64_t mask_str[4],
                  bi_dtype dt,
                  void *ws, size_t ws_bytes,
                  void *stream);

/* Bytes of workspace bi_sdpa needs for these sizes and dtype (0 when there is
 * nothing to do, when the path taken needs none, for Hkv <= 0 or Hq not a
 * multiple of Hkv, or for an unknown dtype). */
size_t bi_sdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, bi_dtype dt);

/*
 * bi_sdpa with every mask form and attention sinks (README, section "How the
 * kernels work", attention paragraph: the mask forms of the single-pass
 * kernel; section "Limitations": attention sinks).  Arguments as bi_sdpa,
 * plus:
 *   mask_kind: BI_MASK_NONE (mask ignored), BI_MASK_BOOL (uint8, nonzero =
 *     may attend) or BI_MASK_ADD (elements of dt, added to the scaled scores;
 *     -inf removes the key, a finite value weights it by exp(value));
 *     element strides mask_str[0..3] over (B, Hq, Lq, S), 0 broadcasts.
 *   sinks: NULL, or Hq fp32 logits in device memory, one per query head: an
 *     extra softmax term on the scale of the scaled scores that carries no
 *     value, so a query's weights sum to less than one.
 * Arithmetic, in the exp2 domain of the bi_sdpa contract: an additive value
 * a turns a key's score into fmaf(a, log2e, S * c) (c = scale * log2e,
 * log2e rounded to fp32); a sink enters every fold of split partials as its
 * first partial, (m, l, O) = (sink * log2e, 1, 0), before split 0.  Keys
 * masked with -inf, like keys masked by a boolean mask, are identity steps,
 * so appending them never changes an earlier result.  A query that sees no
 * key produces zeros, with or without a sink.  Workspace as bi_sdpa.
 */
typedef enum { BI_MASK_NONE = 0, BI_MASK_BOOL = 1, BI_MASK_ADD = 2 } bi_mask_kind;
bi_status bi_sdpa_ex(const void *q, const int64_t q_str[4],
                     const void *k, const int64_t k_str[4],
                     const void *v, const int64_t v_str[4],
                     void *o, const int64_t o_str[4],
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D,
                     float scale, int causal,
                     int mask_kind, const void *mask, const int64_t mask_str[4],
                     const float *sinks,
                     bi_dtype dt,
                     void *ws, size_t ws_bytes,
                     void *stream);

/*
 * bi_sdpa_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments, results and bits as bi_sdpa_ex, without ws / ws_bytes: the
 * split partials (the bytes bi_sdpa_workspace_bytes reports) go to a
 * scratch array of bi_sdpa_scratch_limit() bytes (64 MiB) that the library
 * holds on each GPU it runs on until the process ends; this call allocates
 * and frees nothing.  Sizes needing more return BI_ERR_UNSUPPORTED before
 * anything is enqueued.  Every call on a GPU uses that GPU's one array (the
 * device current on the calling thread), so calls that overlap on one GPU
 * (other streams, other threads) race and must not be made; the array's
 * contents on entry do not matter and are left as the last call wrote them.
 * The first call that needs the array on a device looks up its address
 * there (hipGetSymbolAddress), so make that first call outside graph
 * capture.
 */
bi_status bi_sdpa_ex_noalloc(const void *q, const int64_t q_str[4],
                             const void *k, const int64_t k_str[4],
                             const void *v, const int64_t v_str[4],
                             void *o, const int64_t o_str[4],
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D,
                             float scale, int causal,
                             int mask_kind, const void *mask, const int64_t mask_str[4],
                             const float *sinks,
                             bi_dtype dt,
                             void *stream);
/* Bytes of the per-GPU scratch array bi_sdpa_ex_noalloc uses (its size limit). */
size_t bi_sdpa_scratch_limit(void);

/*
 * Batch-VARIANT comparator, for measurement only.  It runs the same
 * kernels bi_linear picks for this M (the strip, pipelined and ring tile
 * kernels, or the generic ones where bi_linear uses those), with the same
 * fragment loads, MFMA instruction and epilogue, but cuts K into `splits`
 * contiguous ranges (a grid dimension) whose fp32 partial sums are added in
 * ascending order in a second pass -- the M-dependent split-K tuning that the
 * README (section "Why MLX is not invariant", matmul paragraph) identifies
 * as the source of batch variance.  Its results are NOT batch-invariant by
 * design.  splits must be in 1..16; K is cut into that many ranges of whole
 * LDS stages (128 k in the strip kernel, 64 or 128 k in the tile kernels) or
 * k-groups (generic kernels), as even as possible.  ws must hold bi_variant_workspace_bytes(M, N, splits)
 * bytes (256-byte aligned device memory); same dtype / alignment rules as
 * bi_linear.
 * bi_variant_splits(M) is the M-keyed policy: 8 for M <= 16, 4 for M <= 64,
 * 2 for M <= 128, 1 above.
 */
bi_status bi_variant_linear(const void *x, int64_t ldx,
                            const void *w, int64_t ldw,
                            const void *bias,
                            void *y, int64_t ldy,
                            int64_t M, int64_t N, int64_t K,
                            bi_dtype in_dt, bi_dtype out_dt,
                            int splits, void *ws, size_t ws_bytes,
                            void *stream);
size_t bi_variant_workspace_bytes(int64_t M, int64_t N, int splits);
int bi_variant_splits(int64_t M);

/*
 * Batch-VARIANT attention comparator, for measurement only (README, section
 * "Why MLX is not invariant", attention: the split-KV count follows the GQA
 * factor times the query count, and growing the cache past 4096 keys switches
 * from one pass to two).  Arguments as bi_sdpa.  The generic split kernel and
 * the combine run with a split length taken from the call's shape,
 * bi_variant_sdpa_split_len(G = Hq / Hkv, Lq, S): the whole cache (rounded up
 * to 64 keys) as one split up to S = 4096, above that ceil(S / n) rounded up
 * to 64 keys with n = 64 splits when G * Lq >= 4, else 32.  A token's bits
 * therefore move with the query count and the cache length, while every
 * result stays within the oracle tolerance.  ws must hold
 * bi_variant_sdpa_workspace_bytes(B, Hq, Hkv, Lq, S, D) bytes, 256-byte
 * aligned.
 */
bi_status bi_variant_sdpa(const void *q, const int64_t q_str[4],
                          const void *k, const int64_t k_str[4],
                          const void *v, const int64_t v_str[4],
                          void *o, const int64_t o_str[4],
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D,
                          float scale, int causal,
                          const uint8_t *mask, const int64_t mask_str[4],
                          bi_dtype dt,
                          void *ws, size_t ws_bytes,
                          void *stream);
size_t bi_variant_sdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D);
int64_t bi_variant_sdpa_split_len(int64_t G, int64_t Lq, int64_t S);

/*
 * Row sum / row mean over the last dimension (README, section "Why MLX is not
 * invariant", the paragraph listing the ops a batch-invariant stack relies on
 * besides matmul and attention: sum and mean among them).
 *
 * y[m] = round_to_dt( sum over n < N of x[m, n] ), or that sum divided by N
 * (one IEEE fp32 division) when mean != 0.  x: M rows of N elements, row m at
 * x + m * ldx (ldx >= N, in elements; ignored when M == 1).  y: M contiguous
 * elements of dtype dt (F32, F16 or BF16, the same as x).  Each row is reduced
 * in fp32 in an order fixed by N alone: 256 threads, thread t adds elements
 * t, t + 256, ... in ascending order from +0, the 64 partials of a wavefront
 * are combined over lane distances 32, 16, ..., 1, the four wavefront sums as
 * (w0 + w1) + (w2 + w3).  No row depends on M or on the other rows.  N == 0
 * gives 0 (sum) or NaN (mean).  M == 0 enqueues nothing.
 */
bi_status bi_rowsum(const void *x, int64_t ldx, void *y, int64_t M, int64_t N, int mean, bi_dtype dt,
                    void *stream);

/*
 * Quantized linear (README, section "Quantized models": 2, 4 and 8-bit
 * group-wise affine weights, unpacked inside the K loop of the invariant
 * kernel, with no narrower kernel for small batches).
 *
 *   y (M,N) = x (M,K) . W^T + bias,   W[n, k] = round_dt(fmaf(s, q[n, k], b))
 *
 * with s = scales[n, k / group_size], b = biases[n, k / group_size] (fp32
 * fma of the two 16-bit values and the integer field, one rounding to dt) and
 * q[n, k] the bits-wide field k mod (32 / bits) of word k / (32 / bits) of
 * row n of wq, lowest bits first.  The MFMA chain and the epilogue are those
 * of bi_linear, so y equals bi_linear(x, W, bias) bit for bit, and row m of y
 * does not depend on M or on the other rows.
 *
 * x: M rows of K elements of dt at x + m * ldx (16-byte aligned, ldx >= K and
 * a multiple of 8).  wq: N rows of ldwq uint32 words (ldwq >= K * bits / 32;
 * 4-byte aligned for 2 bits; 16-byte aligned with ldwq a multiple of 4 for 4
 * and 8 bits, which every contiguous packing satisfies).  scales, biases: N
 * rows of ldsb elements of dt (ldsb >= K / group_size).  Row pitches of 2^24
 * (x), 2^25 (wq) or 2^26 (scales, biases) elements or more are refused with
 * BI_ERR_UNSUPPORTED.  bias: N elements of dt or
 * NULL.  y: M rows of N elements of dt at y + m * ldy (ldy >= N).
 * dt: BI_BF16 or BI_F16.  bits: 2, 4 or 8 (3, 5 and 6-bit packings and
 * anything else are refused with BI_ERR_UNSUPPORTED).  group_size: 32, 64 or
 * 128, and K a multiple of it.  All device memory; enqueued on `stream`.
 * M == 0 or N == 0 enqueues nothing; K == 0 writes the bias (or zeros).
 * ws: bi_quantized_linear_workspace_bytes(M, N, K, dt) bytes of 256-byte
 * aligned device memory, or NULL when that is 0 (up to 64 rows, and any
 * number of rows when K is a multiple of 128, the weights are unpacked inside
 * the kernels: in the strip kernel's K loop, or in the tile kernel on their
 * way into LDS).  Above 64 rows with other K, chunks of at most 8192 columns
 * are dequantised into ws with the same arithmetic and bi_linear's kernels run
 * on them; the result is the same bits in every case.  Too small a workspace
 * is refused with BI_ERR_WORKSPACE.
 */
bi_status bi_quantized_linear(const void *x, int64_t ldx,
                              const uint32_t *wq, int64_t ldwq,
                              const void *scales, const void *biases, int64_t ldsb,
                              int bits, int64_t group_size,
                              const void *bias,
                              void *y, int64_t ldy,
                              int64_t M, int64_t N, int64_t K,
                              bi_dtype dt, void *ws, size_t ws_bytes, void *stream);
size_t bi_quantized_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, bi_dtype dt);

/* Which kernel configuration a GEMM of this shape runs on ("gemm_skinny_nk/fm1",
 * "gemm16_strip_kn/w16_a8", "gemm_tiled_kn/128x128", ...; b_kn != 0 for a row-major (K, N) operand of
 * bi_matmul / bi_addmm, 0 for bi_linear and for column-major operands).  Informational: every configuration computes the same bits.
 * Returns "none" for empty or oversized shapes. */
const char *bi_gemm_kernel_name(int64_t M, int64_t N, int64_t K, bi_dtype in_dt, int b_kn);

/* Which attention kernels a bi_sdpa call of these sizes runs.  For 16-bit dt
 * and D <= 128: "sdpa_prefill16" when Lq >= 384 and its grid,
 * ceil(ceil((Hq / Hkv) Lq / 16) / 4) x B x Hkv workgroups, exceeds 64; else "sdpa_quad16+combine"
 * ("sdpa_quad16" when S <= 256: one split, folded in the kernel)
 * when the quad grid, ceil(S / 256) splits x ceil(ceil((Hq / Hkv) Lq / 16) / T)
 * row-tile groups x B x Hkv workgroups with T = 1 or 2 row tiles per
 * workgroup, is at most 256 (one workgroup per CU: every split's K / V
 * requested at once); else "sdpa_prefill16" when a KV head has at least 64
 * query rows ((Hq / Hkv) Lq >= 64) and the prefill grid exceeds 64
 * workgroups; else "sdpa_fused16" when S <= 1024, and
 * "sdpa_split16+combine" (D = 128, and D = 64 on 128-byte key rows) or
 * "sdpa_split+combine" (D = 32, 96) otherwise.  For 16-bit dt and D > 128: "sdpa_prefill16w" when Lq >= 384, or
 * Lq >= 64 with B Lq >= 192 (rows of 256, all output columns in one workgroup);
 * else, for D = 256 with at most 1024 workgroups of two splits and one row
 * tile, "sdpa_split16w+combine"; else "sdpa_split+combine".  fp32 runs "sdpa_split+combine".  16-bit D < 128
 * runs the quad and one-launch kernels on rows zero-padded to 128 (the prefill kernel computes only the
 * head dim's chunks),
 * D = 160 ... 224 the wide prefill on rows zero-padded to 256 (the padding
 * adds exact zeros, so the bits are the split kernel's).
 * Informational: the split / block structure, and with it every output bit,
 * is the same whichever runs.  Returns "none" for empty, oversized or
 * unsupported sizes. */
const char *bi_sdpa_kernel_name(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, bi_dtype dt);

/* Name of a status code ("BI_OK", ...); never NULL. */
const char *bi_status_name(bi_status s);
/* Message describing the last error on the calling thread; "" after success.
 * Valid until the next bi_* call on this thread. */
const char *bi_last_error(void);
/* (ABI major << 16) | bits version.  The bits version changes whenever a
 * compile-time constant that shapes the arithmetic (k-group order, KV block
 * and split sizes) or a rounding step changes, i.e. whenever output bits may
 * change. */
int bi_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
