// Host-visible launch interface of the attention kernels (internal to libbi).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

// Fixed arithmetic constants of the attention recipe.  Changing either
// changes output bits, so they are part of the bits version.
constexpr int KV_SPLIT = 256;   // keys per split, at absolute positions [256 s, 256 s + 256)
constexpr int KV_BLOCK = 64;    // keys per block inside a split

struct SdpaParams {
    const void *q, *k, *v;
    void *o;
    int64_t qs[3], ks[3], vs[3], os[3];   // element strides of dims 0..2 (dim 3 is contiguous)
    const void *mask;                     // nullable: uint8 (nonzero = attend) or, with mask_add, dt values
    int64_t ms[4];                        // element strides of the mask
    int mask_add;                         // the mask is additive (dt, added to the scaled scores)
    int mask_vec;                         // keys contiguous, S % 4 == 0, rows 4-key aligned: 4 keys per load
    const float *sinks;                   // nullable: Hq logits, one extra softmax term per query head
    int B, Hq, Hkv, Lq, S, G;             // G = Hq / Hkv
    int causal;
    int dr;                               // head dim; the 16-bit kernels run D <= 128 as 128 with zero padding
    float c;                              // scale * log2(e), rounded once to fp32
    int nsplit;                           // ceil(S / split_len)
    int split_len;                        // KV_SPLIT; other values only in the batch-variant comparator
    float *ws_ml;                         // [rows][nsplit][2]  (m, l)
    float *ws_o;                          // [rows][nsplit][D]
};

// Which kernels serve a call.  Every path computes the same bits; the split,
// wide split and quad paths use a workspace.
enum SdpaPath {
    SDPA_FUSED16,     // 16-bit, D <= 128, at most four splits: one launch, fold in LDS
    SDPA_PREFILL16,   // 16-bit, long caches with many query rows: fold in registers (D > 128: rows of 256)
    SDPA_QUAD16,      // 16-bit, D <= 128, small grids: one wavefront per block, combine kernel
    SDPA_SPLIT16W,    // 16-bit, D = 256, moderate grids: 512-byte rows, combine kernel
    SDPA_SPLIT        // split kernel + combine kernel through the workspace
};
// Hkv >= 1 and Hq % Hkv == 0 (the callers validate).
SdpaPath sdpa_path(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, int dt);
size_t sdpa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, int dt);
// Calls whose split partials would exceed SDPA_WS_CAP bytes run in chunks of this many query rows (each a
// call of its own with the keys up to its last row when causal: every row's arithmetic is unchanged), so
// the workspace stays bounded as Lq and S grow; Lq when the call runs whole.
constexpr int64_t SDPA_WS_CAP = int64_t(256) << 20;
int64_t sdpa_chunk_rows(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, int dt);
// Carves ws into ws_ml / ws_o (p.nsplit must be set).
void sdpa_bind_workspace(SdpaParams &p, void *ws);
hipError_t launch_sdpa(const SdpaParams &p, int dt, int D, hipStream_t stream);
// Batch-variant comparator: the generic split kernel + combine with a split length chosen from the call's
// shape (sdpa_variant_split_len), so that the reduction order moves with the query count and the cache
// length.  Not invariant; measurement only.
int64_t sdpa_variant_split_len(int64_t G, int64_t Lq, int64_t S);
size_t sdpa_variant_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D);
hipError_t launch_sdpa_variant(const SdpaParams &p, int dt, int D, hipStream_t stream);
// Names of the kernels launch_sdpa runs ("sdpa_fused16", ...).
const char *sdpa_kernel_name(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t S, int64_t D, int dt);

}  // namespace bi
