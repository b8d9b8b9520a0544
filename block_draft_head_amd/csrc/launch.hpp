// Host-side launchers behind the C ABI (one per operation).  Arguments are
// already validated by api.cpp; each launcher only enqueues kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dflash2.h"

namespace dflash2 {

// Workspaces start with a 256-byte header holding the device status word.
constexpr size_t kStatusBytes = 256;
// Bit of the status word set when a token id is outside [0, vocab).
constexpr uint32_t kStatusIdRange = 1u;

struct LmheadPlan {
    bool streaming, big;  // big: 256 x 256 bf16 MFMA tiles (many rows)
    bool dma;             // streaming, weights copied into LDS (bf16, at most 8 rows)
    int ksplit;           // dma: waves sharing each tile (each multiplies 1 / ksplit of H)
    int n_mt;
    int nw, prefetch, n_tiles;
    int grid_x, grid_y, n_lists;
    int list_len;  // keys per partial list (>= K; the big kernel keeps a power of two)
    int merge_rows;
    size_t lds, merge_lds, partial_bytes;
    size_t tiles_offset;  // big: byte offset of the exact-path tile buffers after the partial lists
    size_t lse_offset;    // byte offset of the per-list log-sum-exp partials (float2 [M][n_lists])
};
LmheadPlan plan_lmhead(int dtype, int64_t M, int H, int V, int K);
// Forces the number of vocabulary slabs of every later plan (0 = automatic).
void set_forced_slabs(int n);

// LDS of one walk workgroup: the block's best-successor keys, their scores,
// the candidate ids and (sampling) the noise.
inline size_t walk_lds_bytes(int bs, int K) { return (size_t)bs * K * (8 + 4 + 4 + 4); }

// Workspace of the selector CE backward, byte offsets (256-byte aligned).
// g / gv [N, r], ag [N, r] float32, dg (float32 [N, r] or bf16 packed); per (row, slot) entries
// (slot K is the predecessor row) with their weight, target and sorted
// order; per-target counts and offsets over the 2V targets (successor rows,
// then predecessor rows) plus one; and the scan's per-tile prefixes.
constexpr int kScanTile = 4096;
struct CeBwdLayout {
    size_t g, ag, dg, wgt, tgt, src, counts, offsets, tiles, total;
};
inline CeBwdLayout ce_bwd_layout(int64_t N, int V, int r, int K) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t E = (size_t)N * (K + 1), C = 2 * (size_t)V + 1;
    CeBwdLayout L;
    L.g = kStatusBytes;
    L.ag = L.g + up((size_t)N * r * 4);
    L.dg = L.ag + up((size_t)N * r * 4);
    // dg: float32 [N, r], or (bf16) high and low parts packed 8 rows deep
    L.wgt = L.dg + up((size_t)(N + 7) / 8 * 8 * r * 4);
    L.tgt = L.wgt + up(E * 4);
    L.src = L.tgt + up(E * 4);
    L.counts = L.src + up(E * 4);
    L.offsets = L.counts + up(C * 4);
    L.tiles = L.offsets + up(C * 4);
    L.total = L.tiles + up((C + kScanTile - 1) / kScanTile * 4);
    return L;
}

// Sampling walk: temperature and the generator's 64-bit key.
struct SampleParams {
    float temperature;
    uint64_t seed;
};

hipError_t launch_conv_prepare(int dtype, int64_t N, int bs, int H, int taps, int gs, const void *x,
                               const void *w_proj, const void *base, void *x_out, float *k_post,
                               hipStream_t stream);
hipError_t launch_conv_finish(int dtype, int64_t N, int bs, int H, int taps, int gs, const void *y,
                              const float *k_post, const void *base, void *y_out, hipStream_t stream);
// Unary-logit transform (mult, then softcap cap; 1 and 0: none) and the
// optional per-row metrics of the same pass.
struct UnaryMetrics {
    float mult, cap;
    float *lse;        // [M] log-sum-exp of the transformed logits over the vocabulary, or null
    float *gold_prob;  // [M] softmax probability of the gold id, or null
    uint8_t *hit;      // [M] gold id among the top K, or null
};
// With g (and w_h, r > 0) the call also writes the context projection
// g = h W_Hᵀ, float32 [M, r]: on the many-row bf16 path as extra tiles of the
// LM-head kernel's weight stream, else by its own launch.
hipError_t launch_unary_topk(int dtype, int64_t M, int H, int V, int K, const void *h, const void *w,
                             const int32_t *gold, int32_t *out_ids, float *out_vals,
                             float *gold_logit, void *workspace, hipStream_t stream,
                             const UnaryMetrics *metrics = nullptr, const void *w_h = nullptr, int r = 0,
                             float *g = nullptr);
// Decode head (bf16, at most 8 rows): the LM-head kernel with the context
// projection's rows streamed after the vocabulary's, then one workgroup that
// merges the candidate lists and walks every block.  Workspace: status word,
// the workgroups' partial lists, the context rows g [M, r].
struct DecodeLayout {
    int grid;
    size_t partial, heads, g, total;  // byte offsets: lists, their heads (one key per list), context rows
};
DecodeLayout decode_layout(int64_t M, int H, int V, int r, int K);  // r = 0: no context rows
bool decode_head_supported(int64_t M, int H, int V, int r, int K);
hipError_t launch_decode_head(int64_t M, int H, int V, int K, const void *h, const void *w, int r, const void *w_h,
                              const void *A, const void *B, const int32_t *anchors, int bs, int32_t *out_ids,
                              float *out_vals, int32_t *path, float *path_score, void *workspace, hipStream_t stream);
hipError_t launch_context_proj(int dtype, int64_t N, int H, int r, const void *h, const void *w_h,
                               float *g, uint32_t *status, hipStream_t stream);
// g_in: the context rows g = h W_Hᵀ computed beforehand (float32 [N, r]), or
// null to form them here from h and w_h into the workspace.
hipError_t launch_selector_walk(int dtype, int n_blocks, int bs, int H, int V, int r, int K,
                                const void *h, const void *w_h, const float *g_in, const void *A, const void *B,
                                const int32_t *cand_ids, const float *cand_vals,
                                const int32_t *anchors, int32_t *path, float *path_score,
                                void *workspace, hipStream_t stream, const SampleParams *sample);
// Walk without a caller workspace: the status word and the context rows live
// in a file-scope device array of this many bytes (one copy per GPU).
constexpr size_t kNoAllocScratchBytes = ((size_t)8 << 20) + kStatusBytes;
// Device address of that array on the current device (looked up once per device).
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_selector_tf(int dtype, int64_t N, int H, int V, int r, int K, const void *h,
                              const void *w_h, const float *g_in, const void *A, const void *B,
                              const int32_t *cand_ids,
                              const float *cand_vals, const int32_t *pred_ids,
                              const int32_t *gold_ids, const uint8_t *force,
                              const float *gold_logit, float *out_scores, int32_t *out_best,
                              float *out_ce, uint8_t *out_valid, void *workspace,
                              hipStream_t stream);
hipError_t launch_selector_ce_backward(int dtype, int64_t N, int H, int V, int r, int K, const void *h,
                                       const void *w_h, const void *A, const void *B,
                                       const int32_t *cand_ids, const float *cand_vals,
                                       const int32_t *pred_ids, const int32_t *gold_ids,
                                       const uint8_t *force, const float *gold_logit, const float *grad_ce,
                                       float *grad_pred, float *grad_succ, float *grad_wh, float *out_ce,
                                       uint8_t *out_valid, void *workspace, hipStream_t stream);

}  // namespace dflash2
