// C ABI of the DFlash2 draft-block head: host-side validation, then the
// launchers.  Every error the host can detect is returned before anything is
// enqueued; nothing here allocates or synchronises (except
// dflash2_read_device_status).
#include <cmath>
#include <hip/hip_runtime.h>

#include <array>
#include <climits>
#include <initializer_list>
#include <iterator>
#include <cstdint>

#include "../../include/dflash2.h"
#include "launch.hpp"

using namespace dflash2;

static_assert(DFLASH2_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "header and library agree on the array size");

namespace {

size_t elem_size(int dtype) { return dtype == DFLASH2_F32 ? 4 : 2; }
bool dtype_ok(int dtype) { return dtype == DFLASH2_F32 || dtype == DFLASH2_BF16; }

// true when [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

// A byte range of a call's argument (an empty range when the pointer is NULL).
struct Span {
    const void *p;
    size_t b;
};

// true when two outputs share a byte, or an output shares one with an input
template <class O, class I>
bool aliased(const O &outs, const I &ins) {
    const size_t no = std::size(outs), ni = std::size(ins);
    for (size_t i = 0; i < no; ++i) {
        for (size_t j = i + 1; j < no; ++j)
            if (overlaps(outs[i].p, outs[i].b, outs[j].p, outs[j].b)) return true;
        for (size_t j = 0; j < ni; ++j)
            if (overlaps(outs[i].p, outs[i].b, ins[j].p, ins[j].b)) return true;
    }
    return false;
}

// The bytes of an optional argument: 0 when it is NULL.
size_t opt(const void *p, size_t b) { return p ? b : 0; }

// true when a floating-point array or the workspace (vec16) is off a 16-byte
// boundary or an int32 array (word4) off a 4-byte one; NULL passes
bool misaligned(std::initializer_list<const void *> vec16, std::initializer_list<const void *> word4 = {}) {
    for (const void *p : vec16)
        if (reinterpret_cast<uintptr_t>(p) % 16) return true;
    for (const void *p : word4)
        if (reinterpret_cast<uintptr_t>(p) % 4) return true;
    return false;
}

dflash2_status launched(hipError_t e) { return e == hipSuccess ? DFLASH2_OK : DFLASH2_ERR_LAUNCH; }

// Hidden sizes the contraction kernels tile without a remainder.
bool hidden_supported(int32_t hidden) { return hidden % 64 == 0; }

dflash2_status check_conv(int dtype, int64_t n_tokens, int32_t block_size, int32_t hidden,
                          int32_t taps, int32_t group_size) {
    if (!dtype_ok(dtype)) return DFLASH2_ERR_DTYPE;
    if (n_tokens < 1 || block_size < 1 || hidden < 1 || taps < 1 || group_size < 1) return DFLASH2_ERR_SHAPE;
    if (n_tokens % block_size != 0) return DFLASH2_ERR_SHAPE;  // draft length must be whole blocks
    if (taps > block_size) return DFLASH2_ERR_SHAPE;
    if (hidden % group_size != 0) return DFLASH2_ERR_SHAPE;
    if (taps > DFLASH2_MAX_TAPS || !hidden_supported(hidden)) return DFLASH2_ERR_UNSUPPORTED;
    if (n_tokens > INT_MAX) return DFLASH2_ERR_UNSUPPORTED;
    return DFLASH2_OK;
}

dflash2_status check_selector(int dtype, int64_t n_rows, int32_t hidden, int32_t vocab,
                              int32_t rank, int32_t top_k) {
    if (!dtype_ok(dtype)) return DFLASH2_ERR_DTYPE;
    if (n_rows < 1 || hidden < 1 || vocab < 1 || rank < 1) return DFLASH2_ERR_SHAPE;
    if (top_k < 1 || top_k > vocab) return DFLASH2_ERR_SHAPE;
    if (top_k > DFLASH2_MAX_TOP_K || rank % 8 != 0 || rank > DFLASH2_MAX_RANK || !hidden_supported(hidden))
        return DFLASH2_ERR_UNSUPPORTED;
    if (n_rows > INT_MAX) return DFLASH2_ERR_UNSUPPORTED;
    return DFLASH2_OK;
}

// The walk's and sampler's outputs (the workspace among them) and inputs.
std::array<Span, 3> walk_outputs(int64_t N, const void *path, const void *score, const void *ws, size_t ws_bytes) {
    return {Span{path, (size_t)N * 4}, Span{score, opt(score, (size_t)N * 4)}, Span{ws, ws_bytes}};
}
std::array<Span, 8> walk_inputs(int dtype, int32_t n_blocks, int64_t N, int32_t hidden, int32_t vocab, int32_t rank,
                                int32_t top_k, const void *h, const void *w_h, const float *g, const void *A,
                                const void *B, const void *cand_ids, const void *cand_vals, const void *anchors) {
    const size_t es = elem_size(dtype), nk = (size_t)N * top_k * 4, cb = (size_t)vocab * rank * es;
    return {Span{h, opt(h, (size_t)N * hidden * es)}, Span{w_h, opt(w_h, (size_t)rank * hidden * es)},
            Span{g, opt(g, (size_t)N * rank * 4)}, Span{A, cb}, Span{B, cb}, Span{cand_ids, nk}, Span{cand_vals, nk},
            Span{anchors, (size_t)n_blocks * 4}};
}

}  // namespace

extern "C" {

const char *dflash2_version(void) { return "dflash2-gfx950 0.1.0"; }

dflash2_status dflash2_debug_force_slabs(int32_t n_slabs) {
    if (n_slabs < 0 || n_slabs > 4096) return DFLASH2_ERR_SHAPE;
    set_forced_slabs(n_slabs);
    return DFLASH2_OK;
}

const char *dflash2_status_str(int s) {
    switch (s) {
        case DFLASH2_OK: return "ok";
        case DFLASH2_ERR_NULL: return "a required pointer is null";
        case DFLASH2_ERR_SHAPE: return "sizes break a rule of the method";
        case DFLASH2_ERR_DTYPE: return "unknown dtype";
        case DFLASH2_ERR_UNSUPPORTED: return "sizes beyond what the kernels support";
        case DFLASH2_ERR_ALIAS: return "an output overlaps an input";
        case DFLASH2_ERR_WORKSPACE: return "workspace too small";
        case DFLASH2_ERR_LAUNCH: return "kernel launch failed";
        case DFLASH2_ERR_DEVICE_ID_RANGE: return "a token id was outside [0, vocab)";
        default: return "unknown status";
    }
}

size_t dflash2_workspace_bytes(int op, int64_t n_rows, int32_t hidden, int32_t vocab, int32_t rank,
                               int32_t top_k) {
    if (n_rows < 1 || n_rows > INT_MAX) return 0;
    switch (op) {
        case DFLASH2_OP_UNARY_TOPK: {
            if (hidden < 1 || vocab < 1 || top_k < 1 || top_k > DFLASH2_MAX_TOP_K) return 0;
            // the plan depends on the element size only through the streaming
            // fragment buffer; take the larger of the two dtypes' needs
            const LmheadPlan a = plan_lmhead(DFLASH2_F32, n_rows, hidden, vocab, top_k);
            const LmheadPlan b = plan_lmhead(DFLASH2_BF16, n_rows, hidden, vocab, top_k);
            const size_t p = a.partial_bytes > b.partial_bytes ? a.partial_bytes : b.partial_bytes;
            return kStatusBytes + p;
        }
        case DFLASH2_OP_SELECTOR_WALK:
        case DFLASH2_OP_SELECTOR_TF:
            if (rank < 1) return 0;
            return kStatusBytes + (size_t)n_rows * (size_t)rank * 4;
        case DFLASH2_OP_SELECTOR_CE_BACKWARD:
            if (rank < 1 || vocab < 1 || top_k < 1) return 0;
            return ce_bwd_layout(n_rows, vocab, rank, top_k).total;
        case DFLASH2_OP_DECODE_HEAD:
            if (hidden < 1 || vocab < 1 || rank < 0 || top_k < 1 || top_k > DFLASH2_MAX_TOP_K) return 0;
            return decode_layout(n_rows, hidden, vocab, rank, top_k).total;
        default: return 0;
    }
}

dflash2_status dflash2_conv_prepare(int dtype, int64_t n_tokens, int32_t block_size, int32_t hidden,
                                    int32_t taps, int32_t group_size, const void *x,
                                    const void *w_proj, const void *base, void *x_out,
                                    float *k_post, void *stream) {
    dflash2_status s = check_conv(dtype, n_tokens, block_size, hidden, taps, group_size);
    if (s != DFLASH2_OK) return s;
    if (!x || !w_proj || !base || !x_out || !k_post) return DFLASH2_ERR_NULL;
    const size_t es = elem_size(dtype);
    const size_t act = (size_t)n_tokens * hidden * es;
    const size_t kp = (size_t)n_tokens * taps * (hidden / group_size) * 4;
    const size_t G = (size_t)(hidden / group_size);
    if (misaligned({x, w_proj, base, x_out, k_post})) return DFLASH2_ERR_UNSUPPORTED;
    const Span outs[] = {{x_out, act}, {k_post, kp}};
    const Span ins[] = {{x, act}, {w_proj, 2 * (size_t)taps * G * hidden * es}, {base, 2 * (size_t)taps * hidden * es}};
    if (aliased(outs, ins)) return DFLASH2_ERR_ALIAS;
    return launched(launch_conv_prepare(dtype, n_tokens, block_size, hidden, taps, group_size, x,
                                        w_proj, base, x_out, k_post, (hipStream_t)stream));
}

dflash2_status dflash2_conv_finish(int dtype, int64_t n_tokens, int32_t block_size, int32_t hidden,
                                   int32_t taps, int32_t group_size, const void *y,
                                   const float *k_post, const void *base, void *y_out,
                                   void *stream) {
    dflash2_status s = check_conv(dtype, n_tokens, block_size, hidden, taps, group_size);
    if (s != DFLASH2_OK) return s;
    if (!y || !k_post || !base || !y_out) return DFLASH2_ERR_NULL;
    const size_t es = elem_size(dtype);
    const size_t act = (size_t)n_tokens * hidden * es;
    const size_t kp = (size_t)n_tokens * taps * (hidden / group_size) * 4;
    if (misaligned({y, k_post, base, y_out})) return DFLASH2_ERR_UNSUPPORTED;
    const Span outs[] = {{y_out, act}};
    const Span ins[] = {{y, act}, {k_post, kp}, {base, 2 * (size_t)taps * hidden * es}};
    if (aliased(outs, ins)) return DFLASH2_ERR_ALIAS;
    return launched(launch_conv_finish(dtype, n_tokens, block_size, hidden, taps, group_size, y,
                                       k_post, base, y_out, (hipStream_t)stream));
}

dflash2_status dflash2_unary_topk(int dtype, int64_t n_rows, int32_t hidden, int32_t vocab,
                                  int32_t top_k, const void *h, const void *w_lm,
                                  const int32_t *gold_ids, int32_t *out_ids, float *out_vals,
                                  float *out_gold_logit, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    if (!dtype_ok(dtype)) return DFLASH2_ERR_DTYPE;
    if (n_rows < 1 || hidden < 1 || vocab < 1) return DFLASH2_ERR_SHAPE;
    if (top_k < 1 || top_k > vocab) return DFLASH2_ERR_SHAPE;
    if (top_k > DFLASH2_MAX_TOP_K || !hidden_supported(hidden) || n_rows > INT_MAX)
        return DFLASH2_ERR_UNSUPPORTED;
    if (!h || !w_lm || !out_ids || !out_vals || !workspace) return DFLASH2_ERR_NULL;
    if (gold_ids && !out_gold_logit) return DFLASH2_ERR_NULL;
    if (workspace_bytes < dflash2_workspace_bytes(DFLASH2_OP_UNARY_TOPK, n_rows, hidden, vocab, 0, top_k))
        return DFLASH2_ERR_WORKSPACE;
    if (misaligned({h, w_lm, out_vals, out_gold_logit, workspace}, {gold_ids, out_ids}))
        return DFLASH2_ERR_UNSUPPORTED;
    const size_t nk = (size_t)n_rows * top_k, n = (size_t)n_rows, es = elem_size(dtype);
    const Span outs[] = {{out_ids, nk * 4}, {out_vals, nk * 4}, {out_gold_logit, opt(out_gold_logit, n * 4)},
                         {workspace, workspace_bytes}};
    const Span ins[] = {{h, n * hidden * es}, {w_lm, (size_t)vocab * hidden * es}, {gold_ids, opt(gold_ids, n * 4)}};
    if (aliased(outs, ins)) return DFLASH2_ERR_ALIAS;
    return launched(launch_unary_topk(dtype, n_rows, hidden, vocab, top_k, h, w_lm, gold_ids, out_ids,
                                      out_vals, out_gold_logit, workspace, (hipStream_t)stream));
}

dflash2_status dflash2_unary_topk_ex(int dtype, int64_t n_rows, int32_t hidden, int32_t vocab, int32_t top_k,
                                     const void *h, const void *w_lm, const int32_t *gold_ids,
                                     float output_multiplier, float final_logit_softcapping, const void *w_h,
                                     int32_t rank, int32_t *out_ids, float *out_vals, float *out_gold_logit,
                                     float *out_lse, float *out_gold_prob, uint8_t *out_gold_hit, float *out_g,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    if (!dtype_ok(dtype)) return DFLASH2_ERR_DTYPE;
    if (n_rows < 1 || hidden < 1 || vocab < 1) return DFLASH2_ERR_SHAPE;
    if (top_k < 1 || top_k > vocab) return DFLASH2_ERR_SHAPE;
    if (!(output_multiplier > 0.f) || !std::isfinite(output_multiplier)) return DFLASH2_ERR_SHAPE;
    if (!(final_logit_softcapping >= 0.f) || !std::isfinite(final_logit_softcapping)) return DFLASH2_ERR_SHAPE;
    if (top_k > DFLASH2_MAX_TOP_K || !hidden_supported(hidden) || n_rows > INT_MAX)
        return DFLASH2_ERR_UNSUPPORTED;
    if (!h || !w_lm || !out_ids || !out_vals || !workspace) return DFLASH2_ERR_NULL;
    if (gold_ids && !out_gold_logit) return DFLASH2_ERR_NULL;
    if ((out_gold_prob || out_gold_hit) && !gold_ids) return DFLASH2_ERR_NULL;
    if (!w_h != !out_g) return DFLASH2_ERR_NULL;  // the context projection takes both
    if (out_g) {
        if (rank < 1) return DFLASH2_ERR_SHAPE;
        if (rank % 8 != 0 || rank > DFLASH2_MAX_RANK) return DFLASH2_ERR_UNSUPPORTED;
    }
    if (workspace_bytes < dflash2_workspace_bytes(DFLASH2_OP_UNARY_TOPK, n_rows, hidden, vocab, 0, top_k))
        return DFLASH2_ERR_WORKSPACE;
    if (misaligned({h, w_lm, w_h, out_vals, out_gold_logit, out_lse, out_gold_prob, out_g, workspace},
                   {gold_ids, out_ids}))
        return DFLASH2_ERR_UNSUPPORTED;
    const size_t nk = (size_t)n_rows * top_k, n = (size_t)n_rows, es = elem_size(dtype);
    const size_t r = out_g ? (size_t)rank : 0;
    const Span outs[] = {{out_ids, nk * 4}, {out_vals, nk * 4}, {out_gold_logit, opt(out_gold_logit, n * 4)},
                         {out_lse, opt(out_lse, n * 4)}, {out_gold_prob, opt(out_gold_prob, n * 4)},
                         {out_gold_hit, opt(out_gold_hit, n)}, {out_g, n * r * 4}, {workspace, workspace_bytes}};
    const Span ins[] = {{h, n * hidden * es}, {w_lm, (size_t)vocab * hidden * es}, {gold_ids, opt(gold_ids, n * 4)},
                        {w_h, r * hidden * es}};
    if (aliased(outs, ins)) return DFLASH2_ERR_ALIAS;
    const UnaryMetrics um{output_multiplier, final_logit_softcapping, out_lse, out_gold_prob, out_gold_hit};
    return launched(launch_unary_topk(dtype, n_rows, hidden, vocab, top_k, h, w_lm, gold_ids, out_ids, out_vals,
                                      out_gold_logit, workspace, (hipStream_t)stream, &um, w_h, (int)r, out_g));
}

dflash2_status dflash2_selector_walk(int dtype, int32_t n_blocks, int32_t block_size, int32_t hidden,
                                     int32_t vocab, int32_t rank, int32_t top_k, const void *h,
                                     const void *w_h, const float *g, const void *cb_pred, const void *cb_succ,
                                     const int32_t *cand_ids, const float *cand_vals,
                                     const int32_t *anchor_ids, int32_t *out_path,
                                     float *out_path_score, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (n_blocks < 1 || block_size < 1) return dtype_ok(dtype) ? DFLASH2_ERR_SHAPE : DFLASH2_ERR_DTYPE;
    const int64_t N = (int64_t)n_blocks * block_size;
    dflash2_status s = check_selector(dtype, N, hidden, vocab, rank, top_k);
    if (s != DFLASH2_OK) return s;
    if (block_size > DFLASH2_MAX_BLOCK_SIZE) return DFLASH2_ERR_UNSUPPORTED;
    if (!(g || (h && w_h)) || !cb_pred || !cb_succ || !cand_ids || !cand_vals || !anchor_ids || !out_path ||
        !workspace)
        return DFLASH2_ERR_NULL;
    if (workspace_bytes < dflash2_workspace_bytes(DFLASH2_OP_SELECTOR_WALK, N, hidden, vocab, rank, top_k))
        return DFLASH2_ERR_WORKSPACE;
    if (misaligned({h, w_h, g, cb_pred, cb_succ, cand_vals, out_path_score, workspace},
                   {cand_ids, anchor_ids, out_path}))
        return DFLASH2_ERR_UNSUPPORTED;
    if (aliased(walk_outputs(N, out_path, out_path_score, workspace, workspace_bytes),
                walk_inputs(dtype, n_blocks, N, hidden, vocab, rank, top_k, h, w_h, g, cb_pred, cb_succ, cand_ids,
                            cand_vals, anchor_ids)))
        return DFLASH2_ERR_ALIAS;
    return launched(launch_selector_walk(dtype, n_blocks, block_size, hidden, vocab, rank, top_k, h, w_h, g,
                                         cb_pred, cb_succ, cand_ids, cand_vals, anchor_ids, out_path,
                                         out_path_score, workspace, (hipStream_t)stream, nullptr));
}

dflash2_status dflash2_selector_walk_noalloc(int dtype, int32_t n_blocks, int32_t block_size, int32_t hidden,
                                             int32_t vocab, int32_t rank, int32_t top_k, const void *h,
                                             const void *w_h, const float *g, const void *cb_pred,
                                             const void *cb_succ,
                                             const int32_t *cand_ids, const float *cand_vals,
                                             const int32_t *anchor_ids, int32_t *out_path, float *out_path_score,
                                             void *stream) {
    if (n_blocks < 1 || block_size < 1) return dtype_ok(dtype) ? DFLASH2_ERR_SHAPE : DFLASH2_ERR_DTYPE;
    const int64_t N = (int64_t)n_blocks * block_size;
    dflash2_status s = check_selector(dtype, N, hidden, vocab, rank, top_k);
    if (s != DFLASH2_OK) return s;
    if (block_size > DFLASH2_MAX_BLOCK_SIZE) return DFLASH2_ERR_UNSUPPORTED;
    if (dflash2_workspace_bytes(DFLASH2_OP_SELECTOR_WALK, N, hidden, vocab, rank, top_k) > kNoAllocScratchBytes)
        return DFLASH2_ERR_UNSUPPORTED;
    if (!(g || (h && w_h)) || !cb_pred || !cb_succ || !cand_ids || !cand_vals || !anchor_ids || !out_path)
        return DFLASH2_ERR_NULL;
    if (misaligned({h, w_h, g, cb_pred, cb_succ, cand_vals, out_path_score}, {cand_ids, anchor_ids, out_path}))
        return DFLASH2_ERR_UNSUPPORTED;
    if (aliased(walk_outputs(N, out_path, out_path_score, nullptr, 0),
                walk_inputs(dtype, n_blocks, N, hidden, vocab, rank, top_k, h, w_h, g, cb_pred, cb_succ, cand_ids,
                            cand_vals, anchor_ids)))
        return DFLASH2_ERR_ALIAS;
    void *scratch = nullptr;
    if (noalloc_scratch(&scratch) != hipSuccess) return DFLASH2_ERR_LAUNCH;
    return launched(launch_selector_walk(dtype, n_blocks, block_size, hidden, vocab, rank, top_k, h, w_h, g,
                                         cb_pred, cb_succ, cand_ids, cand_vals, anchor_ids, out_path,
                                         out_path_score, scratch, (hipStream_t)stream, nullptr));
}

dflash2_status dflash2_selector_sample(int dtype, int32_t n_blocks, int32_t block_size, int32_t hidden,
                                       int32_t vocab, int32_t rank, int32_t top_k, const void *h,
                                       const void *w_h, const float *g, const void *cb_pred, const void *cb_succ,
                                       const int32_t *cand_ids, const float *cand_vals,
                                       const int32_t *anchor_ids, float temperature, uint64_t seed,
                                       int32_t *out_path, float *out_path_score, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    if (n_blocks < 1 || block_size < 1) return dtype_ok(dtype) ? DFLASH2_ERR_SHAPE : DFLASH2_ERR_DTYPE;
    const int64_t N = (int64_t)n_blocks * block_size;
    dflash2_status s = check_selector(dtype, N, hidden, vocab, rank, top_k);
    if (s != DFLASH2_OK) return s;
    if (!(temperature > 0.0f) || !std::isfinite(temperature)) return DFLASH2_ERR_SHAPE;
    if (block_size > DFLASH2_MAX_BLOCK_SIZE) return DFLASH2_ERR_UNSUPPORTED;
    if (!(g || (h && w_h)) || !cb_pred || !cb_succ || !cand_ids || !cand_vals || !anchor_ids || !out_path ||
        !workspace)
        return DFLASH2_ERR_NULL;
    if (workspace_bytes < dflash2_workspace_bytes(DFLASH2_OP_SELECTOR_WALK, N, hidden, vocab, rank, top_k))
        return DFLASH2_ERR_WORKSPACE;
    if (misaligned({h, w_h, g, cb_pred, cb_succ, cand_vals, out_path_score, workspace},
                   {cand_ids, anchor_ids, out_path}))
        return DFLASH2_ERR_UNSUPPORTED;
    if (aliased(walk_outputs(N, out_path, out_path_score, workspace, workspace_bytes),
                walk_inputs(dtype, n_blocks, N, hidden, vocab, rank, top_k, h, w_h, g, cb_pred, cb_succ, cand_ids,
                            cand_vals, anchor_ids)))
        return DFLASH2_ERR_ALIAS;
    const SampleParams sp{temperature, seed};
    return launched(launch_selector_walk(dtype, n_blocks, block_size, hidden, vocab, rank, top_k, h, w_h, g,
                                         cb_pred, cb_succ, cand_ids, cand_vals, anchor_ids, out_path,
                                         out_path_score, workspace, (hipStream_t)stream, &sp));
}

dflash2_status dflash2_decode_head(int dtype, int32_t n_blocks, int32_t block_size, int32_t hidden, int32_t vocab,
                                   int32_t rank, int32_t top_k, const void *h, const void *w_lm, const void *w_h,
                                   const void *cb_pred, const void *cb_succ, const int32_t *anchor_ids,
                                   int32_t *out_ids, float *out_vals, int32_t *out_path, float *out_path_score,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    if (!dtype_ok(dtype)) return DFLASH2_ERR_DTYPE;
    if (n_blocks < 1 || block_size < 1 || hidden < 1 || vocab < 1) return DFLASH2_ERR_SHAPE;
    if (top_k < 1 || top_k > vocab) return DFLASH2_ERR_SHAPE;
    const bool sel = w_h || cb_pred || cb_succ || anchor_ids || out_path || out_path_score;
    if (sel) {
        if (rank < 1) return DFLASH2_ERR_SHAPE;
        if (rank % 8 != 0 || rank > DFLASH2_MAX_RANK) return DFLASH2_ERR_UNSUPPORTED;
    }
    const int64_t N = (int64_t)n_blocks * block_size;
    const int r = sel ? rank : 0;
    if (dtype != DFLASH2_BF16 || block_size > DFLASH2_MAX_BLOCK_SIZE || !hidden_supported(hidden) ||
        !decode_head_supported(N, hidden, vocab, r, top_k))
        return DFLASH2_ERR_UNSUPPORTED;
    if (!h || !w_lm || !out_ids || !out_vals || !workspace) return DFLASH2_ERR_NULL;
    if (sel && (!w_h || !cb_pred || !cb_succ || !anchor_ids || !out_path)) return DFLASH2_ERR_NULL;
    if (workspace_bytes < dflash2_workspace_bytes(DFLASH2_OP_DECODE_HEAD, N, hidden, vocab, r, top_k))
        return DFLASH2_ERR_WORKSPACE;
    if (misaligned({h, w_lm, w_h, cb_pred, cb_succ, out_vals, out_path_score, workspace},
                   {anchor_ids, out_ids, out_path}))
        return DFLASH2_ERR_UNSUPPORTED;
    const size_t nk = (size_t)N * top_k * 4, np = (size_t)N * 4, cb = (size_t)vocab * r * 2;
    const Span outs[] = {{out_ids, nk}, {out_vals, nk}, {out_path, opt(out_path, np)},
                         {out_path_score, opt(out_path_score, np)}, {workspace, workspace_bytes}};
    const Span ins[] = {{h, (size_t)N * hidden * 2}, {w_lm, (size_t)vocab * hidden * 2},
                        {w_h, opt(w_h, (size_t)r * hidden * 2)}, {cb_pred, opt(cb_pred, cb)},
                        {cb_succ, opt(cb_succ, cb)}, {anchor_ids, opt(anchor_ids, (size_t)n_blocks * 4)}};
    if (aliased(outs, ins)) return DFLASH2_ERR_ALIAS;
    return launched(launch_decode_head(N, hidden, vocab, top_k, h, w_lm, r, sel ? w_h : nullptr, cb_pred, cb_succ,
                                       anchor_ids, block_size, out_ids, out_vals, out_path, out_path_score,
                                       workspace, (hipStream_t)stream));
}

dflash2_status dflash2_selector_score_tf(int dtype, int64_t n_rows, int32_t hidden, int32_t vocab,
                                         int32_t rank, int32_t top_k, const void *h, const void *w_h,
                                         const float *g, const void *cb_pred, const void *cb_succ,
                                         const int32_t *cand_ids, const float *cand_vals,
                                         const int32_t *pred_ids, const int32_t *gold_ids,
                                         const uint8_t *force, const float *gold_logit,
                                         float *out_scores, int32_t *out_best_ids, float *out_ce,
                                         uint8_t *out_valid, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    dflash2_status s = check_selector(dtype, n_rows, hidden, vocab, rank, top_k);
    if (s != DFLASH2_OK) return s;
    if (!(g || (h && w_h)) || !cb_pred || !cb_succ || !cand_ids || !cand_vals || !pred_ids || !out_scores ||
        !out_best_ids || !workspace)
        return DFLASH2_ERR_NULL;
    if (force && !gold_ids) return DFLASH2_ERR_NULL;
    if (force && !gold_logit) return DFLASH2_ERR_NULL;
    if (gold_ids && (!out_ce || !out_valid)) return DFLASH2_ERR_NULL;
    if (workspace_bytes < dflash2_workspace_bytes(DFLASH2_OP_SELECTOR_TF, n_rows, hidden, vocab, rank, top_k))
        return DFLASH2_ERR_WORKSPACE;
    if (misaligned({h, w_h, g, cb_pred, cb_succ, cand_vals, gold_logit, out_scores, out_ce, workspace},
                   {cand_ids, pred_ids, gold_ids, out_best_ids}))
        return DFLASH2_ERR_UNSUPPORTED;
    const size_t nk = (size_t)n_rows * top_k * 4, n = (size_t)n_rows, es = elem_size(dtype);
    const size_t cb = (size_t)vocab * rank * es;
    const Span outs[] = {{out_scores, nk}, {out_best_ids, n * 4}, {out_ce, opt(out_ce, n * 4)},
                         {out_valid, opt(out_valid, n)}, {workspace, workspace_bytes}};
    const Span ins[] = {{h, opt(h, n * hidden * es)}, {w_h, opt(w_h, (size_t)rank * hidden * es)},
                        {g, opt(g, n * rank * 4)}, {cb_pred, cb}, {cb_succ, cb}, {cand_ids, nk}, {cand_vals, nk},
                        {pred_ids, n * 4}, {gold_ids, opt(gold_ids, n * 4)}, {force, opt(force, n)},
                        {gold_logit, opt(gold_logit, n * 4)}};
    if (aliased(outs, ins)) return DFLASH2_ERR_ALIAS;
    return launched(launch_selector_tf(dtype, n_rows, hidden, vocab, rank, top_k, h, w_h, g, cb_pred,
                                       cb_succ, cand_ids, cand_vals, pred_ids, gold_ids, force,
                                       gold_logit, out_scores, out_best_ids, out_ce, out_valid,
                                       workspace, (hipStream_t)stream));
}

dflash2_status dflash2_selector_ce_backward(int dtype, int64_t n_rows, int32_t hidden, int32_t vocab,
                                            int32_t rank, int32_t top_k, const void *h, const void *w_h,
                                            const void *cb_pred, const void *cb_succ,
                                            const int32_t *cand_ids, const float *cand_vals,
                                            const int32_t *pred_ids, const int32_t *gold_ids,
                                            const uint8_t *force, const float *gold_logit,
                                            const float *grad_ce, float *grad_pred, float *grad_succ,
                                            float *grad_wh, float *out_ce, uint8_t *out_valid,
                                            void *workspace, size_t workspace_bytes, void *stream) {
    dflash2_status s = check_selector(dtype, n_rows, hidden, vocab, rank, top_k);
    if (s != DFLASH2_OK) return s;
    if (!h || !w_h || !cb_pred || !cb_succ || !cand_ids || !cand_vals || !pred_ids || !gold_ids || !grad_ce ||
        !grad_pred || !grad_succ || !grad_wh || !workspace)
        return DFLASH2_ERR_NULL;
    if (force && !gold_logit) return DFLASH2_ERR_NULL;
    // (row, slot) entries and the 2V + 1 per-target offsets are int32
    if (n_rows * (int64_t)(top_k + 1) > INT_MAX || 2 * (int64_t)vocab + 1 > INT_MAX) return DFLASH2_ERR_UNSUPPORTED;
    if (workspace_bytes <
        dflash2_workspace_bytes(DFLASH2_OP_SELECTOR_CE_BACKWARD, n_rows, hidden, vocab, rank, top_k))
        return DFLASH2_ERR_WORKSPACE;
    if (misaligned({h, w_h, cb_pred, cb_succ, cand_vals, gold_logit, grad_ce, grad_pred, grad_succ, grad_wh, out_ce,
                    workspace},
                   {cand_ids, pred_ids, gold_ids}))
        return DFLASH2_ERR_UNSUPPORTED;
    const size_t es = elem_size(dtype);
    const size_t cb = (size_t)vocab * rank * 4, wh = (size_t)rank * hidden * 4;
    const size_t n = (size_t)n_rows, nk = n * top_k;
    const Span outs[] = {{grad_pred, cb}, {grad_succ, cb}, {grad_wh, wh}, {out_ce, opt(out_ce, n * 4)},
                         {out_valid, opt(out_valid, n)}};
    const Span ins[] = {{h, n * hidden * es}, {w_h, (size_t)rank * hidden * es},
                        {cb_pred, (size_t)vocab * rank * es}, {cb_succ, (size_t)vocab * rank * es},
                        {cand_ids, nk * 4}, {cand_vals, nk * 4}, {pred_ids, n * 4}, {gold_ids, n * 4},
                        {force, opt(force, n)}, {gold_logit, opt(gold_logit, n * 4)}, {grad_ce, n * 4},
                        {workspace, workspace_bytes}};
    if (aliased(outs, ins)) return DFLASH2_ERR_ALIAS;
    return launched(launch_selector_ce_backward(dtype, n_rows, hidden, vocab, rank, top_k, h, w_h, cb_pred,
                                                cb_succ, cand_ids, cand_vals, pred_ids, gold_ids, force,
                                                gold_logit, grad_ce, grad_pred, grad_succ, grad_wh, out_ce,
                                                out_valid, workspace, (hipStream_t)stream));
}

dflash2_status dflash2_read_device_status(const void *workspace, void *stream) {
    if (!workspace) return DFLASH2_ERR_NULL;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DFLASH2_ERR_LAUNCH;
    uint32_t word = 0;
    if (hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return DFLASH2_ERR_LAUNCH;
    return (word & kStatusIdRange) ? DFLASH2_ERR_DEVICE_ID_RANGE : DFLASH2_OK;
}

}  // extern "C"
