// Candidate selector: S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)>.
//
// Both modes score with one routine, pair_tile: a 16 x 16 tile of transition
// terms sum_r B[cand, r] * (A[pred, r] * g[n, r]) on the float32 MFMA units,
// candidates on the rows and predecessors on the columns, the rank index
// visited in the same order.  The greedy walk scores every adjacent pair of a
// block at once and reduces each predecessor's row to its best successor, then
// one wave chases those pointers from the anchor; with many blocks (bf16) the
// walk instead follows the path, one position at a time against the previous
// pick only, with that pick in column 0 (selector_chase_kernel).  Teacher
// forcing places its one predecessor in column 0 of the same routine, so
// replaying a walk's own predecessors reproduces the walk's scores bit for bit.
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "gemv.hpp"
#include "launch.hpp"
#include "selector.hpp"

namespace dflash2 {

template <typename T, int NJ, bool SAMPLE>
__global__ __launch_bounds__(512) void selector_walk_kernel(
    const float *__restrict__ g, const T *__restrict__ A, const T *__restrict__ B,
    const int32_t *__restrict__ cand_ids, const float *__restrict__ cand_vals,
    const int32_t *__restrict__ anchors, int bs, int V, int r, int K, int32_t *__restrict__ path,
    float *__restrict__ path_score, uint32_t *__restrict__ status, float temperature, uint32_t k0, uint32_t k1) {
    extern __shared__ __align__(16) uint8_t wsm[];
    walk_block<T, NJ, SAMPLE>(blockIdx.x, wsm, g, A, B, cand_ids, cand_vals, anchors, bs, V, r, K, path,
                              path_score, status, temperature, k0, k1);
}

// ------------------------------------------------------------------ walk, one pick at a time
// With many blocks the pair walk is bound by its gathers: at every position
// it fetches the A rows of all K slots of C_{t-1}, though the path follows
// only one of them.  This greedy variant (bf16 codebooks) scores one step at
// a time.  For position t the workgroup copies the K successor rows of B, the
// context row and the single A row of the previous pick straight into LDS
// (global_load_lds, 1 KB per wave instruction): one round trip to memory per
// step and about half the pair walk's bytes.  Wave w then scores successor
// tile w with the predecessor in column 0 of pair_tiles, as teacher forcing
// does, so every score equals the pair walk's bit for bit and so does the path.
// LDS layout (ChaseLayout): candidate ids [bs][K] int; B rows, each r + 8
// elements apart when r is a multiple of 512 (the 16 rows a wave reads at one
// rank offset then fall in 16 different bank groups), else packed r apart in
// whole 1 KB copies (lanes past the last row fetch row 0's first chunk into
// the slack); the context row [r] float and the A row [r] bf16, each in whole
// 1 KB copies; the waves' best keys.
typedef __attribute__((address_space(3))) void chase_lds_t;
constexpr int kChaseThreads = 256;
constexpr int kChaseMinBlocks = 128;
constexpr size_t kChaseMaxLds = 96 * 1024;
struct ChaseLayout {
    int padded, bstride, b_copies, g_copies, a_copies;
    size_t b_off, g_off, a_off, key_off, total;
};
static ChaseLayout chase_layout(int bs, int K, int r) {
    ChaseLayout L;
    L.padded = r % 512 == 0;
    L.bstride = L.padded ? r + 8 : r;
    const size_t rowbytes = (size_t)r * 2;
    L.b_copies = L.padded ? K * (r / 512) : (int)(((size_t)K * rowbytes + 1023) / 1024);
    L.g_copies = (r + 255) / 256;
    L.a_copies = (r + 511) / 512;
    L.b_off = ((size_t)bs * K * 4 + 255) / 256 * 256;
    L.g_off = L.b_off + (L.padded ? (size_t)K * (rowbytes + 16) : (size_t)L.b_copies * 1024);
    L.g_off = (L.g_off + 255) / 256 * 256;
    L.a_off = L.g_off + (size_t)L.g_copies * 1024;
    L.key_off = L.a_off + (size_t)L.a_copies * 1024;
    L.total = L.key_off + 4 * 8;
    return L;
}

__global__ __launch_bounds__(kChaseThreads) void selector_chase_kernel(
    const float *__restrict__ g, const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const int32_t *__restrict__ cand_ids, const float *__restrict__ cand_vals, const int32_t *__restrict__ anchors,
    int bs, int V, int r, int K, ChaseLayout L, int32_t *__restrict__ path, float *__restrict__ path_score,
    uint32_t *__restrict__ status) {
    extern __shared__ __align__(16) uint8_t csm[];
    int32_t *ids = reinterpret_cast<int32_t *>(csm);
    uint8_t *bsm = csm + L.b_off, *gsm = csm + L.g_off, *asm_ = csm + L.a_off;
    uint64_t *keys = reinterpret_cast<uint64_t *>(csm + L.key_off);
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int blk = blockIdx.x, n_it = (K + 15) >> 4, rc = r >> 3;
    const size_t row0 = (size_t)blk * bs;
    const int anchor = anchors[blk];
    const bool anchor_ok = anchor >= 0 && anchor < V;
    if (!anchor_ok && tid == 0) flag_status(status, kStatusIdRange);
    for (int i = tid; i < bs * K; i += kChaseThreads) {
        const int id = cand_ids[row0 * K + i];
        const bool ok = id >= 0 && id < V;
        if (i >= K && !ok) flag_status(status, kStatusIdRange);  // positions 1.. are scored
        ids[i] = ok ? id : -1;
    }
    if (tid == 0) {
        path[row0] = anchor_ok ? anchor : -1;
        if (path_score) path_score[row0] = 0.f;
    }
    __syncthreads();
    int pid = anchor_ok ? anchor : -1;  // the previous pick (workgroup-uniform); -1 once the path has ended
    for (int t = 1; t < bs; ++t) {
        const size_t n = row0 + t;
        if (pid < 0) {
            if (tid == 0) {
                path[n] = -1;
                if (path_score) path_score[n] = __builtin_nanf("");
            }
            continue;
        }
        const int32_t *idt = ids + t * K;
        for (int k = wave; k < L.b_copies; k += kChaseThreads / 64) {
            int j, ch;
            uint8_t *dst;
            if (L.padded) {
                const int bpr = r / 512;
                j = k / bpr;
                ch = (k - j * bpr) * 64 + lane;
                dst = bsm + (size_t)j * (r * 2 + 16) + (size_t)(k - j * bpr) * 1024;
            } else {
                const int f = k * 64 + lane;
                j = f / rc;
                ch = f - j * rc;
                dst = bsm + (size_t)k * 1024;
            }
            int id = j < K ? idt[j] : -1;
            if (id < 0) id = 0, ch = 0;  // slack or an invalid slot: an in-bounds chunk that is never read
            __builtin_amdgcn_global_load_lds(B + (size_t)id * r + ch * 8, (chase_lds_t *)dst, 16, 0, 0);
        }
        for (int k = wave; k < L.g_copies; k += kChaseThreads / 64) {
            const int f = k * 64 + lane, ch = f < (r >> 2) ? f : 0;
            __builtin_amdgcn_global_load_lds(g + n * r + ch * 4, (chase_lds_t *)(gsm + k * 1024), 16, 0, 0);
        }
        for (int k = wave; k < L.a_copies; k += kChaseThreads / 64) {
            const int f = k * 64 + lane, ch = f < rc ? f : 0;
            __builtin_amdgcn_global_load_lds(A + (size_t)pid * r + ch * 8, (chase_lds_t *)(asm_ + k * 1024), 16, 0,
                                             0);
        }
        float uv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int jj = wave * 16 + 4 * q + i;
            uv[i] = (wave < n_it && jj < K) ? cand_vals[n * K + jj] : 0.f;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (wave < n_it) {
            const int j = wave * 16 + c;
            const int cid[1] = {(j < K && idt[j] >= 0) ? j : -1};
            f32x4 P[1];
            pair_tiles<uint16_t, 1>(reinterpret_cast<const uint16_t *>(asm_), reinterpret_cast<const uint16_t *>(bsm),
                                    reinterpret_cast<const float *>(gsm), c == 0 ? 0 : -1, cid, r, L.bstride, P);
            uint64_t local = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int jj = wave * 16 + 4 * q + i;
                const bool ok = c == 0 && jj < K && idt[jj] >= 0;
                const float s = jj < K ? uv[i] + P[0][i] : 0.f;
                const uint64_t key = ok ? make_key(s, (uint32_t)jj) : 0ull;
                local = key > local ? key : local;
            }
            uint64_t o = shfl_xor_u64(local, 16);
            local = o > local ? o : local;
            o = shfl_xor_u64(local, 32);
            local = o > local ? o : local;
            if (lane == 0) keys[wave] = local;
        }
        __syncthreads();
        uint64_t key = 0;
        for (int w = 0; w < n_it; ++w) key = keys[w] > key ? keys[w] : key;
        pid = key ? idt[key_id(key)] : -1;
        if (tid == 0) {
            path[n] = pid;
            if (path_score) path_score[n] = key ? key_val(key) : __builtin_nanf("");
        }
    }
}

// ------------------------------------------------------------------ teacher forcing
// One wave per row: the given predecessor sits in column 0 of pair_tile.
template <typename T>
__global__ __launch_bounds__(256) void selector_tf_kernel(
    const float *__restrict__ g, const T *__restrict__ A, const T *__restrict__ B,
    const int32_t *__restrict__ cand_ids, const float *__restrict__ cand_vals,
    const int32_t *__restrict__ pred_ids, const int32_t *__restrict__ gold_ids,
    const uint8_t *__restrict__ force, const float *__restrict__ gold_logit, long long N, int V, int r,
    int K, float *__restrict__ out_scores, int32_t *__restrict__ out_best, float *__restrict__ out_ce,
    uint8_t *__restrict__ out_valid, uint32_t *__restrict__ status) {
    extern __shared__ __align__(16) float gsm[];  // [4 waves][r]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const long long n = (long long)blockIdx.x * 4 + wave;
    if (n >= N) return;
    float *grow = gsm + wave * r;
    for (int i = lane; i < r / 4; i += 64)
        reinterpret_cast<float4 *>(grow)[i] = reinterpret_cast<const float4 *>(g + (size_t)n * r)[i];
    wave_lds_fence();
    const int c = lane & 15;
    const int p = pred_ids[n];
    const bool p_ok = p >= 0 && p < V;
    const int pid = (c == 0 && p_ok) ? p : -1;
    const int n_jt = (K + 15) / 16;
    // lane k (< K) ends up with the score of slot k
    float s = -__builtin_inff();
    bool mine_ok = false;
    const int qk = c >> 2, ik = lane & 3;
    for (int jt = 0; jt < n_jt; ++jt) {
        const int j = jt * 16 + c;
        int cid = j < K ? cand_ids[(size_t)n * K + j] : -1;
        const bool cok = j < K && cid >= 0 && cid < V;
        if (!cok) cid = -1;
        const f32x4 P = pair_tile<T>(A, B, grow, pid, cid, r);
        const float v0 = __shfl(P[0], 16 * qk), v1 = __shfl(P[1], 16 * qk);
        const float v2 = __shfl(P[2], 16 * qk), v3 = __shfl(P[3], 16 * qk);
        const float pk = ik == 0 ? v0 : ik == 1 ? v1 : ik == 2 ? v2 : v3;
        if ((lane >> 4) == jt && lane < K) {
            mine_ok = cok && p_ok;
            s = mine_ok ? cand_vals[(size_t)n * K + lane] + pk : __builtin_nanf("");
        }
    }
    if (lane < K) out_scores[(size_t)n * K + lane] = s;
    const uint64_t bestkey = wave_max_u64((lane < K && mine_ok) ? make_key(s, (uint32_t)lane) : 0ull);
    const bool all_ok = __all(lane >= K || mine_ok) != 0;
    if (!all_ok && lane == 0) flag_status(status, kStatusIdRange);
    if (lane == 0) out_best[n] = bestkey ? cand_ids[(size_t)n * K + key_id(bestkey)] : -1;
    if (!gold_ids) return;
    const int gid = gold_ids[n];
    const bool g_ok = gid >= 0 && gid < V;
    if (!g_ok && lane == 0) flag_status(status, kStatusIdRange);
    const int my_id = lane < K ? cand_ids[(size_t)n * K + lane] : -1;
    const unsigned long long hit = __ballot(lane < K && g_ok && my_id == gid);
    int kg = hit ? __ffsll(hit) - 1 : -1;
    if (kg < 0 && g_ok && force && force[n]) {
        const f32x4 P = pair_tile<T>(A, B, grow, pid, c == 0 ? gid : -1, r);
        const float sg = gold_logit[n] + __shfl(P[0], 0);
        kg = K - 1;
        if (lane == kg) s = sg;
    }
    const bool valid = kg >= 0 && all_ok;
    float ce = 0.f;
    if (valid) {
        const float m = wave_max_f32(lane < K ? s : -__builtin_inff());
        const float e = lane < K ? expf(s - m) : 0.f;
        const float sum = wave_sum_f32(e);
        ce = m + logf(sum) - __shfl(s, kg);
    }
    if (lane == 0) {
        if (out_ce) out_ce[n] = ce;
        if (out_valid) out_valid[n] = valid ? 1 : 0;
    }
}

// ------------------------------------------------------------------ host side

// The selector's context rows: the caller's g_in as given (then only the
// status word is cleared, by a one-thread kernel rather than a memset node),
// or g = h W_Hᵀ formed into the workspace after its status word.
__global__ void clear_status_kernel(uint32_t *status) { *status = 0u; }

static hipError_t context_rows(int dtype, int64_t N, int H, int r, const void *h, const void *w_h, const float *g_in,
                               void *workspace, const float **g, hipStream_t stream) {
    uint32_t *status = reinterpret_cast<uint32_t *>(workspace);
    if (g_in) {
        *g = g_in;
        hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, stream, status);
        return hipGetLastError();
    }
    float *gw = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(workspace) + kStatusBytes);
    *g = gw;
    return launch_context_proj(dtype, N, H, r, h, w_h, gw, status, stream);
}

hipError_t launch_selector_walk(int dtype, int n_blocks, int bs, int H, int V, int r, int K,
                                const void *h, const void *w_h, const float *g_in, const void *A, const void *B,
                                const int32_t *cand_ids, const float *cand_vals,
                                const int32_t *anchors, int32_t *path, float *path_score,
                                void *workspace, hipStream_t stream, const SampleParams *sample) {
    uint32_t *status = reinterpret_cast<uint32_t *>(workspace);
    const int64_t N = (int64_t)n_blocks * bs;
    const size_t lds = walk_lds_bytes(bs, K);
    const float *g = nullptr;
    hipError_t e = context_rows(dtype, N, H, r, h, w_h, g_in, workspace, &g, stream);
    if (e != hipSuccess) return e;
    const int n_it = (K + 15) / 16;
    const int items = bs >= 2 ? 1 + (bs - 2) * n_it : 1;
    int waves = items < 8 ? items : 8;
    const dim3 block(64 * waves);
    const float temp = sample ? sample->temperature : 1.f;
    const uint32_t k0 = sample ? (uint32_t)sample->seed : 0u, k1 = sample ? (uint32_t)(sample->seed >> 32) : 0u;
    auto launch = [&](auto kern, const auto *Ap, const auto *Bp) -> hipError_t {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3(n_blocks), block, lds, stream, g, Ap, Bp, cand_ids, cand_vals, anchors, bs, V,
                           r, K, path, path_score, status, temp, k0, k1);
        return hipGetLastError();
    };
    // one kernel per successor tile count (K <= 64) and mode
    auto pick = [&](const auto *Ap, const auto *Bp, auto samplec) -> hipError_t {
        using T = std::remove_cv_t<std::remove_pointer_t<decltype(Ap)>>;
        constexpr bool S = decltype(samplec)::value;
        return n_it == 1 ? launch(selector_walk_kernel<T, 1, S>, Ap, Bp)
               : n_it == 2 ? launch(selector_walk_kernel<T, 2, S>, Ap, Bp)
               : n_it == 3 ? launch(selector_walk_kernel<T, 3, S>, Ap, Bp)
                           : launch(selector_walk_kernel<T, 4, S>, Ap, Bp);
    };
    auto mode = [&](const auto *Ap, const auto *Bp) -> hipError_t {
        return sample ? pick(Ap, Bp, std::true_type{}) : pick(Ap, Bp, std::false_type{});
    };
    if (dtype == 0) return mode((const float *)A, (const float *)B);
    const ChaseLayout L = chase_layout(bs, K, r);
    if (!sample && n_blocks >= kChaseMinBlocks && bs >= 2 && L.total <= kChaseMaxLds) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(selector_chase_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.total);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(selector_chase_kernel, dim3(n_blocks), dim3(kChaseThreads), L.total, stream, g,
                           (const uint16_t *)A, (const uint16_t *)B, cand_ids, cand_vals, anchors, bs, V, r, K, L,
                           path, path_score, status);
        return hipGetLastError();
    }
    return mode((const uint16_t *)A, (const uint16_t *)B);
}

// ------------------------------------------------------------------ walk without a caller workspace
// The walk's workspace (status word, then the context rows g [N, r] float32)
// in a file-scope device array, for callers that cannot allocate.  Each GPU
// holds its own copy at its own address; host code never uses the array's
// name as a device address, only the address looked up here once per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex lock;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(lock);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_selector_tf(int dtype, int64_t N, int H, int V, int r, int K, const void *h,
                              const void *w_h, const float *g_in, const void *A, const void *B,
                              const int32_t *cand_ids,
                              const float *cand_vals, const int32_t *pred_ids,
                              const int32_t *gold_ids, const uint8_t *force,
                              const float *gold_logit, float *out_scores, int32_t *out_best,
                              float *out_ce, uint8_t *out_valid, void *workspace,
                              hipStream_t stream) {
    uint32_t *status = reinterpret_cast<uint32_t *>(workspace);
    const float *g = nullptr;
    hipError_t e = context_rows(dtype, N, H, r, h, w_h, g_in, workspace, &g, stream);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((N + 3) / 4);
    if (dtype == 0)
        hipLaunchKernelGGL(selector_tf_kernel<float>, dim3(grid), dim3(256), (size_t)4 * r * 4, stream, g,
                           (const float *)A, (const float *)B, cand_ids, cand_vals, pred_ids, gold_ids,
                           force, gold_logit, (long long)N, V, r, K, out_scores, out_best, out_ce,
                           out_valid, status);
    else
        hipLaunchKernelGGL(selector_tf_kernel<uint16_t>, dim3(grid), dim3(256), (size_t)4 * r * 4, stream, g,
                           (const uint16_t *)A, (const uint16_t *)B, cand_ids, cand_vals, pred_ids,
                           gold_ids, force, gold_logit, (long long)N, V, r, K, out_scores, out_best,
                           out_ce, out_valid, status);
    return hipGetLastError();
}

}  // namespace dflash2
