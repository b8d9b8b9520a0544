// Unary LM-head logits over the full vocabulary with a fused per-row top-K.
//
// U[n, v] = <h[n], w_lm[v]> is formed tile by tile on the MFMA units and
// filtered into per-row sorted candidate lists in LDS; logits never reach HBM.
// Each workgroup emits one sorted list of K keys per row for its slice of the
// vocabulary, and topk_merge_kernel merges the slices.  A key orders
// candidates by value, then by lower id (see make_key), so the result does not
// depend on how the vocabulary was split.
#include "common.hpp"
#include "gemm.hpp"
#include "launch.hpp"

namespace dflash2 {

// Merge `n_lists` descending lists of K keys (list c starts at src + c*stride)
// into the top K, by one wave: every lane tracks the heads of the lists
// lane, lane + 64, ...; each round the wave takes the largest head.  Lane k
// returns the k-th key of the result (0 where fewer than K keys exist).
template <int MAXL>
__device__ uint64_t wave_merge_lists(const uint64_t *src, int n_lists, int stride, int K) {
    const int l = lane_id();
    int ptr[MAXL];
    uint64_t head[MAXL];
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < MAXL; ++j) {
        const int c = l + 64 * j;
        ptr[j] = 0;
        head[j] = c < n_lists ? src[(size_t)c * stride] : 0ull;
        best = head[j] > best ? head[j] : best;
    }
    uint64_t mine = 0;
    for (int k = 0; k < K; ++k) {
        const uint64_t w = wave_max_u64(best);
        if (l == k) mine = w;
        if (w == 0) break;
        if (best == w) {  // keys are unique: exactly one lane owns the winner
            best = 0;
#pragma unroll
            for (int j = 0; j < MAXL; ++j) {
                if (head[j] == w) {
                    ++ptr[j];
                    head[j] = ptr[j] < K ? src[(size_t)(l + 64 * j) * stride + ptr[j]] : 0ull;
                }
                best = head[j] > best ? head[j] : best;
            }
        }
    }
    return mine;
}

// Bitonic sort, descending, of 128 keys held two per lane (element 2*lane+h).
__device__ __forceinline__ void bitonic128_desc(uint64_t &x0, uint64_t &x1) {
    const int l = lane_id();
#pragma unroll
    for (int k = 2; k <= 128; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j == 1) {
                const bool desc = ((2 * l) & k) == 0;
                const uint64_t hi = x0 > x1 ? x0 : x1, lo = x0 > x1 ? x1 : x0;
                x0 = desc ? hi : lo;
                x1 = desc ? lo : hi;
            } else {
                const int lm = j >> 1;
                const uint64_t y0 = shfl_xor_u64(x0, lm), y1 = shfl_xor_u64(x1, lm);
                const bool lower = (l & lm) == 0;
                const bool d0 = ((2 * l) & k) == 0, d1 = ((2 * l + 1) & k) == 0;
                const bool m0 = d0 == lower, m1 = d1 == lower;
                x0 = m0 ? (x0 > y0 ? x0 : y0) : (x0 > y0 ? y0 : x0);
                x1 = m1 ? (x1 > y1 ? x1 : y1) : (x1 > y1 ? y1 : x1);
            }
        }
    }
}

// Insert every key of this lane's `key` that beats the row's threshold into
// the wave-held list `cur` (one entry per lane in lanes < K).
__device__ __forceinline__ void insert_survivors(uint64_t &cur, uint64_t &thr, uint64_t key, int K) {
    unsigned long long mask = __ballot(key > thr);
    while (mask) {
        const int src = __ffsll((unsigned long long)mask) - 1;
        mask &= mask - 1;
        const uint64_t k = shfl_u64(key, src);
        cur = sorted_insert(cur, k, K);
        thr = shfl_u64(cur, K - 1);
    }
}

// ---------------------------------------------------------------- streaming
//
// At most 8 rows.  Every wave owns a contiguous run of 16-row vocabulary
// tiles and streams each tile's rows of w_lm through MFMA (A = h from LDS).
// Lane (n = l % 16, q = l / 16) holds the logits of vocabulary row
// tile*16 + n for rows 4q .. 4q+3.  Each wave keeps its own sorted list per
// row in LDS; the workgroup merges its waves' lists at the end.
template <typename T, int NW>
__global__ __launch_bounds__(64 * NW) void lmhead_stream_kernel(
    const T *__restrict__ h, const T *__restrict__ w, int M, int H, int V, int K, int n_tiles,
    int tiles_per_wave, const int32_t *__restrict__ gold, float *__restrict__ gold_logit,
    uint64_t *__restrict__ partial, uint32_t *__restrict__ status) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int KC = 16 / (int)sizeof(T);
    const int S = H / kstep_elems<T>();
    uint4 *afrag = reinterpret_cast<uint4 *>(smem);
    uint64_t *lists = reinterpret_cast<uint64_t *>(smem + (size_t)S * 32 * 16);  // [NW][8][K]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    if (blockIdx.x == 0 && threadIdx.x == 0 && status) *status = 0u;

    load_afrag<T>(afrag, h, M, H);
    for (int i = threadIdx.x; i < NW * 8 * K; i += blockDim.x) lists[i] = 0ull;
    __syncthreads();

    uint64_t *mylists = lists + wave * 8 * K;
    const int n = lane & 15, q = lane >> 4;
    int grow[4];
    uint64_t thr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = 4 * q + e;
        grow[e] = (gold && row < M) ? gold[row] : -1;
        thr[e] = 0ull;
    }
    const int gw = blockIdx.x * NW + wave;
    const int t0 = gw * tiles_per_wave;
    const int t1 = min(t0 + tiles_per_wave, n_tiles);
    for (int t = t0; t < t1; ++t) {
        const int v = t * 16 + n;
        const T *brow = w + (size_t)min(v, V - 1) * H + q * KC;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        stream_accumulate<T>(acc, afrag, brow, 0, S);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 4 * q + e;
            const bool ok = row < M && v < V;
            const uint64_t key = ok ? make_key(acc[e], (uint32_t)v) : 0ull;
            if (ok && grow[e] == v) gold_logit[row] = acc[e];
            unsigned long long mask = __ballot(key > thr[e]);
            while (mask) {
                const int src = __ffsll((unsigned long long)mask) - 1;
                mask &= mask - 1;
                const uint64_t k = shfl_u64(key, src);
                const int r = 4 * (src >> 4) + e;
                uint64_t *L = mylists + r * K;
                uint64_t cur = lane < K ? L[lane] : 0ull;
                cur = sorted_insert(cur, k, K);
                if (lane < K) L[lane] = cur;
                const uint64_t tail = shfl_u64(cur, K - 1);
                if (4 * q + e == r) thr[e] = tail;
            }
        }
    }
    __syncthreads();
    for (int row = wave; row < M; row += NW) {
        const uint64_t key = wave_merge_lists<(NW + 63) / 64>(lists + row * K, NW, 8 * K, K);
        if (lane < K) partial[((size_t)row * gridDim.x + blockIdx.x) * K + lane] = key;
    }
}

// ---------------------------------------------------------------- tiled
//
// Many rows.  Workgroup (slab, mt) owns rows [128 mt, 128 mt + 128) and the
// vocabulary tiles of its slab; each 128 x 128 logit tile goes through LDS,
// and wave w merges the new values of rows w, w + 4, ... into their lists
// (bitonic sort for the first tile, threshold-filtered insertion after).
template <typename T>
__global__ __launch_bounds__(256) void lmhead_tiled_kernel(
    const T *__restrict__ h, const T *__restrict__ w, int M, int H, int V, int K, int n_vtiles,
    const int32_t *__restrict__ gold, float *__restrict__ gold_logit, uint64_t *__restrict__ partial,
    uint32_t *__restrict__ status) {
    using Cfg = TiledCfg<T, 128, 128>;
    constexpr int BIG = Cfg::STAGE_BYTES > Cfg::CTILE_BYTES ? Cfg::STAGE_BYTES : Cfg::CTILE_BYTES;
    extern __shared__ __align__(16) uint8_t smem[];
    float *ctile = reinterpret_cast<float *>(smem);
    uint64_t *lists = reinterpret_cast<uint64_t *>(smem + BIG);  // [128][K]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int slab = blockIdx.x, n_slabs = gridDim.x, mt = blockIdx.y;
    const int m0 = mt * Cfg::BM;
    if (slab == 0 && mt == 0 && threadIdx.x == 0 && status) *status = 0u;
    const int vt0 = (int)((long long)slab * n_vtiles / n_slabs);
    const int vt1 = (int)((long long)(slab + 1) * n_vtiles / n_slabs);
    for (int i = threadIdx.x; i < Cfg::BM * K; i += blockDim.x) lists[i] = 0ull;

    for (int vt = vt0; vt < vt1; ++vt) {
        const int v0 = vt * Cfg::BN;
        f32x4 acc[Cfg::TM][Cfg::TN];
        tiled_mainloop<T, Cfg>(
            acc, smem,
            [&](int i) -> const T * { const int r = m0 + i; return r < M ? h + (size_t)r * H : nullptr; },
            [&](int j) -> const T * { const int v = v0 + j; return v < V ? w + (size_t)v * H : nullptr; },
            H);
        __syncthreads();
        tiled_store_c<Cfg>(ctile, acc);
        __syncthreads();
        for (int r = wave; r < Cfg::BM; r += 4) {
            const int gr = m0 + r;
            if (gr >= M) break;
            uint64_t *L = lists + r * K;
            const int va = v0 + lane, vb = v0 + 64 + lane;
            const float fa = ctile[r * Cfg::CSTRIDE + lane], fb = ctile[r * Cfg::CSTRIDE + 64 + lane];
            uint64_t ka = va < V ? make_key(fa, (uint32_t)va) : 0ull;
            uint64_t kb = vb < V ? make_key(fb, (uint32_t)vb) : 0ull;
            if (gold) {
                const int g = gold[gr];
                if (g == va && va < V) gold_logit[gr] = fa;
                if (g == vb && vb < V) gold_logit[gr] = fb;
            }
            if (vt == vt0) {
                // element 2l+h after the sort is the (2l+h)-th best of the tile
                uint64_t x0 = ka, x1 = kb;
                bitonic128_desc(x0, x1);
                if (2 * lane < K) L[2 * lane] = x0;
                if (2 * lane + 1 < K) L[2 * lane + 1] = x1;
            } else {
                uint64_t cur = lane < K ? L[lane] : 0ull;
                uint64_t thr = shfl_u64(cur, K - 1);
                insert_survivors(cur, thr, ka, K);
                insert_survivors(cur, thr, kb, K);
                if (lane < K) L[lane] = cur;
            }
        }
        __syncthreads();
    }
    for (int r = wave; r < Cfg::BM; r += 4) {
        const int gr = m0 + r;
        if (gr >= M) break;
        if (lane < K) partial[((size_t)gr * n_slabs + slab) * K + lane] = lists[r * K + lane];
    }
}

// ---------------------------------------------------------------- merge
// One wave per row: merge the row's per-slab lists into the final top-K.
__global__ __launch_bounds__(256) void topk_merge_kernel(const uint64_t *__restrict__ partial, int M,
                                                         int n_lists, int K, int V,
                                                         int32_t *__restrict__ out_ids,
                                                         float *__restrict__ out_vals,
                                                         const int32_t *__restrict__ gold,
                                                         float *__restrict__ gold_logit,
                                                         uint32_t *__restrict__ status) {
    const int lane = lane_id();
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const uint64_t key = wave_merge_lists<16>(partial + (size_t)row * n_lists * K, n_lists, K, K);
    if (lane < K) {
        out_ids[(size_t)row * K + lane] = key ? (int32_t)key_id(key) : -1;
        out_vals[(size_t)row * K + lane] = key ? key_val(key) : -__builtin_inff();
    }
    if (gold && lane == 0) {
        const int g = gold[row];
        if (g < 0 || g >= V) {
            gold_logit[row] = __builtin_nanf("");
            flag_status(status, kStatusIdRange);
        }
    }
}

// ---------------------------------------------------------------- host side

LmheadPlan plan_lmhead(int dtype, int64_t M, int H, int V, int K) {
    LmheadPlan p{};
    const int es = dtype == 0 ? 4 : 2;
    const size_t stream_lds = (size_t)(H / (4 * (16 / es))) * 32 * 16 + (size_t)8 * 8 * K * 8;
    if (M <= kStreamMaxRows && stream_lds <= 160 * 1024) {
        p.streaming = true;
        p.nw = 8;
        const int n_tiles = (V + 15) / 16;
        const int target_waves = 256 * 16;  // 256 CUs x 16 resident waves
        p.tiles_per_wave = (n_tiles + target_waves - 1) / target_waves;
        const int n_waves = (n_tiles + p.tiles_per_wave - 1) / p.tiles_per_wave;
        p.grid_x = (n_waves + p.nw - 1) / p.nw;
        p.grid_y = 1;
        p.n_lists = p.grid_x;
        p.n_tiles = n_tiles;
        p.lds = stream_lds;
    } else {
        p.streaming = false;
        const int n_mt = (int)((M + 127) / 128);
        const int n_vt = (V + 127) / 128;
        int slabs = (512 + n_mt - 1) / n_mt;
        slabs = slabs < 1 ? 1 : slabs;
        slabs = slabs > n_vt ? n_vt : slabs;
        slabs = slabs > 1024 ? 1024 : slabs;
        p.grid_x = slabs;
        p.grid_y = n_mt;
        p.n_lists = slabs;
        p.n_tiles = n_vt;
        const size_t stage = (size_t)(128 + 128) * (8 * 16 + 16);
        const size_t ctile = (size_t)128 * (128 + 4) * 4;
        p.lds = (stage > ctile ? stage : ctile) + (size_t)128 * K * 8;
    }
    p.partial_bytes = (size_t)M * p.n_lists * K * 8;
    return p;
}

template <typename T, class F>
static hipError_t set_lds(F *kernel, size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <typename T>
static hipError_t run_lmhead(const LmheadPlan &p, int64_t M, int H, int V, int K, const void *h,
                             const void *w, const int32_t *gold, int32_t *out_ids, float *out_vals,
                             float *gold_logit, uint64_t *partial, uint32_t *status,
                             hipStream_t stream) {
    hipError_t e;
    if (p.streaming) {
        auto kern = lmhead_stream_kernel<T, 8>;
        if ((e = set_lds<T>(kern, p.lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(p.grid_x), dim3(64 * 8), p.lds, stream, (const T *)h,
                           (const T *)w, (int)M, H, V, K, p.n_tiles, p.tiles_per_wave, gold,
                           gold_logit, partial, status);
    } else {
        auto kern = lmhead_tiled_kernel<T>;
        if ((e = set_lds<T>(kern, p.lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(p.grid_x, p.grid_y), dim3(256), p.lds, stream, (const T *)h,
                           (const T *)w, (int)M, H, V, K, p.n_tiles, gold, gold_logit, partial,
                           status);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream,
                       partial, (int)M, p.n_lists, K, V, out_ids, out_vals, gold, gold_logit, status);
    return hipGetLastError();
}

hipError_t launch_unary_topk(int dtype, int64_t M, int H, int V, int K, const void *h, const void *w,
                             const int32_t *gold, int32_t *out_ids, float *out_vals,
                             float *gold_logit, void *workspace, hipStream_t stream) {
    const LmheadPlan p = plan_lmhead(dtype, M, H, V, K);
    uint32_t *status = reinterpret_cast<uint32_t *>(workspace);
    uint64_t *partial = reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(workspace) + kStatusBytes);
    if (dtype == 0)
        return run_lmhead<float>(p, M, H, V, K, h, w, gold, out_ids, out_vals, gold_logit, partial, status, stream);
    return run_lmhead<uint16_t>(p, M, H, V, K, h, w, gold, out_ids, out_vals, gold_logit, partial, status, stream);
}

}  // namespace dflash2
