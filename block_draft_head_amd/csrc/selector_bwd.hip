// Selector CE backward: gradients of sum_n w[n] CE[n] (the teacher-forced CE
// of the candidate selector) with respect to its own parameters, the
// predecessor codebook A, the successor codebook B and the context
// projection W_H.  The selector's inputs (the backbone hidden states and the
// unary logits) are constants here ([verl PR] "Selector training objective":
// its inputs are detached; [SpecForge] "Selector objective and schedule":
// the stop-gradient switch).
//
// With S'[n, k] = U'[n, k] + <A[p_n] * g[n], B[c'_k]> over the forced set C'
// and d[n, k] = w[n] (softmax(S'[n])_k - [k = k_gold]):
//   dB[c'_k] += d[n, k] (A[p_n] * g[n])
//   dA[p_n]  += g[n] * v[n],  v[n] = sum_k d[n, k] B[c'_k]
//   dg[n]     = A[p_n] * v[n]
//   dW_H     += sum_n dg[n] (outer) h[n]
//
// Kernels, after the context projection g = W_H h:
//  * ce_grad_rows_kernel: one wave per row; recomputes the forced-set scores,
//    the softmax and d; writes ag[n] = A[p_n] * g[n], gv[n] = g[n] * v[n]
//    (over g[n]) and dg[n]; emits one entry per (row, slot): slot k < K
//    targets successor row c'_k with weight d[n, k], slot K the predecessor
//    row p_n with weight 1; and counts the entries of every target.
//  * a counting sort of the entries by target (tile sums, tile prefixes,
//    offsets, placement), then ce_scatter_kernel: one wave per chunk of a
//    target's entries sums their weighted ag / gv rows and adds the sum into
//    the gradient row.  Each gradient row is read and written once instead
//    of taking one float atomic per contribution and element; only a target
//    with more than kSegChunk entries (a token in many rows' candidate sets)
//    adds its chunks atomically.
//  * dW_H += dg^T h, a contraction over the rows: for bf16 inputs on the bf16
//    MFMA with dg split into bf16 high and low parts (wh_grad_bf16_kernel),
//    for float32 inputs on the float32 MFMA (wh_grad_kernel); the eight waves
//    of a workgroup split the rows of one 64 x 64 tile and reduce their
//    partial tiles through LDS.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace dflash2 {

namespace {

// 4 consecutive codebook / activation elements as float32.
template <typename T> __device__ __forceinline__ f32x4 load4(const T *p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <> __device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

__device__ __forceinline__ float readlane_f32(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Float add into ordinary (coarse-grained) device memory; the return value
// is unused, so this is the returnless hardware atomic.
__device__ __forceinline__ void atomic_add(float *p, float v) { unsafeAtomicAdd(p, v); }

}  // namespace

// ------------------------------------------------------------------ per-row kernel
// One wave per row.  Lane l holds elements 4 l + 256 c .. +3 of the rank
// dimension for chunk c < NC (r <= 256 NC).  Lane k < K holds slot k's id,
// score and d.  dg goes to dg_row (float32 inputs) or to the wave's LDS row
// dgs_row (bf16 inputs, packed by the workgroup afterwards).
template <typename T, int NC>
__device__ __forceinline__ void ce_grad_row(
    long long n, float *g, const T *__restrict__ A, const T *__restrict__ B, const int32_t *__restrict__ cand_ids,
    const float *__restrict__ cand_vals, const int32_t *__restrict__ pred_ids,
    const int32_t *__restrict__ gold_ids, const uint8_t *__restrict__ force,
    const float *__restrict__ gold_logit, const float *__restrict__ grad_ce, int V, int r, int K,
    float *__restrict__ ag_out, float *__restrict__ dg, float *dgs_row, int32_t *__restrict__ tgt,
    float *__restrict__ wgt, int32_t *__restrict__ counts, float *__restrict__ out_ce,
    uint8_t *__restrict__ out_valid, uint32_t *__restrict__ status) {
    const int lane = lane_id();
    const size_t nk = (size_t)n * K, e0 = (size_t)n * (K + 1);
    int my_id = lane < K ? cand_ids[nk + lane] : 0;
    float my_u = lane < K ? cand_vals[nk + lane] : 0.f;
    const int p = pred_ids[n], gold = gold_ids[n];
    const bool ids_ok = __all(lane >= K || (my_id >= 0 && my_id < V)) != 0 && p >= 0 && p < V && gold >= 0 &&
                        gold < V;
    if (!ids_ok && lane == 0) flag_status(status, kStatusIdRange);
    const unsigned long long hit = __ballot(lane < K && my_id == gold);
    int kg = -1;
    if (ids_ok) {
        if (hit) {
            kg = __ffsll(hit) - 1;
        } else if (force && force[n]) {
            kg = K - 1;  // the gold replaces the weakest slot, with its own logit
            if (lane == kg) {
                my_id = gold;
                my_u = gold_logit[n];
            }
        }
    }
    float *dg_row = dg + (size_t)n * r;
    auto put_dg = [&](int e, f32x4 v) {
        *reinterpret_cast<f32x4 *>((sizeof(T) == 2 ? dgs_row : dg_row) + e) = v;
    };
    if (kg < 0) {  // excluded row: no CE, no gradient, no entries
        for (int e = 4 * lane; e < r; e += 256) put_dg(e, f32x4{0.f, 0.f, 0.f, 0.f});
        for (int j = lane; j <= K; j += 64) tgt[e0 + j] = -1;
        if (lane == 0) {
            if (out_ce) out_ce[n] = 0.f;
            if (out_valid) out_valid[n] = 0;
        }
        return;
    }
    const T *a_row = A + (size_t)p * r;
    float *g_row = g + (size_t)n * r;  // read here, then overwritten by gv
    f32x4 ag[NC], gr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int e = 4 * lane + 256 * c;
        gr[c] = e < r ? *reinterpret_cast<const f32x4 *>(g_row + e) : f32x4{0.f, 0.f, 0.f, 0.f};
        ag[c] = e < r ? load4<T>(a_row + e) * gr[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // scores over the forced set
    float s = -__builtin_inff();
    for (int k = 0; k < K; ++k) {
        const T *b_row = B + (size_t)__builtin_amdgcn_readlane(my_id, k) * r;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = 4 * lane + 256 * c;
            if (e < r) part += dot4(ag[c], load4<T>(b_row + e));
        }
        const float pair = wave_sum_f32(part);
        if (lane == k) s = my_u + pair;
    }
    const float m = wave_max_f32(s);
    const float ex = lane < K ? expf(s - m) : 0.f;
    const float sum = wave_sum_f32(ex);
    const float w = grad_ce[n];
    const float d = lane < K ? w * (ex / sum - (lane == kg ? 1.f : 0.f)) : 0.f;
    if (lane == 0) {
        if (out_ce) out_ce[n] = m + logf(sum) - readlane_f32(s, kg);
        if (out_valid) out_valid[n] = 1;
    }
    // v = sum_k d_k B[c'_k]
    f32x4 v[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) v[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
        const T *b_row = B + (size_t)__builtin_amdgcn_readlane(my_id, k) * r;
        const float dk = readlane_f32(d, k);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int e = 4 * lane + 256 * c;
            if (e < r) v[c] += dk * load4<T>(b_row + e);
        }
    }
    float *ag_row = ag_out + (size_t)n * r;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int e = 4 * lane + 256 * c;
        if (e < r) {
            put_dg(e, load4<T>(a_row + e) * v[c]);
            *reinterpret_cast<f32x4 *>(g_row + e) = gr[c] * v[c];
            *reinterpret_cast<f32x4 *>(ag_row + e) = ag[c];
        }
    }
    // entries: slot k -> successor row c'_k, slot K -> predecessor row (target V + p)
    if (lane < K) {
        tgt[e0 + lane] = my_id;
        wgt[e0 + lane] = d;
        atomicAdd(counts + my_id, 1);
    }
    if (lane == 0) {
        tgt[e0 + K] = V + p;
        wgt[e0 + K] = 1.f;
        atomicAdd(counts + V + p, 1);
    }
}

// Eight rows per workgroup.  bf16: the rows' dg meet in LDS and go out as
// their truncated bf16 high part and the bf16 of the remainder, packed 8 rows
// deep (element (n, i) at ((n / 8) r + i) 8 + n % 8 of each half; rows past N
// are zero), one 16-byte store per rank element and half.
template <typename T, int NC>
__global__ __launch_bounds__(512) void ce_grad_rows_kernel(
    float *g, const T *__restrict__ A, const T *__restrict__ B, const int32_t *__restrict__ cand_ids,
    const float *__restrict__ cand_vals, const int32_t *__restrict__ pred_ids,
    const int32_t *__restrict__ gold_ids, const uint8_t *__restrict__ force,
    const float *__restrict__ gold_logit, const float *__restrict__ grad_ce, long long N, int V, int r, int K,
    float *__restrict__ ag_out, float *__restrict__ dg, int32_t *__restrict__ tgt, float *__restrict__ wgt,
    int32_t *__restrict__ counts, float *__restrict__ out_ce, uint8_t *__restrict__ out_valid,
    uint32_t *__restrict__ status) {
    extern __shared__ __align__(16) float dgs[];  // bf16: [8][r]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const long long n = (long long)blockIdx.x * 8 + wave;
    float *my_dgs = dgs + (size_t)wave * r;
    if (n < N) {
        ce_grad_row<T, NC>(n, g, A, B, cand_ids, cand_vals, pred_ids, gold_ids, force, gold_logit, grad_ce, V, r,
                           K, ag_out, dg, my_dgs, tgt, wgt, counts, out_ce, out_valid, status);
    } else if constexpr (sizeof(T) == 2) {
        for (int e = 4 * lane; e < r; e += 256) *reinterpret_cast<f32x4 *>(my_dgs + e) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (sizeof(T) == 2) {
        __syncthreads();
        uint16_t *dg_hi = reinterpret_cast<uint16_t *>(dg), *dg_lo = dg_hi + (size_t)(N + 7) / 8 * 8 * r;
        for (int i = threadIdx.x; i < r; i += blockDim.x) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int p = 0; p < 8; p += 2) {
                const float v0 = dgs[(size_t)p * r + i], v1 = dgs[(size_t)(p + 1) * r + i];
                const uint32_t h0 = __float_as_uint(v0) & 0xffff0000u, h1 = __float_as_uint(v1) & 0xffff0000u;
                const uint32_t l0 = __float_as_uint(v0 - __uint_as_float(h0)) & 0xffff0000u;
                const uint32_t l1 = __float_as_uint(v1 - __uint_as_float(h1)) & 0xffff0000u;
                hw[p / 2] = (h0 >> 16) | h1;
                lw[p / 2] = (l0 >> 16) | l1;
            }
            const size_t at = ((size_t)blockIdx.x * r + i) * 8;
            *reinterpret_cast<uint4 *>(dg_hi + at) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            *reinterpret_cast<uint4 *>(dg_lo + at) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
    }
}

// ------------------------------------------------------------------ counting sort by target
// Offsets over C = 2V + 1 counters (the last one stays 0, so offsets[2V] is
// the number of entries), in tiles of kScanTile: per-tile sums, an exclusive
// scan of those sums, then each tile's exclusive scan plus its prefix.  The
// last pass also zeroes the counters, which the placement reuses as cursors.
constexpr int kScanThreads = 256, kScanPer = kScanTile / kScanThreads;  // 16 counters per thread

__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t *__restrict__ p, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = 0;
}

// Exclusive scan of one value per thread over a 256-thread workgroup; every
// thread of the workgroup must call it.  `total` gets the sum of all values.
__device__ __forceinline__ int block_exclusive_scan(int x, int *lds4, int &total) {
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    int inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) lds4[wave] = inc;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int t = lds4[w];
        if (w < wave) before += t;
        total += t;
    }
    __syncthreads();
    return before + inc - x;
}

__global__ __launch_bounds__(256) void scan_tile_sums_kernel(const int32_t *__restrict__ counts, int C,
                                                             int32_t *__restrict__ tile_sum) {
    __shared__ int lds4[4];
    const long long base = (long long)blockIdx.x * kScanTile + threadIdx.x * kScanPer;
    int x = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i)
        if (base + i < C) x += counts[base + i];
    int total;
    block_exclusive_scan(x, lds4, total);
    if (threadIdx.x == 0) tile_sum[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the tile sums, in place.
__global__ __launch_bounds__(256) void scan_tile_prefix_kernel(int32_t *__restrict__ tile_sum, int n_tiles) {
    __shared__ int lds4[4];
    int carry = 0;
    for (int b = 0; b < n_tiles; b += 256) {
        const int i = b + (int)threadIdx.x;
        const int x = i < n_tiles ? tile_sum[i] : 0;
        int total;
        const int ex = block_exclusive_scan(x, lds4, total);
        if (i < n_tiles) tile_sum[i] = carry + ex;
        carry += total;
    }
}

// own_prefix: tile_prefix holds the tile sums, and each workgroup adds up
// those before its own tile (used for at most kScanOwnPrefixTiles tiles)
constexpr int kScanOwnPrefixTiles = 1024;
__global__ __launch_bounds__(256) void scan_apply_kernel(int32_t *__restrict__ counts, int C,
                                                         const int32_t *__restrict__ tile_prefix,
                                                         int32_t *__restrict__ offsets, int own_prefix) {
    __shared__ int lds4[4];
    const long long base = (long long)blockIdx.x * kScanTile + threadIdx.x * kScanPer;
    int v[kScanPer], x = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        v[i] = base + i < C ? counts[base + i] : 0;
        x += v[i];
    }
    int total;
    int prefix;
    if (own_prefix) {
        int part = 0;
        for (int b = threadIdx.x; b < (int)blockIdx.x; b += kScanThreads) part += tile_prefix[b];
        int all;
        block_exclusive_scan(part, lds4, all);
        prefix = all;
    } else {
        prefix = tile_prefix[blockIdx.x];
    }
    int run = block_exclusive_scan(x, lds4, total) + prefix;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i)
        if (base + i < C) {
            offsets[base + i] = run;
            counts[base + i] = 0;
            run += v[i];
        }
}

__global__ __launch_bounds__(256) void place_entries_kernel(const int32_t *__restrict__ tgt, long long E,
                                                            const int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ cursor, int32_t *__restrict__ src) {
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    const int t = tgt[e];
    if (t < 0) return;
    src[offsets[t] + atomicAdd(cursor + t, 1)] = (int32_t)e;
}

// ------------------------------------------------------------------ segmented scatter
// Wave p looks at sorted entry p; it works only if p starts a chunk of
// kSegChunk entries of its target's segment, and then sums that chunk.
constexpr int kSegChunk = 64;

template <int NC>
__global__ __launch_bounds__(256) void ce_scatter_kernel(const int32_t *__restrict__ src,
                                                         const int32_t *__restrict__ tgt,
                                                         const float *__restrict__ wgt,
                                                         const int32_t *__restrict__ offsets,
                                                         const float *__restrict__ ag, const float *__restrict__ gv,
                                                         long long E, int V, int r, int K, float *__restrict__ dA,
                                                         float *__restrict__ dB) {
    const int lane = lane_id();
    const long long p = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= E || p >= offsets[2 * V]) return;
    const int t = tgt[src[p]];
    const int start = offsets[t], end = offsets[t + 1];
    if ((p - start) % kSegChunk != 0) return;
    const int len = (int)min((long long)kSegChunk, (long long)end - p);
    const int my_e = lane < len ? src[p + lane] : 0;
    const float my_w = lane < len ? wgt[my_e] : 0.f;
    const bool succ = t < V;
    const float *rows = succ ? ag : gv;
    f32x4 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < len; ++j) {
        const int e = __builtin_amdgcn_readlane(my_e, j);
        const float w = readlane_f32(my_w, j);
        const float *row = rows + (size_t)(e / (K + 1)) * r;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int x = 4 * lane + 256 * c;
            if (x < r) acc[c] += w * *reinterpret_cast<const f32x4 *>(row + x);
        }
    }
    float *out = succ ? dB + (size_t)t * r : dA + (size_t)(t - V) * r;
    const bool shared = end - start > kSegChunk;  // other waves add chunks of the same row
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int x = 4 * lane + 256 * c;
        if (x >= r) continue;
        if (shared) {
#pragma unroll
            for (int i = 0; i < 4; ++i) atomic_add(out + x + i, acc[c][i]);
        } else {
            *reinterpret_cast<f32x4 *>(out + x) = *reinterpret_cast<const f32x4 *>(out + x) + acc[c];
        }
    }
}

// ------------------------------------------------------------------ dW_H += dg^T h
// One workgroup of 8 waves per 64 (rank) x 64 (hidden) tile of dW_H; wave w
// takes row quads w, w + 8, ...  MFMA 16x16x4 f32, 4 x 4 tiles per wave:
// lane l feeds rank rows i0 + 4 (l % 16) + s (s = 0..3, one float4 of dg) and
// hidden columns j0 + 4 (l % 16) + t (t = 0..3, one 4-element load of h) at
// row 4 quad + l / 16, so tile (s, t) holds
// C[i0 + 16 (l / 16) + 4 q + s][j0 + 4 (l % 16) + t] in register q of lane l.
// The eight partial tiles meet in LDS and their sum is added into dW_H.
constexpr int kWhTile = 64, kWhWaves = 8;
constexpr int kWhSteps = 4;  // row quads in flight per wave
constexpr size_t kWhLds = (size_t)kWhWaves * kWhTile * kWhTile * 4;

template <typename T>
__global__ __launch_bounds__(512) void wh_grad_kernel(const float *__restrict__ dg, const T *__restrict__ h, int N,
                                                       int H, int r, float *__restrict__ dW) {
    extern __shared__ __align__(16) float part[];  // [wave][64][64]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int i0 = blockIdx.x * kWhTile, j0 = blockIdx.y * kWhTile;
    const int q16 = lane & 15, kq = lane >> 4;
    const int ia = i0 + 4 * q16, jb = j0 + 4 * q16;
    const bool a_ok = ia < r;  // r % 8 == 0: a float4 group is wholly in or out
    const int n_quads = (N + 3) / 4;
    f32x4 acc[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[s][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 a_buf[kWhSteps], b_buf[kWhSteps];
    auto fetch = [&](int quad, f32x4 &a, f32x4 &b) {
        const int n = 4 * quad + kq;
        const bool ok = n < N;
        const int nn = ok ? n : 0;  // stays in bounds; the value is zeroed
        a = a_ok ? *reinterpret_cast<const f32x4 *>(dg + (size_t)nn * r + ia) : f32x4{0.f, 0.f, 0.f, 0.f};
        b = load4<T>(h + (size_t)nn * H + jb);
        if (!ok) a = f32x4{0.f, 0.f, 0.f, 0.f};
    };
#pragma unroll
    for (int u = 0; u < kWhSteps; ++u) fetch(wave + kWhWaves * u, a_buf[u], b_buf[u]);
    for (int q0 = wave; q0 < n_quads; q0 += kWhWaves * kWhSteps) {
#pragma unroll
        for (int u = 0; u < kWhSteps; ++u) {
            const f32x4 a = a_buf[u], b = b_buf[u];
            fetch(q0 + kWhWaves * (u + kWhSteps), a_buf[u], b_buf[u]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[s][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[t], acc[s][t], 0, 0, 0);
        }
    }
    float *mine = part + (size_t)wave * kWhTile * kWhTile;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int il = 16 * kq + 4 * q + s;
            *reinterpret_cast<f32x4 *>(mine + il * kWhTile + 4 * q16) =
                f32x4{acc[s][0][q], acc[s][1][q], acc[s][2][q], acc[s][3][q]};
        }
    __syncthreads();
    // thread x sums outputs 8x .. 8x + 7 (one row, 8 columns) over the waves
    const int il = (8 * (int)threadIdx.x) / kWhTile, jl = (8 * (int)threadIdx.x) % kWhTile;
    f32x4 s0{0.f, 0.f, 0.f, 0.f}, s1{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWhWaves; ++w) {
        const float *pw = part + (size_t)w * kWhTile * kWhTile + il * kWhTile + jl;
        s0 += *reinterpret_cast<const f32x4 *>(pw);
        s1 += *reinterpret_cast<const f32x4 *>(pw + 4);
    }
    if (i0 + il < r) {
        float *out = dW + (size_t)(i0 + il) * H + j0 + jl;
        *reinterpret_cast<f32x4 *>(out) = *reinterpret_cast<const f32x4 *>(out) + s0;
        *reinterpret_cast<f32x4 *>(out + 4) = *reinterpret_cast<const f32x4 *>(out + 4) + s1;
    }
}

// bf16 operands: dW_H += (dg_hi + dg_lo)^T h on the bf16 MFMA 16x16x32, k =
// 32 rows per step.  Lane l (m = l % 16, q = l / 16) feeds rank rows
// i0 + 4 m + s of tile s (one 16-byte load of 8 packed rows per half) and
// hidden columns j0 + 4 m + t of tile t: it loads 4 columns of each of its 8
// rows (8 bytes each) and rearranges them into one 8-row fragment per column.
// Tile (s, t) then holds C[i0 + 4 (4 q + e) + s][j0 + 4 m + t] in register e.
// The eight waves of a workgroup take the 32-row steps in turn and sum their
// partial tiles in LDS.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__global__ __launch_bounds__(512) void wh_grad_bf16_kernel(const uint16_t *__restrict__ dg_hi,
                                                           const uint16_t *__restrict__ dg_lo,
                                                           const uint16_t *__restrict__ h, int N, int H, int r,
                                                           float *__restrict__ dW) {
    extern __shared__ __align__(16) float part[];  // [wave][64][64]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int i0 = blockIdx.x * kWhTile, j0 = blockIdx.y * kWhTile;
    const int m = lane & 15, q = lane >> 4;
    const int ia = i0 + 4 * m, jb = j0 + 4 * m;
    const bool a_ok = ia < r;  // r % 8 == 0: the 4 rows of a lane are wholly in or out
    const int n_steps = (N + 31) / 32;
    f32x4 acc[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[s][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    struct Ops {
        uint4 hi[4], lo[4];
        uint2 hv[8];
    };
    auto fetch = [&](int step, Ops &o) {
        const int g8 = step * 4 + q;  // this lane group's 8-row group
        const bool ok = step < n_steps && g8 < (N + 7) / 8;
        const size_t abase = ((size_t)(ok ? g8 : 0) * r + (a_ok ? ia : 0)) * 8;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            o.hi[s] = (ok && a_ok) ? *reinterpret_cast<const uint4 *>(dg_hi + abase + 8 * s) : make_uint4(0u, 0u, 0u, 0u);
            o.lo[s] = (ok && a_ok) ? *reinterpret_cast<const uint4 *>(dg_lo + abase + 8 * s) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int n = g8 * 8 + p;
            const bool rok = ok && n < N;  // rows past N: dg is zero there, h is not read
            o.hv[p] = rok ? *reinterpret_cast<const uint2 *>(h + (size_t)n * H + jb) : make_uint2(0u, 0u);
        }
    };
    Ops cur, nxt;
    fetch(wave, cur);
    for (int step = wave; step < n_steps; step += kWhWaves) {
        fetch(step + kWhWaves, nxt);
        uint4 b[4];  // column t of the 8 rows, rows in pairs
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint2 x = cur.hv[2 * d], y = cur.hv[2 * d + 1];
            reinterpret_cast<uint32_t *>(&b[0])[d] = pack_lo16(x.x, y.x);
            reinterpret_cast<uint32_t *>(&b[1])[d] = pack_hi16(x.x, y.x);
            reinterpret_cast<uint32_t *>(&b[2])[d] = pack_lo16(x.y, y.y);
            reinterpret_cast<uint32_t *>(&b[3])[d] = pack_hi16(x.y, y.y);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.hi[s]),
                                                                    __builtin_bit_cast(bf16x8, b[t]), acc[s][t], 0, 0, 0);
                acc[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.lo[s]),
                                                                    __builtin_bit_cast(bf16x8, b[t]), acc[s][t], 0, 0, 0);
            }
        cur = nxt;
    }
    float *mine = part + (size_t)wave * kWhTile * kWhTile;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int il = 4 * (4 * q + e) + s;
            *reinterpret_cast<f32x4 *>(mine + il * kWhTile + 4 * m) =
                f32x4{acc[s][0][e], acc[s][1][e], acc[s][2][e], acc[s][3][e]};
        }
    __syncthreads();
    const int il = (8 * (int)threadIdx.x) / kWhTile, jl = (8 * (int)threadIdx.x) % kWhTile;
    f32x4 s0{0.f, 0.f, 0.f, 0.f}, s1{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWhWaves; ++w) {
        const float *pw = part + (size_t)w * kWhTile * kWhTile + il * kWhTile + jl;
        s0 += *reinterpret_cast<const f32x4 *>(pw);
        s1 += *reinterpret_cast<const f32x4 *>(pw + 4);
    }
    if (i0 + il < r) {
        float *out = dW + (size_t)(i0 + il) * H + j0 + jl;
        *reinterpret_cast<f32x4 *>(out) = *reinterpret_cast<const f32x4 *>(out) + s0;
        *reinterpret_cast<f32x4 *>(out + 4) = *reinterpret_cast<const f32x4 *>(out + 4) + s1;
    }
}

// ------------------------------------------------------------------ host side

hipError_t launch_selector_ce_backward(int dtype, int64_t N, int H, int V, int r, int K, const void *h,
                                       const void *w_h, const void *A, const void *B,
                                       const int32_t *cand_ids, const float *cand_vals,
                                       const int32_t *pred_ids, const int32_t *gold_ids,
                                       const uint8_t *force, const float *gold_logit, const float *grad_ce,
                                       float *grad_pred, float *grad_succ, float *grad_wh, float *out_ce,
                                       uint8_t *out_valid, void *workspace, hipStream_t stream) {
    const CeBwdLayout L = ce_bwd_layout(N, V, r, K);
    uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
    uint32_t *status = reinterpret_cast<uint32_t *>(ws);
    float *g = reinterpret_cast<float *>(ws + L.g);
    float *ag = reinterpret_cast<float *>(ws + L.ag);
    float *dg = reinterpret_cast<float *>(ws + L.dg);
    float *wgt = reinterpret_cast<float *>(ws + L.wgt);
    int32_t *tgt = reinterpret_cast<int32_t *>(ws + L.tgt);
    int32_t *src = reinterpret_cast<int32_t *>(ws + L.src);
    int32_t *counts = reinterpret_cast<int32_t *>(ws + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    int32_t *tiles = reinterpret_cast<int32_t *>(ws + L.tiles);
    const long long E = (long long)N * (K + 1);
    const int C = 2 * V + 1;
    const int n_tiles = (C + kScanTile - 1) / kScanTile;

    const long long zgrid = (C + 255) / 256 < 1024 ? (C + 255) / 256 : 1024;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)zgrid), dim3(256), 0, stream, counts, (long long)C);
    hipError_t e = launch_context_proj(dtype, N, H, r, h, w_h, g, status, stream);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((N + 7) / 8);
    const int nc = (r + 255) / 256;
    auto rows = [&](const auto *Ap, const auto *Bp) -> hipError_t {
        using T = std::remove_cv_t<std::remove_pointer_t<decltype(Ap)>>;
        const size_t lds = sizeof(T) == 2 ? (size_t)8 * r * 4 : 0;
        auto go = [&](auto kern) {
            hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (err != hipSuccess) return err;
            hipLaunchKernelGGL(kern, dim3(grid), dim3(512), lds, stream, g, Ap, Bp, cand_ids, cand_vals, pred_ids,
                               gold_ids, force, gold_logit, grad_ce, (long long)N, V, r, K, ag, dg, tgt, wgt, counts,
                               out_ce, out_valid, status);
            return hipGetLastError();
        };
        return nc <= 1 ? go(ce_grad_rows_kernel<T, 1>)
               : nc <= 2 ? go(ce_grad_rows_kernel<T, 2>)
               : nc <= 4 ? go(ce_grad_rows_kernel<T, 4>)
               : nc <= 8 ? go(ce_grad_rows_kernel<T, 8>)
                         : go(ce_grad_rows_kernel<T, 16>);
    };
    e = dtype == 0 ? rows((const float *)A, (const float *)B) : rows((const uint16_t *)A, (const uint16_t *)B);
    if (e != hipSuccess) return e;

    hipLaunchKernelGGL(scan_tile_sums_kernel, dim3(n_tiles), dim3(256), 0, stream, counts, C, tiles);
    const int own = n_tiles <= kScanOwnPrefixTiles ? 1 : 0;
    if (!own) hipLaunchKernelGGL(scan_tile_prefix_kernel, dim3(1), dim3(256), 0, stream, tiles, n_tiles);
    hipLaunchKernelGGL(scan_apply_kernel, dim3(n_tiles), dim3(256), 0, stream, counts, C, tiles, offsets, own);
    hipLaunchKernelGGL(place_entries_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, stream, tgt, E,
                       offsets, counts, src);
    auto scatter = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, stream, src, tgt, wgt, offsets, ag, g,
                           E, V, r, K, grad_pred, grad_succ);
    };
    if (nc <= 1) scatter(ce_scatter_kernel<1>);
    else if (nc <= 2) scatter(ce_scatter_kernel<2>);
    else if (nc <= 4) scatter(ce_scatter_kernel<4>);
    else if (nc <= 8) scatter(ce_scatter_kernel<8>);
    else scatter(ce_scatter_kernel<16>);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const dim3 wgrid((unsigned)((r + kWhTile - 1) / kWhTile), (unsigned)(H / kWhTile));
    auto wh = [&](auto kern, const auto *hp) -> hipError_t {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWhLds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, wgrid, dim3(64 * kWhWaves), kWhLds, stream, dg, hp, (int)N, H, r, grad_wh);
        return hipGetLastError();
    };
    if (dtype == 0) return wh(wh_grad_kernel<float>, (const float *)h);
    const uint16_t *dg_hi = reinterpret_cast<const uint16_t *>(dg);
    const uint16_t *dg_lo = dg_hi + (size_t)(N + 7) / 8 * 8 * r;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(wh_grad_bf16_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWhLds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(wh_grad_bf16_kernel, wgrid, dim3(64 * kWhWaves), kWhLds, stream, dg_hi, dg_lo,
                       (const uint16_t *)h, (int)N, H, r, grad_wh);
    return hipGetLastError();
}

}  // namespace dflash2
