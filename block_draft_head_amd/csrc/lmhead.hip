// Unary LM-head logits over the full vocabulary with a fused per-row top-K.
//
// U[n, v] = <h[n], w_lm[v]> is formed tile by tile on the MFMA units and
// filtered into per-row candidate lists in LDS; logits never reach HBM.
// Each workgroup emits one sorted list of K keys per row for its slice of the
// vocabulary, and topk_merge_kernel merges the slices.  A key orders
// candidates by value, then by lower id (see make_key), so the result does not
// depend on how the vocabulary was split.
#include <atomic>
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "gemm.hpp"
#include "launch.hpp"
#include "selector.hpp"

namespace dflash2 {

constexpr int kMergeChunk = 512;

// ---------------------------------------------------------------- unary transform, log-sum-exp
// U' = softcap(mult * U), softcap(x) = cap tanh(x / cap) (cap 0: off).  The
// transform is increasing, so the kernels select on raw logits and apply it
// to the K values; the log-sum-exp runs over the transformed logits.
struct UnaryEpi {
    float mult, cap;
    float2 *lse_part;  // per (row, list): running max and sum of exp(U' - max); null: not wanted
};
__device__ __forceinline__ float unary_transform(float x, float mult, float cap) {
    x *= mult;
    return cap > 0.f ? cap * tanhf(x / cap) : x;
}
// (m, s) += one transformed logit t
__device__ __forceinline__ void lse_add(float &m, float &s, float t) {
    const float mn = fmaxf(m, t);
    s = s * __expf(m - mn) + __expf(t - mn);
    m = mn;
}
// (m, s) += (m2, s2)
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    if (mn == -__builtin_inff()) return;  // both empty
    s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
    m = mn;
}
// (m, s) over the 16 lanes of this lane's quarter (lanes with equal lane / 16)
__device__ __forceinline__ void lse_merge16(float &m, float &s) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) lse_merge(m, s, __shfl_xor(m, o), __shfl_xor(s, o));
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
// At most 8 rows (decode).  One workgroup per CU owns a balanced contiguous
// range of 16-row vocabulary tiles; its waves pull tiles from an LDS counter
// and stream each tile's rows of w_lm through MFMA (A = h, from LDS in
// fragment order).  A ring of P 16-byte loads per lane runs across tile
// boundaries, so the next tile is already in flight while a tile's logits are
// filtered.  Lane (n = l % 16, q = l / 16) holds the logits of vocabulary row
// tile*16 + n for rows 4q .. 4q+3.  Each wave appends the logits above its
// per-row threshold to an LDS candidate buffer (ballot compaction, no sort)
// and shrinks a buffer only when it fills; the workgroup reduces its waves'
// lists at the end.
constexpr int kStreamWGs = 256;       // one per CU of an MI355X
constexpr int kStreamMinLds = 81 * 1024;  // > half the CU's LDS: one workgroup per CU
constexpr int kCandCap = 128;             // candidate slots per wave and row

// Shrinks a wave's candidate buffer B (n keys, K < n <= 128) in place and
// returns the row's new filter threshold (a key passes when it is greater).
// The buffer need not hold a sorted top K, only every key that can still be
// among the row's K best: a bit search over the keys' high words (the order
// image of the value) takes the first cut that keeps between K and about 2K
// of them (at most 64), and since at least K keys reach the cut, no key below
// it can be among the K best.  That costs a handful of ballots; only keys
// tied in their high word past 64 fall back to the exact selection.
__device__ __forceinline__ uint64_t shrink_candidates(uint64_t *B, int &n, int K, uint64_t *scratch) {
    const int lane = lane_id();
    uint64_t k[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) k[i] = lane + 64 * i < n ? B[lane + 64 * i] : 0ull;
    // empty slots have high word 0, below every cut
    const uint32_t h0 = (uint32_t)(k[0] >> 32), h1 = (uint32_t)(k[1] >> 32);
    const int lim = K <= 16 ? 32 : K <= 32 ? 2 * K : 64;
    uint32_t v = 0;
    int c = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t t = v | (1u << b);
        const int ct = __popcll(__ballot(h0 >= t)) + __popcll(__ballot(h1 >= t));
        if (ct >= K) {
            v = t;
            c = ct;
            if (ct <= lim) break;
        }
    }
    if (c >= K && c <= 64) {
        const bool p0 = h0 >= v, p1 = h1 >= v;
        const unsigned long long m0 = __ballot(p0), m1 = __ballot(p1);
        const int c0 = __popcll(m0);
        wave_lds_fence();
        if (p0) B[lanes_below(m0)] = k[0];
        if (p1) B[c0 + lanes_below(m1)] = k[1];
        wave_lds_fence();
        n = c;
        return ((uint64_t)v << 32) - 1ull;
    }
    const uint64_t top = wave_topk<2>(k, K, scratch);
    if (lane < K) B[lane] = top;
    n = K;
    return readlane_u64(top, K - 1);
}

template <typename T, int NW, int P, bool LSE>
__global__ __launch_bounds__(64 * NW) void lmhead_stream_kernel(
    const T *__restrict__ h, const T *__restrict__ w, int M, int H, int V, int K, int n_tiles,
    const int32_t *__restrict__ gold, float *__restrict__ gold_logit, uint64_t *__restrict__ partial,
    uint32_t *__restrict__ status, UnaryEpi ue) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int KC = 16 / (int)sizeof(T);
    constexpr int KS = 4 * KC;
    const int S = H / KS;
    uint4 *afrag = reinterpret_cast<uint4 *>(smem);
    uint64_t *bufs = reinterpret_cast<uint64_t *>(smem + (size_t)S * 32 * 16);  // [NW][8][kCandCap]
    uint64_t *scratch = bufs + NW * 8 * kCandCap;                                // [NW][128]
    int *cnts = reinterpret_cast<int *>(scratch + NW * 128);                     // [NW][8]
    int *qctr = cnts + NW * 8;
    float2 *lse_sm = reinterpret_cast<float2 *>(smem + (size_t)S * 32 * 16 + (size_t)NW * (8 * kCandCap + 128) * 8 +
                                                (size_t)NW * 8 * 4 + 16);  // [NW][8]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    if (blockIdx.x == 0 && threadIdx.x == 0 && status) *status = 0u;

    load_afrag<T>(afrag, h, M, H);
    if (threadIdx.x == 0) *qctr = 0;
    __syncthreads();

    const int t0 = (int)((long long)blockIdx.x * n_tiles / gridDim.x);
    const int t1 = (int)((long long)(blockIdx.x + 1) * n_tiles / gridDim.x);
    auto grab = [&]() -> int {
        int v = 0;
        if (lane == 0) v = atomicAdd(qctr, 1);
        return t0 + __shfl(v, 0);
    };
    uint64_t *mybuf = bufs + wave * 8 * kCandCap;
    const int n = lane & 15, q = lane >> 4;
    int grow[4];
    uint64_t thr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = 4 * q + e;
        grow[e] = (gold && row < M) ? gold[row] : -1;
        thr[e] = 0ull;
    }
    int cnt[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) cnt[r] = 0;
    float lm[4], ls[4];  // log-sum-exp of rows 4 q + e over this lane's logits
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lm[e] = -__builtin_inff();
        ls[e] = 0.f;
    }
    uint64_t *myscratch = scratch + wave * 128;
    // Shrink row r's candidates and raise its threshold.
    auto compact = [&](int r) {
        const uint64_t nt = shrink_candidates(mybuf + r * kCandCap, cnt[r], K, myscratch);
        if (q == (r >> 2)) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e == (r & 3)) thr[e] = nt;
        }
    };
    auto row_ptr = [&](int t) -> const T * {
        return w + (size_t)min(t * 16 + n, V - 1) * H + q * KC;
    };

    int t = grab();
    if (t < t1) {
        uint4 ring[P];
        const T *cur = row_ptr(t);
#pragma unroll
        for (int i = 0; i < P; ++i) ring[i] = *reinterpret_cast<const uint4 *>(cur + (size_t)i * KS);
        while (true) {
            const int tn = grab();
            const T *nxt = row_ptr(tn < t1 ? tn : t);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < S; s0 += P) {
                const bool same = s0 + P < S;
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    const uint4 b = ring[i];
                    if (same)
                        ring[i] = *reinterpret_cast<const uint4 *>(cur + (size_t)(s0 + P + i) * KS);
                    else if (tn < t1)
                        ring[i] = *reinterpret_cast<const uint4 *>(nxt + (size_t)i * KS);
                    mma16<T>(acc, afrag_get(afrag, s0 + i, lane), b);
                }
            }
            const int v = t * 16 + n;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 4 * q + e;
                const bool ok = row < M && v < V;
                const uint64_t key = ok ? make_key(acc[e], (uint32_t)v) : 0ull;
                if (ok && grow[e] == v) gold_logit[row] = acc[e];
                if constexpr (LSE) {
                    if (ok) lse_add(lm[e], ls[e], unary_transform(acc[e], ue.mult, ue.cap));
                }
                const bool pass = key > thr[e];
                const unsigned long long mask = __ballot(pass);
                const int c0 = __popcll(mask & 0xffffull), c1 = __popcll(mask & 0xffff0000ull);
                if (pass) {
                    const int pos = lanes_below(mask) - (q ? c0 : 0);
                    mybuf[row * kCandCap + (q ? cnt[4 + e] : cnt[e]) + pos] = key;
                }
                cnt[e] += c0;
                cnt[4 + e] += c1;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (cnt[r] > kCandCap - 16) compact(r);
            if (tn >= t1) break;
            t = tn;
            cur = nxt;
        }
    }
    if (lane < 8) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (lane == r) cnts[wave * 8 + r] = cnt[r];
    }
    if constexpr (LSE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lse_merge16(lm[e], ls[e]);
            if (n == 0 && 4 * q + e < 8) lse_sm[wave * 8 + 4 * q + e] = make_float2(lm[e], ls[e]);
        }
    }
    __syncthreads();
    // the workgroup's list per row: top K over every wave's candidates
    for (int row = wave; row < M; row += NW) {
        if constexpr (LSE) {
            if (lane == 0) {
                float m = -__builtin_inff(), sm = 0.f;
                for (int ww = 0; ww < NW; ++ww) lse_merge(m, sm, lse_sm[ww * 8 + row].x, lse_sm[ww * 8 + row].y);
                ue.lse_part[(size_t)row * gridDim.x + blockIdx.x] = make_float2(m, sm);
            }
        }
        constexpr int R = 2 * NW;
        uint64_t k[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int ww = i >> 1, slot = lane + 64 * (i & 1);
            k[i] = slot < cnts[ww * 8 + row] ? bufs[(ww * 8 + row) * kCandCap + slot] : 0ull;
        }
        const uint64_t top = wave_topk<R>(k, K, myscratch);
        if (lane < K) partial[((size_t)row * gridDim.x + blockIdx.x) * K + lane] = top;
    }

}

// ---------------------------------------------------------------- streaming through LDS (bf16)
//
// The same job as lmhead_stream_kernel, with the weight rows reaching the
// MFMAs through LDS: each wave copies 2 KB blocks (16 vocabulary rows x 64 k)
// from HBM straight into a private ring of kDmaRing LDS blocks with
// non-temporal global_load_lds_dwordx4 (each instruction reads 8 whole
// 128-byte lines) and reads its B fragments from there.  Streaming a weight
// this way reads HBM about 12% faster than loading it into registers (the
// register loads read 64 bytes of 16 rows each, which the non-temporal
// policy cannot serve well).  Row r of a block holds 16-byte chunk c at
// position c ^ (r & 7): the 8 lanes of a fragment read hit 8 bank groups.
//
// Work split: workgroup b owns an equal contiguous range of vocabulary rows,
// cut into 16-row tiles.  Its waves form groups of KS that share a tile, wave
// p of a group multiplying k-blocks [p Q, p Q + Q) (Q = H / 64 / KS): the
// workgroup then reads its rows close together, which streams HBM a few
// percent faster than one 16-row tile per wave.  A group sums its partial
// tiles through LDS (one barrier per tile) and each wave filters the logits
// of the rows 4 q + e with e % KS == p into its own candidate buffers.
//
// One wave runs per SIMD, so every instruction of the block loop is issue
// time that the copies cannot hide behind another wave: the loop is unrolled
// over one turn of the ring (a wave's share of a tile holds whole turns) so
// that ring slots, fragment registers and block offsets are compile-time
// immediates, and fragments are read ahead of their MFMAs so that LDS
// latency is not on the path either.  A wave waits only for its own copies
// (counted waits), and the group barrier waits for LDS alone, so the copy
// stream never drains inside the kernel.
constexpr int kDmaWaves = 4;
constexpr int kDmaRing = 8;        // 2 KB blocks per wave
constexpr int kDmaCandCap = 96;    // candidate slots per wave and row (>= top-K limit + 16)
constexpr int kDmaAhead = 1;       // fragments are read this many blocks before their MFMAs
constexpr int kDmaLead = 5;        // a block is copied this many blocks before its MFMAs (a deeper lead streams slower)

// K split of a tile among the waves that share it: the largest of 4, 2, 1
// whose share of H holds whole ring turns (0: none does)
inline int dma_ksplit(int H) {
    return H % (64 * kDmaRing * 4) == 0 ? 4 : H % (64 * kDmaRing * 2) == 0 ? 2 : H % (64 * kDmaRing) == 0 ? 1 : 0;
}

inline size_t dma_lds_bytes(int H, int KS) {
    // (plus the log-sum-exp of each wave's rows: kDmaWaves x 8 float2)
    // A fragments (each K share followed by its first two blocks again, read
    // ahead across a tile boundary), rings, candidate buffers, two sets of
    // partial tiles (K split only), merge scratch, counts
    return (size_t)(H / 64 + 2 * KS) * 1024 + (size_t)kDmaWaves * kDmaRing * 2048 +
           (size_t)kDmaWaves * (8 / KS) * kDmaCandCap * 8 + (KS > 1 ? (size_t)2 * kDmaWaves * 1024 : 0) +
           (size_t)kDmaWaves * 128 * 8 + (size_t)kDmaWaves * 8 * 4 + (size_t)kDmaWaves * 8 * 8 + 16;
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>) in order
template <int N, typename F> __device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A fragments of h (bf16, at most 8 rows) in load_afrag's order, except that
// 64-k block b of share p = b / Q sits at block p (Q + 2) + b % Q, and each
// share is followed by its first two blocks again.
__device__ void load_afrag_shares(uint4 *afrag, const uint16_t *__restrict__ A, int M, int H, int Q) {
    for (int i = threadIdx.x; i < H; i += blockDim.x) {
        const int m = i & 7, q = (i >> 3) & 3, s = i >> 5;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (m < M) v = *reinterpret_cast<const uint4 *>(A + (size_t)m * H + (size_t)(4 * s + q) * 8);
        const int b = i >> 6, bl = b % Q;
        const int dst = ((b / Q) * (Q + 2) + bl) * 64 + (i & 63);
        afrag[dst] = v;
        if (bl < 2) afrag[dst + Q * 64] = v;
    }
}

// The decode head: the context projection's rows stream after the
// vocabulary's through the same kernel (their tiles write g instead of
// candidates), so the selector adds no pass over h of its own.
struct DecodeFuse {
    const uint16_t *wh;  // [r, H], or null: no context projection
    int r;
    float *g;            // [M, r] float32 context rows
};

template <int KS, bool LSE, bool FUSED>
__global__ __launch_bounds__(64 * kDmaWaves) void lmhead_dma_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ w, int M, int H, int V, int K,
    const int32_t *__restrict__ gold, float *__restrict__ gold_logit, uint64_t *__restrict__ partial,
    uint32_t *__restrict__ status, UnaryEpi ue, DecodeFuse fu, uint64_t *__restrict__ heads) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NW = kDmaWaves, NB = kDmaRing, CAP = kDmaCandCap, AH = kDmaAhead, LD = kDmaLead;
    constexpr int G = NW / KS;   // wave groups
    constexpr int OWN = 8 / KS;  // rows whose candidates one wave keeps
    static_assert(NW % KS == 0 && 4 % KS == 0, "a K split divides the waves and the rows of a lane");
    static_assert(AH >= 1 && AH <= 2 && AH < LD && LD <= NB && NB % 4 == 0,
                  "at most two tile-wrapping fragment reads, copies ahead of them, four fragment buffers");
    const int Q = H / 64 / KS;  // blocks of one K share, a multiple of NB
    uint4 *afrag = reinterpret_cast<uint4 *>(smem);
    uint8_t *rings = smem + (size_t)(H / 64 + 2 * KS) * 1024;                        // [NW][NB][2048]
    uint64_t *bufs = reinterpret_cast<uint64_t *>(rings + (size_t)NW * NB * 2048);   // [NW][OWN][CAP]
    f32x4 *parts = reinterpret_cast<f32x4 *>(bufs + NW * OWN * CAP);                // [2][NW][64]
    uint64_t *scratch = reinterpret_cast<uint64_t *>(parts + (KS > 1 ? 2 * NW * 64 : 0));  // [NW][128]
    int *cnts = reinterpret_cast<int *>(scratch + NW * 128);                         // [NW][OWN]
    float2 *lse_sm = reinterpret_cast<float2 *>(cnts + NW * 8);                     // [NW][8]
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gi = wave / KS, kp = wave % KS;
    if (blockIdx.x == 0 && threadIdx.x == 0 && status) *status = 0u;

    load_afrag_shares(afrag, h, M, H, Q);
    __syncthreads();

    // workgroup b owns 16-row tiles [t0, t1) of the vocabulary's tiles, then
    // (fused decode head) the context projection's tiles
    // (the fused head's fields as scalars: read through the struct, which the
    // lambdas below would capture by address, they would count as divergent)
    const uint16_t *const wh = FUSED ? fu.wh : nullptr;
    const int rk = FUSED && wh ? fu.r : 0;
    float *const gout = FUSED ? fu.g : nullptr;
    const int tiles_v = (V + 15) / 16;
    const int n_all = tiles_v + (rk + 15) / 16;
    const int t0 = (int)((long long)blockIdx.x * n_all / gridDim.x);
    const int ntile = (int)((long long)(blockIdx.x + 1) * n_all / gridDim.x) - t0;
    // group gi takes tiles gi, gi + G, ...; with a K split every wave runs the
    // same number of iterations (they meet at barriers), a group with one
    // tile fewer repeating its last tile with no row valid
    const int nit = KS == 1 ? (ntile - gi + G - 1) / G : (ntile + G - 1) / G;
    uint64_t *mybuf = bufs + wave * OWN * CAP;
    const int n = lane & 15, q = lane >> 4;
    int grow[4];
    uint64_t thr[4];
    float gval[4];
    bool ghit[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = 4 * q + e;
        grow[e] = (gold && row < M) ? gold[row] : -1;
        thr[e] = 0ull;
        gval[e] = 0.f;
        ghit[e] = false;
    }
    // take the gold ids now: the compiler, which does not count the copies,
    // would otherwise wait for every load in flight at their first use
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" ::"v"(grow[e]));
    int cnt[OWN];
#pragma unroll
    for (int r = 0; r < OWN; ++r) cnt[r] = 0;
    float lm[4], ls[4];  // log-sum-exp of rows 4 q + e (e % KS == kp) over this lane's logits
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lm[e] = -__builtin_inff();
        ls[e] = 0.f;
    }
    uint64_t *myscratch = scratch + wave * 128;

    // copies: lane L of copy j of a block fills row 8 j + L / 8, position L % 8,
    // with the row's chunk (L % 8) ^ (row & 7).  Rows past the range read row 0
    // instead (a few lines per partial tile, L2 hits).
    uint8_t *ring = rings + (size_t)wave * NB * 2048;
    const uint32_t ring_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t *)ring;
    const int crow = lane >> 3, cpos = lane & 7;
    // byte offsets of this lane's chunk of its two copy rows in the tile of
    // iteration `it`, first block of the wave's K share; returns the matrix
    // the tile's rows belong to (w_lm, or w_h past the vocabulary's tiles)
    auto tile_rows = [&](int it, uint32_t (&ro)[2]) -> const uint16_t * {
        const int gt = t0 + min(it * G + gi, ntile - 1);
        const bool ht = FUSED && gt >= tiles_v;
        const int row0 = ht ? (gt - tiles_v) * 16 : gt * 16, lim = ht ? rk : V;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = 8 * j + crow, vrow = row0 + row;
            ro[j] = (uint32_t)((cpos ^ (row & 7)) * 16 + kp * Q * 128) +
                    (vrow < lim ? (uint32_t)vrow * (uint32_t)H * 2u : 0u);
        }
        // (wave-uniform; read from the first lane so that the copies can take
        // it as their scalar base whatever the compiler proves about it)
        return readfirstlane_ptr(ht ? wh : w);
    };
    // block `src` + I of the rows `ro` into ring slot I.  The instruction's
    // immediate offset moves the LDS destination as well as the global
    // address, so M0 is set that much lower.  s_nop 4: the wait states that
    // an SGPR or M0 written just before needs (the compiler adds none to
    // inline assembly).  `held` are the B fragments last
    // read from the slot: naming them as inputs makes the compiler wait for
    // those reads before the copy overwrites it.
    auto copy_block = [&](const uint32_t (&ro)[2], const uint16_t *src_in, auto slotc, const uint4 (&held)[2]) {
        constexpr int I = decltype(slotc)::value;
        // with two matrices in the stream the base is chosen per tile; it is
        // wave-uniform, and read from the first lane again here so that the
        // copy can take it as its scalar base whatever the compiler proves
        const uint16_t *src = FUSED ? readfirstlane_ptr(src_in) : src_in;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t dst = ring_lds + (uint32_t)(I * (2048 - 128) + j * 1024);
            asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 offset:%2 nt" ::"v"(ro[j]), "s"(src), "n"(I * 128),
                         "{m0}"(dst), "v"(__builtin_bit_cast(big::u32x4, held[0])),
                         "v"(__builtin_bit_cast(big::u32x4, held[1]))
                         : "memory");
        }
    };
    // fragments: B from ring slot I, A from the block that `ablk` points at
    // (rows 8..15 of A only reach output rows 8..15, which are never read)
    const uint32_t bq0 = (uint32_t)(n * 128 + (((0 + q) ^ (n & 7)) << 4));
    const uint32_t bq1 = (uint32_t)(n * 128 + (((4 + q) ^ (n & 7)) << 4));
    const uint4 *arow = afrag + (size_t)kp * (Q + 2) * 64 + q * 8 + (n & 7);
    auto frags = [&](auto slotc, const uint4 *ablk, uint4 (&fb)[2], uint4 (&fa)[2]) {
        constexpr int I = decltype(slotc)::value;
        fb[0] = *reinterpret_cast<const uint4 *>(ring + I * 2048 + bq0);
        fb[1] = *reinterpret_cast<const uint4 *>(ring + I * 2048 + bq1);
        fa[0] = ablk[0];
        fa[1] = ablk[32];
    };

    if (nit > 0) {
        // Stream position P (iteration P / Q, block P % Q of the K share) lives
        // in ring slot P % NB.  Step I of the turn starting at block g: wait
        // for block g + I + AH (the copies of the LD - 1 - AH blocks after it
        // may still be in flight), read its fragments into buffer
        // (I + AH) % 4, multiply block g + I from buffer I % 4, then copy
        // block g + I + LD into its slot, whose previous block has been
        // multiplied by then.
        uint32_t cur[2], nxt[2];
        const uint16_t *cbase = tile_rows(0, cur);
        const uint16_t *nbase = tile_rows(nit > 1 ? 1 : 0, nxt);
        uint4 fb[4][2], fa[4][2];
        const uint4 none[2] = {};
        static_for<LD>([&](auto ic) { copy_block(cur, cbase, ic, none); });
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (LD - AH)) : "memory");  // blocks 0 .. AH-1 have landed
        static_for<AH>([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            frags(ic, arow + I * 64, fb[I], fa[I]);
        });
        // One turn of the ring.  MODE 0: inside an iteration; 1: an
        // iteration's last turn, whose copies past it take the next tile's
        // first blocks; 2: the stream's last turn, which copies nothing past it.
        auto turn = [&](int g, f32x4 &acc, auto modec) {
            constexpr int MODE = decltype(modec)::value;
            const uint4 *ablk = arow + (size_t)(g + AH) * 64;
            static_for<NB>([&](auto ic) {
                constexpr int I = decltype(ic)::value;
                constexpr bool wrap = I + LD >= NB;  // the copy's block is in the next turn
                constexpr int S = wrap ? I + LD - NB : I + LD;
                // copies that may still be in flight once block g + I + AH has landed
                constexpr int fly = MODE == 2 ? ((LD - 1 < NB - 1 - I) ? LD - 1 : NB - 1 - I) - AH : LD - 1 - AH;
                if constexpr (MODE != 2 || I + AH < NB) {
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(fly > 0 ? 2 * fly : 0) : "memory");
                    frags(std::integral_constant<int, (I + AH) % NB>{}, ablk + I * 64, fb[(I + AH) % 4],
                          fa[(I + AH) % 4]);
                }
                mma16<uint16_t>(acc, fa[I % 4][0], fb[I % 4][0]);
                mma16<uint16_t>(acc, fa[I % 4][1], fb[I % 4][1]);
                if constexpr (MODE != 2 || !wrap) {
                    constexpr bool next_tile = MODE == 1 && wrap;
                    const uint16_t *src = next_tile ? nbase : cbase + (size_t)(g + (wrap ? NB : 0)) * 64;
                    // with LD == NB the slot is the one just multiplied from
                    copy_block(next_tile ? nxt : cur, src, std::integral_constant<int, S>{},
                               LD == NB ? fb[I % 4] : none);
                }
                // keep each step's instructions together: the scheduler would
                // otherwise pull every MFMA up to the reads of its own fragments
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        for (int it = 0;; ++it) {
            const bool last = it + 1 >= nit;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int g = 0; g < Q - NB; g += NB) turn(g, acc, std::integral_constant<int, 0>{});
            if (!last) turn(Q - NB, acc, std::integral_constant<int, 1>{});
            else turn(Q - NB, acc, std::integral_constant<int, 2>{});
            if constexpr (KS > 1) {
                // the group's partial tiles, summed in share order by each of
                // its waves; two sets, so one barrier per tile keeps a set
                // from being overwritten before every wave has read it.  The
                // barrier waits for LDS only: the copies stay in flight.
                f32x4 *set = parts + (it & 1) * NW * 64;
                set[wave * 64 + lane] = acc;
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                acc = set[(gi * KS) * 64 + lane];
#pragma unroll
                for (int p = 1; p < KS; ++p) acc += set[(gi * KS + p) * 64 + lane];
            }
            const int ti = it * G + gi;
            const int gt = t0 + ti;
            if (FUSED && gt >= tiles_v) {
                // a tile of the context projection: g[row, rho] (every tile
                // row that is a real row of w_h)
                const int rho = (gt - tiles_v) * 16 + n;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (e % KS != kp) continue;
                    const int row = 4 * q + e;
                    if (ti < ntile && rho < rk && row < M) gout[(size_t)row * rk + rho] = acc[e];
                }
                if (last) break;
                cur[0] = nxt[0];
                cur[1] = nxt[1];
                cbase = nbase;
                nbase = tile_rows(it + 2 < nit ? it + 2 : it + 1, nxt);
                continue;
            }
            const int v = gt * 16 + n;
            const bool vok = ti < ntile && v < V;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (e % KS != kp) continue;
                const int row = 4 * q + e;
                const int s0 = e / KS, s1 = 4 / KS + e / KS;  // buffers of rows e and 4 + e
                const bool ok = vok && row < M;
                const uint64_t key = ok ? make_key(acc[e], (uint32_t)v) : 0ull;
                if (ok && grow[e] == v) {
                    gval[e] = acc[e];
                    ghit[e] = true;
                }
                if constexpr (LSE) {
                    if (ok) lse_add(lm[e], ls[e], unary_transform(acc[e], ue.mult, ue.cap));
                }
                const bool pass = key > thr[e];
                const unsigned long long mask = __ballot(pass);
                const int c0 = __popcll(mask & 0xffffull), c1 = __popcll(mask & 0xffff0000ull);
                if (pass) {
                    const int pos = lanes_below(mask) - (q ? c0 : 0);
                    mybuf[(q ? s1 : s0) * CAP + (q ? cnt[s1] : cnt[s0]) + pos] = key;
                }
                cnt[s0] += c0;
                cnt[s1] += c1;
            }
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (e % KS != kp) continue;
                    const int sl = qq * (4 / KS) + e / KS;
                    if (cnt[sl] > CAP - 16) {
                        const uint64_t nt = shrink_candidates(mybuf + sl * CAP, cnt[sl], K, myscratch);
                        if (q == qq) thr[e] = nt;
                    }
                }
            }
            if (last) break;
            cur[0] = nxt[0];
            cur[1] = nxt[1];
            cbase = nbase;
            nbase = tile_rows(it + 2 < nit ? it + 2 : it + 1, nxt);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (ghit[e]) gold_logit[4 * q + e] = gval[e];
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < OWN; ++r) cnts[wave * OWN + r] = cnt[r];
    }
    if constexpr (LSE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e % KS != kp) continue;
            lse_merge16(lm[e], ls[e]);
            if (n == 0 && 4 * q + e < 8) lse_sm[wave * 8 + 4 * q + e] = make_float2(lm[e], ls[e]);
        }
    }
    __syncthreads();
    // row 4 q + e: candidates of wave e % KS of every group, buffer
    // q (4 / KS) + e / KS
    for (int row = wave; row < M; row += NW) {
        constexpr int R = 2 * G;
        const int e = row & 3, sl = (row >> 2) * (4 / KS) + e / KS;
        if constexpr (LSE) {
            if (lane == 0) {
                float m = -__builtin_inff(), sm = 0.f;
                for (int gg = 0; gg < G; ++gg) {
                    const int ww = gg * KS + e % KS;
                    lse_merge(m, sm, lse_sm[ww * 8 + row].x, lse_sm[ww * 8 + row].y);
                }
                ue.lse_part[(size_t)row * gridDim.x + blockIdx.x] = make_float2(m, sm);
            }
        }
        uint64_t k[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int ww = (i >> 1) * KS + e % KS, slot = lane + 64 * (i & 1);
            k[i] = slot < cnts[ww * OWN + sl] ? bufs[(ww * OWN + sl) * CAP + slot] : 0ull;
        }
        const uint64_t top = wave_topk<R>(k, K, myscratch);
        if (lane < K) partial[((size_t)row * gridDim.x + blockIdx.x) * K + lane] = top;
        // the list's head again, beside the other workgroups' heads of the row
        if (heads && lane == 0) heads[(size_t)row * gridDim.x + blockIdx.x] = top;
    }
}

// ---------------------------------------------------------------- tiled
//
// Many rows.  Workgroup (slab, mt) owns rows [128 mt, 128 mt + 128) and the
// vocabulary tiles of its slab; each 128 x 128 logit tile goes through LDS,
// and wave w merges the new values of rows w, w + 4, ... into their lists
// (bitonic sort for the first tile, threshold-filtered insertion after).
template <typename T, bool LSE>
__global__ __launch_bounds__(256) void lmhead_tiled_kernel(
    const T *__restrict__ h, const T *__restrict__ w, int M, int H, int V, int K, int n_vtiles,
    const int32_t *__restrict__ gold, float *__restrict__ gold_logit, uint64_t *__restrict__ partial,
    uint32_t *__restrict__ status, UnaryEpi ue) {
    using Cfg = TiledCfg<T, 128, 128>;
    constexpr int BIG = Cfg::STAGE_BYTES > Cfg::CTILE_BYTES ? Cfg::STAGE_BYTES : Cfg::CTILE_BYTES;
    extern __shared__ __align__(16) uint8_t smem[];
    float *ctile = reinterpret_cast<float *>(smem);
    uint64_t *lists = reinterpret_cast<uint64_t *>(smem + BIG);  // [128][K]
    float2 *lse_sm = reinterpret_cast<float2 *>(lists + Cfg::BM * K);  // [128]: row r's, kept by wave r % 4
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int slab = blockIdx.x, n_slabs = gridDim.x, mt = blockIdx.y;
    const int m0 = mt * Cfg::BM;
    if (slab == 0 && mt == 0 && threadIdx.x == 0 && status) *status = 0u;
    const int vt0 = (int)((long long)slab * n_vtiles / n_slabs);
    const int vt1 = (int)((long long)(slab + 1) * n_vtiles / n_slabs);
    for (int i = threadIdx.x; i < Cfg::BM * K; i += blockDim.x) lists[i] = 0ull;
    if constexpr (LSE) {
        for (int i = threadIdx.x; i < Cfg::BM; i += blockDim.x) lse_sm[i] = make_float2(-__builtin_inff(), 0.f);
    }

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
            if constexpr (LSE) {
                const float ta = va < V ? unary_transform(fa, ue.mult, ue.cap) : -__builtin_inff();
                const float tb = vb < V ? unary_transform(fb, ue.mult, ue.cap) : -__builtin_inff();
                const float mx = wave_max_f32(fmaxf(ta, tb));  // column 0 of the tile is always real
                const float sm = wave_sum_f32((va < V ? __expf(ta - mx) : 0.f) + (vb < V ? __expf(tb - mx) : 0.f));
                if (lane == 0) {
                    float2 run = lse_sm[r];
                    lse_merge(run.x, run.y, mx, sm);
                    lse_sm[r] = run;
                }
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
        if constexpr (LSE) {
            if (lane == 0) ue.lse_part[(size_t)gr * n_slabs + slab] = lse_sm[r];
        }
    }
}

// ---------------------------------------------------------------- many rows, bf16
//
// Workgroup (mt, slab) owns rows [256 mt, 256 mt + 256) and the 256-wide
// vocabulary tiles of its slab; big::mainloop forms each 256 x 256 logit tile
// in the accumulators.  Thread r owns tile row r: the row's running top-KL
// list (KL = K rounded up to a power of two; keeping more than K keys per
// list never changes the merged top K) lives in the workspace as the slab's
// partial list, the value of its KL-th key in LDS as the row's threshold.
//
// After a tile, every lane compares its accumulators with their rows'
// thresholds and appends each logit at or above one to that row's LDS slots;
// the owners then insert their slots into their lists and raise their
// thresholds.  A slab's first tile has no thresholds yet: for KL <= 16 each
// row takes as its threshold the KL-th largest of its 64 lane maxima (see
// lane_max_bound), else the tile takes the exact path.  On the exact path the
// tile's logits go to a per-workgroup buffer in the workspace and an owner
// scans its whole row there; when the tile was also scanned, only the rows
// whose hits overflowed their slots do (the others take their slots).
// Insertion keeps the exact top-KL under the key order, so the result does
// not depend on the tiling or on which path a tile took.
constexpr int kRowCand = 32;        // candidate slots per tile row (over the second stage buffer)
constexpr int kCandPerThread = 16;  // exact path: buffers merged once one holds more (16 more land per step)
constexpr int kCandStride = kCandPerThread + 16;
constexpr size_t kBigTileFloats = (size_t)big::BM * big::BN;  // exact path buffer per workgroup
static_assert(big::BM * kRowCand * 8 <= big::STAGE, "candidate slots over one stage buffer");
static_assert(big::NT * 64 * 4 <= big::STAGE, "register-scan scratch over one stage buffer");
static_assert(big::NT * kCandStride * 8 <= big::STAGE, "exact-path buffers over one stage buffer");
static_assert(64 * big::BM * 4 <= big::STAGE, "lane maxima over one stage buffer");

// (row tile, slab) of workgroup `bid`: the workgroups of one XCD (bid % 8)
// take a block of up to 4 row tiles x consecutive slabs, so they share the
// A rows and B rows they stream in that XCD's L2.
__device__ __forceinline__ void big_tile_of(int bid, int G, int n_mt, int n_slabs, int &mt, int &slab) {
    int L = bid;
    if (G % 8 == 0) L = (bid & 7) * (G >> 3) + (bid >> 3);
    const int Mx = (n_mt % 4 == 0) ? 4 : (n_mt % 2 == 0) ? 2 : 1;
    mt = (L / (Mx * n_slabs)) * Mx + L % Mx;
    slab = (L / Mx) % n_slabs;
}

// A row's partial list: KL keys in descending order (0 = empty slot).
template <int KL>
__device__ __forceinline__ void list_insert(uint64_t (&L)[KL], uint64_t x) {
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const uint64_t y = L[j];
        const bool gt = x > y;
        L[j] = gt ? x : y;
        x = gt ? y : x;
    }
}
template <int KL>
__device__ __forceinline__ void load_list(uint64_t (&L)[KL], const uint64_t *src) {
#pragma unroll
    for (int j = 0; j < KL; j += 2) {
        const big::u32x4 v = *reinterpret_cast<const big::u32x4 *>(src + j);
        L[j] = (uint64_t)v.x | ((uint64_t)v.y << 32);
        L[j + 1] = (uint64_t)v.z | ((uint64_t)v.w << 32);
    }
}
template <int KL>
__device__ __forceinline__ void store_list(const uint64_t (&L)[KL], uint64_t *dst) {
#pragma unroll
    for (int j = 0; j < KL; j += 2)
        *reinterpret_cast<big::u32x4 *>(dst + j) =
            big::u32x4{(uint32_t)L[j], (uint32_t)(L[j] >> 32), (uint32_t)L[j + 1], (uint32_t)(L[j + 1] >> 32)};
}

// The accumulators stay in AGPRs: every use outside the MFMAs goes through
// these, whose operands are AGPRs (left to itself the compiler moves all 256
// to VGPRs for the compares and spills everything else).
__device__ __forceinline__ float agpr_read(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}
template <int OFF>
__device__ __forceinline__ void agpr_store_global(float *p, float a) {
    asm volatile("global_store_dword %0, %1, off offset:%2" ::"v"(p), "a"(a), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void agpr_store_lds4(float *p, f32x4 a) {
    asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"((uint32_t)(size_t)(__attribute__((address_space(3))) float *)p),
                 "a"(a), "i"(OFF)
                 : "memory");
}

// Register scan of one finished tile (every column real).  For each of its
// four 32-row groups a lane forms, in vector registers only, the mask of its
// 64 accumulators at or above their rows' thresholds (kept in LDS).  A group
// with a hit in any lane is copied to the wave's LDS scratch, and each lane
// walks its own hits: value by index from the scratch, a slot of the row
// claimed with an LDS atomic (a row's hits come from two waves), the key
// written there.  A row with more than kRowCand hits sets *ovf.
// The tile's share of each row's log-sum-exp, shifted by the row's running
// maximum `shift` (LDS): lanes sum exp(U' - shift) over their values of a row,
// the 32 lanes of a half-wave reduce it, and one lane per half-wave and wave
// adds it to tile_sum.  A value more than 60 above its shift (the sum could
// leave float32 range) flags the tile for the exact path instead.
constexpr float kLseSpan = 60.f;
__device__ __forceinline__ float fast_transform(float x, float mult, float cap) {
    x *= mult;
    // cap tanh(x / cap) as cap (1 - 2 / (exp(2 x / cap) + 1)): one exp and a
    // divide; absolute error ~1e-7 cap, which the sum of exponentials absorbs
    return cap > 0.f ? cap * (1.f - 2.f / (__expf(2.f * x / cap) + 1.f)) : x;
}
__device__ __forceinline__ void register_lse(const big::f32x16 (&acc)[4][4], const float *shift, float *tile_sum,
                                             uint32_t *ovf, float mult, float cap) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1;
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const int hl = (lane >> 5) + zero;
    bool far = false;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int rbase = wm * 128 + tm * 32 + 4 * hl;  // rows of acc[tm][*][i]: rbase + 8 (i / 4) + i % 4
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 c4 = *reinterpret_cast<const float4 *>(shift + rbase + 8 * g);
            const float c[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float sum = 0.f;
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) {
                    const float d = fast_transform(agpr_read(acc[tm][tn][4 * g + e]), mult, cap) - c[e];
                    far = far || d > kLseSpan;
                    sum += __expf(d);
                }
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) sum += __shfl_xor(sum, o);
                if ((lane & 31) == 0) atomicAdd(tile_sum + rbase + 8 * g + e, sum);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (far) *ovf = 1u;
}

// Thresholds from the tile itself, for a slab's first tiles.  A tile row's
// 256 logits sit in 64 lanes (32 columns in each of two waves) holding 4 each;
// the KL-th largest of the row's 64 lane maxima is reached by at least KL
// distinct logits of the row (the lanes' own maxima), so it is at most the
// KL-th largest logit of the row's list and this tile together, and the
// larger of it and the row's threshold is still a threshold.  For KL <= 16
// about KL + 4 logits of the tile reach it on average and almost never more
// than the row's kRowCand slots: the register scan can take the first tile
// (no list yet), and with it the second, where the row's threshold alone
// lets about KL logits through and some row of 256 overflows its slots in
// most slabs.  The maxima meet in LDS (lm, 64 slots x 256 rows, a row's
// group of 4 at a slot moved by 4 (slot mod 16) rows so that the owners'
// reads hit distinct banks); the owner of row t forms its bound with a max /
// min network.  Rows past M keep +inf.  Ends with a barrier: thr is set and
// lm is free again.
template <int KL>
__device__ __forceinline__ void lane_max_bound(const big::f32x16 (&acc)[4][4], float *lm, float *thr, bool my_ok) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
    const int slot = wn * 32 + (lane & 31), sw = 4 * (slot & 15);
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float m[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * g + e;
                m[e] = fmaxf(fmaxf(agpr_read(acc[tm][0][i]), agpr_read(acc[tm][1][i])),
                             fmaxf(agpr_read(acc[tm][2][i]), agpr_read(acc[tm][3][i])));
            }
            const int rb = big::acc_row(wm, tm, 4 * g, lane);  // rows rb .. rb + 3 (rb % 4 == 0)
            *reinterpret_cast<float4 *>(lm + slot * big::BM + (rb ^ sw)) = make_float4(m[0], m[1], m[2], m[3]);
        }
    __syncthreads();
    float top[KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) top[j] = -__builtin_inff();
#pragma unroll 8
    for (int s = 0; s < 64; ++s) {
        float m = lm[s * big::BM + (t ^ (4 * (s & 15)))];
#pragma unroll
        for (int j = 0; j < KL; ++j) {
            const float hi = fmaxf(top[j], m);
            m = fminf(top[j], m);
            top[j] = hi;
        }
    }
    if (my_ok) thr[t] = fmaxf(thr[t], top[KL - 1]);
    __syncthreads();
}

__device__ __forceinline__ void register_scan(const big::f32x16 (&acc)[4][4], const float *thr, uint32_t *cnt,
                                              uint64_t *slots, uint32_t *ovf, float *scr, int v0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
    // an opaque zero: the addresses below are formed where they are used
    // instead of being hoisted out of the tile loop (and spilled)
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const int hl = (lane >> 5) + zero;
    const uint32_t col0 = (uint32_t)(v0 + wn * 128 + (lane & 31));
    // the lane's 64 values: 16-byte chunk q at (q ^ lane % 16), so each 16 lanes
    // writing one chunk hit 16 different bank groups
    float *sc = scr + (wave * 64 + lane) * 64;
    const int swz = lane & 15;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int rbase = wm * 128 + tm * 32 + 4 * hl;  // rows of acc[tm][*][i]: rbase + 8 (i / 4) + i % 4
        float th[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 t4 = *reinterpret_cast<const float4 *>(thr + rbase + 8 * g);
            th[4 * g] = t4.x;
            th[4 * g + 1] = t4.y;
            th[4 * g + 2] = t4.z;
            th[4 * g + 3] = t4.w;
        }
        uint64_t bits = 0;  // bit 16 tn + i: acc[tm][tn][i] is a hit
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            uint32_t hb = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) hb |= agpr_read(acc[tm][tn][i]) >= th[i] ? (1u << i) : 0u;
            bits |= (uint64_t)hb << (16 * tn);
        }
        if (__ballot(bits != 0)) {
#define DF2_SCR(TN, Q)                                                                                        \
    agpr_store_lds4<0>(sc + 4 * ((4 * TN + Q) ^ swz),                                                         \
                       __builtin_shufflevector(acc[tm][TN], acc[tm][TN], 4 * Q, 4 * Q + 1, 4 * Q + 2, 4 * Q + 3))
            DF2_SCR(0, 0); DF2_SCR(0, 1); DF2_SCR(0, 2); DF2_SCR(0, 3);
            DF2_SCR(1, 0); DF2_SCR(1, 1); DF2_SCR(1, 2); DF2_SCR(1, 3);
            DF2_SCR(2, 0); DF2_SCR(2, 1); DF2_SCR(2, 2); DF2_SCR(2, 3);
            DF2_SCR(3, 0); DF2_SCR(3, 1); DF2_SCR(3, 2); DF2_SCR(3, 3);
#undef DF2_SCR
            while (bits) {
                const int j = __builtin_ctzll(bits);
                bits &= bits - 1;
                const int tn = j >> 4, i = j & 15;
                const int r = rbase + 8 * (i >> 2) + (i & 3);
                const uint32_t sl = atomicAdd(cnt + r, 1u);
                if (sl < (uint32_t)kRowCand)
                    slots[r * kRowCand + sl] = make_key(sc[4 * ((j >> 2) ^ swz) + (j & 3)], col0 + 32 * tn);
                else *ovf = 1u;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Exact path, one owner thread per row over the tile's logits in `row`
// (256 floats, nvalid of them real columns).  Pass 1: a lower bound of the
// row's KL-th largest logit in the tile, the KL-th largest of the maxima of
// its 64 runs of 4 (KL distinct logits reach it), by a branch-free max / min
// network.  Pass 2: logits at or above max(threshold, bound) go to the
// thread's LDS buffer, 16 at a time; a buffer past kCandPerThread is merged
// into the list and the threshold raised.
// (Not inlined: it runs on rare tiles, and inlined its registers would crowd
// the accumulators of the common path.)
// (Out of line, so its pointers carry their address spaces explicitly: as
// generic pointers every access would be a flat access with full waits.)
typedef __attribute__((address_space(1))) const f32x4 gfloat4;
typedef __attribute__((address_space(1))) uint64_t gu64;
typedef __attribute__((address_space(3))) uint64_t lu64;
typedef __attribute__((address_space(3))) float lfloat;
template <int KL>
__device__ __attribute__((noinline)) void exact_row_scan(gfloat4 *__restrict__ row4, int nvalid, int v0, bool fresh,
                                                         gu64 *list, lfloat *thr_out, lu64 *buf, lfloat *lse_m,
                                                         lfloat *lse_s, float mult, float cap) {
    float rowmax = -__builtin_inff();
    float top[KL];
#pragma unroll
    for (int j = 0; j < KL; ++j) top[j] = -__builtin_inff();
    for (int q0 = 0; q0 < big::BN / 4; q0 += 16) {  // 16 loads in flight per round trip
        f32x4 v4[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v4[u] = row4[q0 + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int c = 4 * (q0 + u);
            float m = fmaxf(fmaxf(v4[u].x, c + 1 < nvalid ? v4[u].y : -__builtin_inff()),
                            fmaxf(c + 2 < nvalid ? v4[u].z : -__builtin_inff(),
                                  c + 3 < nvalid ? v4[u].w : -__builtin_inff()));
            if (c >= nvalid) m = -__builtin_inff();
            rowmax = fmaxf(rowmax, m);
#pragma unroll
            for (int j = 0; j < KL; ++j) {
                const float hi = fmaxf(top[j], m);
                m = fminf(top[j], m);
                top[j] = hi;
            }
        }
    }
    float th = fmaxf(*thr_out, top[KL - 1]);
    // log-sum-exp of the tile row (transformed logits), shifted by its maximum
    const float tmax = lse_m ? unary_transform(rowmax, mult, cap) : 0.f;
    float esum = 0.f;
    bool loaded = false, changed = false;
    uint64_t L[KL];
    int n = 0;
    auto flush = [&]() {
        if (!loaded) {
            if (fresh) {
#pragma unroll
                for (int j = 0; j < KL; ++j) L[j] = 0ull;
            } else {
#pragma unroll
                for (int j = 0; j < KL; ++j) L[j] = list[j];
            }
            loaded = true;
        }
        for (int i = 0; i < n; ++i) list_insert<KL>(L, buf[i]);
        if (L[KL - 1]) th = fmaxf(th, key_val(L[KL - 1]));
        changed = true;
        n = 0;
    };
    for (int q0 = 0; q0 < big::BN / 4; q0 += 16) {
        f32x4 v4[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v4[u] = row4[q0 + u];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {  // 16 values per step, then the buffer check
#pragma unroll
            for (int u = 4 * s4; u < 4 * s4 + 4; ++u) {
                const float vv[4] = {v4[u].x, v4[u].y, v4[u].z, v4[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 4 * (q0 + u) + e;
                    if (vv[e] >= th && c < nvalid) buf[n++] = make_key(vv[e], (uint32_t)(v0 + c));
                    if (lse_m && c < nvalid) esum += __expf(unary_transform(vv[e], mult, cap) - tmax);
                }
            }
            // all lanes merge together once any buffer is past the mark (a merge
            // per lane at its own step would run the wave through every one)
            if (__any(n > kCandPerThread)) flush();
        }
    }
    if (n) flush();
    if (lse_m) {
        float m = *lse_m, sm = *lse_s;
        lse_merge(m, sm, tmax, esum);
        *lse_m = m;
        *lse_s = sm;
    }
    if (changed) {
#pragma unroll
        for (int j = 0; j < KL; ++j) list[j] = L[j];
        *thr_out = th;
    }
}

template <int KL, bool LSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void lmhead_big_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ w, int M, int H, int V, int n_mt, int n_slabs,
    int n_vt, uint64_t *__restrict__ partial, float *__restrict__ tiles, uint32_t *__restrict__ status,
    UnaryEpi ue, DecodeFuse ctx) {
    using namespace big;
    __shared__ __align__(16) uint8_t st0[STAGE];
    __shared__ __align__(16) uint8_t st1[STAGE];
    // B-slice touches for the short lists (off for the long ones, whose
    // epilogue they slow)
    constexpr bool kTouch = KL <= 16;
    __shared__ __align__(16) uint8_t touch_sink[kTouch ? TOUCH_SINK : 16];
    uint64_t *slots = reinterpret_cast<uint64_t *>(st1);  // register-scan hits, [BM][kRowCand]
    __shared__ __align__(16) float thr[BM];  // per tile row: value of its KL-th key (+inf: not a row)
    __shared__ uint32_t cnt[BM];             // per tile row: register-scan hits this tile
    __shared__ uint32_t ovf[2];              // per tile parity: some row overflowed its slots
    // per tile row: running log-sum-exp (max, sum of exp(U' - max)) and this tile's share
    __shared__ __align__(16) float lse_m[LSE ? BM : 1];
    __shared__ float lse_s[LSE ? BM : 1], lse_t[LSE ? BM : 1];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
    int mt, slab;
    big_tile_of(blockIdx.x, gridDim.x, n_mt, n_slabs, mt, slab);
    const int m0 = mt * BM;
    if (blockIdx.x == 0 && t == 0 && status) *status = 0u;
    // the slabs split the vocabulary's tiles and then the context
    // projection's (W_H rows, ctx.r > 0) as one sequence, so the extra tiles
    // land at the ends of the last slabs without unbalancing them
    const int n_ct = ctx.r > 0 ? (ctx.r + BN - 1) / BN : 0, n_all = n_vt + n_ct;
    const int vt0 = (int)((long long)slab * n_all / n_slabs), vt1 = (int)((long long)(slab + 1) * n_all / n_slabs);
    const int vt1v = vt1 < n_vt ? vt1 : n_vt;  // end of this slab's vocabulary tiles
    const bool my_ok = m0 + t < M;
    uint64_t *my_list = partial + ((size_t)(my_ok ? m0 + t : 0) * n_slabs + slab) * KL;
    float *tile = tiles + (size_t)blockIdx.x * kBigTileFloats;  // exact path: [256 rows][256 cols]
    thr[t] = my_ok ? -__builtin_inff() : __builtin_inff();
    cnt[t] = 0u;
    if constexpr (LSE) {
        lse_m[t] = -__builtin_inff();
        lse_s[t] = 0.f;
        lse_t[t] = 0.f;
    }
    if (t < 2) ovf[t] = 0u;
    // (the mainloop's barriers order these before their first use)
    // A tile is kept in the workspace buffer ("stored") when it is the slab's
    // first or follows a tile that overflowed; an overflow in a tile that was
    // not stored drops its slots and forms the tile again, stored.  So no
    // accumulator is live past the register scan.
    // the register scan takes a slab's first tile (and with KL = 16 its
    // second) with thresholds raised by lane_max_bound; else the first tiles
    // are stored for the exact path
    constexpr bool kBoundFirst = !LSE && KL <= 16;
    bool store = !kBoundFirst;
    int pass = 0;  // parity of the overflow flag: per pass, a tile formed twice takes two
    // short lists live in their owner's registers between tiles (written to
    // the workspace around exact-path tiles and at the end)
    constexpr bool kRegList = KL <= 16;
    uint64_t RL[kRegList ? KL : 1];
#pragma unroll
    for (int j = 0; j < (kRegList ? KL : 1); ++j) RL[j] = 0ull;
    bool prefilled = false;
    if (vt0 >= n_vt) {
        // a slab of context tiles only: its lists stay empty
        if constexpr (!kRegList) {
            if (my_ok)
                for (int j = 0; j < KL; ++j) my_list[j] = 0ull;
        }
    }
    for (int vt = vt0; vt < vt1; ++pass) {
        if (vt >= n_vt) {
            // a context projection tile: g[m0 + row][c0 + col] = <h row, W_H row c0 + col>,
            // the accumulators stored as they are (rows past M or r dropped)
            const int c0 = (vt - n_vt) * BN;
            f32x16 acc[4][4];
            mainloop<kTouch>(acc, st0, st1, touch_sink, h + (size_t)m0 * H, M - m0, ctx.wh + (size_t)c0 * H,
                             ctx.r - c0, H, false);
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int row = m0 + acc_row(wm, tm, i, lane), col = c0 + wn * 128 + tn * 32 + (lane & 31);
                        const float v = agpr_read(acc[tm][tn][i]);
                        if (row < M && col < ctx.r) ctx.g[(size_t)row * ctx.r + col] = v;
                    }
            __syncthreads();  // every wave is done with the stage buffers
            ++vt;
            continue;
        }
        const int v0 = vt * BN, par = pass & 1;
        const bool fresh = vt == vt0;
        // The tile with the vocabulary's tail takes the exact path too (the
        // register scan assumes every column real), and so do a slab's first
        // KL / 16 tiles: after j tiles a row expects about KL / j hits in the
        // next, and a tile in which any of its 256 rows overflows the 32
        // slots would be formed twice, so the register scan starts once
        // that expectation is down to 16.
        const bool bound = kBoundFirst && !store && v0 + BN <= V && (fresh || (KL == 16 && vt - vt0 == 1));
        const bool scan = bound || (!fresh && v0 + BN <= V && (vt - vt0) * 16 >= KL);
        store = store || !scan;
        f32x16 acc[4][4];
        mainloop<kTouch>(acc, st0, st1, touch_sink, h + (size_t)m0 * H, M - m0, w + (size_t)v0 * H, V - v0, H,
                         prefilled);
        prefilled = false;
        if (store) {
            // straight from the accumulators, one base address per 4-row group
            // (an opaque zero keeps the compiler from hoisting all sixteen out of the loop)
            int zero;
            asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
            float *tile_z = tile + zero;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float *b = tile_z + acc_row(wm, tm, 4 * g, lane) * BN + wn * 128 + (lane & 31);
#define DF2_ST(E, TN) agpr_store_global<(E * BN + TN * 32) * 4>(b, acc[tm][TN][4 * g + E])
                    DF2_ST(0, 0); DF2_ST(0, 1); DF2_ST(0, 2); DF2_ST(0, 3);
                    DF2_ST(1, 0); DF2_ST(1, 1); DF2_ST(1, 2); DF2_ST(1, 3);
                    DF2_ST(2, 0); DF2_ST(2, 1); DF2_ST(2, 2); DF2_ST(2, 3);
                    DF2_ST(3, 0); DF2_ST(3, 1); DF2_ST(3, 2); DF2_ST(3, 3);
#undef DF2_ST
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        bool over = true;
        uint32_t n_hits = 0;  // this row's hits in the scan (slots hold them all up to kRowCand)
        if (scan) {
            if (bound) lane_max_bound<KL>(acc, reinterpret_cast<float *>(st0), thr, my_ok);
            // the idle stage buffers hold the scan's scratch
            register_scan(acc, thr, cnt, slots, &ovf[par], reinterpret_cast<float *>(st0), v0);
            if constexpr (LSE) register_lse(acc, lse_m, lse_t, &ovf[par], ue.mult, ue.cap);
            __syncthreads();
            over = ovf[par] != 0u;
            if (t == 0) ovf[par ^ 1] = 0u;  // last read a pass ago; next written a pass from now
            const uint32_t n = cnt[t];
            n_hits = n;
            cnt[t] = 0u;
            if constexpr (LSE) {
                // the tile's share, relative to the same shift; dropped if the
                // tile is formed again for the exact path
                if (!over) lse_s[t] += lse_t[t];
                lse_t[t] = 0.f;
            }
            if (!over && vt + 1 < vt1v) {
                // the next tile's first k-slice loads under the list insertion (the
                // barrier above ended the scan's use of st0)
                const int v1 = v0 + BN;
                prefill(st0, h + (size_t)m0 * H, M - m0, w + (size_t)v1 * H, V - v1, H);
                prefilled = true;
            }
            if (!over && n) {
                // the row's hits go into its list
                if constexpr (kRegList) {
                    for (uint32_t i = 0; i < n; ++i) list_insert<KL>(RL, slots[t * kRowCand + i]);
                    thr[t] = RL[KL - 1] ? key_val(RL[KL - 1]) : -__builtin_inff();
                } else {
                    uint64_t L[KL];
                    load_list<KL>(L, my_list);
                    for (uint32_t i = 0; i < n; ++i) list_insert<KL>(L, slots[t * kRowCand + i]);
                    store_list<KL>(L, my_list);
                    thr[t] = L[KL - 1] ? key_val(L[KL - 1]) : -__builtin_inff();
                }
            }
        } else {
            __syncthreads();  // the stored tile is visible to the workgroup
        }
        if (!over) {
            store = false;
            ++vt;
            continue;
        }
        if (store) {
            // exact path over the stored tile: every row when the tile was not
            // scanned (or with the log-sum-exp, whose tile share was dropped),
            // else only the rows whose hits overflowed their slots, the others
            // inserting their slots as above
            if (kBoundFirst && scan && n_hits <= (uint32_t)kRowCand) {
                if (my_ok && n_hits) {
                    if constexpr (kRegList) {
                        for (uint32_t i = 0; i < n_hits; ++i) list_insert<KL>(RL, slots[t * kRowCand + i]);
                        thr[t] = RL[KL - 1] ? key_val(RL[KL - 1]) : -__builtin_inff();
                    } else {
                        uint64_t L[KL];
                        load_list<KL>(L, my_list);
                        for (uint32_t i = 0; i < n_hits; ++i) list_insert<KL>(L, slots[t * kRowCand + i]);
                        store_list<KL>(L, my_list);
                        thr[t] = L[KL - 1] ? key_val(L[KL - 1]) : -__builtin_inff();
                    }
                }
            } else if (my_ok) {
                if constexpr (kRegList) {
                    if (!fresh) store_list<KL>(RL, my_list);
                }
                exact_row_scan<KL>((gfloat4 *)(tile + t * BN), V - v0, v0, fresh, (gu64 *)my_list,
                                   (lfloat *)&thr[t], (lu64 *)(reinterpret_cast<uint64_t *>(st0) + t * kCandStride),
                                   LSE ? (lfloat *)&lse_m[t] : nullptr, LSE ? (lfloat *)&lse_s[t] : nullptr, ue.mult,
                                   ue.cap);
                if constexpr (kRegList) load_list<KL>(RL, my_list);
            }
            __syncthreads();  // the buffers in st0 are the next mainloop's first stage
            ++vt;
        }
        store = true;  // next: this tile again if it was not stored, else the next tile, stored
    }
    if constexpr (kRegList) {
        if (my_ok) store_list<KL>(RL, my_list);
    }
    if constexpr (LSE) {
        if (my_ok) ue.lse_part[(size_t)(m0 + t) * n_slabs + slab] = make_float2(lse_m[t], lse_s[t]);
    }
}

// ---------------------------------------------------------------- merge
// One workgroup of 8 waves per row.  The row's n_lists sorted lists (K keys
// each) are cut into chunks of 512 keys; each wave reduces chunks to their
// top K in LDS; the survivors are reduced again until one chunk is left.

__device__ __forceinline__ void merge_stage(const uint64_t *src, int n, int K, uint64_t *dst,
                                            bool final_stage, int32_t *out_ids, float *out_vals,
                                            uint64_t *scratch, float mult, float cap) {
    const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int chunks = (n + kMergeChunk - 1) / kMergeChunk;
    for (int c = wave; c < chunks; c += nw) {
        const int base = c * kMergeChunk, nc = min(kMergeChunk, n - base);
        uint64_t top;
        if (nc <= 128) {
            // small chunk: two keys per lane, so most lanes hold a key
            uint64_t k[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) k[i] = lane + 64 * i < nc ? src[base + lane + 64 * i] : 0ull;
            top = wave_topk<2>(k, K, scratch + wave * 128);
        } else {
            // lane l holds keys [8l, 8l + 8): runs of sorted lists, so the
            // lane maxima are mostly list heads
            uint64_t k[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) k[i] = lane * 8 + i < nc ? src[base + lane * 8 + i] : 0ull;
            top = wave_topk<8>(k, K, scratch + wave * 128);
        }
        if (lane < K) {
            if (final_stage) {
                out_ids[lane] = top ? (int32_t)key_id(top) : -1;
                out_vals[lane] = top ? unary_transform(key_val(top), mult, cap) : -__builtin_inff();
            } else {
                dst[(size_t)c * K + lane] = top;
            }
        }
    }
}

// After the merge, a kernel whose tiles do not see the gold column (gold_h
// set) has the workgroup form the gold logit as a float32 dot product.
template <typename T>
__global__ __launch_bounds__(512) void topk_merge_kernel(const uint64_t *__restrict__ partial, int M,
                                                         int n_keys, int K, int V,
                                                         int32_t *__restrict__ out_ids,
                                                         float *__restrict__ out_vals,
                                                         const int32_t *__restrict__ gold,
                                                         float *__restrict__ gold_logit,
                                                         uint32_t *__restrict__ status, int lds_keys,
                                                         const T *__restrict__ gold_h, const T *__restrict__ gold_w,
                                                         int H, UnaryEpi ue, int n_lists, float *__restrict__ out_lse,
                                                         float *__restrict__ out_prob, uint8_t *__restrict__ out_hit) {
    extern __shared__ __align__(16) uint8_t smem[];
    uint64_t *bufA = reinterpret_cast<uint64_t *>(smem);
    uint64_t *bufB = bufA + lds_keys;
    uint64_t *scratch = bufB + lds_keys;  // 8 waves x 128 keys
    const int row = blockIdx.x;
    int n = n_keys;  // the row's partial lists, back to back
    const uint64_t *src = partial + (size_t)row * n;
    uint64_t *dst = bufA;
    int32_t *oi = out_ids + (size_t)row * K;
    float *ov = out_vals + (size_t)row * K;
    while (true) {
        const bool fin = n <= kMergeChunk;
        merge_stage(src, n, K, dst, fin, oi, ov, scratch, ue.mult, ue.cap);
        if (fin) break;
        __syncthreads();
        n = (n + kMergeChunk - 1) / kMergeChunk * K;
        src = dst;
        dst = dst == bufA ? bufB : bufA;
    }
    // log-sum-exp over the full vocabulary from the lists' partial sums
    float lse = 0.f;
    if (ue.lse_part) {
        __syncthreads();  // scratch is free again
        float m = -__builtin_inff(), sm = 0.f;
        for (int i = threadIdx.x; i < n_lists; i += blockDim.x) {
            const float2 ps = ue.lse_part[(size_t)row * n_lists + i];
            lse_merge(m, sm, ps.x, ps.y);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) lse_merge(m, sm, __shfl_xor(m, o), __shfl_xor(sm, o));
        float2 *part = reinterpret_cast<float2 *>(scratch);
        if (lane_id() == 0) part[threadIdx.x >> 6] = make_float2(m, sm);
        __syncthreads();
        m = -__builtin_inff();
        sm = 0.f;
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) lse_merge(m, sm, part[i].x, part[i].y);
        lse = m + logf(sm);
        if (out_lse && threadIdx.x == 0) out_lse[row] = lse;
    }
    if (!gold) return;
    const int g = gold[row];
    const bool g_ok = g >= 0 && g < V;
    if (out_hit) {
        __syncthreads();  // the final stage's ids are visible to the workgroup
        if (threadIdx.x < 64) {
            const bool hit = g_ok && (int)threadIdx.x < K && oi[threadIdx.x] == g;
            const unsigned long long b = __ballot(hit);
            if (threadIdx.x == 0) out_hit[row] = b ? 1 : 0;
        }
    }
    if (gold_h && g_ok) {
        __syncthreads();  // scratch is free again
        const T *x = gold_h + (size_t)row * H, *y = gold_w + (size_t)g * H;
        float acc = 0.f;
        for (int c = threadIdx.x; c < H / 8; c += blockDim.x) {
            float a[8], b[8];
            load8<T>(x + c * 8, a);
            load8<T>(y + c * 8, b);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(a[e], b[e], acc);
        }
        acc = wave_sum_f32(acc);
        float *part = reinterpret_cast<float *>(scratch);
        if (lane_id() == 0) part[threadIdx.x >> 6] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            float sum = 0.f;
            for (int i = 0; i < (int)(blockDim.x >> 6); ++i) sum += part[i];
            gold_logit[row] = sum;
        }
    }
    if (!g_ok && threadIdx.x == 0) {
        gold_logit[row] = __builtin_nanf("");
        flag_status(status, kStatusIdRange);
    }
    // the gold logit (written above, or by the LM-head kernel before this
    // launch) in transformed form, and its probability
    if (g_ok && threadIdx.x == 0) {
        const float u = unary_transform(gold_logit[row], ue.mult, ue.cap);
        gold_logit[row] = u;
        if (out_prob) out_prob[row] = __expf(u - lse);
    }
}

// Rows whose lists hold at most kMergeRowsKeys keys in all: one wave per row,
// four rows per workgroup (the workgroup-per-row kernel would leave most of
// its eight waves idle), the wave taking the row's keys kMergeChunk at a time
// with its running top K beside them.  Same keys selected as
// topk_merge_kernel; the gold dot product is summed in another order.
constexpr int kMergeRowsKeys = 2 * kMergeChunk;
template <typename T>
__global__ __launch_bounds__(256) void topk_merge_rows_kernel(const uint64_t *__restrict__ partial, int M, int n_keys,
                                                              int K, int V, int32_t *__restrict__ out_ids,
                                                              float *__restrict__ out_vals,
                                                              const int32_t *__restrict__ gold,
                                                              float *__restrict__ gold_logit,
                                                              uint32_t *__restrict__ status,
                                                              const T *__restrict__ gold_h,
                                                              const T *__restrict__ gold_w, int H, UnaryEpi ue,
                                                              int n_lists, float *__restrict__ out_lse,
                                                              float *__restrict__ out_prob,
                                                              uint8_t *__restrict__ out_hit) {
    __shared__ uint64_t scratch[4 * 128];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wave;
    if (row >= M) return;
    const uint64_t *src = partial + (size_t)row * n_keys;
    uint64_t top = 0;  // lane j < K: the j-th best key so far
    for (int base = 0; base < n_keys; base += kMergeChunk) {
        uint64_t k[9];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = base + lane * 8 + i;
            k[i] = idx < n_keys ? src[idx] : 0ull;
        }
        k[8] = top;
        top = wave_topk<9>(k, K, scratch + wave * 128);
    }
    int32_t *oi = out_ids + (size_t)row * K;
    if (lane < K) {
        oi[lane] = top ? (int32_t)key_id(top) : -1;
        out_vals[(size_t)row * K + lane] = top ? unary_transform(key_val(top), ue.mult, ue.cap) : -__builtin_inff();
    }
    float lse = 0.f;
    if (ue.lse_part) {
        float m = -__builtin_inff(), sm = 0.f;
        for (int i = lane; i < n_lists; i += 64) {
            const float2 ps = ue.lse_part[(size_t)row * n_lists + i];
            lse_merge(m, sm, ps.x, ps.y);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) lse_merge(m, sm, __shfl_xor(m, o), __shfl_xor(sm, o));
        lse = m + logf(sm);
        if (out_lse && lane == 0) out_lse[row] = lse;
    }
    if (!gold) return;
    const int g = gold[row];
    const bool g_ok = g >= 0 && g < V;
    if (out_hit) {
        const bool hit = g_ok && lane < K && top && (int32_t)key_id(top) == g;
        const unsigned long long b = __ballot(hit);
        if (lane == 0) out_hit[row] = b ? 1 : 0;
    }
    float u = 0.f;
    if (gold_h && g_ok) {
        const T *x = gold_h + (size_t)row * H, *y = gold_w + (size_t)g * H;
        float acc = 0.f;
        for (int c = lane; c < H / 8; c += 64) {
            float a[8], bb[8];
            load8<T>(x + c * 8, a);
            load8<T>(y + c * 8, bb);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(a[e], bb[e], acc);
        }
        u = wave_sum_f32(acc);
    } else if (g_ok) {
        u = gold_logit[row];  // written by the LM-head kernel
    }
    if (lane == 0) {
        if (!g_ok) {
            gold_logit[row] = __builtin_nanf("");
            flag_status(status, kStatusIdRange);
        } else {
            u = unary_transform(u, ue.mult, ue.cap);
            gold_logit[row] = u;
            if (out_prob) out_prob[row] = __expf(u - lse);
        }
    }
}

// ---------------------------------------------------------------- decode head tail
// One workgroup of 8 waves after the LM-head kernel of at most 8 rows: wave w
// merges row w's partial lists (n_lists <= 256 sorted lists of K keys), then
// the workgroup walks every block on the merged lattice.
//
// The merge reads list heads first (the stream kernel writes each list's head
// a second time into the row's array of heads, so a wave's load of them is
// consecutive words rather than one cache line per list).  With v the largest value such that at
// least K heads have a high word (the order image of the logit) >= v, any key
// whose high word is below v has K larger keys and is not among the row's K
// best; so only lists whose head reaches v, and only their keys that do,
// remain.  Those survivors (usually K to 2K of them) are sorted by a bitonic
// network of 128 keys; when more than 128 survive (massive ties) every key
// of the qualifying lists is ranked by wave_topk instead.  Two dependent
// loads (the heads, then those lists) and no serial ranking loop.  The walk's
// anchors and context rows are copied to LDS while the heads load.
constexpr int kTailWaves = 8;
constexpr int kTailChunk = 512;      // keys a wave scans per step (8 per lane)
constexpr int kTailCtxFloats = 8192; // context rows held in LDS (else read from global memory)

// Largest v such that at least K of the wave's keys have a high word >= v
// (0 when fewer than K keys are set).
template <int R>
__device__ __forceinline__ uint32_t high_word_bound(const uint64_t (&k)[R], int K) {
    uint32_t v = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t t = v | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < R; ++i) cnt += __popcll(__ballot((uint32_t)(k[i] >> 32) >= t));
        if (cnt >= K) v = t;
    }
    return v;
}

template <int NJ, bool WALK>
__global__ __launch_bounds__(64 * kTailWaves) void decode_tail_kernel(
    const uint64_t *__restrict__ partial, const uint64_t *__restrict__ heads, int M, int n_lists, int K, int V,
    int32_t *__restrict__ out_ids,
    float *__restrict__ out_vals, const float *__restrict__ g, const uint16_t *__restrict__ A,
    const uint16_t *__restrict__ B, const int32_t *__restrict__ anchors, int bs, int r, int32_t *__restrict__ path,
    float *__restrict__ path_score, uint32_t *__restrict__ status) {
    __shared__ uint64_t cand[kTailWaves][128];     // per row: survivors, then the sorted top
    __shared__ uint64_t scratch[kTailWaves * 128];  // wave_topk (many ties)
    __shared__ int sel[kTailWaves][256];            // per row: the lists that reach the bound
    __shared__ int32_t ids_sm[kStreamMaxRows * DFLASH2_MAX_TOP_K];
    __shared__ float vals_sm[kStreamMaxRows * DFLASH2_MAX_TOP_K];
    __shared__ int32_t anchors_sm[kStreamMaxRows];
    __shared__ __align__(16) float g_sm[WALK ? kTailCtxFloats : 1];
    __shared__ __align__(16) uint8_t wsm[kStreamMaxRows * DFLASH2_MAX_TOP_K * 20];  // walk_lds_bytes(bs <= 8, K <= 64)
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int row = wave;
    const uint64_t *rl = partial + (size_t)row * n_lists * K;
    uint64_t hk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int li = lane + 64 * i;
        hk[i] = (row < M && li < n_lists) ? heads[(size_t)row * n_lists + li] : 0ull;
    }
    const bool g_in_lds = WALK && M * r <= kTailCtxFloats;
    if constexpr (WALK) {
        // issued after the heads, so both loads are in flight together
        if ((int)threadIdx.x < M / bs) anchors_sm[threadIdx.x] = anchors[threadIdx.x];
        if (g_in_lds)
            for (int i = threadIdx.x; i < M * r / 4; i += blockDim.x)
                reinterpret_cast<float4 *>(g_sm)[i] = reinterpret_cast<const float4 *>(g)[i];
    }
    uint64_t top = 0ull;
    if (row < M) {
        const uint32_t v = high_word_bound<4>(hk, K);
        const uint64_t lb = (uint64_t)v << 32;
        int C = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool q = hk[i] != 0ull && hk[i] >= lb;
            const unsigned long long m = __ballot(q);
            if (q) sel[wave][C + lanes_below(m)] = lane + 64 * i;
            C += __popcll(m);
        }
        wave_lds_fence();
        // the survivors: keys of those lists at or above the bound
        const int n = C * K;
        int S = 0;
        for (int base = 0; base < n; base += kTailChunk) {
            uint64_t k[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = base + lane + 64 * i;
                k[i] = e < n ? rl[(size_t)sel[wave][e / K] * K + e % K] : 0ull;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool keep = k[i] != 0ull && k[i] >= lb;
                const unsigned long long m = __ballot(keep);
                const int pos = S + lanes_below(m);
                if (keep && pos < 128) cand[wave][pos] = k[i];
                S += __popcll(m);
            }
        }
        wave_lds_fence();
        if (S <= 128) {
            uint64_t x0 = 2 * lane < S ? cand[wave][2 * lane] : 0ull;
            uint64_t x1 = 2 * lane + 1 < S ? cand[wave][2 * lane + 1] : 0ull;
            bitonic128_desc(x0, x1);  // element 2 l + h: the (2 l + h)-th largest
            wave_lds_fence();
            cand[wave][2 * lane] = x0;
            cand[wave][2 * lane + 1] = x1;
            wave_lds_fence();
            top = lane < K ? cand[wave][lane] : 0ull;
        } else {
            // more than 128 keys tie at the bound: rank every key of the lists
            top = 0ull;
            for (int base = 0; base < n; base += kTailChunk) {
                uint64_t k[9];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = base + lane + 64 * i;
                    k[i] = e < n ? rl[(size_t)sel[wave][e / K] * K + e % K] : 0ull;
                }
                k[8] = top;
                top = wave_topk<9>(k, K, scratch + wave * 128);
            }
        }
    }
    if (row < M) {
        if (lane < K) {
            const int32_t id = top ? (int32_t)key_id(top) : -1;
            const float val = top ? key_val(top) : -__builtin_inff();
            out_ids[(size_t)row * K + lane] = id;
            out_vals[(size_t)row * K + lane] = val;
            ids_sm[row * K + lane] = id;
            vals_sm[row * K + lane] = val;
        }
    }
    if constexpr (WALK) {
        __syncthreads();
        const float *gw = g_in_lds ? g_sm : g;
        for (int blk = 0; blk < M / bs; ++blk) {
            walk_block<uint16_t, NJ, false>(blk, wsm, gw, A, B, ids_sm, vals_sm, anchors_sm, bs, V, r, K, path,
                                            path_score, status, 1.f, 0u, 0u);
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------- host side

// Debug knob: a fixed number of vocabulary slabs (partial top-K lists per
// row), 0 = the automatic choice.  Each logit is formed the same way whatever
// the split, and the merge orders keys totally, so the merged lists must not
// depend on it; the determinism tests change it and compare.
static std::atomic<int> g_forced_slabs{0};

void set_forced_slabs(int n) { g_forced_slabs.store(n, std::memory_order_relaxed); }

// The slab count: `automatic`, or the forced count, within [1, limit].
static int slab_count(int automatic, int limit) {
    const int f = g_forced_slabs.load(std::memory_order_relaxed);
    const int n = f > 0 ? f : automatic;
    return n < 1 ? 1 : n > limit ? limit : n;
}

// Workgroups for a weight stream of n tiles over at most `cap`: as few as
// keep the largest share at ceil(n / cap) tiles, so that every workgroup
// carries that share but a few (the stream is bound by HBM, not by the
// workgroup count, and the one-tile-longer workgroups set its end).
static int balanced_stream_grid(int n, int cap) {
    if (n <= cap) return n;
    const int per = (n + cap - 1) / cap;
    return (n + per - 1) / per;
}

static int first_stage_keys(int n_keys, int K) {
    return (n_keys + kMergeChunk - 1) / kMergeChunk * K;
}

LmheadPlan plan_lmhead(int dtype, int64_t M, int H, int V, int K) {
    LmheadPlan p{};
    const int es = dtype == 0 ? 4 : 2;
    const int S = H / (4 * (16 / es));
    const int nw = 8;
    size_t stream_lds = (size_t)S * 32 * 16 + (size_t)nw * (8 * kCandCap + 128) * 8 + (size_t)nw * 8 * 4 + 16 +
                        (size_t)nw * 8 * 8;
    if (stream_lds < (size_t)kStreamMinLds) stream_lds = kStreamMinLds;
    const int ks = dma_ksplit(H);
    if (dtype != 0 && M <= kStreamMaxRows && ks > 0 && dma_lds_bytes(H, ks) <= 160 * 1024 &&
        (uint64_t)V * H * 2 < (1ull << 32)) {
        // weights through LDS
        p.streaming = true;
        p.dma = true;
        p.ksplit = ks;
        p.n_tiles = (V + 15) / 16;
        p.grid_x = slab_count(balanced_stream_grid(p.n_tiles, kStreamWGs), p.n_tiles < kStreamWGs ? p.n_tiles : kStreamWGs);
        p.grid_y = 1;
        p.n_lists = p.grid_x;
        p.lds = dma_lds_bytes(H, ks);
    } else if (M <= kStreamMaxRows && stream_lds <= 160 * 1024) {
        p.streaming = true;
        p.nw = nw;
        p.n_tiles = (V + 15) / 16;
        p.grid_x = slab_count(balanced_stream_grid(p.n_tiles, kStreamWGs), p.n_tiles < kStreamWGs ? p.n_tiles : kStreamWGs);
        p.grid_y = 1;
        p.n_lists = p.grid_x;
        p.lds = stream_lds;
        p.prefetch = S % 16 == 0 ? 16 : S % 8 == 0 ? 8 : S % 4 == 0 ? 4 : S % 2 == 0 ? 2 : 1;
    } else if (dtype != 0 && (uint64_t)big::BM * H * 2 < (1ull << 32)) {  // 32-bit offsets within a tile
        p.streaming = false;
        p.big = true;
        p.n_mt = (int)((M + big::BM - 1) / big::BM);
        p.n_tiles = (V + big::BN - 1) / big::BN;
        const int slabs = slab_count((256 + p.n_mt - 1) / p.n_mt, p.n_tiles);
        p.grid_x = p.n_mt * slabs;
        p.grid_y = 1;
        p.n_lists = slabs;
        p.lds = 0;  // static LDS only
        p.list_len = K <= 8 ? 8 : K <= 16 ? 16 : K <= 32 ? 32 : 64;
    } else {
        p.streaming = false;
        const int n_mt = (int)((M + 127) / 128);
        const int n_vt = (V + 127) / 128;
        const int slabs = slab_count((512 + n_mt - 1) / n_mt, n_vt < 1024 ? n_vt : 1024);
        p.grid_x = slabs;
        p.grid_y = n_mt;
        p.n_lists = slabs;
        p.n_tiles = n_vt;
        const size_t stage = (size_t)(128 + 128) * (8 * 16 + 16);
        const size_t ctile = (size_t)128 * (128 + 4) * 4;
        p.lds = (stage > ctile ? stage : ctile) + (size_t)128 * K * 8 + (size_t)128 * 8;
    }
    // merge: LDS for the first reduction stage's survivors (later stages are smaller)
    if (!p.big) p.list_len = K;
    const int first = first_stage_keys(p.n_lists * p.list_len, K);
    p.merge_rows = 1;
    p.merge_lds = (size_t)2 * first * 8 + 8 * 128 * 8;
    p.partial_bytes = (size_t)M * p.n_lists * p.list_len * 8;
    if (p.big) {  // then the exact-path tile buffers, one per workgroup
        p.partial_bytes = (p.partial_bytes + 255) / 256 * 256;
        p.tiles_offset = p.partial_bytes;
        p.partial_bytes += (size_t)p.grid_x * kBigTileFloats * 4;
    }
    // then each list's log-sum-exp partial (float2)
    p.partial_bytes = (p.partial_bytes + 255) / 256 * 256;
    p.lse_offset = p.partial_bytes;
    p.partial_bytes += (size_t)M * p.n_lists * 8;
    return p;
}

template <class F>
static hipError_t set_lds(F *kernel, size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <typename T, int P, bool LSE>
static hipError_t launch_stream(const LmheadPlan &p, int64_t M, int H, int V, int K, const void *h,
                                const void *w, const int32_t *gold, float *gold_logit, uint64_t *partial,
                                uint32_t *status, const UnaryEpi &ue, hipStream_t stream) {
    auto kern = lmhead_stream_kernel<T, 8, P, LSE>;
    hipError_t e = set_lds(kern, p.lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(p.grid_x), dim3(64 * 8), p.lds, stream, (const T *)h, (const T *)w,
                       (int)M, H, V, K, p.n_tiles, gold, gold_logit, partial, status, ue);
    return hipGetLastError();
}

template <typename T, bool LSE>
static hipError_t run_lmhead(const LmheadPlan &p, int64_t M, int H, int V, int K, const void *h,
                             const void *w, const int32_t *gold, int32_t *out_ids, float *out_vals,
                             float *gold_logit, uint64_t *partial, uint32_t *status, const UnaryEpi &ue,
                             const UnaryMetrics &um, const DecodeFuse &ctx, hipStream_t stream) {
    hipError_t e;
    if (p.dma) {
        if constexpr (sizeof(T) == 2) {
            auto launch = [&](auto kern) -> hipError_t {
                hipError_t err = set_lds(kern, p.lds);
                if (err != hipSuccess) return err;
                hipLaunchKernelGGL(kern, dim3(p.grid_x), dim3(64 * kDmaWaves), p.lds, stream, (const uint16_t *)h,
                                   (const uint16_t *)w, (int)M, H, V, K, gold, gold_logit, partial, status, ue,
                                   DecodeFuse{}, nullptr);
                return hipGetLastError();
            };
            e = p.ksplit == 4 ? launch(lmhead_dma_kernel<4, LSE, false>)
                : p.ksplit == 2 ? launch(lmhead_dma_kernel<2, LSE, false>)
                                : launch(lmhead_dma_kernel<1, LSE, false>);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (p.streaming) {
#define DF2_STREAM(PP) launch_stream<T, PP, LSE>(p, M, H, V, K, h, w, gold, gold_logit, partial, status, ue, stream)
        switch (p.prefetch) {
            case 16: e = DF2_STREAM(16); break;
            case 8: e = DF2_STREAM(8); break;
            case 4: e = DF2_STREAM(4); break;
            case 2: e = DF2_STREAM(2); break;
            default: e = DF2_STREAM(1); break;
        }
#undef DF2_STREAM
    } else if (p.big) {
        if constexpr (sizeof(T) == 2) {
            auto kern = p.list_len == 8    ? lmhead_big_kernel<8, LSE>
                        : p.list_len == 16 ? lmhead_big_kernel<16, LSE>
                        : p.list_len == 32 ? lmhead_big_kernel<32, LSE>
                                           : lmhead_big_kernel<64, LSE>;
            float *tiles = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(partial) + p.tiles_offset);
            hipLaunchKernelGGL(kern, dim3(p.grid_x), dim3(big::NT), p.lds, stream, (const uint16_t *)h,
                               (const uint16_t *)w, (int)M, H, V, p.n_mt, p.n_lists, p.n_tiles, partial, tiles,
                               status, ue, ctx);
            e = hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        auto kern = lmhead_tiled_kernel<T, LSE>;
        if ((e = set_lds(kern, p.lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(p.grid_x, p.grid_y), dim3(256), p.lds, stream, (const T *)h,
                           (const T *)w, (int)M, H, V, K, p.n_tiles, gold, gold_logit, partial,
                           status, ue);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    const int n_keys = p.n_lists * p.list_len;
    if (n_keys <= kMergeChunk || (n_keys <= kMergeRowsKeys && M >= 1024)) {
        hipLaunchKernelGGL(topk_merge_rows_kernel<T>, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream, partial,
                           (int)M, n_keys, K, V, out_ids, out_vals, gold, gold_logit, status,
                           p.big ? (const T *)h : nullptr, p.big ? (const T *)w : nullptr, H, ue, p.n_lists, um.lse,
                           um.gold_prob, um.hit);
        return hipGetLastError();
    }
    auto merge = topk_merge_kernel<T>;
    if ((e = set_lds(merge, p.merge_lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(merge, dim3((unsigned)M), dim3(512), p.merge_lds, stream, partial, (int)M, n_keys, K, V,
                       out_ids, out_vals, gold, gold_logit, status, first_stage_keys(n_keys, K),
                       p.big ? (const T *)h : nullptr, p.big ? (const T *)w : nullptr, H, ue, p.n_lists, um.lse,
                       um.gold_prob, um.hit);
    return hipGetLastError();
}

// ---------------------------------------------------------------- decode head, host side

DecodeLayout decode_layout(int64_t M, int H, int V, int r, int K) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    DecodeLayout L{};
    const int tiles_v = (V + 15) / 16, tiles = tiles_v + (r > 0 ? (r + 15) / 16 : 0);
    auto grid_of = [](int n) { return slab_count(balanced_stream_grid(n, kStreamWGs), n < kStreamWGs ? n : kStreamWGs); };
    L.grid = grid_of(tiles);
    // room for the lists of either call (with W_H's tiles the grid may be the
    // smaller one), so a workspace sized for the walk serves the lattice alone
    const int lists = L.grid > grid_of(tiles_v) ? L.grid : grid_of(tiles_v);
    L.partial = kStatusBytes;
    L.heads = L.partial + up((size_t)M * lists * K * 8);
    L.g = L.heads + up((size_t)M * lists * 8);
    L.total = L.g + up((size_t)M * (r > 0 ? r : 0) * 4);
    return L;
}

bool decode_head_supported(int64_t M, int H, int V, int r, int K) {
    const int ks = dma_ksplit(H);
    return M >= 1 && M <= kStreamMaxRows && ks > 0 && dma_lds_bytes(H, ks) <= 160 * 1024 && K >= 1 &&
           K <= DFLASH2_MAX_TOP_K && (uint64_t)V * H * 2 < (1ull << 32) && (uint64_t)(r > 0 ? r : 0) * H * 2 < (1ull << 32);
}

hipError_t launch_decode_head(int64_t M, int H, int V, int K, const void *h, const void *w, int r, const void *w_h,
                              const void *A, const void *B, const int32_t *anchors, int bs, int32_t *out_ids,
                              float *out_vals, int32_t *path, float *path_score, void *workspace, hipStream_t stream) {
    const bool walk = w_h != nullptr;
    const DecodeLayout L = decode_layout(M, H, V, walk ? r : 0, K);
    uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
    uint32_t *status = reinterpret_cast<uint32_t *>(ws);
    uint64_t *partial = reinterpret_cast<uint64_t *>(ws + L.partial);
    uint64_t *heads = reinterpret_cast<uint64_t *>(ws + L.heads);
    float *g = reinterpret_cast<float *>(ws + L.g);
    const DecodeFuse fu{(const uint16_t *)w_h, walk ? r : 0, g};
    const int ks = dma_ksplit(H);
    const size_t lds = dma_lds_bytes(H, ks);
    auto stream_kernel = [&](auto kern) -> hipError_t {
        hipError_t err = set_lds(kern, lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(kern, dim3(L.grid), dim3(64 * kDmaWaves), lds, stream, (const uint16_t *)h,
                           (const uint16_t *)w, (int)M, H, V, K, nullptr, nullptr, partial, status,
                           UnaryEpi{1.f, 0.f, nullptr}, fu, heads);
        return hipGetLastError();
    };
    hipError_t e = ks == 4 ? stream_kernel(lmhead_dma_kernel<4, false, true>)
                   : ks == 2 ? stream_kernel(lmhead_dma_kernel<2, false, true>)
                             : stream_kernel(lmhead_dma_kernel<1, false, true>);
    if (e != hipSuccess) return e;
    auto tail = [&](auto kern) -> hipError_t {
        hipLaunchKernelGGL(kern, dim3(1), dim3(64 * kTailWaves), 0, stream, partial, heads, (int)M, L.grid, K, V, out_ids,
                           out_vals, g, (const uint16_t *)A, (const uint16_t *)B, anchors, bs, walk ? r : 0, path,
                           path_score, status);
        return hipGetLastError();
    };
    if (!walk) return tail(decode_tail_kernel<1, false>);
    const int nj = (K + 15) >> 4;
    return nj == 1 ? tail(decode_tail_kernel<1, true>)
           : nj == 2 ? tail(decode_tail_kernel<2, true>)
           : nj == 3 ? tail(decode_tail_kernel<3, true>)
                     : tail(decode_tail_kernel<4, true>);
}

hipError_t launch_unary_topk(int dtype, int64_t M, int H, int V, int K, const void *h, const void *w,
                             const int32_t *gold, int32_t *out_ids, float *out_vals,
                             float *gold_logit, void *workspace, hipStream_t stream, const UnaryMetrics *metrics,
                             const void *w_h, int r, float *g) {
    const LmheadPlan p = plan_lmhead(dtype, M, H, V, K);
    uint32_t *status = reinterpret_cast<uint32_t *>(workspace);
    uint64_t *partial = reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(workspace) + kStatusBytes);
    const UnaryMetrics um = metrics ? *metrics : UnaryMetrics{1.f, 0.f, nullptr, nullptr, nullptr};
    const bool lse = um.lse || um.gold_prob;
    UnaryEpi ue{um.mult, um.cap,
                lse ? reinterpret_cast<float2 *>(reinterpret_cast<uint8_t *>(partial) + p.lse_offset) : nullptr};
    // the context projection: extra tiles of the many-row kernel's stream,
    // else its own launch ahead of the LM head
    DecodeFuse ctx{};
    if (g && r > 0) {
        if (p.big) {
            ctx = DecodeFuse{(const uint16_t *)w_h, r, g};
        } else {
            hipError_t e = launch_context_proj(dtype, M, H, r, h, w_h, g, nullptr, stream);
            if (e != hipSuccess) return e;
        }
    }
    if (dtype == 0)
        return lse ? run_lmhead<float, true>(p, M, H, V, K, h, w, gold, out_ids, out_vals, gold_logit, partial,
                                             status, ue, um, ctx, stream)
                   : run_lmhead<float, false>(p, M, H, V, K, h, w, gold, out_ids, out_vals, gold_logit, partial,
                                              status, ue, um, ctx, stream);
    return lse ? run_lmhead<uint16_t, true>(p, M, H, V, K, h, w, gold, out_ids, out_vals, gold_logit, partial,
                                            status, ue, um, ctx, stream)
               : run_lmhead<uint16_t, false>(p, M, H, V, K, h, w, gold, out_ids, out_vals, gold_logit, partial,
                                             status, ue, um, ctx, stream);
}

}  // namespace dflash2
