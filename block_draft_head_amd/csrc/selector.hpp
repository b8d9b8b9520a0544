// Selector scoring routines shared by the selector kernels and the fused
// decode head: the pair-term MFMA tiles, the counter-based Gumbel noise and
// the per-block walk (every adjacent pair scored at once, then the pointer
// chase).  S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)>.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace dflash2 {

// 8 codebook elements as packed 16-byte words (one for bf16, two for float32),
// unpacked to float32 at their MFMA step.
template <typename T> constexpr int kWords8 = (int)sizeof(T) / 2;
__device__ __forceinline__ void unpack_words8(const uint4 (&w)[1], float (&o)[8]) { unpack16(w[0], o); }
__device__ __forceinline__ void unpack_words8(const uint4 (&w)[2], float (&o)[8]) {
    float a[4], b[4];
    unpack16(w[0], a);
    unpack16(w[1], b);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = a[e], o[4 + e] = b[e];
}

// v = hi + lo + d with hi, lo bf16 and |d| < 2^-15 |v|: hi is v truncated to
// bf16 (the float32 remainder v - hi is exact), lo that remainder truncated.
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], uint4 &hi, uint4 &lo) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = __float_as_uint(v[e]) & 0xffff0000u;
        l[e] = __float_as_uint(v[e] - __uint_as_float(h[e])) & 0xffff0000u;
    }
    hi = make_uint4((h[0] >> 16) | h[1], (h[2] >> 16) | h[3], (h[4] >> 16) | h[5], (h[6] >> 16) | h[7]);
    lo = make_uint4((l[0] >> 16) | l[1], (l[2] >> 16) | l[3], (l[4] >> 16) | l[5], (l[6] >> 16) | l[7]);
}

// P[m][c] = sum_r B[cid_m, r] * (A[pid_c, r] * grow[r]) where lane l holds
// candidate cid (row l % 16) and predecessor pid (column l % 16); a negative
// id is a zero row/column.  r is a multiple of 8; grow is the context row (r
// floats, global memory or LDS).  The rank index is visited 32 at a time (8
// per lane group); B rows sit bstride elements apart (r in global memory,
// padded in LDS).  pair_tiles forms NJ such tiles over the same
// predecessors (tile j from candidates cid[j]): the predecessor rows and the
// context are loaded and multiplied once for all of them, and a batch of
// steps (as many as keep its operands within about 128 registers) has all of
// its gathers and context loads issued before its MFMAs.
//   bf16 codebooks: the B rows enter a bf16 MFMA exactly; A(a) * g is split
//   into bf16 high and low parts (relative error below 2^-15), two 16x16x32
//   MFMAs per step, summed in two accumulators.
//   float32 codebooks: 16x16x4 float32 MFMAs, element e of a step feeding
//   accumulator e % 4.
// A tile's MFMAs run in the same order whatever NJ and the batch size, so
// equal inputs give bit-equal tiles in every caller.
// P[j][i] of lane l is tile j's P[4 * (l / 16) + i][l % 16].
template <typename T, int NJ>
__device__ __forceinline__ void pair_tiles(const T *__restrict__ A, const T *__restrict__ B, const float *grow,
                                           int pid, const int (&cid)[NJ], int r, int bstride, f32x4 (&P)[NJ]) {
    constexpr int W = kWords8<T>;
    constexpr int PER = 4 * W * (1 + NJ) + 8;  // registers of one step's operands
    constexpr int S = 128 / PER >= 8 ? 8 : 128 / PER >= 4 ? 4 : 128 / PER >= 2 ? 2 : 1;
    const int q = lane_id() >> 4;
    const T *arow = pid >= 0 ? A + (size_t)pid * r : nullptr;
    const T *brow[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) brow[j] = cid[j] >= 0 ? B + (size_t)cid[j] * bstride : nullptr;
    f32x4 acc[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int rho0 = 0; rho0 < r; rho0 += 32 * S) {
        uint4 ra[S][W], rb[S][NJ][W];
        float gg[S][8];
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int rho = rho0 + u * 32 + q * 8;
            const bool in = rho < r;
#pragma unroll
            for (int i = 0; i < W; ++i) {
                ra[u][i] = (in && arow) ? reinterpret_cast<const uint4 *>(arow + rho)[i] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    rb[u][j][i] =
                        (in && brow[j]) ? reinterpret_cast<const uint4 *>(brow[j] + rho)[i] : make_uint4(0u, 0u, 0u, 0u);
            }
            const float4 g0 = in ? reinterpret_cast<const float4 *>(grow + rho)[0] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 g1 = in ? reinterpret_cast<const float4 *>(grow + rho)[1] : make_float4(0.f, 0.f, 0.f, 0.f);
            gg[u][0] = g0.x, gg[u][1] = g0.y, gg[u][2] = g0.z, gg[u][3] = g0.w;
            gg[u][4] = g1.x, gg[u][5] = g1.y, gg[u][6] = g1.z, gg[u][7] = g1.w;
        }
#pragma unroll
        for (int u = 0; u < S; ++u) {
            float a[8], ag[8];
            unpack_words8(ra[u], a);
#pragma unroll
            for (int e = 0; e < 8; ++e) ag[e] = a[e] * gg[u][e];
            if constexpr (sizeof(T) == 2) {
                uint4 hi, lo;
                split_bf16x8(ag, hi, lo);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    mma16<uint16_t>(acc[j][0], rb[u][j][0], hi);
                    mma16<uint16_t>(acc[j][1], rb[u][j][0], lo);
                }
            } else {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    float b[8];
                    unpack_words8(rb[u][j], b);
#pragma unroll
                    for (int e = 0; e < 8; ++e) mma16_f32x1(acc[j][e & 3], b[e], ag[e]);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) P[j] = (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
}

template <typename T>
__device__ __forceinline__ f32x4 pair_tile(const T *__restrict__ A, const T *__restrict__ B, const float *grow,
                                           int pid, int cid, int r) {
    const int c[1] = {cid};
    f32x4 P[1];
    pair_tiles<T, 1>(A, B, grow, pid, c, r, r, P);
    return P[0];
}

// ------------------------------------------------------------------ walk
// One workgroup per anchor block.  Work item (t, it): position t and the
// predecessor tile it (16 slots of C_{t-1}; at t = 1 the single anchor).  A
// wave reads its item's candidate ids and context row from global memory, so
// its gathers start at once, and keeps each predecessor's best successor as a
// key (score, lowest slot on ties) in LDS.  Wave 0 then chases the pointers:
// the keys of 8 positions at a time sit in its registers (lane = slot) and
// each step is a register read-lane.
// LDS (walk_lds_bytes): best [bs][K] u64, ids [bs][K] int, best_s [bs][K]
// float, noise [bs][K] float (sampling).  NJ = ceil(K / 16).
//
// SAMPLE: the pick maximises S / temperature + G instead of S, G standard
// Gumbel noise drawn per (block, position, slot) from Philox4x32-10 (the key
// order then ranks the noisy scores; the clean S of each predecessor's pick
// is kept beside its key for the path score).
//
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011): ten rounds of
// (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)), the key advanced by the Weyl increments between rounds; the
// first output word.
__device__ __forceinline__ uint32_t philox_first_word(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                     uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}
// Standard Gumbel noise of slot j at position t of block b: -log(-log(u)),
// u the centred top 24 bits of the first Philox word at counter (j, t, b, 0).
__device__ __forceinline__ float walk_gumbel(int j, int t, int b, uint32_t k0, uint32_t k1) {
    const uint32_t x = philox_first_word((uint32_t)j, (uint32_t)t, (uint32_t)b, 0u, k0, k1);
    const float u = ((float)(x >> 8) + 0.5f) * 0x1p-24f;
    return -logf(-logf(u));
}

template <typename T, int NJ, bool SAMPLE>
__device__ __forceinline__ void walk_block(int blk, uint8_t *wsm, const float *__restrict__ g, const T *__restrict__ A,
                           const T *__restrict__ B, const int32_t *__restrict__ cand_ids,
                           const float *__restrict__ cand_vals, const int32_t *__restrict__ anchors, int bs,
                           int V, int r, int K, int32_t *__restrict__ path, float *__restrict__ path_score,
                           uint32_t *__restrict__ status, float temperature, uint32_t k0, uint32_t k1) {
    uint64_t *best = reinterpret_cast<uint64_t *>(wsm);
    int32_t *cids = reinterpret_cast<int32_t *>(best + bs * K);
    float *best_s = reinterpret_cast<float *>(cids + bs * K);
    float *noise = best_s + bs * K;
    const int lane = lane_id(), wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int n_it = NJ;
    const int n_items = bs >= 2 ? 1 + (bs - 2) * n_it : 0;
    const size_t row0 = (size_t)blk * bs;
    const int anchor = anchors[blk];
    const bool anchor_ok = anchor >= 0 && anchor < V;
    if (!anchor_ok && threadIdx.x == 0) flag_status(status, kStatusIdRange);
    for (int i = threadIdx.x; i < bs * K; i += blockDim.x) cids[i] = cand_ids[row0 * K + i];  // for the chase
    if constexpr (SAMPLE) {
        // the block's noise, once per (position, slot): every predecessor of a
        // position sees the same draws
        for (int i = threadIdx.x; i < bs * K; i += blockDim.x) noise[i] = walk_gumbel(i % K, i / K, blk, k0, k1);
        __syncthreads();
    }

    for (int item = wave; item < n_items; item += nwaves) {
        const int t = item == 0 ? 1 : 2 + (item - 1) / n_it;
        const int it = item == 0 ? 0 : (item - 1) % n_it;
        const size_t n = row0 + t;
        int pid = -1;
        bool col_used;
        if (t == 1) {
            col_used = c == 0;
            pid = (col_used && anchor_ok) ? anchor : -1;
        } else {
            const int i = it * 16 + c;
            col_used = i < K;
            if (col_used) {
                pid = cand_ids[(n - 1) * K + i];
                if (pid < 0 || pid >= V) pid = -1;  // flagged when its own row is scored
            }
        }
        // every successor tile at once: ids and unary values first, then one
        // pass over the rank for all NJ tiles
        int cid[NJ];
        bool cok[NJ];
        float uv[NJ][4];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            const int j = jt * 16 + c;
            cid[jt] = j < K ? cand_ids[n * K + j] : -1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int jj = jt * 16 + 4 * q + i;
                uv[jt][i] = jj < K ? cand_vals[n * K + jj] : 0.f;
            }
        }
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            const int j = jt * 16 + c;
            cok[jt] = j < K && cid[jt] >= 0 && cid[jt] < V;
            if (j < K && !cok[jt]) flag_status(status, kStatusIdRange);
            if (!cok[jt]) cid[jt] = -1;
        }
        f32x4 P[NJ];
        pair_tiles<T, NJ>(A, B, g + n * r, pid, cid, r, r, P);
        // noise of this lane's slots
        float gn[NJ][4];
        if constexpr (SAMPLE) {
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int jj = jt * 16 + 4 * q + i;
                    gn[jt][i] = jj < K ? noise[t * K + jj] : 0.f;
                }
        }
        uint64_t bestkey = 0;
        float bests = 0.f;  // S of the best key's slot (sampling)
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            uint64_t local = 0;
            float locs = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int jj = jt * 16 + 4 * q + i;
                const bool ok = __shfl((int)cok[jt], 4 * q + i) != 0;
                const float s = jj < K ? uv[jt][i] + P[jt][i] : 0.f;
                float z = s;
                if constexpr (SAMPLE) z = s / temperature + gn[jt][i];
                const uint64_t key = (ok && pid >= 0) ? make_key(z, (uint32_t)jj) : 0ull;
                if (key > local) {
                    local = key;
                    locs = s;
                }
            }
            uint64_t o = shfl_xor_u64(local, 16);
            float os = __shfl_xor(locs, 16);
            if (o > local) {
                local = o;
                locs = os;
            }
            o = shfl_xor_u64(local, 32);
            os = __shfl_xor(locs, 32);
            if (o > local) {
                local = o;
                locs = os;
            }
            if (local > bestkey) {
                bestkey = local;
                bests = locs;
            }
        }
        if (q == 0 && col_used) {
            const int e = t * K + (t == 1 ? 0 : it * 16 + c);
            best[e] = bestkey;
            best_s[e] = bests;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const size_t p0 = row0;
        if (lane == 0) {
            path[p0] = anchor_ok ? anchor : -1;
            if (path_score) path_score[p0] = 0.f;
        }
        bool alive = anchor_ok;
        int slot = 0;  // wave-uniform
        for (int t0 = 1; t0 < bs; t0 += 8) {
            // 8 positions' keys, scores and ids in registers (lane = slot), so
            // each step of the chase is a handful of register reads
            uint64_t kk[8];
            float ks[8];
            int ci[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u;
                const bool in = t < bs && lane < K;
                kk[u] = in ? best[t * K + lane] : 0ull;
                ks[u] = in ? best_s[t * K + lane] : 0.f;
                ci[u] = in ? cids[t * K + lane] : -1;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u;
                if (t >= bs) break;
                const uint64_t key = alive ? readlane_u64(kk[u], slot) : 0ull;
                // S of the pick (the key holds the noisy score when sampling)
                const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ks[u]), slot));
                if (key == 0) alive = false;
                else slot = (int)key_id(key);
                const int pick = __builtin_amdgcn_readlane(ci[u], slot);
                if (lane == 0) {
                    path[p0 + t] = alive ? pick : -1;
                    if (path_score) path_score[p0 + t] = alive ? (SAMPLE ? sc : key_val(key)) : __builtin_nanf("");
                }
            }
        }
    }
}

}  // namespace dflash2
