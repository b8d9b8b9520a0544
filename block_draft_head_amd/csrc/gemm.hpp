// Contraction building blocks: C[m][c] = sum_k A[m][k] * B[c][k] with A and B
// row-major [rows, H] (the [out, in] layout of a linear layer for B).
//
// Two regimes:
//  * streaming (at most 8 rows of A): A sits in LDS in MFMA-fragment order and
//    every lane streams 16-byte chunks of its B row from HBM straight into the
//    MFMA operand registers.  B is read exactly once; nothing is staged.
//  * tiled (many rows): BM x BN output tiles, 4 waves in a 2 x 2 grid, A and B
//    k-slices staged through padded LDS with a register double buffer.
#pragma once

#include "common.hpp"

namespace dflash2 {

// ------------------------------------------------------------------ streaming

constexpr int kStreamMaxRows = 8;

// k-steps of one 16x16 MFMA tile: 4 lane groups x 16 bytes.
template <typename T> __host__ __device__ constexpr int kstep_elems() { return 4 * (16 / (int)sizeof(T)); }

// A fragments for the streaming regime: entry (s, q, m) holds 16 bytes of A
// row m at k-chunk 4*s + q; rows m >= M are zero.  S = H / kstep.
template <typename T>
__device__ void load_afrag(uint4 *afrag, const T *__restrict__ A, int M, int H) {
    constexpr int KC = 16 / (int)sizeof(T);
    const int S = H / kstep_elems<T>();
    for (int i = threadIdx.x; i < S * 32; i += blockDim.x) {
        const int m = i & 7, q = (i >> 3) & 3, s = i >> 5;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (m < M) v = *reinterpret_cast<const uint4 *>(A + (size_t)m * H + (size_t)(4 * s + q) * KC);
        afrag[i] = v;
    }
}

__device__ __forceinline__ uint4 afrag_get(const uint4 *afrag, int s, int lane) {
    const int m = lane & 15, q = lane >> 4;
    return m < kStreamMaxRows ? afrag[s * 32 + q * 8 + m] : make_uint4(0u, 0u, 0u, 0u);
}

// acc += steps [s0, s1) of (A fragments) x (this lane's B row).  `brow`
// points at the lane's B row already offset by its lane group's 16-byte
// chunk; a null row contributes zero.  Up to 8 loads in flight per wave.
template <typename T>
__device__ __forceinline__ void stream_accumulate(f32x4 &acc, const uint4 *afrag, const T *brow,
                                                  int s0, int s1) {
    constexpr int KS = kstep_elems<T>();
    const int lane = lane_id();
    for (int s = s0; s < s1; s += 8) {
        uint4 b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            b[i] = make_uint4(0u, 0u, 0u, 0u);
            if (s + i < s1 && brow) b[i] = *reinterpret_cast<const uint4 *>(brow + (size_t)(s + i) * KS);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (s + i < s1) mma16<T>(acc, afrag_get(afrag, s + i, lane), b[i]);
    }
}

// ------------------------------------------------------------------ tiled

template <typename T, int BM_, int BN_>
struct TiledCfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int KC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
    static constexpr int CH = 8;                     // chunks per row per stage (128 bytes)
    static constexpr int BK = CH * KC;               // elements per stage
    static constexpr int ROWB = CH * 16 + 16;        // LDS bytes per staged row (padded)
    static constexpr int WM = BM / 2, WN = BN / 2;   // wave tile
    static constexpr int TM = WM / 16, TN = WN / 16; // 16x16 MFMA tiles per wave
    static constexpr int A_PER_T = BM * CH / 256;    // chunks each thread moves
    static constexpr int B_PER_T = BN * CH / 256;
    static constexpr int STAGE_BYTES = (BM + BN) * ROWB;
    static constexpr int CSTRIDE = BN + 4;           // floats per row of the C tile in LDS
    static constexpr int CTILE_BYTES = BM * CSTRIDE * 4;
    static_assert(BM * CH % 256 == 0 && BN * CH % 256 == 0, "tile must split over 256 threads");
};

// One BM x BN tile over all of H.  arow(i) / brow(j) return the start of A
// row i / B row j of the tile, or nullptr for a zero row.  H must be a
// multiple of BK.  `stage` is STAGE_BYTES of LDS.  On return acc holds the
// wave's TM x TN tiles; the caller must __syncthreads() before reusing LDS.
template <typename T, class Cfg, class ARow, class BRow>
__device__ __forceinline__ void tiled_mainloop(f32x4 (&acc)[Cfg::TM][Cfg::TN], uint8_t *stage,
                                               ARow arow, BRow brow, int H) {
    const int t = threadIdx.x;
    const int lane = lane_id(), wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int chunk = t % Cfg::CH;
    const T *ap[Cfg::A_PER_T];
    const T *bp[Cfg::B_PER_T];
#pragma unroll
    for (int i = 0; i < Cfg::A_PER_T; ++i) {
        const T *r = arow(t / Cfg::CH + i * (256 / Cfg::CH));
        ap[i] = r ? r + chunk * Cfg::KC : nullptr;
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_T; ++i) {
        const T *r = brow(t / Cfg::CH + i * (256 / Cfg::CH));
        bp[i] = r ? r + chunk * Cfg::KC : nullptr;
    }
#pragma unroll
    for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
        for (int b = 0; b < Cfg::TN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[Cfg::A_PER_T], rb[Cfg::B_PER_T];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Cfg::A_PER_T; ++i)
            ra[i] = ap[i] ? *reinterpret_cast<const uint4 *>(ap[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < Cfg::B_PER_T; ++i)
            rb[i] = bp[i] ? *reinterpret_cast<const uint4 *>(bp[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
    };
    uint8_t *sa = stage, *sb = stage + Cfg::BM * Cfg::ROWB;
    gload(0);
    for (int k0 = 0; k0 < H; k0 += Cfg::BK) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < Cfg::A_PER_T; ++i)
            *reinterpret_cast<uint4 *>(sa + (t / Cfg::CH + i * (256 / Cfg::CH)) * Cfg::ROWB + chunk * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < Cfg::B_PER_T; ++i)
            *reinterpret_cast<uint4 *>(sb + (t / Cfg::CH + i * (256 / Cfg::CH)) * Cfg::ROWB + chunk * 16) = rb[i];
        __syncthreads();
        if (k0 + Cfg::BK < H) gload(k0 + Cfg::BK);
#pragma unroll
        for (int ks = 0; ks < Cfg::CH / 4; ++ks) {
            uint4 fa[Cfg::TM], fb[Cfg::TN];
            const int c = ks * 4 + (lane >> 4);
#pragma unroll
            for (int a = 0; a < Cfg::TM; ++a)
                fa[a] = *reinterpret_cast<const uint4 *>(sa + (wm * Cfg::WM + a * 16 + (lane & 15)) * Cfg::ROWB + c * 16);
#pragma unroll
            for (int b = 0; b < Cfg::TN; ++b)
                fb[b] = *reinterpret_cast<const uint4 *>(sb + (wn * Cfg::WN + b * 16 + (lane & 15)) * Cfg::ROWB + c * 16);
#pragma unroll
            for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
                for (int b = 0; b < Cfg::TN; ++b) mma16<T>(acc[a][b], fa[a], fb[b]);
        }
    }
}

// Write the wave accumulators to a float C tile in LDS ([BM][CSTRIDE]).
template <class Cfg>
__device__ __forceinline__ void tiled_store_c(float *ctile, const f32x4 (&acc)[Cfg::TM][Cfg::TN]) {
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
        for (int b = 0; b < Cfg::TN; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * Cfg::WM + a * 16 + 4 * (lane >> 4) + i;
                const int c = wn * Cfg::WN + b * 16 + (lane & 15);
                ctile[r * Cfg::CSTRIDE + c] = acc[a][b][i];
            }
}

}  // namespace dflash2
