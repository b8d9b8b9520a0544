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


// ------------------------------------------------------------------ 256 x 256 bf16 tile
//
// The contraction for many rows.  256 threads, 4 waves in a 2 x 2 grid; each
// wave owns a 128 x 128 block of the output as 4 x 4 tiles of the
// 32 x 32 x 16 bf16 MFMA (float32 accumulators, 256 registers).  The k loop
// walks 64-element stages: A and B rows of a stage (128 bytes each) sit in one
// of two LDS buffers, chunk c of row r at slot c ^ ((r >> 1) & 7), so the 16
// rows that one quarter of a wave reads for an MFMA fragment fall on 16
// different 16-byte bank groups.  While a stage is multiplied, the next one
// is copied from global memory straight into the idle buffer; inside a stage
// the fragments of k16 step s + 1 are read from LDS between the MFMAs of
// step s.
namespace big {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int ROWB = BK * 2;                   // bytes per row per stage
constexpr int KS = BK / 16;                    // k16 steps per stage
constexpr int HALF = BM * ROWB;                // 32 KB: the A (or B) part of a stage
constexpr int STAGE = 2 * HALF;                // 64 KB: A rows, then B rows
constexpr int LW = HALF / 1024 / (NT / 64);    // 1 KB copies per wave per operand per stage (8)
constexpr int TOUCH_AHEAD = 2;                 // k-tiles between a B slice's touch and its copies
constexpr int TOUCH_SINK = NT / 64 * 256;      // LDS bytes the touches land in (256 per wave)

__device__ __forceinline__ int swz(int row, int c) { return row * ROWB + ((c ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Output layout: acc[tm][tn][i] of lane l of wave (wm, wn) is
//   C[wm*128 + tm*32 + 8*(i/4) + 4*(l/32) + i%4][wn*128 + tn*32 + l%32].
__device__ __forceinline__ int acc_row(int wm, int tm, int i, int lane) {
    return wm * 128 + tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// The operands go from global memory straight into LDS (global_load_lds_dwordx4):
// one instruction of a wave fills 1 KB of consecutive LDS, 16 bytes per lane,
// so each lane fetches the global chunk that the swizzled layout puts at its
// slot.  No staging registers and no LDS write instructions.  The copies are
// inline assembly, so the compiler neither knows of them nor waits for them:
// the one wait is the count before the barrier that ends each k-tile, and
// every reuse of a stage buffer follows such a barrier.  (Left to the
// compiler, its waits for its own LDS copies drain every load in flight
// before the next LDS read, so nothing could stay in flight across a k-tile.)
//
// Touches (TCH): the last global read of each k-tile is one 4-byte read per
// B row of the k-slice TOUCH_AHEAD tiles ahead, into a scratch word of LDS
// that nothing reads.  Each row's slice is one 128-byte line, so the slice
// reaches L2 before its copies are issued, and the wait that ends the k-tile
// leaves that read in flight (vmcnt(1)); the next k-tile's wait covers it.
// This pays where a B tile is read by few workgroups (few row tiles: most of
// its k-slices come from HBM, whose latency the two-stage ring alone does not
// cover), and is left off for the long lists, whose epilogue it slows.
struct Pipe {
    const uint8_t *A, *B;       // first row of the A tile / B tile
    uint32_t ao[LW], bo[LW];     // byte offset of this lane's chunk of copy j, k-slice 0
    int wbase;                   // wave-uniform LDS offset of this wave's copies
    int aro[4], bro[4], hk;
    uint32_t to;                 // this lane's B row (64 * wave + lane) at k-slice 0, for the touches

    // Rows past a_rows (b_rows) read row a_rows - 1 (b_rows - 1); 256 * H * 2 < 2^32.
    __device__ __forceinline__ void init(const uint16_t *A_, int a_rows, const uint16_t *B_, int b_rows, int H) {
        const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        A = reinterpret_cast<const uint8_t *>(A_);
        B = reinterpret_cast<const uint8_t *>(B_);
        wbase = wave * LW * 1024;
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int row = (wave * LW + j) * 8 + (lane >> 3), c = (lane & 7) ^ ((row >> 1) & 7);
            ao[j] = (uint32_t)min(row, a_rows - 1) * (uint32_t)H * 2u + (uint32_t)c * 16u;
            bo[j] = (uint32_t)min(row, b_rows - 1) * (uint32_t)H * 2u + (uint32_t)c * 16u;
        }
        to = (uint32_t)min(wave * 64 + lane, b_rows - 1) * (uint32_t)H * 2u;
        const int wm = wave >> 1, wn = wave & 1, r32 = lane & 31;
        hk = lane >> 5;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            aro[i] = wm * 128 + i * 32 + r32;
            bro[i] = wn * 128 + i * 32 + r32;
        }
    }
    // (wave-uniform; read from the first lane so that the copies can take it
    // as their scalar base whatever the compiler proves about it)
    static __device__ __forceinline__ const uint8_t *uniform(const uint8_t *p) {
        const uint64_t v = (uint64_t)p;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        return (const uint8_t *)(((uint64_t)hi << 32) | lo);
    }
    static __device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
        return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t *)p;
    }
    // 16 bytes per lane from base + off into LDS at dst + 16 lane.  s_nop 4:
    // the wait states that a scalar base or M0 written just before needs (the
    // compiler adds none to inline assembly).
    static __device__ __forceinline__ void copy16(const uint8_t *base, uint32_t off, const uint8_t *dst) {
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(uniform(base)),
                     "{m0}"(lds_addr(dst))
                     : "memory");
    }
    // 4 bytes of this lane's B row in k-slice k0b into the wave's sink word
    __device__ __forceinline__ void touch(uint32_t k0b, const uint8_t *sink) const {
        asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(to + k0b), "s"(uniform(B)),
                     "{m0}"(lds_addr(sink))
                     : "memory");
    }
    // k-slice at byte offset k0b into stage st
    __device__ __forceinline__ void fill(uint8_t *st, uint32_t k0b) {
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            copy16(A, ao[j] + k0b, st + wbase + j * 1024);
            copy16(B, bo[j] + k0b, st + HALF + wbase + j * 1024);
        }
    }
    __device__ __forceinline__ void frags(const uint8_t *st, int s, u32x4 (&fa)[4], u32x4 (&fb)[4]) const {
        const int c = 2 * s + hk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i] = *reinterpret_cast<const u32x4 *>(st + swz(aro[i], c));
            fb[i] = *reinterpret_cast<const u32x4 *>(st + HALF + swz(bro[i], c));
        }
    }
    // One k-tile from `cur` while k-slice nk fills `nxt` (and, with TCH, B's
    // k-slice tk is touched); the fragments of the first k16 step of `nxt`
    // are read after the closing barrier.  The copies go out during the
    // first two k16 steps, each after one fragment read, between one MFMA
    // and the next (all 16 at the start of the tile measured 6% slower: they
    // queue ahead of the fragment reads).
    static_assert(LW == 8 && KS == 4, "the copies go out four per operand in each of the first two k16 steps");
    template <bool TCH>
    __device__ __forceinline__ void tile(f32x16 (&acc)[4][4], const uint8_t *cur, uint8_t *nxt, uint32_t nk,
                                         u32x4 (&fa)[2][4], u32x4 (&fb)[2][4], uint32_t tk, const uint8_t *sink) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int c0 = s & 1;
            if (s + 1 < KS) {
                const int c = 2 * (s + 1) + hk;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fa[c0 ^ 1][i] = *reinterpret_cast<const u32x4 *>(cur + swz(aro[i], c));
                    if (s < 2) copy16(A, ao[s * 4 + i] + nk, nxt + wbase + (s * 4 + i) * 1024);
                    fb[c0 ^ 1][i] = *reinterpret_cast<const u32x4 *>(cur + HALF + swz(bro[i], c));
                    if (s < 2) copy16(B, bo[s * 4 + i] + nk, nxt + HALF + wbase + (s * 4 + i) * 1024);
                }
            }
            if (TCH && s == 2) touch(tk, sink);  // after every copy of the tile
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = mfma32(fa[c0][tm], fb[c0][tn], acc[tm][tn]);
            if (s + 1 < KS) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wave's copies into nxt have landed (its touch may still be in
        // flight), and its fragment reads of cur are done
        if constexpr (TCH) asm volatile("s_waitcnt vmcnt(1)\n\ts_waitcnt lgkmcnt(0)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
        frags(nxt, 0, fa[0], fb[0]);
    }
};

// acc = A[0 .. 256) . B[0 .. 256)^T over all of H (H % 64 == 0), A and B
// pointing at the tiles' first rows (row r at r * H elements).  st0 and st1
// are two __shared__ buffers of at least STAGE bytes, sink (TCH) one of
// TOUCH_SINK bytes.  On return every copy and touch has landed and all waves
// have passed a barrier after their last fragment read that matters; the
// caller may reuse st0 and st1 after one more barrier (the last fragment
// reads are of a spare slice and unused).
//
// prefilled: the caller has already issued this wave's copies of k-slice 0
// into st0 (prefill below, same operands), so the first stage only waits.
__device__ __forceinline__ void prefill(uint8_t *st0, const uint16_t *A, int a_rows, const uint16_t *B, int b_rows,
                                        int H) {
    Pipe P;
    P.init(A, a_rows, B, b_rows, H);
    P.fill(st0, 0);
}
template <bool TCH>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[4][4], uint8_t *st0, uint8_t *st1, const uint8_t *sink,
                                         const uint16_t *A, int a_rows, const uint16_t *B, int b_rows, int H,
                                         bool prefilled = false) {
    Pipe P;
    P.init(A, a_rows, B, b_rows, H);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
    if (!prefilled) P.fill(st0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    u32x4 fa[2][4], fb[2][4];
    P.frags(st0, 0, fa[0], fb[0]);
    const int KT = H / BK;
    // stage buffers alternate by name, two k-tiles per trip; a tile with no
    // next slice re-fills its idle buffer with the last slice, and one with no
    // slice TOUCH_AHEAD ahead touches the last (in bounds, unused)
    const uint8_t *wsink = sink + (threadIdx.x >> 6) * 256;
    auto ahead = [&](int k) { return (uint32_t)min(k, KT - 1) * BK * 2; };
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
        P.tile<TCH>(acc, st0, st1, ahead(kt + 1), fa, fb, ahead(kt + TOUCH_AHEAD), wsink);
        P.tile<TCH>(acc, st1, st0, ahead(kt + 2), fa, fb, ahead(kt + 1 + TOUCH_AHEAD), wsink);
    }
    if (kt < KT) P.tile<TCH>(acc, st0, st1, ahead(KT - 1), fa, fb, ahead(KT - 1), wsink);
    if constexpr (TCH) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last touch
}

}  // namespace big
}  // namespace dflash2
