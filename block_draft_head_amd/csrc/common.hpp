// Device-side building blocks shared by the DFlash2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash2 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

// float32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7f800000u) == 0x7f800000u) return (uint16_t)((b >> 16) | ((b & 0xffffu) ? 0x40u : 0u));
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// Storage element traits: bf16 is carried as uint16_t bit patterns.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
    static constexpr int kPer16B = 8;  // elements per 16-byte load
    __device__ static float f32(uint16_t v) { return bf16_to_f32(v); }
    __device__ static uint16_t from_f32(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<float> {
    static constexpr int kPer16B = 4;
    __device__ static float f32(float v) { return v; }
    __device__ static float from_f32(float v) { return v; }
};

// Unpack a 16-byte chunk into float32 values.
__device__ __forceinline__ void unpack16(const uint4 v, float (&o)[8]) {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ void unpack16(const uint4 v, float (&o)[4]) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}

// 8 consecutive elements <-> float32 (16-byte bf16 or 32-byte float32 accesses).
template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&o)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float (&o)[8]) {
    unpack16(*reinterpret_cast<const uint4 *>(p), o);
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&o)[8]) {
    const uint4 a = reinterpret_cast<const uint4 *>(p)[0], b = reinterpret_cast<const uint4 *>(p)[1];
    o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y); o[2] = __uint_as_float(a.z); o[3] = __uint_as_float(a.w);
    o[4] = __uint_as_float(b.x); o[5] = __uint_as_float(b.y); o[6] = __uint_as_float(b.z); o[7] = __uint_as_float(b.w);
}
template <typename T>
__device__ __forceinline__ void store8(T *p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t *p, const float (&v)[8]) {
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    *reinterpret_cast<uint4 *>(p) = o;
}
template <>
__device__ __forceinline__ void store8<float>(float *p, const float (&v)[8]) {
    reinterpret_cast<uint4 *>(p)[0] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    reinterpret_cast<uint4 *>(p)[1] = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7]));
}

// ---------------------------------------------------------------- MFMA
//
// One 16x16 output tile, one 16-byte k-chunk per lane.  Lane l supplies row
// (l % 16) of the A operand and column (l % 16) of the B operand; lanes with
// the same l / 16 supply the same k positions for A and for B, so any
// consistent assignment of the dot-product index to (lane group, element)
// gives the same sum.  Output: acc[i] of lane l is C[4 * (l / 16) + i][l % 16].
template <typename T> __device__ __forceinline__ void mma16(f32x4 &acc, uint4 a, uint4 b);

template <> __device__ __forceinline__ void mma16<uint16_t>(f32x4 &acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mma16<float>(f32x4 &acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// fp32 operands, one element per lane (k = lane / 16).
__device__ __forceinline__ void mma16_f32x1(f32x4 &acc, float a, float b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// ---------------------------------------------------------------- top-K keys
//
// A candidate is a 64-bit key: the order-preserving image of its float32
// value in the high word and (0xffffffff - id) in the low word.  The larger
// key is the better candidate: higher value first, lower id on an exact tie.
// Key 0 sorts below every real candidate and marks an empty slot.
__device__ __forceinline__ uint32_t ord_f32(float v) {
    if (v == 0.0f) v = 0.0f;  // -0 and +0 are the same value
    uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ uint64_t make_key(float v, uint32_t id) {
    return ((uint64_t)ord_f32(v) << 32) | (uint64_t)(0xffffffffu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xffffffffu - (uint32_t)k; }
__device__ __forceinline__ float key_val(uint64_t k) { return unord_f32((uint32_t)(k >> 32)); }

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    uint32_t lo = __shfl((uint32_t)v, src), hi = __shfl((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
    uint32_t lo = __shfl_up((uint32_t)v, d), hi = __shfl_up((uint32_t)(v >> 32), d);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Insert `key` into a descending list held one entry per lane in lanes
// [0, K) (`cur` is this lane's entry).  Returns the lane's new entry; the
// smallest entry drops out.  Every lane of the wave must call it.
__device__ __forceinline__ uint64_t sorted_insert(uint64_t cur, uint64_t key, int K) {
    const int l = lane_id();
    const unsigned long long gt = __ballot(l < K && cur > key);
    const int pos = __popcll(gt);
    const uint64_t prev = shfl_up_u64(cur, 1);
    if (l < K) {
        if (l == pos) return key;
        if (l > pos) return prev;
    }
    return cur;
}

// readlane of a 64-bit value from a wave-uniform lane.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, src);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

// A wave-uniform pointer read from the first active lane, so that it can sit
// in scalar registers.  readfirstlane returns a signed int: each half is
// widened as unsigned, or a low word with bit 31 set would sign-extend into
// the high word.
template <typename P>
__device__ __forceinline__ P *readfirstlane_ptr(P *p) {
    const uint64_t b = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    return reinterpret_cast<P *>(((uint64_t)hi << 32) | (uint64_t)lo);
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Orders this wave's LDS accesses before and after the call with respect to
// each other (a wave's LDS instructions execute in program order).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Top K (K <= 64) of up to 64*R keys held R per lane (key 0 = empty), by one
// wave.  Lane j < K returns the j-th largest key (0 past the last key).
// `scratch` is 128 keys of LDS owned by the wave.
// A lower bound comes first: the largest v such that at least K lanes hold a
// key whose high word is >= v (those K keys are all >= v << 32), found bit
// by bit from ballot counts.  If that admits more than 64 keys, the bound is
// redone over every key (the K-th largest high word).  The keys above it are
// compacted to one per lane and ranked by one broadcast loop; only when more
// than 64 keys share the bound's high word is every passing key ranked in
// place instead (exact, slower).
template <int R>
__device__ __forceinline__ uint64_t wave_topk(const uint64_t (&k)[R], int K, uint64_t *scratch) {
    const int lane = lane_id();
    uint32_t lmh = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint32_t hw = (uint32_t)(k[i] >> 32);
        lmh = hw > lmh ? hw : lmh;
    }
    uint32_t v = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t t = v | (1u << b);
        if (__popcll(__ballot(lmh >= t)) >= K) v = t;
    }
    int C = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) C += __popcll(__ballot(k[i] != 0ull && (uint32_t)(k[i] >> 32) >= v));
    if (C > 64) {
        // tighten: the largest v with at least K keys whose high word is >= v
        v = 0;
        for (int b = 31; b >= 0; --b) {
            const uint32_t t = v | (1u << b);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < R; ++i) cnt += __popcll(__ballot((uint32_t)(k[i] >> 32) >= t));
            if (cnt >= K) v = t;
        }
    }
    const uint64_t th = (uint64_t)v << 32;
    bool pass[R];
    C = 0;
    wave_lds_fence();
#pragma unroll
    for (int i = 0; i < R; ++i) {
        pass[i] = k[i] != 0ull && k[i] >= th;
        const unsigned long long m = __ballot(pass[i]);
        const int pos = C + lanes_below(m);
        if (pass[i] && pos < 64) scratch[pos] = k[i];
        C += __popcll(m);
    }
    wave_lds_fence();
    if (C <= 64) {
        const uint64_t c = lane < C ? scratch[lane] : 0ull;
        int rank = 0;
        for (int j = 0; j < C; ++j) rank += readlane_u64(c, j) > c ? 1 : 0;
        if (lane < C && rank < K) scratch[64 + rank] = c;
    } else {
        int rank[R];
#pragma unroll
        for (int i = 0; i < R; ++i) rank[i] = 0;
#pragma unroll
        for (int i2 = 0; i2 < R; ++i2) {
            unsigned long long m = __ballot(pass[i2]);
            while (m) {
                const int src = __builtin_ctzll(m);
                m &= m - 1;
                const uint64_t cand = readlane_u64(k[i2], src);
#pragma unroll
                for (int i = 0; i < R; ++i) rank[i] += cand > k[i] ? 1 : 0;
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (pass[i] && rank[i] < K) scratch[64 + rank[i]] = k[i];
    }
    wave_lds_fence();
    const int kept = C < K ? C : K;
    const uint64_t out = lane < kept ? scratch[64 + lane] : 0ull;
    wave_lds_fence();
    return out;
}

// Sets a bit of the status word (kernels that meet an out-of-range id).
__device__ __forceinline__ void flag_status(uint32_t *status, uint32_t bit) {
    if (status) atomicOr(status, bit);
}

}  // namespace dflash2
