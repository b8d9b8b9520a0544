// Projections of at most 8 rows (weight streaming on the vector ALUs), shared
// by the conv and the selector kernels.
#pragma once

#include "common.hpp"
#include "gemm.hpp"

namespace dflash2 {

// ------------------------------------------------------------ at most 8 rows
//
// A workgroup owns a few weight rows.  Its threads split H into 8-element
// chunks, so every weight byte is loaded exactly once and a thread's loads of
// one round are all in flight together; the x rows (at most 8 x H) are
// re-read from L2 by every workgroup.  A thread keeps R x 8 partial dot
// products; a transposing butterfly sums them over the wave (R*8 values on
// 64 lanes: each exchange halves the values a lane holds) and LDS sums the
// waves.  The summation order is fixed, so results are deterministic.  With
// at most 8 rows the MFMA tile would be half empty and the launch needs many
// workgroups (one per CU or more), which a 16-column MFMA tile per workgroup
// cannot give for a few hundred weight rows.

constexpr int kGemvThreads = 512;
constexpr int kGemvMaxRows = 32;  // weight rows per workgroup (2T <= 32)

// Butterfly over the wave: on entry every lane holds N partial values; on
// exit v[0] of lane l is the wave total of value (l >> (6 - log2 N)) & (N - 1).
template <int N, int O, int NV>
__device__ __forceinline__ void butterfly(float (&v)[NV], int lane) {
    if constexpr (N > 1) {
        const bool upper = (lane & O) != 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float keep = upper ? v[i + N / 2] : v[i];
            const float send = upper ? v[i] : v[i + N / 2];
            v[i] = keep + __shfl_xor(send, O);
        }
        butterfly<N / 2, O / 2>(v, lane);
    } else if constexpr (O >= 1) {
        v[0] += __shfl_xor(v[0], O);
        butterfly<1, O / 2>(v, lane);
    }
}

template <int N> constexpr int ilog2() { return N <= 1 ? 0 : 1 + ilog2<N / 2>(); }

// res[i * 8 + m] = <x[m], W[row_of(i)]> for i < n_rows, m < min(M, 8).
// R = weight rows per pass.
template <typename T, int R, class RowOf>
__device__ __forceinline__ void gemv_rows(const T *__restrict__ x, const T *__restrict__ W, int M, int H,
                                          RowOf row_of, int n_rows, float *res, float *red) {
    constexpr int NV = R * kStreamMaxRows;
    const int lane = lane_id(), wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int nch = H / 8;
    for (int p = 0; p < n_rows; p += R) {
        float acc[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] = 0.f;
        const T *wr[R];
#pragma unroll
        for (int i = 0; i < R; ++i) wr[i] = W + (size_t)row_of(min(p + i, n_rows - 1)) * H;
        for (int c = threadIdx.x; c < nch; c += blockDim.x) {
            float wf[R][8], xf[kStreamMaxRows][8];
#pragma unroll
            for (int i = 0; i < R; ++i) load8<T>(wr[i] + (size_t)c * 8, wf[i]);
#pragma unroll
            for (int m = 0; m < kStreamMaxRows; ++m) load8<T>(x + (size_t)min(m, M - 1) * H + (size_t)c * 8, xf[m]);
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int m = 0; m < kStreamMaxRows; ++m)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[i * kStreamMaxRows + m] = fmaf(wf[i][e], xf[m][e], acc[i * kStreamMaxRows + m]);
        }
        butterfly<NV, 32>(acc, lane);
        constexpr int SH = 6 - ilog2<NV>();
        if ((lane & ((1 << SH) - 1)) == 0) red[wave * NV + (lane >> SH)] = acc[0];
        __syncthreads();
        if ((int)threadIdx.x < NV) {
            float s = 0.f;
            for (int w = 0; w < nwaves; ++w) s += red[w * NV + threadIdx.x];
            const int i = threadIdx.x / kStreamMaxRows, m = threadIdx.x % kStreamMaxRows;
            if (p + i < n_rows) res[(p + i) * kStreamMaxRows + m] = s;
        }
        __syncthreads();
    }
}

// Context projection rows of workgroup b: g[m][b*R + j] = <h[m], w_h[b*R + j]>.
// The walk and teacher forcing both take g from here (same workgroup shape),
// so a replay scores with bit-equal context rows.
constexpr int kCtxRows = 2;
template <typename T>
__device__ __forceinline__ void ctx_rows(const T *__restrict__ h, const T *__restrict__ w_h, int M, int H, int r,
                                         float *__restrict__ g, float *red, float *res) {
    const int r0 = blockIdx.x * kCtxRows, nr = min(kCtxRows, r - r0);
    gemv_rows<T, kCtxRows>(h, w_h, M, H, [&](int i) { return r0 + i; }, nr, res, red);
    for (int i = threadIdx.x; i < nr * M; i += blockDim.x) {
        const int m = i / nr, j = i % nr;
        g[(size_t)m * r + r0 + j] = res[j * kStreamMaxRows + m];
    }
}
constexpr int kCtxRed = (kGemvThreads / 64) * kCtxRows * kStreamMaxRows;

}  // namespace dflash2
