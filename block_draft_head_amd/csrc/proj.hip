// Hidden-state projections with fused epilogues:
//  * conv prepare: c = x w_proj^T, then the block-local taps of the input
//    kernel and the output kernel's dynamic part (k_post), in one kernel;
//  * context projection g = h w_h^T for the selector (float32 out).
// At most 8 rows: weight streaming on the vector ALUs (below).  More rows:
// LDS-tiled MFMA with the epilogue applied to the C tile in LDS.
#include "common.hpp"
#include "gemm.hpp"
#include "gemv.hpp"
#include "launch.hpp"

namespace dflash2 {

// Context projection: workgroup b owns rows [b*R, b*R + R) of w_h.
template <typename T>
__global__ __launch_bounds__(kGemvThreads) void ctx_gemv_kernel(const T *__restrict__ h, const T *__restrict__ w_h,
                                                                int M, int H, int r, float *__restrict__ g,
                                                                uint32_t *__restrict__ status) {
    __shared__ float red[kCtxRed];
    __shared__ float res[kCtxRows * kStreamMaxRows];
    if (blockIdx.x == 0 && threadIdx.x == 0 && status) *status = 0u;
    ctx_rows<T>(h, w_h, M, H, r, g, red, res);
}

// Conv prepare: workgroup g owns group g, i.e. projection rows (s*T + j)*G + g
// for s in {0, 1}, j < T; then applies the input kernel to the group's gs
// channels and writes the output kernel's dynamic part.
//
// The operands of the taps (x and the input base kernel at the group's
// channels) do not depend on the projection: the threads that apply a tap
// fetch them before the contraction.  TMAX bounds the taps at compile time.
template <typename T, int TMAX>
__global__ __launch_bounds__(kGemvThreads) void conv_gemv_kernel(const T *__restrict__ x, const T *__restrict__ w_proj,
                                                                 const T *__restrict__ base, T *__restrict__ x_out,
                                                                 float *__restrict__ k_post, int M, int H, int bs,
                                                                 int taps, int gs) {
    constexpr int R = 4;
    __shared__ float red[(kGemvThreads / 64) * R * kStreamMaxRows];
    __shared__ float res[kGemvMaxRows * kStreamMaxRows];
    const int g = blockIdx.x, G = H / gs, nr = 2 * taps;
    // thread i < M * gs owns output (m, channel g*gs + i % gs)
    const int i_out = threadIdx.x;
    const bool owns = i_out < M * gs && M * gs <= (int)blockDim.x;
    const int m = owns ? i_out / gs : 0, hh = g * gs + (owns ? i_out % gs : 0);
    const int jmax = min(taps - 1, m % bs);
    float bj[TMAX], xj[TMAX];
#pragma unroll
    for (int j = 0; j < TMAX; ++j) {
        bj[j] = xj[j] = 0.f;
        if (owns && j <= jmax) {
            bj[j] = Elem<T>::f32(base[(size_t)j * H + hh]);
            xj[j] = Elem<T>::f32(x[(size_t)(m - j) * H + hh]);
        }
    }
    gemv_rows<T, R>(x, w_proj, M, H, [&](int i) { return i * G + g; }, nr, res, red);
    // k_post[m][j][g] = c[m, s=1, j]
    for (int i = threadIdx.x; i < M * taps; i += blockDim.x) {
        const int mm = i / taps, j = i % taps;
        k_post[((size_t)mm * taps + j) * G + g] = res[(taps + j) * kStreamMaxRows + mm];
    }
    // x_out over the group's channels, taps inside the block only
    if (owns) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < TMAX; ++j)
            if (j <= jmax) acc = fmaf(bj[j] + res[j * kStreamMaxRows + m], xj[j], acc);
        x_out[(size_t)m * H + hh] = Elem<T>::from_f32(acc);
    } else {
        for (int i = threadIdx.x; i < M * gs; i += blockDim.x) {  // groups wider than the workgroup
            const int mm = i / gs, h2 = g * gs + i % gs;
            const int jm = min(taps - 1, mm % bs);
            float acc = 0.f;
            for (int j = 0; j <= jm; ++j)
                acc = fmaf(Elem<T>::f32(base[(size_t)j * H + h2]) + res[j * kStreamMaxRows + mm],
                           Elem<T>::f32(x[(size_t)(mm - j) * H + h2]), acc);
            x_out[(size_t)mm * H + h2] = Elem<T>::from_f32(acc);
        }
    }
}

// ------------------------------------------------------------ tiled epilogues
// An epilogue sees a float C tile in LDS: rows [m0, m0 + nrows) of the
// output, tile columns [0, ncols), row stride cs.  Column c of tile `ct`
// maps to a projection output row through col_row().

struct EpiStore {  // out[m][col] for col < ncol_total; clears the status word
    float *out;
    int M, ncol_total;
    uint32_t *status;
    __device__ int col_row(int ct, int c, int tile_cols) const {
        const int col = ct * tile_cols + c;
        return col < ncol_total ? col : -1;
    }
    __device__ void operator()(const float *C, int cs, int m0, int nrows, int ct, int tile_cols) const {
        if (status && ct == 0 && m0 == 0 && threadIdx.x == 0) *status = 0u;
        for (int i = threadIdx.x; i < nrows * tile_cols; i += blockDim.x) {
            const int r = i / tile_cols, c = i % tile_cols;
            const int col = ct * tile_cols + c;
            if (m0 + r < M && col < ncol_total) out[(size_t)(m0 + r) * ncol_total + col] = C[r * cs + c];
        }
    }
};

// Conv prepare.  Tile ct covers groups [ct*Gw, ct*Gw + Gw); tile column
// c = (s*T + j)*Gw + gl holds c[n, s, j, ct*Gw + gl], i.e. projection row
// (s*T + j)*G + ct*Gw + gl.
template <typename T>
struct EpiConv {
    const T *x, *base;
    T *x_out;
    float *k_post;
    int M, H, bs, taps, gs, G, Gw;
    __device__ int col_row(int ct, int c, int /*tile_cols*/) const {
        const int sj = c / Gw, gl = c % Gw, g = ct * Gw + gl;
        return (sj < 2 * taps && g < G) ? sj * G + g : -1;
    }
    __device__ void operator()(const float *C, int cs, int m0, int nrows, int ct, int /*tile_cols*/) const {
        const int g0 = ct * Gw;
        const int gn = min(G, g0 + Gw) - g0;
        // dynamic part of the output kernel
        for (int i = threadIdx.x; i < nrows * taps * gn; i += blockDim.x) {
            const int r = i / (taps * gn), rem = i % (taps * gn), j = rem / gn, gl = rem % gn;
            const int n = m0 + r;
            if (n < M) k_post[((size_t)n * taps + j) * G + g0 + gl] = C[r * cs + (taps + j) * Gw + gl];
        }
        // input kernel applied block-locally
        const int nc = gn * gs;
        for (int i = threadIdx.x; i < nrows * nc; i += blockDim.x) {
            const int r = i / nc, hc = i % nc;
            const int n = m0 + r;
            if (n >= M) continue;
            const int hh = g0 * gs + hc, gl = hc / gs;
            const int jmax = min(taps - 1, n % bs);
            float acc = 0.f;
            for (int j = 0; j <= jmax; ++j)
                acc = fmaf(Elem<T>::f32(base[(size_t)j * H + hh]) + C[r * cs + j * Gw + gl],
                           Elem<T>::f32(x[(size_t)(n - j) * H + hh]), acc);
            x_out[(size_t)n * H + hh] = Elem<T>::from_f32(acc);
        }
    }
};

// ------------------------------------------------------------ tiled
// 64 x 64 tiles: the projections have few output columns (2·T·G or r), so
// larger tiles would leave most CUs idle.
constexpr int kProjTile = 64;

template <typename T, class Epi>
__global__ __launch_bounds__(256) void proj_tiled_kernel(const T *__restrict__ A, const T *__restrict__ W,
                                                         int M, int H, Epi epi) {
    using Cfg = TiledCfg<T, kProjTile, kProjTile>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int ct = blockIdx.x, m0 = blockIdx.y * Cfg::BM;
    f32x4 acc[Cfg::TM][Cfg::TN];
    tiled_mainloop<T, Cfg>(
        acc, smem,
        [&](int i) -> const T * { const int r = m0 + i; return r < M ? A + (size_t)r * H : nullptr; },
        [&](int j) -> const T * { const int wr = epi.col_row(ct, j, Cfg::BN); return wr >= 0 ? W + (size_t)wr * H : nullptr; },
        H);
    __syncthreads();
    float *C = reinterpret_cast<float *>(smem);
    tiled_store_c<Cfg>(C, acc);
    __syncthreads();
    epi(C, Cfg::CSTRIDE, m0, min(Cfg::BM, M - m0), ct, Cfg::BN);
}

// ------------------------------------------------------------ host side

template <typename T, class Epi>
static hipError_t run_proj_tiled(int64_t M, int H, int n_col_tiles, const void *A, const void *W, const Epi &epi,
                                 hipStream_t stream) {
    using Cfg = TiledCfg<T, kProjTile, kProjTile>;
    const size_t lds = Cfg::STAGE_BYTES > Cfg::CTILE_BYTES ? Cfg::STAGE_BYTES : Cfg::CTILE_BYTES;
    auto kern = proj_tiled_kernel<T, Epi>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_col_tiles, (unsigned)((M + kProjTile - 1) / kProjTile)), dim3(256), lds, stream,
                       (const T *)A, (const T *)W, (int)M, H, epi);
    return hipGetLastError();
}

template <typename T>
static hipError_t run_conv_prepare(int64_t N, int bs, int H, int taps, int gs, const void *x,
                                   const void *w_proj, const void *base, void *x_out, float *k_post,
                                   hipStream_t stream) {
    const int G = H / gs;
    if (N <= kStreamMaxRows) {
        const dim3 grid(G), block(kGemvThreads);
        if (taps <= 2)
            hipLaunchKernelGGL((conv_gemv_kernel<T, 2>), grid, block, 0, stream, (const T *)x, (const T *)w_proj,
                               (const T *)base, (T *)x_out, k_post, (int)N, H, bs, taps, gs);
        else if (taps <= 4)
            hipLaunchKernelGGL((conv_gemv_kernel<T, 4>), grid, block, 0, stream, (const T *)x, (const T *)w_proj,
                               (const T *)base, (T *)x_out, k_post, (int)N, H, bs, taps, gs);
        else
            hipLaunchKernelGGL((conv_gemv_kernel<T, 16>), grid, block, 0, stream, (const T *)x, (const T *)w_proj,
                               (const T *)base, (T *)x_out, k_post, (int)N, H, bs, taps, gs);
        return hipGetLastError();
    }
    EpiConv<T> epi{(const T *)x, (const T *)base, (T *)x_out, k_post, (int)N, H, bs, taps, gs, G, 0};
    epi.Gw = kProjTile / (2 * taps);
    const int n_ct = (G + epi.Gw - 1) / epi.Gw;
    return run_proj_tiled<T>(N, H, n_ct, x, w_proj, epi, stream);
}

hipError_t launch_conv_prepare(int dtype, int64_t N, int bs, int H, int taps, int gs, const void *x,
                               const void *w_proj, const void *base, void *x_out, float *k_post,
                               hipStream_t stream) {
    if (dtype == 0) return run_conv_prepare<float>(N, bs, H, taps, gs, x, w_proj, base, x_out, k_post, stream);
    return run_conv_prepare<uint16_t>(N, bs, H, taps, gs, x, w_proj, base, x_out, k_post, stream);
}

template <typename T>
static hipError_t run_context_proj(int64_t N, int H, int r, const void *h, const void *w_h, float *g,
                                   uint32_t *status, hipStream_t stream) {
    if (N <= kStreamMaxRows) {
        hipLaunchKernelGGL(ctx_gemv_kernel<T>, dim3((r + kCtxRows - 1) / kCtxRows), dim3(kGemvThreads), 0, stream,
                           (const T *)h, (const T *)w_h, (int)N, H, r, g, status);
        return hipGetLastError();
    }
    EpiStore epi{g, (int)N, r, status};
    return run_proj_tiled<T>(N, H, (r + kProjTile - 1) / kProjTile, h, w_h, epi, stream);
}

hipError_t launch_context_proj(int dtype, int64_t N, int H, int r, const void *h, const void *w_h,
                               float *g, uint32_t *status, hipStream_t stream) {
    if (dtype == 0) return run_context_proj<float>(N, H, r, h, w_h, g, status, stream);
    return run_context_proj<uint16_t>(N, H, r, h, w_h, g, status, stream);
}

}  // namespace dflash2
