// Hidden-state projections with fused epilogues:
//  * conv prepare: c = x w_proj^T, then the block-local taps of the input
//    kernel and the output kernel's dynamic part (k_post), in one kernel;
//  * context projection g = h w_h^T for the selector (float32 out).
// Streaming regime for at most 8 rows (weights streamed once, the reduction
// over H split across 16 waves), tiled MFMA regime otherwise.
#include "common.hpp"
#include "gemm.hpp"
#include "launch.hpp"

namespace dflash2 {

// ------------------------------------------------------------ epilogues
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
        const int nch = gn * gs;
        for (int i = threadIdx.x; i < nrows * nch; i += blockDim.x) {
            const int r = i / nch, hc = i % nch;
            const int n = m0 + r;
            if (n >= M) continue;
            const int hh = g0 * gs + hc, gl = hc / gs;
            const int jmax = min(taps - 1, n % bs);
            float acc = 0.f;
            for (int j = 0; j <= jmax; ++j) {
                const float k = Elem<T>::f32(base[(size_t)j * H + hh]) + C[r * cs + j * Gw + gl];
                acc = fmaf(k, Elem<T>::f32(x[(size_t)(n - j) * H + hh]), acc);
            }
            x_out[(size_t)n * H + hh] = Elem<T>::from_f32(acc);
        }
    }
};

// ------------------------------------------------------------ streaming
// Workgroup = 16 waves on one 16-column tile; wave w reduces k-steps
// [w*S/16, (w+1)*S/16) and the partial tiles are summed through LDS.
constexpr int kProjWaves = 16;

template <typename T, class Epi>
__global__ __launch_bounds__(64 * kProjWaves) void proj_stream_kernel(const T *__restrict__ A,
                                                                      const T *__restrict__ W, int M,
                                                                      int H, Epi epi) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int KC = 16 / (int)sizeof(T);
    const int S = H / kstep_elems<T>();
    uint4 *afrag = reinterpret_cast<uint4 *>(smem);
    f32x4 *red = reinterpret_cast<f32x4 *>(smem + (size_t)S * 32 * 16);  // [16 waves][64 lanes]
    float *C = reinterpret_cast<float *>(red + kProjWaves * 64);        // [16][17]
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int ct = blockIdx.x;
    load_afrag<T>(afrag, A, M, H);
    __syncthreads();
    const int wrow = epi.col_row(ct, lane & 15, 16);
    const T *brow = wrow >= 0 ? W + (size_t)wrow * H + (lane >> 4) * KC : nullptr;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    stream_accumulate<T>(acc, afrag, brow, wave * S / kProjWaves, (wave + 1) * S / kProjWaves);
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (threadIdx.x < 256) {
        const int l = threadIdx.x & 63, i = threadIdx.x >> 6;
        float s = 0.f;
        for (int ww = 0; ww < kProjWaves; ++ww) s += red[ww * 64 + l][i];
        C[(4 * (l >> 4) + i) * 17 + (l & 15)] = s;
    }
    __syncthreads();
    epi(C, 17, 0, min(M, kStreamMaxRows), ct, 16);
}

// ------------------------------------------------------------ tiled
template <typename T, class Epi>
__global__ __launch_bounds__(256) void proj_tiled_kernel(const T *__restrict__ A, const T *__restrict__ W,
                                                         int M, int H, Epi epi) {
    using Cfg = TiledCfg<T, 128, 128>;
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
static hipError_t run_proj(int64_t M, int H, int n_col_tiles_stream, int n_col_tiles_tiled,
                           const void *A, const void *W, const Epi &epi, bool streaming,
                           hipStream_t stream) {
    hipError_t e;
    if (streaming) {
        const int S = H / kstep_elems<T>();
        const size_t lds = (size_t)S * 32 * 16 + (size_t)kProjWaves * 64 * 16 + 16 * 17 * 4;
        auto kern = proj_stream_kernel<T, Epi>;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(n_col_tiles_stream), dim3(64 * kProjWaves), lds, stream,
                           (const T *)A, (const T *)W, (int)M, H, epi);
    } else {
        using Cfg = TiledCfg<T, 128, 128>;
        const size_t lds = Cfg::STAGE_BYTES > Cfg::CTILE_BYTES ? Cfg::STAGE_BYTES : Cfg::CTILE_BYTES;
        auto kern = proj_tiled_kernel<T, Epi>;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(n_col_tiles_tiled, (unsigned)((M + 127) / 128)), dim3(256), lds,
                           stream, (const T *)A, (const T *)W, (int)M, H, epi);
    }
    return hipGetLastError();
}

bool proj_streaming(int64_t M, int H, int dtype) {
    // the fragment copy of A must fit in LDS next to the reduction buffers
    const int es = dtype == 0 ? 4 : 2;
    const size_t afrag = (size_t)(H / (4 * (16 / es))) * 32 * 16;
    return M <= kStreamMaxRows && afrag <= 96 * 1024;
}

template <typename T>
static hipError_t run_conv_prepare(int64_t N, int bs, int H, int taps, int gs, const void *x,
                                   const void *w_proj, const void *base, void *x_out, float *k_post,
                                   hipStream_t stream, int dtype) {
    const int G = H / gs;
    const bool streaming = proj_streaming(N, H, dtype) && 2 * taps <= 16;
    EpiConv<T> epi{(const T *)x, (const T *)base, (T *)x_out, k_post, (int)N, H, bs, taps, gs, G, 0};
    if (streaming) {
        epi.Gw = 16 / (2 * taps);
        const int n_ct = (G + epi.Gw - 1) / epi.Gw;
        return run_proj<T>(N, H, n_ct, 0, x, w_proj, epi, true, stream);
    }
    epi.Gw = 128 / (2 * taps);
    const int n_ct = (G + epi.Gw - 1) / epi.Gw;
    return run_proj<T>(N, H, 0, n_ct, x, w_proj, epi, false, stream);
}

hipError_t launch_conv_prepare(int dtype, int64_t N, int bs, int H, int taps, int gs, const void *x,
                               const void *w_proj, const void *base, void *x_out, float *k_post,
                               hipStream_t stream) {
    if (dtype == 0)
        return run_conv_prepare<float>(N, bs, H, taps, gs, x, w_proj, base, x_out, k_post, stream, dtype);
    return run_conv_prepare<uint16_t>(N, bs, H, taps, gs, x, w_proj, base, x_out, k_post, stream, dtype);
}

hipError_t launch_context_proj(int dtype, int64_t N, int H, int r, const void *h, const void *w_h,
                               float *g, uint32_t *status, hipStream_t stream) {
    EpiStore epi{g, (int)N, r, status};
    const bool streaming = proj_streaming(N, H, dtype);
    if (dtype == 0)
        return run_proj<float>(N, H, (r + 15) / 16, (r + 127) / 128, h, w_h, epi, streaming, stream);
    return run_proj<uint16_t>(N, H, (r + 15) / 16, (r + 127) / 128, h, w_h, epi, streaming, stream);
}

}  // namespace dflash2
