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
    struct Pre {};
    __device__ Pre prefetch(int /*ct*/) const { return {}; }
    __device__ void stage(uint8_t * /*lds*/, const Pre &) const {}
    __device__ int col_row(int ct, int c, int tile_cols) const {
        const int col = ct * tile_cols + c;
        return col < ncol_total ? col : -1;
    }
    __device__ void operator()(const float *C, int cs, int m0, int nrows, int ct, int tile_cols,
                               const uint8_t * /*lds*/ = nullptr) const {
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
    // Streaming regime (at most 8 rows): the tile's x rows and input-kernel
    // base are fetched before the contraction (one 16-byte chunk per thread),
    // parked in registers and written to LDS after it.
    struct Pre {
        uint4 xv, bv;
        int xi, bi;
    };
    __device__ int nch(int ct) const { return (min(G, ct * Gw + Gw) - ct * Gw) * gs; }
    __device__ Pre prefetch(int ct) const {
        constexpr int E = 16 / (int)sizeof(T);
        const int h0 = ct * Gw * gs, nc = nch(ct), cpr = nc / E;  // chunks per row
        Pre p;
        p.xi = p.bi = -1;
        const int t = threadIdx.x;
        if (t < min(M, kStreamMaxRows) * cpr) {
            p.xi = t;
            p.xv = *reinterpret_cast<const uint4 *>(x + (size_t)(t / cpr) * H + h0 + (t % cpr) * E);
        }
        if (t < taps * cpr) {
            p.bi = t;
            p.bv = *reinterpret_cast<const uint4 *>(base + (size_t)(t / cpr) * H + h0 + (t % cpr) * E);
        }
        return p;
    }
    __device__ void stage(uint8_t *lds, const Pre &p) const {
        uint4 *xs = reinterpret_cast<uint4 *>(lds);
        if (p.xi >= 0) xs[p.xi] = p.xv;
        if (p.bi >= 0) xs[kStreamMaxRows * 512 / (16 / (int)sizeof(T)) + p.bi] = p.bv;
    }
    __device__ void operator()(const float *C, int cs, int m0, int nrows, int ct, int /*tile_cols*/,
                               const uint8_t *lds = nullptr) const {
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
        const T *xs = reinterpret_cast<const T *>(lds);
        const T *bsm = xs + kStreamMaxRows * 512;
        for (int i = threadIdx.x; i < nrows * nc; i += blockDim.x) {
            const int r = i / nc, hc = i % nc;
            const int n = m0 + r;
            if (n >= M) continue;
            const int hh = g0 * gs + hc, gl = hc / gs;
            const int jmax = min(taps - 1, n % bs);
            float acc = 0.f;
            for (int j = 0; j <= jmax; ++j) {
                float bj, xj;
                if (lds) {  // rows n - j < 8 of this tile, staged in LDS
                    bj = Elem<T>::f32(bsm[j * nc + hc]);
                    xj = Elem<T>::f32(xs[(n - j) * nc + hc]);
                } else {
                    bj = Elem<T>::f32(base[(size_t)j * H + hh]);
                    xj = Elem<T>::f32(x[(size_t)(n - j) * H + hh]);
                }
                acc = fmaf(bj + C[r * cs + j * Gw + gl], xj, acc);
            }
            x_out[(size_t)n * H + hh] = Elem<T>::from_f32(acc);
        }
    }
};

// ------------------------------------------------------------ streaming
// Workgroup = 16 waves on one 16-column tile; wave w reduces k-steps
// [w*S/16, (w+1)*S/16) and the partial tiles are summed through LDS.
constexpr int kProjWaves = 16;
constexpr int kDF2MaxTapsStream = 8;  // 2T <= 16 in the streaming regime

template <typename T, class Epi>
__global__ __launch_bounds__(64 * kProjWaves) void proj_stream_kernel(const T *__restrict__ A,
                                                                      const T *__restrict__ W, int M,
                                                                      int H, Epi epi) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int KC = 16 / (int)sizeof(T);
    constexpr int KS = 4 * KC;
    const int S = H / KS;
    f32x4 *red = reinterpret_cast<f32x4 *>(smem);             // [16 waves][64 lanes]
    float *C = reinterpret_cast<float *>(red + kProjWaves * 64);  // [16][17]
    uint8_t *epi_lds = reinterpret_cast<uint8_t *>(C + 16 * 17);
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int ct = blockIdx.x;
    const typename Epi::Pre pre = epi.prefetch(ct);
    const int m = lane & 15, q = lane >> 4;
    const T *arow = m < M ? A + (size_t)m * H + q * KC : nullptr;
    const int wrow = epi.col_row(ct, m, 16);
    const T *brow = wrow >= 0 ? W + (size_t)wrow * H + q * KC : nullptr;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int s0 = wave * S / kProjWaves, s1 = (wave + 1) * S / kProjWaves;
    for (int s = s0; s < s1; s += 8) {
        uint4 a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = b[i] = make_uint4(0u, 0u, 0u, 0u);
            if (s + i < s1) {
                if (arow) a[i] = *reinterpret_cast<const uint4 *>(arow + (size_t)(s + i) * KS);
                if (brow) b[i] = *reinterpret_cast<const uint4 *>(brow + (size_t)(s + i) * KS);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (s + i < s1) mma16<T>(acc, a[i], b[i]);
    }
    red[wave * 64 + lane] = acc;
    epi.stage(epi_lds, pre);
    __syncthreads();
    if (threadIdx.x < 256) {
        const int l = threadIdx.x & 63, i = threadIdx.x >> 6;
        float sum = 0.f;
        for (int ww = 0; ww < kProjWaves; ++ww) sum += red[ww * 64 + l][i];
        C[(4 * (l >> 4) + i) * 17 + (l & 15)] = sum;
    }
    __syncthreads();
    epi(C, 17, 0, min(M, kStreamMaxRows), ct, 16, epi_lds);
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
        const size_t lds = (size_t)kProjWaves * 64 * 16 + 16 * 17 * 4 +
                           (size_t)(kStreamMaxRows + kDF2MaxTapsStream) * 512 * sizeof(T);
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

bool proj_streaming(int64_t M, int /*H*/, int /*dtype*/) { return M <= kStreamMaxRows; }

template <typename T>
static hipError_t run_conv_prepare(int64_t N, int bs, int H, int taps, int gs, const void *x,
                                   const void *w_proj, const void *base, void *x_out, float *k_post,
                                   hipStream_t stream, int dtype) {
    const int G = H / gs;
    // streaming needs one MFMA tile to hold whole groups (2T <= 16) and the
    // tile's channels to fit the LDS staging (at most 512)
    constexpr int E = 16 / (int)sizeof(T);
    const int gw_s = 2 * taps <= 16 ? 16 / (2 * taps) : 1;
    const bool streaming = proj_streaming(N, H, dtype) && 2 * taps <= 16 && gw_s * gs <= 512 &&
                           (gw_s * gs) % E == 0 && ((G % gw_s) * gs) % E == 0;
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
