// Post-sublayer half of the grouped dynamic causal convolution:
//   y_out[n, h] = sum_{j <= min(T-1, n mod bs)} (base[1, j, h] + k_post[n, j, h / gs]) * y[n - j, h]
// Purely bandwidth-bound.  One thread owns 8 consecutive channels of one row.
// Every tap's loads are issued together: a tap that would reach before the
// block start reads a clamped in-block row and is weighted by zero, so no tap
// crosses an anchor block and no load waits on another.
#include "common.hpp"
#include "launch.hpp"

namespace dflash2 {

template <typename T, int TMAX, bool GS8>
__global__ __launch_bounds__(256) void conv_finish_kernel(const T *__restrict__ y, const float *__restrict__ k_post,
                                                          const T *__restrict__ base, T *__restrict__ y_out,
                                                          long long N, int bs, int H, int taps, int gs, int G) {
    const int chunks = H / 8;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= N * chunks) return;
    const long long n = gid / chunks;
    const int h0 = (int)(gid % chunks) * 8;
    const int p = (int)(n % bs);
    float v[TMAX][8], b[TMAX][8], kp[TMAX][8];
#pragma unroll
    for (int j = 0; j < TMAX; ++j) {
        const int jj = min(j, taps - 1);
        const long long src = n - min(j, p);  // stays inside the block
        load8<T>(y + (size_t)src * H + h0, v[j]);
        load8<T>(base + (size_t)(taps + jj) * H + h0, b[j]);
        const float *kr = k_post + ((size_t)n * taps + jj) * G;
        if constexpr (GS8) {  // the 8 channels share one group
            const float k = kr[h0 / gs];
#pragma unroll
            for (int c = 0; c < 8; ++c) kp[j][c] = k;
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) kp[j][c] = kr[(h0 + c) / gs];
        }
    }
    const int jmax = min(taps - 1, p);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < TMAX; ++j) {
        if (j <= jmax) {
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = fmaf(b[j][c] + kp[j][c], v[j][c], acc[c]);
        }
    }
    store8<T>(y_out + (size_t)n * H + h0, acc);
}

template <typename T, int TMAX>
static void launch_finish(unsigned grid, unsigned block, hipStream_t stream, const void *y, const float *k_post,
                          const void *base, void *y_out, long long N, int bs, int H, int taps, int gs, int G) {
    if (gs % 8 == 0)
        hipLaunchKernelGGL((conv_finish_kernel<T, TMAX, true>), dim3(grid), dim3(block), 0, stream, (const T *)y,
                           k_post, (const T *)base, (T *)y_out, N, bs, H, taps, gs, G);
    else
        hipLaunchKernelGGL((conv_finish_kernel<T, TMAX, false>), dim3(grid), dim3(block), 0, stream, (const T *)y,
                           k_post, (const T *)base, (T *)y_out, N, bs, H, taps, gs, G);
}

template <typename T>
static hipError_t run_finish(int64_t N, int bs, int H, int taps, int gs, const void *y, const float *k_post,
                             const void *base, void *y_out, hipStream_t stream) {
    const long long threads = (long long)N * (H / 8);
    // small launches: narrow workgroups spread the rows over more CUs
    const unsigned block = threads < 256 * 1024 ? 64 : 256;
    const unsigned grid = (unsigned)((threads + block - 1) / block);
    const int G = H / gs;
    if (taps <= 2) launch_finish<T, 2>(grid, block, stream, y, k_post, base, y_out, N, bs, H, taps, gs, G);
    else if (taps <= 4) launch_finish<T, 4>(grid, block, stream, y, k_post, base, y_out, N, bs, H, taps, gs, G);
    else if (taps <= 8) launch_finish<T, 8>(grid, block, stream, y, k_post, base, y_out, N, bs, H, taps, gs, G);
    else launch_finish<T, 16>(grid, block, stream, y, k_post, base, y_out, N, bs, H, taps, gs, G);
    return hipGetLastError();
}

hipError_t launch_conv_finish(int dtype, int64_t N, int bs, int H, int taps, int gs, const void *y,
                              const float *k_post, const void *base, void *y_out, hipStream_t stream) {
    if (dtype == 0) return run_finish<float>(N, bs, H, taps, gs, y, k_post, base, y_out, stream);
    return run_finish<uint16_t>(N, bs, H, taps, gs, y, k_post, base, y_out, stream);
}

}  // namespace dflash2
