// Post-sublayer half of the grouped dynamic causal convolution:
//   y_out[n, h] = sum_{j <= min(T-1, n mod bs)} (base[1, j, h] + k_post[n, j, h / gs]) * y[n - j, h]
// Purely bandwidth-bound.  One thread owns 8 consecutive channels of one row
// and reads the T (or fewer, at a block start) rows it taps; the rows a
// neighbour thread also taps are served from cache.  No tap crosses an anchor
// block.
#include "common.hpp"
#include "launch.hpp"

namespace dflash2 {

template <typename T>
__global__ __launch_bounds__(256) void conv_finish_kernel(const T *__restrict__ y, const float *__restrict__ k_post,
                                                          const T *__restrict__ base, T *__restrict__ y_out,
                                                          long long N, int bs, int H, int taps, int gs, int G) {
    const int chunks = H / 8;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= N * chunks) return;
    const long long n = gid / chunks;
    const int h0 = (int)(gid % chunks) * 8;
    const int jmax = min(taps - 1, (int)(n % bs));
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j <= jmax; ++j) {
        float v[8], b[8];
        load8<T>(y + (size_t)(n - j) * H + h0, v);
        load8<T>(base + (size_t)(taps + j) * H + h0, b);
        const float *kp = k_post + ((size_t)n * taps + j) * G;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(b[c] + kp[(h0 + c) / gs], v[c], acc[c]);
    }
    store8<T>(y_out + (size_t)n * H + h0, acc);
}

hipError_t launch_conv_finish(int dtype, int64_t N, int bs, int H, int taps, int gs, const void *y,
                              const float *k_post, const void *base, void *y_out, hipStream_t stream) {
    const long long threads = (long long)N * (H / 8);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    const int G = H / gs;
    if (dtype == 0)
        hipLaunchKernelGGL(conv_finish_kernel<float>, dim3(grid), dim3(256), 0, stream, (const float *)y,
                           k_post, (const float *)base, (float *)y_out, (long long)N, bs, H, taps, gs, G);
    else
        hipLaunchKernelGGL(conv_finish_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                           (const uint16_t *)y, k_post, (const uint16_t *)base, (uint16_t *)y_out,
                           (long long)N, bs, H, taps, gs, G);
    return hipGetLastError();
}

}  // namespace dflash2
