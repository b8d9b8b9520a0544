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
// (s*T + j)*G + ct*Gw + gl.  TMAX bounds the taps at compile time.
template <typename T, int TMAX>
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
        if constexpr (sizeof(T) == 2) {
            if (nc % 8 == 0 && (g0 * gs) % 8 == 0) {
                // One item: 8 channels (a 16-byte chunk) of one row.  A thread
                // loads every tap operand of IB items before any sum, so the
                // loads overlap instead of each waiting out its latency; the
                // sums keep the tap order of the scalar path below.
                constexpr int IB = TMAX <= 2 ? 4 : TMAX <= 8 ? 2 : 1;
                const int chunks = nc / 8, items = nrows * chunks, h0 = g0 * gs;
                for (int i0 = threadIdx.x; i0 < items; i0 += IB * blockDim.x) {
                    uint4 xv[IB][TMAX], bv[IB][TMAX];
#pragma unroll
                    for (int ib = 0; ib < IB; ++ib) {
                        const int i = i0 + ib * blockDim.x, r = i / chunks, n = m0 + r;
                        const int hh = h0 + (i % chunks) * 8;
                        const bool live = i < items && n < M;
                        const int jmax = live ? min(taps - 1, n % bs) : -1;
#pragma unroll
                        for (int j = 0; j < TMAX; ++j) {
                            const bool ok = j <= jmax;
                            xv[ib][j] = ok ? *reinterpret_cast<const uint4 *>(x + (size_t)(n - j) * H + hh)
                                           : make_uint4(0u, 0u, 0u, 0u);
                            bv[ib][j] = ok ? *reinterpret_cast<const uint4 *>(base + (size_t)j * H + hh)
                                           : make_uint4(0u, 0u, 0u, 0u);
                        }
                    }
#pragma unroll
                    for (int ib = 0; ib < IB; ++ib) {
                        const int i = i0 + ib * blockDim.x, r = i / chunks, n = m0 + r, ch = i % chunks;
                        if (i >= items || n >= M) continue;
                        const int jmax = min(taps - 1, n % bs);
                        float acc[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
                        for (int j = 0; j < TMAX; ++j) {
                            if (j > jmax) break;
                            const uint32_t xw[4] = {xv[ib][j].x, xv[ib][j].y, xv[ib][j].z, xv[ib][j].w};
                            const uint32_t bw[4] = {bv[ib][j].x, bv[ib][j].y, bv[ib][j].z, bv[ib][j].w};
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float xf = bf16_to_f32((xw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
                                const float bf = bf16_to_f32((bw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
                                const int gl = (ch * 8 + e) / gs;
                                acc[e] = fmaf(bf + C[r * cs + j * Gw + gl], xf, acc[e]);
                            }
                        }
                        uint32_t ow[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            ow[e] = (uint32_t)f32_to_bf16(acc[2 * e]) | ((uint32_t)f32_to_bf16(acc[2 * e + 1]) << 16);
                        *reinterpret_cast<uint4 *>(x_out + (size_t)n * H + h0 + ch * 8) =
                            make_uint4(ow[0], ow[1], ow[2], ow[3]);
                    }
                }
                return;
            }
        }
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

// ------------------------------------------------------------ DMA-fed tiles (bf16)
//
// The same tiles for bf16 operands with a deep pipeline: the k loop walks
// 64-element stages through a ring of NS LDS stages that global_load_lds
// fills directly, NS - 1 stages ahead, so a workgroup's loads are not
// serialised behind its MFMAs (the projections have few output tiles, and a
// tile that waits out each load's latency leaves HBM idle).  Each wave waits
// for its own copies (counted waits) and one barrier per stage publishes
// them; the barrier waits for LDS only, so the later stages stay in flight.
// Row r of a stage holds 16-byte chunk c at position c ^ (r & 7): the rows
// one fragment read touches fall on distinct bank groups.
template <int BM_, int BN_, int NS_>
struct DmaTileCfg {
    static constexpr int BM = BM_, BN = BN_, NS = NS_;
    static constexpr int ROWS = BM + BN;
    static constexpr int STAGE = ROWS * 128;     // bytes: 64 k of every row
    static constexpr int CPW = ROWS / 32;        // 8-row copies per wave and stage
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int TM = WM / 16, TN = WN / 16;
    static constexpr int CSTRIDE = BN + 4;
    static constexpr int CTILE_BYTES = BM * CSTRIDE * 4;
    static constexpr int LDS = NS * STAGE > CTILE_BYTES ? NS * STAGE : CTILE_BYTES;
    static_assert(ROWS % 32 == 0 && TM >= 1 && TN >= 1 && NS >= 3, "tile shape");
};

// (row tile, column tile) of workgroup `bid` of n_rt * n_ct.  Workgroups are
// dispatched to the 8 XCDs in turn; each XCD takes a contiguous range of
// tiles, walked in bands of up to kProjBandRows row tiles, column by column,
// so the workgroups that run together on an XCD share A rows and W rows in
// its L2 instead of each XCD re-reading every row tile.
constexpr int kProjBandRows = 4;
__device__ __forceinline__ void proj_tile_of(int bid, int n_rt, int n_ct, int &rt, int &ct) {
    const int n = n_rt * n_ct;
    const int L = n % 8 == 0 ? (bid & 7) * (n >> 3) + (bid >> 3) : bid;
    int SM = kProjBandRows;
    while (n_rt % SM != 0) SM >>= 1;
    const int band = L / (SM * n_ct), rem = L % (SM * n_ct);
    ct = rem / SM;
    rt = band * SM + rem % SM;
}
using DmaTileBig = DmaTileCfg<64, 64, 4>;
using DmaTileSmall = DmaTileCfg<32, 32, 8>;

// KSPLIT = 2 (grids with fewer workgroups than CUs): 8 waves, two groups of
// 4 each with its own ring taking one half of the k stages, so a CU keeps
// twice the bytes in flight; group 1 hands its accumulators to group 0
// through LDS before the epilogue.  The groups run the same number of steps
// (a group with one stage fewer repeats its last copy and skips its MFMAs), so
// every wave meets every barrier.
template <class Cfg, class Epi, int KSPLIT>
__global__ __launch_bounds__(256 * KSPLIT) void proj_dma_kernel(const uint16_t *__restrict__ A,
                                                                const uint16_t *__restrict__ W, int M, int H,
                                                                int n_ct, Epi epi) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int NS = Cfg::NS, CPW = Cfg::CPW;
    int rt, ct;
    proj_tile_of(blockIdx.x, (M + Cfg::BM - 1) / Cfg::BM, n_ct, rt, ct);
    const int m0 = rt * Cfg::BM;
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lw = wave & 3, kg = wave >> 2;  // wave within its group, group
    const int wm = lw >> 1, wn = lw & 1, n = lane & 15, q = lane >> 4;
    uint8_t *ring = smem + (size_t)kg * NS * Cfg::STAGE;
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t *)ring;
    // this lane's chunk of each of its copies: stage row (lw CPW + c) 8 + L / 8
    // (A rows, then W rows), chunk (L % 8) ^ (row % 8).  Rows past M or past
    // the projection read row 0; their outputs are never used.
    const uint8_t *src[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int row = (lw * CPW + c) * 8 + (lane >> 3);
        const uint16_t *rp;
        if (row < Cfg::BM) {
            const int r = m0 + row;
            rp = A + (size_t)(r < M ? r : 0) * H;
        } else {
            const int wr = epi.col_row(ct, row - Cfg::BM, Cfg::BN);
            rp = W + (size_t)(wr >= 0 ? wr : 0) * H;
        }
        src[c] = reinterpret_cast<const uint8_t *>(rp) + (((lane & 7) ^ (row & 7)) << 4);
    }
    const int nk = H / 64;
    const int nk0 = KSPLIT == 1 ? nk : nk / 2;                   // group 0's stages
    const int k_begin = kg == 0 ? 0 : nk0, k_count = kg == 0 ? nk0 : nk - nk0;
    const int steps = nk - nk0 > nk0 ? nk - nk0 : nk0;           // both groups
    // local stage s (the group's last one again past its end) into slot s % NS
    auto issue = [&](int s) {
        const size_t kb = (size_t)(k_begin + (s < k_count ? s : k_count - 1)) * 128;
        const uint32_t base = lds0 + (uint32_t)((s % NS) * Cfg::STAGE + lw * CPW * 1024);
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const uint8_t *p = src[c] + kb;
            const uint32_t dst = base + (uint32_t)(c * 1024);
            // (s_nop: the wait state M0 needs after the SALU write before it;
            // the compiler adds none to inline assembly)
            asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(p), "{m0}"(dst) : "memory");
        }
    };
    f32x4 acc[Cfg::TM][Cfg::TN];
#pragma unroll
    for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
        for (int b = 0; b < Cfg::TN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < NS - 1; ++s) issue(s);
    for (int s = 0; s < steps; ++s) {
        // stage s has landed (the NS - 2 after it may still fly) in every wave,
        // and every wave has finished reading stage s - 1, whose slot is refilled
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(CPW * (NS - 2)) : "memory");
        issue(s + NS - 1);
        if (s >= k_count) continue;
        const uint8_t *st = ring + (s % NS) * Cfg::STAGE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int pos = ((ks * 4 + q) ^ (n & 7)) << 4;
            uint4 fa[Cfg::TM], fb[Cfg::TN];
#pragma unroll
            for (int a = 0; a < Cfg::TM; ++a)
                fa[a] = *reinterpret_cast<const uint4 *>(st + (wm * Cfg::WM + a * 16 + n) * 128 + pos);
#pragma unroll
            for (int b = 0; b < Cfg::TN; ++b)
                fb[b] = *reinterpret_cast<const uint4 *>(st + (Cfg::BM + wn * Cfg::WN + b * 16 + n) * 128 + pos);
#pragma unroll
            for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
                for (int b = 0; b < Cfg::TN; ++b) mma16<uint16_t>(acc[a][b], fa[a], fb[b]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float *C = reinterpret_cast<float *>(smem);
    if constexpr (KSPLIT == 2) {
        // group 1's accumulators, lane by lane, over its idle ring
        f32x4 *part = reinterpret_cast<f32x4 *>(smem + (size_t)NS * Cfg::STAGE) + (size_t)(lw * 64 + lane) * Cfg::TM * Cfg::TN;
        if (kg == 1) {
#pragma unroll
            for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
                for (int b = 0; b < Cfg::TN; ++b) part[a * Cfg::TN + b] = acc[a][b];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int a = 0; a < Cfg::TM; ++a)
#pragma unroll
                for (int b = 0; b < Cfg::TN; ++b) acc[a][b] += part[a * Cfg::TN + b];
            tiled_store_c<Cfg>(C, acc);
        }
    } else {
        tiled_store_c<Cfg>(C, acc);
    }
    __syncthreads();
    epi(C, Cfg::CSTRIDE, m0, min(Cfg::BM, M - m0), ct, Cfg::BN);
}

// ------------------------------------------------------------ host side

template <class Cfg, class Epi>
static hipError_t run_proj_dma(int64_t M, int H, int n_col_tiles, const void *A, const void *W, const Epi &epi,
                               hipStream_t stream) {
    const int n_rt = (int)((M + Cfg::BM - 1) / Cfg::BM);
    auto go = [&](auto kern, int ksplit) -> hipError_t {
        const int lds = ksplit * Cfg::NS * Cfg::STAGE > Cfg::LDS ? ksplit * Cfg::NS * Cfg::STAGE : Cfg::LDS;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(n_rt * n_col_tiles), dim3(256 * ksplit), lds, stream, (const uint16_t *)A,
                           (const uint16_t *)W, (int)M, H, n_col_tiles, epi);
        return hipGetLastError();
    };
    // fewer workgroups than CUs (one per CU): split k over two rings
    if (n_rt * n_col_tiles < 256 && H / 64 >= 2 && 2 * Cfg::NS * Cfg::STAGE <= 160 * 1024)
        return go(proj_dma_kernel<Cfg, Epi, 2>, 2);
    return go(proj_dma_kernel<Cfg, Epi, 1>, 1);
}

// The larger tile once its grid covers half the chip: larger tiles read fewer
// bytes per MFMA, and a workgroup's stream rate is bounded by the bytes its
// ring keeps in flight (measured on 512 rows x 5120 x 1280: 64 x 64 tiles on
// 160 workgroups 41 us, 32 x 32 tiles on 640 workgroups 46 us).
template <class Cfg> static bool proj_fills(int64_t M, int n_col_tiles) {
    return (M + Cfg::BM - 1) / Cfg::BM * n_col_tiles >= 128;
}

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

template <typename T, int TMAX>
static hipError_t run_conv_tiles(int64_t N, int bs, int H, int taps, int gs, const void *x, const void *w_proj,
                                 const void *base, void *x_out, float *k_post, hipStream_t stream) {
    const int G = H / gs;
    EpiConv<T, TMAX> epi{(const T *)x, (const T *)base, (T *)x_out, k_post, (int)N, H, bs, taps, gs, G, 0};
    if constexpr (sizeof(T) == 2) {
        // Gw groups per tile: the 2 T projection rows of each
        auto run = [&](auto cfg) -> hipError_t {
            using Cfg = decltype(cfg);
            epi.Gw = Cfg::BN / (2 * taps);
            return run_proj_dma<Cfg>(N, H, (G + epi.Gw - 1) / epi.Gw, x, w_proj, epi, stream);
        };
        auto n_ct = [&](int bn) { return (G + bn / (2 * taps) - 1) / (bn / (2 * taps)); };
        if (proj_fills<DmaTileBig>(N, n_ct(DmaTileBig::BN))) return run(DmaTileBig{});
        return run(DmaTileSmall{});
    }
    epi.Gw = kProjTile / (2 * taps);
    const int n_ct = (G + epi.Gw - 1) / epi.Gw;
    return run_proj_tiled<T>(N, H, n_ct, x, w_proj, epi, stream);
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
    if (taps <= 2) return run_conv_tiles<T, 2>(N, bs, H, taps, gs, x, w_proj, base, x_out, k_post, stream);
    if (taps <= 4) return run_conv_tiles<T, 4>(N, bs, H, taps, gs, x, w_proj, base, x_out, k_post, stream);
    if (taps <= 8) return run_conv_tiles<T, 8>(N, bs, H, taps, gs, x, w_proj, base, x_out, k_post, stream);
    return run_conv_tiles<T, 16>(N, bs, H, taps, gs, x, w_proj, base, x_out, k_post, stream);
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
    if constexpr (sizeof(T) == 2) {
        auto run = [&](auto cfg) -> hipError_t {
            using Cfg = decltype(cfg);
            return run_proj_dma<Cfg>(N, H, (r + Cfg::BN - 1) / Cfg::BN, h, w_h, epi, stream);
        };
        if (proj_fills<DmaTileBig>(N, (r + DmaTileBig::BN - 1) / DmaTileBig::BN)) return run(DmaTileBig{});
        return run(DmaTileSmall{});
    }
    return run_proj_tiled<T>(N, H, (r + kProjTile - 1) / kProjTile, h, w_h, epi, stream);
}

hipError_t launch_context_proj(int dtype, int64_t N, int H, int r, const void *h, const void *w_h,
                               float *g, uint32_t *status, hipStream_t stream) {
    if (dtype == 0) return run_context_proj<float>(N, H, r, h, w_h, g, status, stream);
    return run_context_proj<uint16_t>(N, H, r, h, w_h, g, status, stream);
}

}  // namespace dflash2
