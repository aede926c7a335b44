// LayerNorm backward, the parameter part: the gradients with respect to
// gamma and beta are sums over the rows (CREDIT paper, Sec. IV-A, the
// LayerNorm workload):
//   dgamma_j = sum_i dy_ij xhat_ij,   dbeta_j = sum_i dy_ij,
//   xhat_ij = (x_ij - mean_i) rstd_i,
// with each row's mean and rstd as the row part wrote them
// (credit_layernorm_backward_stats).  The row kernels hold a row's x and
// gamma * dy in registers; a column sum across rows would need per-column
// accumulators beside them, which the widest tiles have no registers for, so
// the parameter part is its own pair of HBM-bound kernels that read x and dy
// once more:
//   stage 1: workgroup (b, g) sums rows [g R, (g + 1) R) of column block b
//     (one 16-byte vector per thread, coalesced along the row; 256 vectors,
//     or 64 with four row lanes for narrow rows) into partial[g][...], with
//     eight rows' loads per lane in flight and the next eight issued before
//     they are summed;
//   stage 2: four waves per 64 columns add the G partials (each a fixed
//     subset in order) and then their four sums in order.
// Both stages sum in a fixed order, so results are reproducible run to run.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "api_internal.hpp"
#include "common.hpp"
#include "credit.h"

namespace credit {
namespace {

constexpr int kParamsBlock = 256;  // threads per workgroup, one column vector each
constexpr int kRowUnroll = 8;      // rows per row lane whose loads are in flight together
constexpr int kTargetWgs = 2048;   // stage-1 workgroups to aim for (8 per CU)
constexpr int64_t kMinRowsPerGroup = 8;

struct ParamsArgs {
    const void *x;
    const void *dy;
    const float *stats;  // [rows][2]: mean, rstd
    float *partial;      // [2][groups][cols]: dgamma sums, then dbeta sums
    int64_t rows;
    int64_t cols;
    int64_t rows_per_group;
    int64_t groups;
};

// Element e of a 16-byte vector (VB = 16) or the one element (VB = element
// size) of type T, as fp32.
template <class T, int VB>
struct Vec {
    static constexpr int kE = VB / StorageTraits<T>::kBytes;
    uint32_t w[VB >= 4 ? VB / 4 : 1];

    __device__ __forceinline__ void load(const void *base, int64_t elem)
    {
        const char *p = static_cast<const char *>(base) + elem * StorageTraits<T>::kBytes;
        if constexpr (VB == 16) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            w[0] = v.x;
            w[1] = v.y;
            w[2] = v.z;
            w[3] = v.w;
        } else if constexpr (VB == 4) {
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
        } else {
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
        }
    }
    __device__ __forceinline__ float at(int e) const
    {
        if constexpr (StorageTraits<T>::kBytes == 4)
            return __uint_as_float(w[e]);
        else if constexpr (VB == 2)
            return __uint_as_float(w[0] << 16);
        else
            return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
    }
};

// Sum rows rl, rl + RL, ... of rows [r0, r1) of one column vector into sg, sb:
// kRowUnroll rows' loads in flight, the next batch issued before the current
// one is summed.
template <class T, int VB, int RL>
__device__ __forceinline__ void sum_rows(const ParamsArgs &a, int64_t col0, int64_t r0, int64_t n,
                                         float (&sg)[Vec<T, VB>::kE], float (&sb)[Vec<T, VB>::kE])
{
    using V = Vec<T, VB>;
    constexpr int E = V::kE;
    constexpr int U = kRowUnroll;
    auto add = [&](const V &xv, const V &dv, int64_t row) __attribute__((always_inline)) {
        const float mu = a.stats[2 * row], rstd = a.stats[2 * row + 1];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float d = dv.at(e);
            sg[e] = __builtin_fmaf(d, (xv.at(e) - mu) * rstd, sg[e]);
            sb[e] += d;
        }
    };
    int64_t k = 0;
    V xv[U], dv[U];
    if (U <= n) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xv[u].load(a.x, (r0 + u * RL) * a.cols + col0);
            dv[u].load(a.dy, (r0 + u * RL) * a.cols + col0);
        }
    }
    for (; k + U <= n; k += U) {
        V xc[U], dc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xc[u] = xv[u];
            dc[u] = dv[u];
        }
        if (k + 2 * U <= n) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xv[u].load(a.x, (r0 + (k + U + u) * RL) * a.cols + col0);
                dv[u].load(a.dy, (r0 + (k + U + u) * RL) * a.cols + col0);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            add(xc[u], dc[u], r0 + (k + u) * RL);
    }
    for (; k < n; ++k) {
        V x1, d1;
        x1.load(a.x, (r0 + k * RL) * a.cols + col0);
        d1.load(a.dy, (r0 + k * RL) * a.cols + col0);
        add(x1, d1, r0 + k * RL);
    }
}

// Stage 1.  CV column vectors per workgroup: 256 (one row lane), or 64 for
// narrow rows, where the workgroup's four waves take every fourth row of the
// group and their sums are added in wave order through LDS (fewer groups, so
// a smaller workspace and a shorter stage 2).
template <class T, int VB, int CV>
__global__ __launch_bounds__(kParamsBlock) void lnbwd_params_partial_kernel(ParamsArgs a)
{
    constexpr int E = Vec<T, VB>::kE;
    constexpr int RL = kParamsBlock / CV;
    __shared__ float sh[2][RL][CV][E];
    const int lc = threadIdx.x % CV, rl = threadIdx.x / CV;
    const int64_t col0 = (static_cast<int64_t>(blockIdx.x) * CV + lc) * E;
    const int64_t g = blockIdx.y;
    const int64_t r0 = g * a.rows_per_group;
    const int64_t r1 = min(a.rows, r0 + a.rows_per_group);
    const bool active = col0 < a.cols;
    // rows of this lane: r0 + rl + k RL, k < n
    const int64_t n = active && r0 + rl < r1 ? (r1 - r0 - rl + RL - 1) / RL : 0;
    float sg[E], sb[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        sg[e] = sb[e] = 0.0f;
    sum_rows<T, VB, RL>(a, col0, r0 + rl, n, sg, sb);
    if constexpr (RL > 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            sh[0][rl][lc][e] = sg[e];
            sh[1][rl][lc][e] = sb[e];
        }
        __syncthreads();
        if (rl != 0)
            return;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float tg = sh[0][0][lc][e], tb = sh[1][0][lc][e];
#pragma unroll
            for (int i = 1; i < RL; ++i) {
                tg += sh[0][i][lc][e];
                tb += sh[1][i][lc][e];
            }
            sg[e] = tg;
            sb[e] = tb;
        }
    }
    if (!active)
        return;
    float *pg = a.partial + g * a.cols + col0;
    float *pb = a.partial + (a.groups + g) * a.cols + col0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        pg[e] = sg[e];
        pb[e] = sb[e];
    }
}

// Stage 2: 64 columns per workgroup; wave w adds groups w, w + 4, ... and
// the four sums are added in wave order.
constexpr int kFinishCols = 64;
__global__ __launch_bounds__(kParamsBlock) void lnbwd_params_finish_kernel(const float *partial, int64_t groups,
                                                                          int64_t cols, float *dgamma,
                                                                          float *dbeta)
{
    constexpr int W = kParamsBlock / kFinishCols;
    __shared__ float sh[2][W][kFinishCols];
    const int lane = threadIdx.x % kFinishCols, w = threadIdx.x / kFinishCols;
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kFinishCols + lane;
    float sg = 0.0f, sb = 0.0f;
    if (j < cols)
        for (int64_t g = w; g < groups; g += W) {
            sg += partial[g * cols + j];
            sb += partial[(groups + g) * cols + j];
        }
    sh[0][w][lane] = sg;
    sh[1][w][lane] = sb;
    __syncthreads();
    if (w != 0 || j >= cols)
        return;
    float tg = sh[0][0][lane], tb = sh[1][0][lane];
#pragma unroll
    for (int i = 1; i < W; ++i) {
        tg += sh[0][i][lane];
        tb += sh[1][i][lane];
    }
    dgamma[j] = tg;
    dbeta[j] = tb;
}

// Stage-1 shape: column vectors per workgroup (CV), column blocks and row
// groups: about kTargetWgs workgroups, at least kMinRowsPerGroup rows per
// row lane.
struct ParamsGrid {
    int cv;
    int64_t col_blocks, groups, rows_per_group;
};

ParamsGrid params_grid(int64_t rows, int64_t cols, int vb_elems)
{
    ParamsGrid p;
    const int64_t vecs = (cols + vb_elems - 1) / vb_elems;
    p.cv = vecs >= 32 * kParamsBlock ? kParamsBlock : 64;
    const int64_t lanes = kParamsBlock / p.cv;
    p.col_blocks = (vecs + p.cv - 1) / p.cv;
    int64_t g = (kTargetWgs + p.col_blocks - 1) / p.col_blocks;
    g = std::max<int64_t>(1, std::min<int64_t>(g, rows / (kMinRowsPerGroup * lanes)));
    p.rows_per_group = (rows + g - 1) / g;
    p.groups = rows > 0 ? (rows + p.rows_per_group - 1) / p.rows_per_group : 0;
    return p;
}

int elems_per_access(credit_dtype_t dt, int64_t cols)
{
    const int eb = dt == CREDIT_F32 ? 4 : 2;
    return (cols * eb) % 16 == 0 ? 16 / eb : 1;
}

}  // namespace
}  // namespace credit

using namespace credit;

extern "C" credit_status_t credit_layernorm_backward_params_workspace(int64_t rows, int64_t cols, credit_dtype_t dt,
                                                                      size_t *bytes)
{
    if (bytes == nullptr || rows < 0 || cols < 1 || (dt != CREDIT_F32 && dt != CREDIT_BF16))
        return CREDIT_ERR_INVALID_ARG;
    const ParamsGrid pg = params_grid(rows, cols, elems_per_access(dt, cols));
    *bytes = static_cast<size_t>(2 * pg.groups * cols) * sizeof(float);
    return CREDIT_OK;
}

extern "C" credit_status_t credit_layernorm_backward_params(const void *x, const void *dy, const float *row_stats,
                                                            float *dgamma, float *dbeta, int64_t rows, int64_t cols,
                                                            credit_dtype_t dt, void *workspace,
                                                            size_t workspace_bytes, void *stream)
{
    if (dgamma == nullptr || dbeta == nullptr || rows < 0 || cols < 1 || (dt != CREDIT_F32 && dt != CREDIT_BF16) ||
        (rows > 0 && (x == nullptr || dy == nullptr || row_stats == nullptr)))
        return CREDIT_ERR_INVALID_ARG;
    const int epa = elems_per_access(dt, cols);
    const int eb = dt == CREDIT_F32 ? 4 : 2;
    auto misaligned = [](const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) != 0; };
    if ((epa > 1 && (misaligned(x, 16) || misaligned(dy, 16))) || misaligned(x, eb) || misaligned(dy, eb) ||
        misaligned(row_stats, 8) || misaligned(dgamma, 4) || misaligned(dbeta, 4))
        return CREDIT_ERR_ALIGNMENT;
    const ParamsGrid pg = params_grid(rows, cols, epa);
    const size_t need = static_cast<size_t>(2 * pg.groups * cols) * sizeof(float);
    if (rows > 0 && (workspace == nullptr || workspace_bytes < need || misaligned(workspace, 16)))
        return CREDIT_ERR_INVALID_ARG;
    if (pg.col_blocks > 0x7FFFFFFF || pg.groups > 65535)
        return CREDIT_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (rows > 0) {
        ParamsArgs a{x, dy, row_stats, static_cast<float *>(workspace), rows, cols, pg.rows_per_group, pg.groups};
        const dim3 grid(static_cast<unsigned>(pg.col_blocks), static_cast<unsigned>(pg.groups));
        const dim3 block(kParamsBlock);
#define CREDIT_PARAMS_LAUNCH(T, VB)                                                          \
    do {                                                                                     \
        if (pg.cv == kParamsBlock)                                                           \
            hipLaunchKernelGGL((lnbwd_params_partial_kernel<T, VB, kParamsBlock>), grid, block, 0, s, a); \
        else                                                                                 \
            hipLaunchKernelGGL((lnbwd_params_partial_kernel<T, VB, 64>), grid, block, 0, s, a); \
    } while (0)
        if (dt == CREDIT_F32) {
            if (epa > 1)
                CREDIT_PARAMS_LAUNCH(float, 16);
            else
                CREDIT_PARAMS_LAUNCH(float, 4);
        } else {
            if (epa > 1)
                CREDIT_PARAMS_LAUNCH(bf16_t, 16);
            else
                CREDIT_PARAMS_LAUNCH(bf16_t, 2);
        }
#undef CREDIT_PARAMS_LAUNCH
    }
    // zero rows: the sums are zero (no groups)
    const unsigned fb = static_cast<unsigned>((cols + kFinishCols - 1) / kFinishCols);
    hipLaunchKernelGGL(lnbwd_params_finish_kernel, dim3(fb), dim3(kParamsBlock), 0, s,
                       static_cast<const float *>(workspace), pg.groups, cols, dgamma, dbeta);
    if (hipGetLastError() != hipSuccess)
        return CREDIT_ERR_HIP;
    return CREDIT_OK;
}
