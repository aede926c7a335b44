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
//     (kParamsBlock 16-byte vectors, one per thread: coalesced along the row)
//     into partial[g][...]; four rows' loads are issued before their sums;
//   stage 2: one thread per column adds the G partials in order.
// Both stages sum in a fixed order, so results are reproducible run to run.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "api_internal.hpp"
#include "common.hpp"
#include "credit.h"

namespace credit {
namespace {

constexpr int kParamsBlock = 256;  // threads per workgroup, one column vector each
constexpr int kRowUnroll = 4;      // rows whose loads are in flight together
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

template <class T, int VB>
__global__ __launch_bounds__(kParamsBlock) void lnbwd_params_partial_kernel(ParamsArgs a)
{
    using V = Vec<T, VB>;
    constexpr int E = V::kE;
    const int64_t col0 = (static_cast<int64_t>(blockIdx.x) * kParamsBlock + threadIdx.x) * E;
    const int64_t g = blockIdx.y;
    const int64_t r0 = g * a.rows_per_group;
    const int64_t r1 = min(a.rows, r0 + a.rows_per_group);
    if (col0 >= a.cols)
        return;
    float sg[E], sb[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        sg[e] = sb[e] = 0.0f;
    int64_t r = r0;
    for (; r + kRowUnroll <= r1; r += kRowUnroll) {
        V xv[kRowUnroll], dv[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            xv[u].load(a.x, (r + u) * a.cols + col0);
            dv[u].load(a.dy, (r + u) * a.cols + col0);
        }
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const float mu = a.stats[2 * (r + u)], rstd = a.stats[2 * (r + u) + 1];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float d = dv[u].at(e);
                sg[e] = __builtin_fmaf(d, (xv[u].at(e) - mu) * rstd, sg[e]);
                sb[e] += d;
            }
        }
    }
    for (; r < r1; ++r) {
        V xv, dv;
        xv.load(a.x, r * a.cols + col0);
        dv.load(a.dy, r * a.cols + col0);
        const float mu = a.stats[2 * r], rstd = a.stats[2 * r + 1];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float d = dv.at(e);
            sg[e] = __builtin_fmaf(d, (xv.at(e) - mu) * rstd, sg[e]);
            sb[e] += d;
        }
    }
    float *pg = a.partial + g * a.cols + col0;
    float *pb = a.partial + (a.groups + g) * a.cols + col0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        pg[e] = sg[e];
        pb[e] = sb[e];
    }
}

__global__ __launch_bounds__(kParamsBlock) void lnbwd_params_finish_kernel(const float *partial, int64_t groups,
                                                                          int64_t cols, float *dgamma,
                                                                          float *dbeta)
{
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kParamsBlock + threadIdx.x;
    if (j >= cols)
        return;
    float sg = 0.0f, sb = 0.0f;
    for (int64_t g = 0; g < groups; ++g) {
        sg += partial[g * cols + j];
        sb += partial[(groups + g) * cols + j];
    }
    dgamma[j] = sg;
    dbeta[j] = sb;
}

// Row groups of stage 1 for a shape: enough workgroups to fill the chip,
// at least kMinRowsPerGroup rows each.
void params_grid(int64_t rows, int64_t cols, int vb_elems, int64_t *col_blocks, int64_t *groups,
                 int64_t *rows_per_group)
{
    const int64_t vecs = (cols + vb_elems - 1) / vb_elems;
    *col_blocks = (vecs + kParamsBlock - 1) / kParamsBlock;
    int64_t g = (kTargetWgs + *col_blocks - 1) / *col_blocks;
    g = std::max<int64_t>(1, std::min<int64_t>(g, rows / kMinRowsPerGroup));
    *rows_per_group = (rows + g - 1) / g;
    *groups = rows > 0 ? (rows + *rows_per_group - 1) / *rows_per_group : 0;
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
    int64_t cb = 0, g = 0, rpg = 0;
    params_grid(rows, cols, elems_per_access(dt, cols), &cb, &g, &rpg);
    *bytes = static_cast<size_t>(2 * g * cols) * sizeof(float);
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
    int64_t cb = 0, g = 0, rpg = 0;
    params_grid(rows, cols, epa, &cb, &g, &rpg);
    const size_t need = static_cast<size_t>(2 * g * cols) * sizeof(float);
    if (rows > 0 && (workspace == nullptr || workspace_bytes < need || misaligned(workspace, 16)))
        return CREDIT_ERR_INVALID_ARG;
    if (cb > 0x7FFFFFFF || g > 65535)
        return CREDIT_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (rows > 0) {
        ParamsArgs a{x, dy, row_stats, static_cast<float *>(workspace), rows, cols, rpg, g};
        const dim3 grid(static_cast<unsigned>(cb), static_cast<unsigned>(g));
        if (dt == CREDIT_F32) {
            if (epa > 1)
                hipLaunchKernelGGL((lnbwd_params_partial_kernel<float, 16>), grid, dim3(kParamsBlock), 0, s, a);
            else
                hipLaunchKernelGGL((lnbwd_params_partial_kernel<float, 4>), grid, dim3(kParamsBlock), 0, s, a);
        } else {
            if (epa > 1)
                hipLaunchKernelGGL((lnbwd_params_partial_kernel<bf16_t, 16>), grid, dim3(kParamsBlock), 0, s, a);
            else
                hipLaunchKernelGGL((lnbwd_params_partial_kernel<bf16_t, 2>), grid, dim3(kParamsBlock), 0, s, a);
        }
    }
    // zero rows: the sums are zero (g = 0 groups)
    const unsigned fb = static_cast<unsigned>((cols + kParamsBlock - 1) / kParamsBlock);
    hipLaunchKernelGGL(lnbwd_params_finish_kernel, dim3(fb), dim3(kParamsBlock), 0, s,
                       static_cast<const float *>(workspace), g, cols, dgamma, dbeta);
    if (hipGetLastError() != hipSuccess)
        return CREDIT_ERR_HIP;
    return CREDIT_OK;
}
