// Measurement kernels (streaming copy, cache flush).
#include "kernels.hpp"
#include "registry.hpp"

namespace credit {

// ---------------------------------------------------------------------------
// Measurement kernels: a 128-bit streaming copy (the achievable read+write
// ceiling) and a cache flush (read-modify-write of a large buffer).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                   int64_t n16)
{
    constexpr int U = 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k)
            v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
        for (int k = 0; k < U; ++k)
            __builtin_nontemporal_store(v[k], dst + i + k * stride);
    }
    for (; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void flush_kernel(u32x4 *__restrict__ buf, int64_t n16)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
        u32x4 v = buf[i];
        v += 1u;
        buf[i] = v;
    }
}

void register_misc_kernels(std::vector<KernelEntry> &out)
{
    out.push_back(KernelEntry{0, -1, -1, 16, 256, 0, reinterpret_cast<const void *>(&copy_kernel)});
    out.push_back(KernelEntry{0, -2, -1, 16, 256, 0, reinterpret_cast<const void *>(&flush_kernel)});
}

}  // namespace credit
