// Measurement kernels: streaming copy and cache flush.
#include "kernels.hpp"
#include "registry.hpp"

namespace credit {

// 128-bit streaming copy, the achievable read+write ceiling.  One vector per
// thread per grid-stride step: consecutive workgroups cover consecutive 4 KiB
// pieces, so the addresses in flight at any time form one compact window
// (measured on MI355X to stream faster than per-thread multi-vector chunks).
// Loads and stores use the row kernels' cache policies.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                   int64_t n16)
{
    const int64_t step = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * 256; b < n16; b += step) {
        const uint32_t bytes = static_cast<uint32_t>(min<int64_t>(256, n16 - b) * 16);
        const rsrc_t s = make_rsrc(src + b, bytes);
        const rsrc_t d = make_rsrc(dst + b, bytes);
        const uint32_t off = threadIdx.x * 16u;
        buf_store<16, kStreamStore>(buf_load<16, kStream>(s, off), d, off);
    }
}

// Read-modify-write of a large buffer, to evict L2 and the Infinity Cache.
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
