// Instantiates every tile of the ladders in registry.hpp for one operator.
#pragma once

#include "kernels.hpp"
#include "registry.hpp"

namespace credit {

template <OpKind OP, class T, int DT>
void register_op_dtype(std::vector<KernelEntry> &v)
{
    constexpr int VB = 16;
    constexpr int VS = StorageTraits<T>::kBytes;  // one-element access
#define CREDIT_K(kind, vb, block, items, ...) \
    v.push_back(KernelEntry{kind, OP, DT, vb, block, items, reinterpret_cast<const void *>(&__VA_ARGS__)})
    // path 1a
    CREDIT_K(kKindWave, VB, 64, 1, single_wave_kernel<OP, T, VB, 1>);
    CREDIT_K(kKindWave, VB, 64, 2, single_wave_kernel<OP, T, VB, 2>);
    CREDIT_K(kKindWave, VB, 64, 4, single_wave_kernel<OP, T, VB, 4>);
    CREDIT_K(kKindWave, VB, 64, 8, single_wave_kernel<OP, T, VB, 8>);
    CREDIT_K(kKindWave, VB, 64, 16, single_wave_kernel<OP, T, VB, 16>);
    // path 1b
    CREDIT_K(kKindWg, VB, 256, 2, single_wg_kernel<OP, T, VB, 256, 2>);
    CREDIT_K(kKindWg, VB, 256, 4, single_wg_kernel<OP, T, VB, 256, 4>);
    CREDIT_K(kKindWg, VB, 256, 8, single_wg_kernel<OP, T, VB, 256, 8>);
    CREDIT_K(kKindWg, VB, 256, 16, single_wg_kernel<OP, T, VB, 256, 16>);
    CREDIT_K(kKindWg, VB, 512, 4, single_wg_kernel<OP, T, VB, 512, 4>);
    CREDIT_K(kKindWg, VB, 512, 8, single_wg_kernel<OP, T, VB, 512, 8>);
    CREDIT_K(kKindWg, VB, 512, 16, single_wg_kernel<OP, T, VB, 512, 16>);
    CREDIT_K(kKindWg, VB, 1024, 4, single_wg_kernel<OP, T, VB, 1024, 4>);
    CREDIT_K(kKindWg, VB, 1024, 8, single_wg_kernel<OP, T, VB, 1024, 8>);
    CREDIT_K(kKindWg, VB, 1024, 16, single_wg_kernel<OP, T, VB, 1024, 16>);
    // path 2 and its work-free control
    CREDIT_K(kKindSplit, VB, 256, 8, split_kernel<OP, T, VB, 256, 8, false>);
    CREDIT_K(kKindSplit, VB, 256, 16, split_kernel<OP, T, VB, 256, 16, false>);
    CREDIT_K(kKindSplit, VB, 512, 8, split_kernel<OP, T, VB, 512, 8, false>);
    CREDIT_K(kKindSplit, VB, 512, 16, split_kernel<OP, T, VB, 512, 16, false>);
    CREDIT_K(kKindSplit, VB, 1024, 4, split_kernel<OP, T, VB, 1024, 4, false>);
    CREDIT_K(kKindSplit, VB, 1024, 8, split_kernel<OP, T, VB, 1024, 8, false>);
    CREDIT_K(kKindSplit, VB, 1024, 16, split_kernel<OP, T, VB, 1024, 16, false>);
    CREDIT_K(kKindControl, VB, 256, 8, split_kernel<OP, T, VB, 256, 8, true>);
    CREDIT_K(kKindControl, VB, 256, 16, split_kernel<OP, T, VB, 256, 16, true>);
    CREDIT_K(kKindControl, VB, 512, 8, split_kernel<OP, T, VB, 512, 8, true>);
    CREDIT_K(kKindControl, VB, 512, 16, split_kernel<OP, T, VB, 512, 16, true>);
    CREDIT_K(kKindControl, VB, 1024, 4, split_kernel<OP, T, VB, 1024, 4, true>);
    CREDIT_K(kKindControl, VB, 1024, 8, split_kernel<OP, T, VB, 1024, 8, true>);
    CREDIT_K(kKindControl, VB, 1024, 16, split_kernel<OP, T, VB, 1024, 16, true>);
    // path 3
    CREDIT_K(kKindReread, VB, 256, 4, reread_kernel<OP, T, VB, 256, 4>);
    CREDIT_K(kKindReread, VB, 512, 4, reread_kernel<OP, T, VB, 512, 4>);
    CREDIT_K(kKindReread, VB, 1024, 4, reread_kernel<OP, T, VB, 1024, 4>);
    // one-element accesses
    CREDIT_K(kKindWave, VS, 64, 4, single_wave_kernel<OP, T, VS, 4>);
    CREDIT_K(kKindWave, VS, 64, 16, single_wave_kernel<OP, T, VS, 16>);
    CREDIT_K(kKindWg, VS, 1024, 4, single_wg_kernel<OP, T, VS, 1024, 4>);
    CREDIT_K(kKindWg, VS, 1024, 16, single_wg_kernel<OP, T, VS, 1024, 16>);
    CREDIT_K(kKindSplit, VS, 1024, 16, split_kernel<OP, T, VS, 1024, 16, false>);
    CREDIT_K(kKindControl, VS, 1024, 16, split_kernel<OP, T, VS, 1024, 16, true>);
    CREDIT_K(kKindReread, VS, 256, 8, reread_kernel<OP, T, VS, 256, 8>);
#undef CREDIT_K
}

}  // namespace credit
