// Table of compiled kernel instantiations, filled by the per-operator
// translation units and searched by the host library when it plans a launch.
#pragma once

#include <vector>

namespace credit {

enum KernelKind { kKindWave = 1, kKindWg = 2, kKindSplit = 3, kKindReread = 4, kKindControl = 5 };

struct KernelEntry {
    int kind;
    int op;     // credit_op_t
    int dt;     // credit_dtype_t
    int vb;     // bytes per global access
    int block;  // threads per row owner (64 for wave-per-row)
    int items;  // vectors held per thread (paths 1, 2) or streamed per step (path 3)
    const void *fn;
};

void register_softmax_kernels(std::vector<KernelEntry> &out);
void register_layernorm_kernels(std::vector<KernelEntry> &out);
void register_rmsnorm_kernels(std::vector<KernelEntry> &out);
void register_misc_kernels(std::vector<KernelEntry> &out);

// Tile ladders (shared by the instantiation units and the planner).
// Path 1a, one wave per row:    items in {1, 2, 4, 8, 16}.
// Path 1b, one workgroup/row:   (256: 2,4,8,16) (512: 4,8,16) (1024: 4,8,16).
// Path 2, split row:            (256: 8,16) (512: 8,16) (1024: 4,8,16).
// Path 3, reread:               (256: 4) (512: 4) (1024: 4).
// One-element accesses (rows whose byte length is not a multiple of 16):
//   1a items {4, 16}; 1b (1024: 4, 16); 2 (1024: 16); 3 (256: 8).

}  // namespace credit
