// Table of compiled kernel instantiations, filled by the per-operator
// translation units and searched by the host library when it plans a launch.
// The tile ladders are X-macro lists so that the instantiations and the
// planner's ladders come from one definition.
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

// Tile ladders for 16-byte accesses: X(items) for wave-per-row, X(block, items)
// for the others.
#define CREDIT_WAVE_TILES(X) X(1) X(2) X(4) X(8) X(16)
#define CREDIT_WG_TILES(X)                                                                                 \
    X(128, 4) X(128, 8) X(128, 16) X(256, 2) X(256, 4) X(256, 8) X(256, 16) X(512, 2) X(512, 4) X(512, 8)  \
    X(512, 16) X(1024, 1) X(1024, 2) X(1024, 4) X(1024, 8) X(1024, 16)
#define CREDIT_SPLIT_TILES(X) X(256, 8) X(256, 16) X(512, 4) X(512, 8) X(512, 16) X(1024, 4) X(1024, 8) X(1024, 16)
#define CREDIT_REREAD_TILES(X) X(256, 4) X(512, 4) X(1024, 4)

// Tiles left out for one operator: LayerNorm's split kernel at 1024 threads x
// 16 16-byte vectors needs more than the 128 VGPRs that 1024 threads allow (it
// spills), so LayerNorm splits such slices finer instead.
constexpr bool tile_enabled(int op, int kind, int block, int items, int vb)
{
    return !(op == 1 && (kind == kKindSplit || kind == kKindControl) && block == 1024 && items == 16 &&
             vb == 16);
}

// Ladders for one-element accesses (rows whose byte length is not a multiple
// of 16 bytes).
#define CREDIT_WAVE_TILES_1E(X) X(4) X(16)
#define CREDIT_WG_TILES_1E(X) X(1024, 4) X(1024, 16)
#define CREDIT_SPLIT_TILES_1E(X) X(1024, 16)
#define CREDIT_REREAD_TILES_1E(X) X(256, 8)

}  // namespace credit
