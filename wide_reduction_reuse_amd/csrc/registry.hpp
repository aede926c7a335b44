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
    // row shape the kernel holds: 0 whole 16-byte vectors (or one-element
    // tiles), 1 a partial last vector (PART kernels), 2 rows held from the
    // 64-byte boundary below their start (SHIFT kernels)
    int part = 0;
    // vectors per thread held in LDS beside the `items` in registers (the LDS
    // tier of paths 1 and 2; 0 for every other kernel)
    int lds = 0;
};

// Operators with PART kernels (rows whose byte length is a multiple of 4 but
// not of 16, held from their first byte): LayerNorm (whose two parameter
// vectors, realigned to a shifted row, cost it more registers than the
// shift saves on such rows) and fp32 LayerNorm backward (whose parameters
// enter the reduction, g = gamma * dy held in the tile, so its rows cannot be
// shifted against them).  (bf16 LayerNorm backward, whose held rows are
// reduced in the streaming form, which counts whole vectors, keeps
// one-element tiles for such rows.)
constexpr bool op_has_part(int op, int dt) { return op == 1 || (op == 4 && dt == 0); }

// Operators with SHIFT kernels (rows held from the 64-byte boundary below
// their start): all, LayerNorm in bf16 only (for its odd-length rows); the
// parameter vectors of LayerNorm, RMSNorm and LayerNorm backward are
// realigned to each row's shift where they are applied.  Which rows are
// shifted: see the planner's row_is_shifted.
constexpr bool op_has_shift(int op, int dt) { return op != 1 || dt == 1; }

// Whether the split path shifts rows too: fp32 LayerNorm backward shifts on
// path 1 only.  Its split slices keep their parameter vectors for every row of
// the cluster, which realigning them per row gives up: its shifted slices
// measured 1-9% slower on MI355X than the unshifted ones.
constexpr bool op_shifts_split(int op, int dt) { return op_has_shift(op, dt) && op != 4; }

void register_softmax_kernels(std::vector<KernelEntry> &out);
void register_layernorm_kernels(std::vector<KernelEntry> &out);
void register_rmsnorm_kernels(std::vector<KernelEntry> &out);
void register_softmax_bwd_kernels(std::vector<KernelEntry> &out);
void register_layernorm_bwd_kernels(std::vector<KernelEntry> &out);
void register_quantize_kernels(std::vector<KernelEntry> &out);
void register_misc_kernels(std::vector<KernelEntry> &out);

// Row inputs an operator holds per element: x, and dy for the two backward
// operators (credit_op_t 3 and 4).
constexpr int op_inputs(int op) { return (op == 3 || op == 4) ? 2 : 1; }

// Scalars per partial that split workgroups exchange (the host sizes each
// cluster's exchange words from it, the kernels write and read that many).
constexpr int op_stats(int op)
{
    return op == 0 ? 2 : op == 1 ? 3 : op == 2 ? 1 : op == 3 ? 3 : op == 4 ? 5 : 1;
}

// Tile ladders for 16-byte accesses: X(items) for wave-per-row, X(block, items)
// for the others.
#define CREDIT_WAVE_TILES(X) X(1) X(2) X(4) X(8) X(16)
#define CREDIT_WG_TILES(X)                                                                                 \
    X(128, 4) X(128, 8) X(128, 16) X(256, 2) X(256, 4) X(256, 8) X(256, 16) X(512, 2) X(512, 4) X(512, 8)  \
    X(512, 16) X(1024, 1) X(1024, 2) X(1024, 4) X(1024, 8) X(1024, 16)
#define CREDIT_SPLIT_TILES(X) X(256, 8) X(256, 16) X(512, 4) X(512, 8) X(512, 16) X(1024, 4) X(1024, 8) X(1024, 16)
#define CREDIT_REREAD_TILES(X) X(256, 4) X(512, 4) X(1024, 4)

// Tiles left out for one operator (and dtype), each of which spilled
// registers to scratch memory when compiled.  held = register bytes of row
// data a thread holds (all inputs).  At 1024 threads, where a thread has at
// most 128 VGPRs:
//   LayerNorm split 16 x 16 B: the next smaller tiles split such slices finer.
//   softmax-logits backward (x and dy held): more than 256 B (path 1) or
//     128 B (split, which also keeps the exchange state).
//   LayerNorm backward (x and g held, five statistics): more than 64 B; its
//     512-thread tiles hold the same rows.
// At 512 threads (256 VGPRs): bf16 LayerNorm backward, which holds x and dy
// as loaded and converts them for every use, more than 256 B (x and dy of
// 16 vectors each).
//   LayerNorm's SHIFT workgroup tile 1024 x 16 (its parameter vectors are
//     realigned at the output, on top of a tile at the 128-VGPR cap).
// part: the row kind the tile holds (KernelEntry::part).
constexpr bool tile_enabled(int op, int dt, int kind, int block, int items, int vb, int part = 0)
{
    if (part == 2 && op == 1 && kind == kKindWg && block == 1024 && items == 16)
        return false;
    if (op == 4 && dt == 1 && kind != kKindReread && block >= 512 && op_inputs(op) * items * vb > 256)
        return false;
    if (kind == kKindReread || block < 1024)
        return true;
    const bool split = kind == kKindSplit || kind == kKindControl;
    // a 2-byte vector still takes a whole 32-bit register
    const int held = op_inputs(op) * items * (vb < 4 ? 4 : vb);
    if (op == 1 && split && items == 16 && vb == 16)
        return false;
    if (op == 3 && held > (split ? 128 : 256))
        return false;
    if (op == 4 && held > 64)
        return false;
    return true;
}

// The LDS tier (paths 1 and 2, rows of whole 16-byte vectors):
// X(block, items, lds) holds block * items vectors in registers and
// block * lds more in LDS (128 KiB of the 160 KiB a workgroup may use on
// gfx950 for one input at 1024 threads or two at 512).  Two-input operators
// at 1024 threads have no register room beside the LDS part's staging.
#define CREDIT_WG_LDS_TILES(X) X(512, 16, 8) X(1024, 16, 8)
#define CREDIT_SPLIT_LDS_TILES(X) X(512, 16, 8) X(1024, 16, 8)

constexpr bool lds_tile_enabled(int op, int dt, int kind, int block, int items)
{
    // LayerNorm at 1024 threads spilled registers with the LDS part's staging
    return tile_enabled(op, dt, kind, block, items, 16) && ((op_inputs(op) == 1 && op != 1) || block < 1024);
}

// Ladders for one-element accesses (rows whose byte length is not a multiple
// of 16 bytes).  The 32-vector tiles let such rows up to 32768 elements stay
// on one workgroup and wider ones split in fewer, larger slices (4- and 2-byte
// accesses stream at 5.8-6.0 TB/s on MI355X when a thread keeps 32 in flight);
// 48 vectors spilled registers for LayerNorm, RMSNorm bf16 and softmax
// backward.
#define CREDIT_WAVE_TILES_1E(X) X(4) X(16)
#define CREDIT_WG_TILES_1E(X) X(1024, 4) X(1024, 16) X(1024, 32)
#define CREDIT_SPLIT_TILES_1E(X) X(1024, 16) X(1024, 32)
#define CREDIT_REREAD_TILES_1E(X) X(256, 8)

}  // namespace credit
