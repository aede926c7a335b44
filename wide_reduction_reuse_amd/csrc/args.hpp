// Kernel argument blocks and launch constants shared by the kernels and the
// host library (plain structs: no device code).
#pragma once

#include <stdint.h>

namespace credit {

struct RowArgs {
    const void *x;
    const void *gamma;
    const void *beta;
    void *y;
    int64_t rows;
    int64_t cols;
    float eps;
};

// Exchange control block (one per scratch); each counter on its own 128-byte line.
struct SplitCtl {
    uint32_t ticket;
    uint32_t pad0[31];
    uint32_t done;
    uint32_t pad1[31];
    uint32_t epoch;
    uint32_t pad2[31];
    uint32_t error;  // bit 0: a spin-wait gave up
    uint32_t pad3[31];
};

struct SplitArgs {
    RowArgs r;
    SplitCtl *ctl;
    uint64_t *slots;     // [rows in launch][P][Q] words {value bits | epoch << 32}
    int64_t row0;        // first row of this launch
    int32_t p;           // workgroups per row
    uint32_t spin_limit; // polls before a wait gives up and flags ctl->error
};

constexpr int kMaxSplit = 8;
constexpr int kWaveRowsPerWg = 4;  // path 1, wave-per-row: rows per 256-thread workgroup

}  // namespace credit
