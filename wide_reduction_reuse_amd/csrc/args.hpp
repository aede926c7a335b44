// Kernel argument blocks and launch constants shared by the kernels and the
// host library (plain structs: no device code).
#pragma once

#include <stdint.h>

namespace credit {

struct RowArgs {
    const void *x;      // [rows][cols] row input
    const void *gamma;  // [cols] parameters, else null
    const void *beta;
    void *y;            // [rows][cols] output (int8 codes for quantization)
    int64_t rows;
    int64_t cols;
    float eps;
    const void *dy;     // [rows][cols] second row input (backward operators), else null
    void *row_out;      // [rows] fp32 per-row output (quantization scale), else null
};

// Exchange control block (one per scratch); each counter on its own 128-byte line.
struct SplitCtl {
    uint32_t ticket;  // monotonic: every split workgroup takes one ticket when it starts
    uint32_t pad0[31];
    uint32_t error;   // bit 0: a spin-wait gave up
    uint32_t pad1[31];
};

struct SplitArgs {
    RowArgs r;
    uint32_t *ticket;      // &ctl->ticket
    uint32_t *error;       // &ctl->error
    uint64_t *slots;       // [clusters][2][P][Q] words {value bits | tag << 32}
    int32_t p;             // workgroups per row
    int32_t clusters;      // C: cluster k handles rows k, k + C, k + 2C, ...
    uint32_t ticket_base;  // value of *ticket when this launch starts
    uint32_t tag_base;     // row iteration i of this launch exchanges tag tag_base + i
    uint32_t spin_limit;   // polls before a wait gives up and flags *error
};

constexpr int kMaxSplit = 8;
constexpr int kWaveRowsPerWg = 4;  // path 1, wave-per-row: rows per 256-thread workgroup

}  // namespace credit
