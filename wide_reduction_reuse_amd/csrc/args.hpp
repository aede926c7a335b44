// Kernel argument blocks and launch constants shared by the kernels and the
// host library (plain structs: no device code).
#pragma once

#include <hip/hip_runtime.h>
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

// Exchange control block (one per scratch); each word on its own 128-byte
// line.  It carries the state of the split-row protocol from one launch to the
// next on the device itself, so that a launch needs nothing from the host
// but its shape (and a captured launch replays correctly):
//   ticket     tickets taken by the running launch; its workgroups take
//              0, 1, ... in start order, and its last workgroup resets it to 0
//   done       workgroups of the running launch that have finished (reset
//              to 0 by the last one)
//   tags_used  exchange tags issued so far: a launch uses tags
//              tags_used + 1 ... tags_used + iters, and its last workgroup adds
//              iters; once it reaches 2^31 the last workgroup clears every
//              exchange word and sets it back to 0 (so a tag never wraps, and
//              tag 0, the value of a cleared word, is never expected)
//   error      bit 0: a spin-wait gave up (sticky until the host reads it)
//   unmatched  0; a test of the give-up path sets 2^31, which makes every
//              reader wait for its tag + 2^31, a tag no word carries while
//              fewer than 2^30 tags have been issued
// A zero-filled block is the initial state.
struct SplitCtl {
    uint32_t ticket;
    uint32_t pad0[31];
    uint32_t done;
    uint32_t pad1[31];
    uint32_t tags_used;
    uint32_t pad2[31];
    uint32_t error;
    uint32_t pad3[31];
    uint32_t unmatched;
    uint32_t pad4[31];
};

// tags_used at or above this value is reset (with the words cleared) by the
// launch that reaches it; a launch uses at most kMaxSplitIters tags, so tags
// stay below 2^31 + 2^30.
constexpr uint32_t kTagResetAt = 1u << 31;
constexpr uint32_t kMaxSplitIters = 1u << 30;

// A split-row scratch is a SplitCtl followed by kSlotWords 64-bit exchange
// words (1 MiB), 256-byte aligned; a launch's clusters are capped so that
// their words fit.
constexpr int64_t kSlotWords = INT64_C(1) << 17;
constexpr int64_t kScratchBytes = static_cast<int64_t>(sizeof(SplitCtl)) + kSlotWords * 8;

struct SplitArgs {
    RowArgs r;
    SplitCtl *ctl;         // the scratch: control block, then the exchange words
                           // [clusters][2][P][Q] {value bits | tag << 32}
    int32_t p;             // workgroups per row
    int32_t clusters;      // C: cluster k handles rows k, k + C, k + 2C, ...;
                           // rows <= C * kMaxSplitIters
    uint32_t spin_limit;   // polls before a wait gives up (it then flags ctl->error
                           // and poisons its row)
};

// The exchange words of a scratch.
__host__ __device__ inline uint64_t *scratch_slots(SplitCtl *ctl) { return reinterpret_cast<uint64_t *>(ctl + 1); }

// Rows held from the 64-byte boundary at or below their first byte (the
// kernels' SHIFT mode) begin with up to shift_max_bytes of the previous row:
// row r of a tensor whose base is 16-byte aligned starts at
// (base + r * row_bytes) mod 64 bytes into a 64-byte line, a multiple of
// g = the lowest set bit of row_bytes (at most 64) plus a multiple of 16 from
// the base, so at most 64 - min(g, 16).  shift_held_vectors: the 16-byte
// vectors that any row's held span covers, for eb-byte elements.
__host__ __device__ constexpr int shift_max_bytes(int64_t row_bytes)
{
    const int64_t g = row_bytes % 64 == 0 ? 64 : (row_bytes & -row_bytes);
    return 64 - static_cast<int>(g < 16 ? g : 16);
}
__host__ __device__ constexpr int64_t shift_held_vectors(int64_t cols, int eb)
{
    const int64_t e = 16 / eb;
    return (cols + shift_max_bytes(cols * eb) / eb + e - 1) / e;
}

// Vectors per slice of a row of nv held vectors of vb bytes split p ways:
// ceil(nv / p) rounded up to whole 64-byte lines, so that every slice of a
// line-aligned row starts on a line boundary (the last slice takes the rest).
__host__ __device__ constexpr int64_t slice_vectors(int64_t nv, int p, int vb)
{
    const int64_t q = (nv + p - 1) / p;
    const int64_t line = vb >= 64 ? 1 : 64 / vb;
    return (q + line - 1) / line * line;
}

constexpr int kMaxSplit = 8;
constexpr int kWaveRowsPerWg = 4;  // path 1, wave-per-row: rows per 256-thread workgroup

}  // namespace credit
