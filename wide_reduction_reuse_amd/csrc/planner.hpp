// Host-only planner: which tiles can hold a row (or slice) on chip, and the
// cost model that picks among path 1 (one owner per row), path 2 (P workgroups
// per row) and path 3 (reread).  No HIP calls: everything here is arithmetic on
// shapes, tile ladders and a device/calibration description, so it runs and is
// tested without a GPU.
//
// Cost model: CREDIT paper, Sec. III-D.  Eq. 3 gives legality (the retained
// slice plus fixed scratch must fit the per-workgroup on-chip budget); Eq. 7
// prices the avoided reread at the bandwidth the baseline actually achieves,
// T_save = (b_reread / b_B) * T_B; Eq. 8 counts sequential cluster waves
// W = ceil(M / floor(S / P)) and the replay and exchange times; Eq. 9 takes
// dT = T_save - T_ctrl - T_replay - T_deposit - T_DSM, plus, on gfx950, the
// time a baseline that leaves CUs idle gives back when its rows are split
// over them (T_occ).
#pragma once

#include <stdint.h>

#include <array>
#include <functional>
#include <map>
#include <string>
#include <vector>

namespace credit {

enum PathId { kPathAuto = 0, kPathSingle = 1, kPathSplit = 2, kPathReread = 3 };

constexpr int kNumOps = 6;  // credit_op_t values 0..5

struct TileSpec {
    int kind = 0;   // KernelKind
    int block = 0;  // threads per row owner (64: one wave per row)
    int items = 0;  // vectors per thread (held) or per step (reread)
    int vb = 16;    // bytes per access
    int lds = 0;    // vectors per thread held in LDS beside `items` (the LDS tier)
};

// What the planner knows about the device.  Defaults describe an MI355X.
struct DeviceModel {
    int cus = 256;
    int xcds = 8;
    double clock_ghz = 2.4;
    double hbm_peak_gbs = 8000.0;
    double l2_bytes_per_xcd = 4.0 * 1024 * 1024;
    double mall_bytes = 256.0 * 1024 * 1024;
    double lds_bytes_per_cu = 160.0 * 1024;
    double vgpr_bytes_per_cu = 512.0 * 1024;
};

// One measured candidate of a calibration table: a plan for rows of `cols`
// elements of one operator and dtype, with its median kernel time (us) at
// several row counts (ascending).
struct CalibEntry {
    int op = 0, dt = 0;
    int64_t cols = 0;
    int path = 0, split_p = 1, block = 0, items = 0, vb = 16, wgs_per_cu = 0, lds = 0;
    std::vector<double> rows, us;
};

// Time of `e` at `rows`, interpolated piecewise linearly in (log rows,
// log time) between its measurements and extrapolated along the end segments.
double calib_time_us(const CalibEntry &e, double rows);

// Constants of the analytic model (fitted to exhaustive timings of
// calibration shapes by model_fit.py; these defaults are MI355X's).
struct ModelConsts {
    double bw_gbs = 5100.5492;     // rate the kernels stream at with enough bytes in flight
    double lat_us = 0.6889;        // a CU's bytes in flight / lat_us = the rate it can sustain
    double owner_gbs = 44.5709;    // the most one owner streams: its row's bytes / owner_gbs bound its time
    double miss3 = 0.3980;         // fraction of path 3's second read served from HBM
    double l0_us = 2.2005;         // least time of one owner's row: a fixed part
    double item_us = 0.2123;       // ... and a part per vector each thread holds or streams
    double own3_us = 1.6787;       // ... and, for a reread owner, its second pass
    double launch_us = 3.5074;     // one launch
    double exch_us = 3.5980;       // one split-row exchange per row wave (Eq. 8's control cost)
    double split_launch_us = 6.2248; // a split launch's control cost beyond its row waves
    double eta3 = 1.2562;          // bytes multiplier of reread launches (their streaming efficiency)
    double persist = 1.0084;       // ... of persistent owners on path 1
    double word_gbs = 10.0;        // exchange-word rate of one workgroup (T_DSM)
};

// A compiled kernel, for its occupancy: credit_op_t, credit_dtype_t,
// KernelKind, threads, vectors per thread, bytes per access, row kind
// (held_row_kind; 0 for the reread path), LDS vectors per thread.
struct OccKey {
    int op = 0, dt = 0, kind = 0, block = 0, items = 0, vb = 0, part = 0, lds = 0;
    std::array<int, 8> tuple() const { return {op, dt, kind, block, items, vb, part, lds}; }
};

// What the planner knows beyond the tile ladders (from a calibration file,
// else defaults).
struct Calibration {
    bool loaded = false;
    // ablation of the paper's Table V (first row): price streaming at the
    // device's peak HBM bandwidth instead of the achieved rate
    bool peak_bandwidth = false;
    DeviceModel device;
    bool has_device = false;
    ModelConsts model;
    // resident workgroups per CU of the compiled kernels: occ_query (set by
    // the host library from the HIP runtime) first, then this table (from the
    // calibration file), else an estimate from the tile's registers
    std::function<int(const OccKey &)> occ_query;
    std::map<std::array<int, 8>, int> occupancy;
    // measured candidates; shapes whose (op, dtype, cols) appear here are
    // planned from them, all others by the analytic model
    std::vector<CalibEntry> table;
};

struct PlanRequest {
    int op = 0;  // credit_op_t
    int dt = 0;  // credit_dtype_t
    int64_t rows = 0;
    int64_t cols = 0;
};

struct PathEstimate {
    bool legal = false;
    int split_p = 1;
    TileSpec tile;
    double us = -1.0;
    // model terms, kept for reporting and tests (path 2: split_terms)
    double t_save_us = 0.0;
    double t_occ_us = 0.0;
    double t_ctrl_us = 0.0;
    double t_dsm_us = 0.0;
    double delta_us = 0.0;
    double waves = 0.0;
};

// The terms of Eq. 7-9 for splitting a shape's rows over P workgroups with
// tile t, against the non-split baseline (base_path with base_tile, whose
// time is t_base_us).
struct SplitTerms {
    double t_base_us = 0.0;  // T_B
    double b_base = 0.0;     // bytes per element the baseline moves
    double b_reread = 0.0;   // of which its reread (Eq. 4)
    double t_save_us = 0.0;  // Eq. 7: (b_reread / b_B) T_B
    double t_occ_us = 0.0;   // gfx950: (T_B - T_save)(1 - u_B / u_split), u = fraction of CUs given work
    double resident = 0.0;   // S: split workgroups the device holds at once
    double waves = 0.0;      // Eq. 8: W = ceil(M / floor(S / P))
    double t_ctrl_us = 0.0;  // W exchanges and the split launch's control cost
    double t_dsm_us = 0.0;   // s W (P - 1) q / B_w (not multiplied by P)
    double delta_us = 0.0;   // Eq. 9: T_save + T_occ - T_ctrl - T_DSM (T_replay = T_deposit = 0)
    double t_split_us = 0.0; // T_B - dT
};

// Resident workgroups per CU of the kernel `path` runs with tile t.
int occupancy_of(const PlanRequest &req, const Calibration &cal, int path, const TileSpec &t);
// Predicted time of one launch of a plan on path 1 or 3 (path 2 is priced by
// split_terms); wgs_per_cu_mode as credit_plan_t::wgs_per_cu.
double stream_time_us(const PlanRequest &req, const Calibration &cal, int path, const TileSpec &t,
                      int wgs_per_cu_mode);
SplitTerms split_terms(const PlanRequest &req, const Calibration &cal, int P, const TileSpec &t, int base_path,
                       const TileSpec &base_tile, double t_base_us);
// The analytic model's non-split baseline for a shape: path 1's tile when one
// holds the row, else path 3's fastest tile; false only for bad arguments.
bool analytic_baseline(const PlanRequest &req, const Calibration &cal, int *path, TileSpec *tile, double *us);

struct Plan {
    int path = kPathSingle;
    int split_p = 1;
    int wgs_per_cu = 0;  // credit_plan_t::wgs_per_cu
    TileSpec tile;
    PathEstimate est[3];  // paths 1..3
};

int elem_bytes(int dt);
int n_params(int op);
int stats_per_partial(int op);  // q: scalars exchanged per partial
int in_bytes(int op, int dt);   // bytes per element of all row inputs (x, and dy for backward operators)
int out_bytes(int op, int dt);  // bytes per output element (1 for int8 codes)
int row_out_bytes(int op);      // bytes written per row besides the row (quantization scale)
bool op_supported(int op, int dt);  // a compiled (operator, dtype) pair

// Bytes per global access for a row of `cols` elements: 16 when the row's byte
// length is a multiple of 16 (rows stay 16-byte aligned), else one element.
int vec_bytes_for(int dt, int64_t cols);
// Rows whose byte length is a multiple of 4 but not of 16, of an operator
// with PART kernels, that `path` (kPathSingle / kPathSplit) does not shift:
// held as 16-byte vectors whose last one is partial (PART kernels mask its
// missing elements).
bool row_is_partial(int op, int dt, int64_t cols, int path);
// Rows whose byte length is not a multiple of 64, of an operator with SHIFT
// kernels on `path` (for LayerNorm: odd-length bf16 rows only; LayerNorm
// backward: path 1 only, fp32 rows of whole 16-byte vectors and bf16 rows
// that are not): held as 16-byte vectors from the 64-byte boundary below each
// row's start.
bool row_is_shifted(int op, int dt, int64_t cols, int path);
// The kernels' row kind for the held tiles of `path` (1 or 2): 0 whole
// vectors or one-element tiles, 1 partial last vector (row_is_partial),
// 2 shifted (row_is_shifted).
int held_row_kind(int op, int dt, int64_t cols, int path);
// Bytes per access of the held tiles (paths 1, 2): 16 for PART and SHIFT rows too.
int held_vec_bytes(int op, int dt, int64_t cols, int path);
// Bytes per access that `path` (kPathSingle / kPathSplit / kPathReread) uses.
int path_vec_bytes(int op, int dt, int64_t cols, int path);
// 16-byte vectors of a row that the LDS tier holds: rows of whole 16-byte
// vectors, held as they are (no shift) by the LDS-tier kernels; else 0.
int64_t lds_row_vectors(int dt, int64_t cols);
// The row kind of the kernel a plan runs: held_row_kind for register tiles
// of paths 1 and 2, 0 for the reread path and the LDS tier.
int plan_row_kind(int op, int dt, int64_t cols, int path, int lds);
// Vectors of held_vec_bytes covering a row on `path` (1 or 2), the last one
// possibly partial (SHIFT rows: the most that any row's held span covers,
// shift_held_vectors).
int64_t held_vectors(int op, int dt, int64_t cols, int path);

// Tile ladders, mirroring the compiled instantiations.
const std::vector<TileSpec> &tiles_for(int kind, int vb_is_16);

// Path 1: the tile that holds a row of `cols`, or false if none can: a
// register tile where one holds it, else an LDS-tier tile.
bool single_tile(int op, int dt, int64_t cols, TileSpec *out);
// Path 2: the tile that holds a 1/p slice, or false if none can (registers
// first, then the LDS tier, as for path 1).
bool split_tile(int op, int dt, int64_t cols, int p, TileSpec *out);
// The LDS-tier tiles of `kind` (kKindWg or kKindSplit) that `op` compiles;
// empty for rows the tier does not hold (not whole 16-byte vectors).
std::vector<TileSpec> lds_ladder(int op, int dt, int64_t cols, int kind);
// Path 3: always possible.
TileSpec reread_tile(int dt, int64_t cols);

// Retained bytes per workgroup for a held tile (Eq. 3's S_CTA: registers and
// LDS) and the budget.
double tile_capacity_bytes(const TileSpec &t);
double onchip_budget_bytes(const DeviceModel &d);

// Every legal (path, P, tile) for a shape, each with the model's estimate.
struct Candidate {
    int path;
    int split_p;
    PathEstimate est;
    int wgs_per_cu = 0;
};
void enumerate_candidates(const PlanRequest &req, const Calibration &cal, std::vector<Candidate> *out);

// Plan with the cost model; forced_path / forced_p restrict the choice
// (0 = free).  Returns false if the forced choice is illegal for the shape.
bool make_plan(const PlanRequest &req, const Calibration &cal, int forced_path, int forced_p, Plan *out);

// Parse a calibration JSON document (the subset written by the calibration
// script: one object of numbers and nested number arrays).  Returns false and
// leaves *out untouched on any syntax or schema error.
bool parse_calibration(const std::string &text, Calibration *out);

}  // namespace credit
