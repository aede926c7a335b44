// Host-only planner and cost model (see planner.hpp).
#include "planner.hpp"

#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstdlib>
#include <map>

#include "args.hpp"
#include "registry.hpp"

namespace credit {

int elem_bytes(int dt) { return dt == 1 ? 2 : 4; }

// Per operator (credit_op_t order: softmax, LayerNorm, RMSNorm, softmax-logits
// backward, LayerNorm backward, int8 quantization).
int n_params(int op)
{
    static const int v[kNumOps] = {0, 2, 1, 0, 1, 0};
    return op >= 0 && op < kNumOps ? v[op] : 0;
}
int stats_per_partial(int op) { return op_stats(op); }
int in_bytes(int op, int dt) { return op_inputs(op) * elem_bytes(dt); }
int out_bytes(int op, int dt) { return op == 5 ? 1 : elem_bytes(dt); }
int row_out_bytes(int op) { return op == 5 ? 4 : 0; }
bool op_supported(int op, int dt) { return op >= 0 && op < kNumOps && (dt == 0 || dt == 1); }

int vec_bytes_for(int dt, int64_t cols)
{
    return (cols * elem_bytes(dt)) % 16 == 0 ? 16 : elem_bytes(dt);
}

bool row_is_shifted(int op, int dt, int64_t cols, int path)
{
    // LayerNorm shifts only the rows it has no 16-byte kernels for otherwise
    // (odd bf16 lengths): on its other rows the PART and whole-vector kernels
    // measured as fast or faster.  LayerNorm backward shifts on path 1 only
    // (measured on MI355X, every legal plan of each width timed): fp32 rows
    // of whole 16-byte vectors (2-10% faster than held as they are; its rows
    // with a partial last vector were no faster shifted, -4% to +5%, than
    // held by the PART kernels, which fetch the parameters unshifted), and
    // bf16 rows that are not whole 16-byte vectors (1.39-1.99x faster than
    // the one-element tiles and the reread path; its rows of whole 16-byte
    // vectors ran 20% slower shifted than held as they are).
    const int64_t bytes = cols * elem_bytes(dt);
    const bool shifts = path == kPathSplit ? op_shifts_split(op, dt) : op_has_shift(op, dt);
    if (op == 4)
        return shifts && bytes % 64 != 0 && (dt == 0) == (bytes % 16 == 0);
    return shifts && bytes % 64 != 0 && (op != 1 || bytes % 4 != 0);
}

bool row_is_partial(int op, int dt, int64_t cols, int path)
{
    const int64_t bytes = cols * elem_bytes(dt);
    return op_has_part(op, dt) && bytes % 16 != 0 && bytes % 4 == 0 && !row_is_shifted(op, dt, cols, path);
}

int held_row_kind(int op, int dt, int64_t cols, int path)
{
    return row_is_partial(op, dt, cols, path) ? 1 : (row_is_shifted(op, dt, cols, path) ? 2 : 0);
}

int held_vec_bytes(int op, int dt, int64_t cols, int path)
{
    return held_row_kind(op, dt, cols, path) != 0 ? 16 : vec_bytes_for(dt, cols);
}

int path_vec_bytes(int op, int dt, int64_t cols, int path)
{
    return path == kPathReread ? vec_bytes_for(dt, cols) : held_vec_bytes(op, dt, cols, path);
}

int64_t lds_row_vectors(int dt, int64_t cols)
{
    const int64_t bytes = cols * elem_bytes(dt);
    return bytes % 16 == 0 ? bytes / 16 : 0;
}

int plan_row_kind(int op, int dt, int64_t cols, int path, int lds)
{
    return (path == kPathReread || lds > 0) ? 0 : held_row_kind(op, dt, cols, path);
}

int64_t held_vectors(int op, int dt, int64_t cols, int path)
{
    if (held_row_kind(op, dt, cols, path) == 2)
        return shift_held_vectors(cols, elem_bytes(dt));
    const int64_t vb = held_vec_bytes(op, dt, cols, path);
    return (cols * elem_bytes(dt) + vb - 1) / vb;
}

// ---------------------------------------------------------------------------
// Tile ladders: the same X-macro lists the kernel instantiations expand.
// ---------------------------------------------------------------------------
static std::vector<TileSpec> make_ladder(int kind, bool v16)
{
    std::vector<TileSpec> t;
    const int vb = v16 ? 16 : 0;
#define ADD1(it) t.push_back(TileSpec{kind, 64, it, vb});
#define ADD2(b, it) t.push_back(TileSpec{kind, b, it, vb});
    if (v16) {
        switch (kind) {
        case kKindWave:
            CREDIT_WAVE_TILES(ADD1)
            break;
        case kKindWg:
            CREDIT_WG_TILES(ADD2)
            break;
        case kKindSplit:
        case kKindControl:
            CREDIT_SPLIT_TILES(ADD2)
            break;
        case kKindReread:
            CREDIT_REREAD_TILES(ADD2)
            break;
        }
    } else {
        switch (kind) {
        case kKindWave:
            CREDIT_WAVE_TILES_1E(ADD1)
            break;
        case kKindWg:
            CREDIT_WG_TILES_1E(ADD2)
            break;
        case kKindSplit:
        case kKindControl:
            CREDIT_SPLIT_TILES_1E(ADD2)
            break;
        case kKindReread:
            CREDIT_REREAD_TILES_1E(ADD2)
            break;
        }
    }
#undef ADD1
#undef ADD2
    return t;
}

const std::vector<TileSpec> &tiles_for(int kind, int vb_is_16)
{
    static std::map<int, std::vector<TileSpec>> cache[2];
    auto &m = cache[vb_is_16 ? 1 : 0];
    auto it = m.find(kind);
    if (it == m.end())
        it = m.emplace(kind, make_ladder(kind, vb_is_16 != 0)).first;
    return it->second;
}

// Preference among tiles that can hold `nv` vectors: the smallest capacity,
// then the one whose thread count is nearest 512, then fewer vectors per
// thread.  On the calibration shapes of MI355X (every legal plan timed), this
// rule picks a tile within 1% of the fastest of its path more often than
// preferring two vectors per thread, the most resident waves or the most
// bytes in flight.
static bool pick_holding_tile(const std::vector<TileSpec> &ladder, int64_t nv, TileSpec *out)
{
    bool found = false;
    TileSpec best;
    int64_t best_cap = 0;
    for (const TileSpec &t : ladder) {
        const int64_t cap = static_cast<int64_t>(t.block) * t.items;
        if (cap < nv)
            continue;
        bool better = !found || cap < best_cap;
        if (found && cap == best_cap) {
            auto from512 = [](int block) { return std::abs(std::log2(static_cast<double>(block)) - 9.0); };
            const double d_new = from512(t.block), d_old = from512(best.block);
            better = d_new < d_old || (d_new == d_old && t.items < best.items);
        }
        if (better) {
            best = t;
            best_cap = cap;
            found = true;
        }
    }
    if (found)
        *out = best;
    return found;
}

// The held-tile ladders of path 1 (wave and workgroup tiles) that `op`
// compiles for rows of `vb`-byte vectors.
static std::vector<TileSpec> single_ladder(int op, int dt, int vb, int part)
{
    std::vector<TileSpec> ladder;
    for (int kind : {kKindWave, kKindWg})
        for (const TileSpec &u : tiles_for(kind, vb == 16))
            if (tile_enabled(op, dt, kind, u.block, u.items, vb, part))
                ladder.push_back(u);
    return ladder;
}

// The held tiles of an LDS ladder that `kind` compiles for `op`.
static std::vector<TileSpec> lds_tiles(int op, int dt, int kind)
{
    std::vector<TileSpec> out;
#define CREDIT_LDS_ADD(b, it, lt)                            \
    if (lds_tile_enabled(op, dt, kind, b, it))               \
        out.push_back(TileSpec{kind, b, it, 16, lt});
    if (kind == kKindWg) {
        CREDIT_WG_LDS_TILES(CREDIT_LDS_ADD)
    } else if (kind == kKindSplit) {
        CREDIT_SPLIT_LDS_TILES(CREDIT_LDS_ADD)
    }
#undef CREDIT_LDS_ADD
    return out;
}

std::vector<TileSpec> lds_ladder(int op, int dt, int64_t cols, int kind)
{
    if (lds_row_vectors(dt, cols) == 0)
        return {};
    return lds_tiles(op, dt, kind);
}

// The LDS-tier tile that holds `need` vectors with the fewest LDS vectors
// per thread (then fewer registers), or false.
static bool pick_lds_tile(const std::vector<TileSpec> &ladder, int64_t need, TileSpec *out)
{
    bool found = false;
    for (const TileSpec &t : ladder) {
        const int64_t cap = static_cast<int64_t>(t.block) * (t.items + t.lds);
        if (cap < need)
            continue;
        if (!found || static_cast<int64_t>(t.block) * t.lds < static_cast<int64_t>(out->block) * out->lds) {
            *out = t;
            found = true;
        }
    }
    return found;
}

bool single_tile(int op, int dt, int64_t cols, TileSpec *out)
{
    const int vb = held_vec_bytes(op, dt, cols, kPathSingle);
    const int64_t nv = held_vectors(op, dt, cols, kPathSingle);
    const std::vector<TileSpec> ladder = single_ladder(op, dt, vb, held_row_kind(op, dt, cols, kPathSingle));
    TileSpec t;
    if (!pick_holding_tile(ladder, nv, &t) &&
        !pick_lds_tile(lds_ladder(op, dt, cols, kKindWg), lds_row_vectors(dt, cols), &t))
        return false;
    t.vb = vb;
    *out = t;
    return true;
}

bool split_tile(int op, int dt, int64_t cols, int p, TileSpec *out)
{
    if (p != 2 && p != 4 && p != 8)
        return false;
    const int vb = held_vec_bytes(op, dt, cols, kPathSplit);
    const int64_t nv = held_vectors(op, dt, cols, kPathSplit);
    const int64_t per = slice_vectors(nv, p, vb);
    if (per * (p - 1) >= nv)
        return false;  // the last slice would be empty: too narrow to split p ways
    std::vector<TileSpec> ladder;
    for (const TileSpec &u : tiles_for(kKindSplit, vb == 16))
        if (tile_enabled(op, dt, kKindSplit, u.block, u.items, vb, held_row_kind(op, dt, cols, kPathSplit)))
            ladder.push_back(u);
    // the LDS tier holds rows of whole 16-byte vectors as they are (no shift)
    const int64_t nvl = lds_row_vectors(dt, cols);
    const int64_t perl = slice_vectors(nvl, p, 16);
    TileSpec t;
    if (!pick_holding_tile(ladder, per, &t) &&
        !(perl * (p - 1) < nvl && pick_lds_tile(lds_ladder(op, dt, cols, kKindSplit), perl, &t)))
        return false;
    t.vb = vb;
    *out = t;
    return true;
}

TileSpec reread_tile(int dt, int64_t cols)
{
    const int vb = vec_bytes_for(dt, cols);
    const int64_t nv = cols * elem_bytes(dt) / vb;
    const auto &ladder = tiles_for(kKindReread, vb == 16);
    TileSpec t = ladder.front();
    if (vb == 16) {
        // enough threads to give each one a few vectors per pass
        for (const TileSpec &c : ladder)
            if (static_cast<int64_t>(c.block) * c.items * 2 <= nv)
                t = c;
    }
    t.vb = vb;
    return t;
}

double tile_capacity_bytes(const TileSpec &t) { return static_cast<double>(t.block) * (t.items + t.lds) * t.vb; }

double onchip_budget_bytes(const DeviceModel &d) { return d.vgpr_bytes_per_cu + d.lds_bytes_per_cu; }

// ---------------------------------------------------------------------------
// Cost model (CREDIT paper, Sec. III-D), for gfx950.
//
// stream_time_us prices one launch of a non-split plan from its shape, its
// tile and the compiled kernel's occupancy: owners (rows, or row slices)
// run in rounds of the resident slots; a round streams its bytes at the
// device rate unless the bytes in flight per CU are too few to cover the
// memory latency (occupancy enters here), and no owner finishes a row faster
// than a fixed latency plus a cost per vector each thread holds.  The split
// path is priced the paper's way, relative to the best non-split baseline
// (split_terms: Eq. 7's saved reread at the baseline's own rate, Eq. 8's row
// waves, Eq. 9's difference), with one term added for gfx950: a baseline that
// leaves CUs idle (fewer owners than CUs) gains from splitting rows across
// them even when it rereads nothing.  The constants are fitted to exhaustive
// timings of calibration shapes (model_fit.py) and can be replaced by a
// calibration file.
// ---------------------------------------------------------------------------
namespace {

constexpr double kExchangeWordBytes = 8.0;  // one {value, tag} exchange word

// b_in: bytes per element of all row inputs (the bytes a reread reads again);
// b_out: bytes per element written; row_bytes = N (b_in + b_out).
struct Shape {
    double M, N, b_in, b_out, row_bytes, bytes_io;
    int inputs;
};

Shape shape_of(const PlanRequest &req)
{
    Shape s;
    s.M = static_cast<double>(req.rows);
    s.N = static_cast<double>(req.cols);
    s.b_in = in_bytes(req.op, req.dt);
    s.b_out = out_bytes(req.op, req.dt);
    s.inputs = op_inputs(req.op);
    s.row_bytes = s.N * (s.b_in + s.b_out);
    s.bytes_io = s.M * s.N * (s.b_in + s.b_out) + s.N * elem_bytes(req.dt) * n_params(req.op) +
                 s.M * row_out_bytes(req.op);
    return s;
}

// Estimated resident workgroups per CU for a tile when the compiled
// kernel's occupancy is not known: VGPRs from the held data plus a fixed
// overhead, 512 VGPRs per SIMD lane, 4 SIMDs, at most 8 waves per SIMD.
int estimate_wgs_per_cu(const TileSpec &t, int inputs, const DeviceModel &d)
{
    const int waves = t.kind == kKindWave ? 4 : std::max(1, t.block / 64);
    const int data_vgprs = inputs * ((t.kind == kKindReread) ? t.items * t.vb / 4 * 2 : t.items * t.vb / 4);
    const int vgprs = (data_vgprs + 32 + 7) / 8 * 8;
    const int waves_per_simd = std::min(8, 512 / vgprs);
    int wgs = std::max(1, (4 * waves_per_simd) / waves);
    if (t.lds > 0)  // the LDS part: block * lds vectors per input
        wgs = std::min(wgs, std::max(1, static_cast<int>(d.lds_bytes_per_cu /
                                                         (static_cast<double>(t.block) * t.lds * t.vb * inputs))));
    return wgs;
}

int kind_of(int path, const TileSpec &t)
{
    if (path == kPathSplit)
        return kKindSplit;
    if (path == kPathReread)
        return kKindReread;
    return t.block == 64 ? kKindWave : kKindWg;
}

}  // namespace

int occupancy_of(const PlanRequest &req, const Calibration &cal, int path, const TileSpec &t)
{
    OccKey k;
    k.op = req.op;
    k.dt = req.dt;
    k.kind = kind_of(path, t);
    k.block = t.block;
    k.items = t.items;
    k.vb = t.vb;
    k.part = plan_row_kind(req.op, req.dt, req.cols, path, t.lds);
    k.lds = t.lds;
    if (cal.occ_query) {
        const int o = cal.occ_query(k);
        if (o > 0)
            return o;
    }
    auto it = cal.occupancy.find(k.tuple());
    if (it != cal.occupancy.end() && it->second > 0)
        return it->second;
    TileSpec u = t;
    u.kind = k.kind;
    return estimate_wgs_per_cu(u, op_inputs(req.op), cal.device);
}

double stream_time_us(const PlanRequest &req, const Calibration &cal, int path, const TileSpec &t,
                      int wgs_per_cu_mode)
{
    const ModelConsts &m = cal.model;
    const DeviceModel &d = cal.device;
    const Shape s = shape_of(req);
    const double cus = d.cus;
    const double bw = (cal.peak_bandwidth ? d.hbm_peak_gbs : m.bw_gbs) * 1e3;  // bytes per us
    const double occ = occupancy_of(req, cal, path, t);
    const bool wave = path == kPathSingle && t.block == 64;
    const double own_per_wg = wave ? 4.0 : 1.0;  // a wave-per-row workgroup holds four rows
    const double slots = occ * cus * own_per_wg;  // rows resident at once
    const double extra = path == kPathReread ? s.N * s.b_in * m.miss3 : 0.0;
    const bool persistent = path == kPathSingle && wgs_per_cu_mode == 0;
    const double n_conc = std::min(s.M, slots);
    const double cus_active = std::max(1.0, std::min(cus, std::ceil(n_conc / (occ * own_per_wg))));
    double own_in = s.N * s.b_in;
    if (path == kPathReread)  // the reread kernel holds one streamed chunk per input
        own_in = std::min(own_in, static_cast<double>(t.block) * t.items * t.vb * s.inputs);
    const double inflight_cu = n_conc / cus_active * own_in;
    const double bw_eff = std::max(1.0, std::min(bw, cus_active * inflight_cu / m.lat_us));
    const double eta = (path == kPathReread ? m.eta3 : 1.0) * (persistent ? m.persist : 1.0);
    const double per = (s.row_bytes + extra) * eta;
    const double t_min = m.l0_us + m.item_us * (t.items + t.lds) + (path == kPathReread ? m.own3_us : 0.0) +
                         (s.row_bytes + extra) / (m.owner_gbs * 1e3);
    if (persistent) {
        const double iters = std::ceil(s.M / std::max(1.0, n_conc));
        return m.launch_us + iters * std::max(n_conc * per / bw_eff, t_min);
    }
    const double rounds = std::ceil(s.M / slots);
    const double last = s.M - (rounds - 1.0) * slots;
    const double t_full = std::max(slots * per / bw_eff, t_min);
    const double t_last = std::max(last * per / bw_eff, t_min);
    return m.launch_us + (rounds - 1.0) * t_full + t_last;
}

SplitTerms split_terms(const PlanRequest &req, const Calibration &cal, int P, const TileSpec &t, int base_path,
                       const TileSpec &base_tile, double t_base_us)
{
    const ModelConsts &m = cal.model;
    const DeviceModel &d = cal.device;
    const Shape s = shape_of(req);
    SplitTerms r;
    r.t_base_us = t_base_us;
    // bytes per element the baseline schedule moves, and its reread (Eq. 4)
    r.b_reread = base_path == kPathReread ? s.b_in : 0.0;
    r.b_base = s.b_in + s.b_out + r.b_reread;
    r.t_save_us = r.b_reread / r.b_base * t_base_us;  // Eq. 7
    // the fraction of the CUs each schedule gives work (workgroups are spread
    // over the CUs before any CU takes a second one)
    auto busy = [&](double wgs) { return std::min(1.0, wgs / d.cus); };
    const double u_base = busy(base_path == kPathSingle && base_tile.block == 64 ? std::ceil(s.M / 4.0) : s.M);
    const double u_split = busy(s.M * P);
    r.t_occ_us = (t_base_us - r.t_save_us) * std::max(0.0, 1.0 - u_base / u_split);
    // Eq. 8: sequential row waves of the persistent clusters, each one exchange
    r.resident = static_cast<double>(occupancy_of(req, cal, kPathSplit, t)) * d.cus;
    const double clusters = std::max(1.0, std::min(std::floor(r.resident / P), s.M));
    r.waves = std::ceil(s.M / clusters);
    r.t_ctrl_us = r.waves * m.exch_us + m.split_launch_us;
    // remote words: each workgroup publishes q words that P - 1 peers read;
    // the P workgroups do so at once, so the elapsed cost is not P times one
    // workgroup's (Eq. 8)
    r.t_dsm_us = kExchangeWordBytes * r.waves * (P - 1) * stats_per_partial(req.op) / (m.word_gbs * 1e3);
    r.delta_us = r.t_save_us + r.t_occ_us - r.t_ctrl_us - r.t_dsm_us;  // Eq. 9 (T_replay = T_deposit = 0)
    r.t_split_us = t_base_us - r.delta_us;
    return r;
}

double calib_time_us(const CalibEntry &e, double rows)
{
    const size_t n = e.rows.size();
    if (n == 0)
        return -1.0;
    if (n == 1)
        return e.us[0] * rows / e.rows[0];
    size_t i = 0;
    while (i + 2 < n && rows > e.rows[i + 1])
        ++i;
    const double l1 = std::log(e.rows[i]), l2 = std::log(e.rows[i + 1]);
    const double t1 = std::log(e.us[i]), t2 = std::log(e.us[i + 1]);
    const double lx = std::log(std::max(rows, 1.0));
    return std::exp(t1 + (t2 - t1) * (lx - l1) / (l2 - l1));
}

namespace {

// Whether a table entry's tile is compiled for this width's row kind and
// holds the row (or its widest slice) as that kind: a table measured on
// another kernel set (before a width's rows were shifted, say) can hold
// plans the library would now refuse.
bool entry_holds(const PlanRequest &req, const CalibEntry &e)
{
    if (e.path == kPathReread)
        return true;
    const int kind = e.path == kPathSplit ? kKindSplit : (e.block == 64 ? kKindWave : kKindWg);
    const int vb = held_vec_bytes(req.op, req.dt, req.cols, e.path);
    if (e.lds > 0 ? !lds_tile_enabled(req.op, req.dt, kind, e.block, e.items)
                  : !tile_enabled(req.op, req.dt, kind, e.block, e.items, vb,
                                  plan_row_kind(req.op, req.dt, req.cols, e.path, 0)))
        return false;
    const int64_t nv = e.lds > 0 ? lds_row_vectors(req.dt, req.cols) : held_vectors(req.op, req.dt, req.cols, e.path);
    int64_t need = nv;
    if (e.path == kPathSplit) {
        need = slice_vectors(nv, e.split_p, e.lds > 0 ? 16 : vb);
        if (need * (e.split_p - 1) >= nv)
            return false;
    }
    return nv > 0 && need <= static_cast<int64_t>(e.block) * (e.items + e.lds);
}

// Plan from the calibration table when it measured this (op, dtype, cols)
// and holds a candidate the forced path / P allow: every such candidate's
// time at req.rows is interpolated from its measurements, and the fastest
// wins.  Returns false when the table cannot decide, or measured this width
// with an access width no longer planned (then the neighbours price it).
// Entries whose tile no longer holds the row as the library holds it now are
// passed over, and a width where a held path the library now offers has no
// entry is left to the neighbours.
bool plan_from_table(const PlanRequest &req, const Calibration &cal, int forced_path, int forced_p, Plan *out)
{
    Plan p;
    const CalibEntry *best = nullptr;
    double best_us = 0.0;
    for (const CalibEntry &e : cal.table) {
        if (e.op != req.op || e.dt != req.dt || e.cols != req.cols)
            continue;
        if (forced_path != kPathAuto && e.path != forced_path)
            continue;
        if (forced_p != 0 && e.path == kPathSplit && e.split_p != forced_p)
            continue;
        if (e.vb != path_vec_bytes(req.op, req.dt, req.cols, e.path))
            return false;  // measured with an access width no longer planned: price from the neighbours
        if (!entry_holds(req, e))
            continue;
        const double us = calib_time_us(e, static_cast<double>(req.rows));
        PathEstimate &pe = p.est[e.path - 1];
        if (!pe.legal || us < pe.us) {
            pe.legal = true;
            pe.us = us;
            pe.split_p = e.split_p;
            pe.tile = TileSpec{0, e.block, e.items, e.vb, e.lds};
        }
        if (best == nullptr || us < best_us) {
            best = &e;
            best_us = us;
        }
    }
    if (best == nullptr)
        return false;
    if (forced_path == kPathAuto) {
        // a held path the library offers at this width now but the table never
        // timed here (it was timed on another kernel set): the table cannot
        // weigh it, the neighbours price it
        TileSpec t;
        bool split_now = false;
        for (int P : {2, 4, 8})
            split_now = split_now || ((forced_p == 0 || P == forced_p) && split_tile(req.op, req.dt, req.cols, P, &t));
        if ((!p.est[0].legal && single_tile(req.op, req.dt, req.cols, &t)) || (!p.est[1].legal && split_now))
            return false;
    }
    p.path = best->path;
    p.split_p = best->split_p;
    p.wgs_per_cu = best->wgs_per_cu;
    p.tile = TileSpec{0, best->block, best->items, best->vb, best->lds};
    *out = p;
    return true;
}

// Time of candidate `cd` at a width the table did not measure, from the same
// plan's measurements at the nearest calibrated widths below and above:
// each is read at the row count that moves the same bytes, and the two are
// interpolated in (log cols, log time); one side alone is used as it is.
// A held plan (paths 1, 2) runs partial-vector kernels on rows that end in a
// partial 16-byte vector and ODD kernels on odd-length bf16 rows, which
// stream slower than whole-vector rows: widths are priced from widths of the
// same kind (held_row_kind), and another kind serves only where the plan was
// never measured on the same kind.
// Negative when the table never measured the plan.
double neighbour_time_us(const PlanRequest &req, const Calibration &cal, const Candidate &cd)
{
    const CalibEntry *lo = nullptr, *hi = nullptr;
    const bool held = cd.path != kPathReread;
    const int kind = plan_row_kind(req.op, req.dt, req.cols, cd.path, cd.est.tile.lds);
    for (int same_kind = 1; same_kind >= 0 && lo == nullptr && hi == nullptr; --same_kind)
        for (const CalibEntry &e : cal.table) {
            if (e.op != req.op || e.dt != req.dt || e.path != cd.path || e.split_p != cd.split_p ||
                e.block != cd.est.tile.block || e.items != cd.est.tile.items || e.vb != cd.est.tile.vb ||
                e.lds != cd.est.tile.lds ||
                e.wgs_per_cu != cd.wgs_per_cu || e.rows.empty())
                continue;
            if (same_kind && held && plan_row_kind(e.op, e.dt, e.cols, e.path, e.lds) != kind)
                continue;
            if (e.cols <= req.cols && (lo == nullptr || e.cols > lo->cols))
                lo = &e;
            if (e.cols >= req.cols && (hi == nullptr || e.cols < hi->cols))
                hi = &e;
        }
    const double bytes_rows = static_cast<double>(req.rows) * static_cast<double>(req.cols);
    auto at = [&](const CalibEntry *e) { return calib_time_us(*e, bytes_rows / static_cast<double>(e->cols)); };
    if (lo == nullptr && hi == nullptr)
        return -1.0;
    if (lo == nullptr || lo == hi)
        return at(hi);
    if (hi == nullptr)
        return at(lo);
    const double w = std::log(static_cast<double>(req.cols) / lo->cols) / std::log(static_cast<double>(hi->cols) / lo->cols);
    return std::exp((1.0 - w) * std::log(at(lo)) + w * std::log(at(hi)));
}

// Plan for a width the table did not measure: every legal candidate the
// table measured at some width is priced by neighbour_time_us and the
// fastest wins.  Returns false when no candidate was ever measured (odd
// widths without odd-width calibration, another device's table).
bool plan_from_neighbours(const PlanRequest &req, const Calibration &cal, int forced_path, int forced_p, Plan *out)
{
    std::vector<Candidate> cands;
    enumerate_candidates(req, cal, &cands);
    Plan p;
    const Candidate *best = nullptr;
    double best_us = 0.0;
    for (const Candidate &cd : cands) {
        if (forced_path != kPathAuto && cd.path != forced_path)
            continue;
        if (forced_p != 0 && cd.path == kPathSplit && cd.split_p != forced_p)
            continue;
        const double us = neighbour_time_us(req, cal, cd);
        if (us < 0.0)
            continue;
        PathEstimate &pe = p.est[cd.path - 1];
        if (!pe.legal || us < pe.us) {
            pe = cd.est;
            pe.legal = true;
            pe.us = us;
        }
        if (best == nullptr || us < best_us) {
            best = &cd;
            best_us = us;
        }
    }
    if (best == nullptr)
        return false;
    p.path = best->path;
    p.split_p = best->split_p;
    p.wgs_per_cu = best->wgs_per_cu;
    p.tile = best->est.tile;
    *out = p;
    return true;
}

}  // namespace

// A held tile is a candidate when it holds `need` vectors and is at least
// half used (or is the smallest tile that holds them).
static bool worth_holding(const std::vector<TileSpec> &ladder, const TileSpec &t, int64_t need)
{
    const int64_t cap = static_cast<int64_t>(t.block) * t.items;
    if (cap < need)
        return false;
    if (cap < 2 * need)
        return true;
    for (const TileSpec &u : ladder) {
        const int64_t c = static_cast<int64_t>(u.block) * u.items;
        if (c >= need && c < cap)
            return false;
    }
    return true;
}

// The path-1 tiles worth pricing for a row: the register tiles that hold it
// and are at least half used, and the LDS-tier tiles whose register part the
// row fills (otherwise the same registers alone hold it).  A shifted row
// whose span no register tile holds, though its whole 16-byte vectors would
// fit one, is held unshifted by an LDS-tier tile.  vb is set on each.
static std::vector<TileSpec> held_candidates(int op, int dt, int64_t cols)
{
    const int vb = held_vec_bytes(op, dt, cols, kPathSingle);
    const int64_t nv = held_vectors(op, dt, cols, kPathSingle);
    const int part = held_row_kind(op, dt, cols, kPathSingle);
    const std::vector<TileSpec> held = single_ladder(op, dt, vb, part);
    std::vector<TileSpec> out;
    bool reg_holds = false;
    for (TileSpec t : held) {
        reg_holds = reg_holds || static_cast<int64_t>(t.block) * t.items >= nv;
        if (!worth_holding(held, t, nv))
            continue;
        t.vb = vb;
        out.push_back(t);
    }
    const int64_t nvl = lds_row_vectors(dt, cols);
    for (const TileSpec &t : lds_ladder(op, dt, cols, kKindWg)) {
        const int64_t reg = static_cast<int64_t>(t.block) * t.items;
        if ((nvl <= reg && reg_holds) || nvl > reg + static_cast<int64_t>(t.block) * t.lds)
            continue;
        out.push_back(t);
    }
    return out;
}

// The split tiles worth pricing at width p: the register tiles that hold a
// slice and are at least half used, and the LDS-tier tiles that hold an
// (unshifted) slice no register tile holds or whose register part it fills.
static std::vector<TileSpec> split_candidates(int op, int dt, int64_t cols, int p)
{
    const int vb = held_vec_bytes(op, dt, cols, kPathSplit);
    const int64_t nv = held_vectors(op, dt, cols, kPathSplit);
    const int part = held_row_kind(op, dt, cols, kPathSplit);
    const int64_t nvl = lds_row_vectors(dt, cols);
    const int64_t per = slice_vectors(nv, p, vb);
    const int64_t perl = slice_vectors(nvl, p, 16);
    const bool reg_ok = per * (p - 1) < nv;
    const bool lds_ok = nvl > 0 && perl * (p - 1) < nvl;
    std::vector<TileSpec> tiles;
    if (!reg_ok && !lds_ok)
        return tiles;
    std::vector<TileSpec> ladder;
    for (const TileSpec &u : tiles_for(kKindSplit, vb == 16))
        if (tile_enabled(op, dt, kKindSplit, u.block, u.items, vb, part))
            ladder.push_back(u);
    for (TileSpec t : ladder)
        if (reg_ok && worth_holding(ladder, t, per)) {
            t.vb = vb;
            tiles.push_back(t);
        }
    const bool reg_holds_slice = !tiles.empty();
    for (const TileSpec &t : lds_ladder(op, dt, cols, kKindSplit)) {
        const int64_t reg = static_cast<int64_t>(t.block) * t.items;
        if (lds_ok && (perl > reg || !reg_holds_slice) && perl <= reg + static_cast<int64_t>(t.block) * t.lds)
            tiles.push_back(t);
    }
    return tiles;
}

bool make_plan(const PlanRequest &req, const Calibration &cal, int forced_path, int forced_p, Plan *out)
{
    if (!cal.table.empty() && plan_from_table(req, cal, forced_path, forced_p, out))
        return true;
    if (!cal.table.empty() && plan_from_neighbours(req, cal, forced_path, forced_p, out))
        return true;
    // The analytic model.  The non-split baseline is path 1 when a tile holds
    // the row (a held row is never reread: path 3 moves b_in more bytes per
    // element at the same rate), else path 3; each split width P is priced
    // against it by Eq. 7-9 (split_terms) and the fastest prediction wins.
    // Within a path the tile is the one pick_holding_tile prefers.  Taking
    // the candidate tile this model prices fastest instead scored worse on
    // MI355X (61 against 74 of the 90 width-sweep shapes within 1% of the
    // fastest plan): the model's terms that depend on the tile, occupancy and
    // vectors per thread, rank the tiles of one path worse than that rule.
    Plan p;
    TileSpec t1;
    if (single_tile(req.op, req.dt, req.cols, &t1)) {
        PathEstimate &e = p.est[0];
        e.legal = true;
        e.tile = t1;
        e.us = stream_time_us(req, cal, kPathSingle, t1, -1);
    }
    {
        PathEstimate &e = p.est[2];
        for (TileSpec t : tiles_for(kKindReread, vec_bytes_for(req.dt, req.cols) == 16)) {
            t.kind = kKindReread;
            t.vb = vec_bytes_for(req.dt, req.cols);
            const double us = stream_time_us(req, cal, kPathReread, t, 0);
            if (!e.legal || us < e.us) {
                e.legal = true;
                e.tile = t;
                e.us = us;
            }
        }
    }
    const bool single_legal = p.est[0].legal;
    const int base_path = single_legal ? kPathSingle : kPathReread;
    const PathEstimate &base = p.est[base_path - 1];
    for (int P : {2, 4, 8}) {
        if (forced_p != 0 && P != forced_p)
            continue;
        TileSpec t;
        if (!split_tile(req.op, req.dt, req.cols, P, &t))
            continue;
        const SplitTerms st = split_terms(req, cal, P, t, base_path, base.tile, base.us);
        PathEstimate e;
        e.legal = true;
        e.split_p = P;
        e.tile = t;
        e.us = st.t_split_us;
        e.t_save_us = st.t_save_us;
        e.t_occ_us = st.t_occ_us;
        e.t_ctrl_us = st.t_ctrl_us;
        e.t_dsm_us = st.t_dsm_us;
        e.delta_us = st.delta_us;
        e.waves = st.waves;
        if (!p.est[1].legal || e.us < p.est[1].us)
            p.est[1] = e;
    }

    int path = forced_path;
    if (path == kPathAuto)
        path = p.est[1].legal && p.est[1].delta_us > 0.0 ? kPathSplit : base_path;
    if (path < 1 || path > 3 || !p.est[path - 1].legal)
        return false;
    p.path = path;
    p.split_p = path == kPathSplit ? p.est[1].split_p : 1;
    // path 1: one row per owner (measured at least as fast as owners that loop)
    p.wgs_per_cu = path == kPathSingle ? -1 : 0;
    p.tile = p.est[path - 1].tile;
    *out = p;
    return true;
}

bool analytic_baseline(const PlanRequest &req, const Calibration &cal, int *path, TileSpec *tile, double *us)
{
    Calibration c = cal;
    c.table.clear();
    Plan p;
    if (!make_plan(req, c, kPathAuto, 0, &p))
        return false;
    *path = p.est[0].legal ? kPathSingle : kPathReread;
    *tile = p.est[*path - 1].tile;
    *us = p.est[*path - 1].us;
    return true;
}

void enumerate_candidates(const PlanRequest &req, const Calibration &cal, std::vector<Candidate> *out)
{
    out->clear();
    // held tiles (paths 1, 2) and the reread tiles of path 3 can differ in
    // access width: a partial row is held as 16-byte vectors, reread by element
    for (const TileSpec &t : held_candidates(req.op, req.dt, req.cols))
        for (int mode : {0, -1}) {
            PathEstimate e;
            e.legal = true;
            e.tile = t;
            e.us = stream_time_us(req, cal, kPathSingle, t, mode);
            out->push_back(Candidate{kPathSingle, 1, e, mode});
        }
    const int rvb = vec_bytes_for(req.dt, req.cols);
    for (TileSpec t : tiles_for(kKindReread, rvb == 16)) {
        t.vb = rvb;
        PathEstimate e;
        e.legal = true;
        e.tile = t;
        e.us = stream_time_us(req, cal, kPathReread, t, 0);
        out->push_back(Candidate{kPathReread, 1, e, 0});
    }
    int base_path = 0;
    TileSpec base_tile;
    double base_us = 0.0;
    if (!analytic_baseline(req, cal, &base_path, &base_tile, &base_us))
        return;
    for (int P : {2, 4, 8})
        for (const TileSpec &t : split_candidates(req.op, req.dt, req.cols, P)) {
            const SplitTerms st = split_terms(req, cal, P, t, base_path, base_tile, base_us);
            PathEstimate e;
            e.legal = true;
            e.split_p = P;
            e.tile = t;
            e.us = st.t_split_us;
            e.t_save_us = st.t_save_us;
            e.t_occ_us = st.t_occ_us;
            e.t_ctrl_us = st.t_ctrl_us;
            e.t_dsm_us = st.t_dsm_us;
            e.delta_us = st.delta_us;
            e.waves = st.waves;
            out->push_back(Candidate{kPathSplit, P, e, 0});
        }
}

// ---------------------------------------------------------------------------
// Minimal JSON reader for the calibration file: objects, arrays, numbers,
// strings, true/false/null.  Values are flattened to "a.b.c" -> number and
// "a.b[i][j]" -> number.
// ---------------------------------------------------------------------------
namespace {

struct JsonReader {
    const std::string &s;
    size_t i = 0;
    std::map<std::string, double> nums;
    explicit JsonReader(const std::string &t) : s(t) {}

    void ws()
    {
        while (i < s.size() && std::isspace(static_cast<unsigned char>(s[i])))
            ++i;
    }
    bool lit(const char *w)
    {
        size_t n = std::char_traits<char>::length(w);
        if (s.compare(i, n, w) == 0) {
            i += n;
            return true;
        }
        return false;
    }
    bool str(std::string *out)
    {
        ws();
        if (i >= s.size() || s[i] != '"')
            return false;
        ++i;
        std::string r;
        while (i < s.size() && s[i] != '"') {
            if (s[i] == '\\') {
                if (i + 1 >= s.size())
                    return false;
                r.push_back(s[i + 1]);
                i += 2;
            } else {
                r.push_back(s[i++]);
            }
        }
        if (i >= s.size())
            return false;
        ++i;
        *out = r;
        return true;
    }
    bool value(const std::string &path, int depth)
    {
        if (depth > 16)
            return false;
        ws();
        if (i >= s.size())
            return false;
        const char c = s[i];
        if (c == '{') {
            ++i;
            ws();
            if (i < s.size() && s[i] == '}') {
                ++i;
                return true;
            }
            for (;;) {
                std::string k;
                if (!str(&k))
                    return false;
                ws();
                if (i >= s.size() || s[i] != ':')
                    return false;
                ++i;
                if (!value(path.empty() ? k : path + "." + k, depth + 1))
                    return false;
                ws();
                if (i < s.size() && s[i] == ',') {
                    ++i;
                    continue;
                }
                if (i < s.size() && s[i] == '}') {
                    ++i;
                    return true;
                }
                return false;
            }
        }
        if (c == '[') {
            ++i;
            ws();
            if (i < s.size() && s[i] == ']') {
                ++i;
                return true;
            }
            for (int idx = 0;; ++idx) {
                if (!value(path + "[" + std::to_string(idx) + "]", depth + 1))
                    return false;
                ws();
                if (i < s.size() && s[i] == ',') {
                    ++i;
                    continue;
                }
                if (i < s.size() && s[i] == ']') {
                    ++i;
                    return true;
                }
                return false;
            }
        }
        if (c == '"') {
            std::string tmp;
            return str(&tmp);
        }
        if (lit("true")) {
            nums[path] = 1.0;
            return true;
        }
        if (lit("false")) {
            nums[path] = 0.0;
            return true;
        }
        if (lit("null"))
            return true;
        const char *begin = s.c_str() + i;
        char *end = nullptr;
        const double v = std::strtod(begin, &end);
        if (end == begin)
            return false;
        i += static_cast<size_t>(end - begin);
        nums[path] = v;
        return true;
    }
};

}  // namespace

bool parse_calibration(const std::string &text, Calibration *out)
{
    JsonReader r(text);
    if (!r.value("", 0))
        return false;
    r.ws();
    if (r.i != text.size())
        return false;
    Calibration c;
    auto get = [&](const char *k, double *dst) {
        auto it = r.nums.find(k);
        if (it != r.nums.end())
            *dst = it->second;
    };
    if (r.nums.find("version") == r.nums.end())
        return false;
    double peak = 0.0;
    get("model_peak_bandwidth", &peak);
    c.peak_bandwidth = peak != 0.0;
    // the analytic model's constants (model_fit.py); the control kernel's
    // measured exchange cost per row wave (ctrlbench.py) is Eq. 8's T_ctrl
    // per wave when the file has no fitted one
    get("exchange_us", &c.model.exch_us);
    ModelConsts &m = c.model;
    const std::pair<const char *, double *> consts[] = {
        {"model.bw_gbs", &m.bw_gbs},       {"model.lat_us", &m.lat_us},
        {"model.miss3", &m.miss3},         {"model.l0_us", &m.l0_us},
        {"model.item_us", &m.item_us},     {"model.own3_us", &m.own3_us},
        {"model.launch_us", &m.launch_us}, {"model.exch_us", &m.exch_us},
        {"model.split_launch_us", &m.split_launch_us}, {"model.eta3", &m.eta3},
        {"model.persist", &m.persist},     {"model.owner_gbs", &m.owner_gbs},
        {"model.word_gbs", &m.word_gbs}};
    for (const auto &kv : consts)
        get(kv.first, kv.second);
    if (!(m.bw_gbs > 0) || !(m.lat_us > 0) || !(m.word_gbs > 0) || !(m.owner_gbs > 0) || m.miss3 < 0 || m.eta3 <= 0 || m.persist <= 0)
        return false;
    // Version 3 rows carry the LDS-tier vectors per thread (version 2 rows
    // describe register-only tiles).
    const bool v3 = r.nums["version"] >= 3.0;
    const int nkey = v3 ? 8 : 7;
    // occupancy[i] = [op, dt, kind, block, items, vec_bytes, row kind, (lds,) workgroups per CU]
    for (int i = 0;; ++i) {
        const std::string pre = "occupancy[" + std::to_string(i) + "]";
        std::array<int, 8> key{};
        double v = 0.0;
        auto it = r.nums.find(pre + "[0]");
        if (it == r.nums.end())
            break;
        for (int j = 0; j < nkey; ++j) {
            auto jt = r.nums.find(pre + "[" + std::to_string(j) + "]");
            if (jt == r.nums.end())
                return false;
            key[j] = static_cast<int>(jt->second);
        }
        auto vt = r.nums.find(pre + "[" + std::to_string(nkey) + "]");
        if (vt == r.nums.end())
            return false;
        v = vt->second;
        if (v < 1 || v > 64)
            return false;
        c.occupancy[key] = static_cast<int>(v);
    }
    // table[i] = [op, dt, cols, path, split_p, block, items, (lds,) vec_bytes, wgs_per_cu, n,
    //             rows_1, us_1, ..., rows_n, us_n]
    for (int i = 0;; ++i) {
        const std::string pre = "table[" + std::to_string(i) + "]";
        auto at = [&](int j, double *v) {
            auto it = r.nums.find(pre + "[" + std::to_string(j) + "]");
            if (it == r.nums.end())
                return false;
            *v = it->second;
            return true;
        };
        const int nfix = v3 ? 11 : 10;
        double f[11];
        if (!at(0, &f[0]))
            break;
        for (int j = 1; j < nfix; ++j)
            if (!at(j, &f[j]))
                return false;
        const int o = v3 ? 1 : 0;  // columns after `items` shift by one in version 3
        CalibEntry e;
        e.op = static_cast<int>(f[0]);
        e.dt = static_cast<int>(f[1]);
        e.cols = static_cast<int64_t>(f[2]);
        e.path = static_cast<int>(f[3]);
        e.split_p = static_cast<int>(f[4]);
        e.block = static_cast<int>(f[5]);
        e.items = static_cast<int>(f[6]);
        e.lds = v3 ? static_cast<int>(f[7]) : 0;
        e.vb = static_cast<int>(f[7 + o]);
        e.wgs_per_cu = static_cast<int>(f[8 + o]);
        const int n = static_cast<int>(f[9 + o]);
        if (!op_supported(e.op, e.dt) || e.cols < 1 || e.path < 1 || e.path > 3 || n < 1 || n > 64 || e.lds < 0 ||
            e.lds > 64)
            return false;
        for (int j = 0; j < n; ++j) {
            double rr = 0.0, tt = 0.0;
            if (!at(nfix + 2 * j, &rr) || !at(nfix + 1 + 2 * j, &tt) || !(rr >= 1.0) || !(tt > 0.0))
                return false;
            if (!e.rows.empty() && rr <= e.rows.back())
                return false;
            e.rows.push_back(rr);
            e.us.push_back(tt);
        }
        c.table.push_back(e);
    }
    double cus = -1;
    get("device.cus", &cus);
    if (cus > 0) {
        c.has_device = true;
        c.device.cus = static_cast<int>(cus);
        get("device.xcds", &cus);
        c.device.xcds = std::max(1, static_cast<int>(cus));
        get("device.clock_ghz", &c.device.clock_ghz);
        get("device.hbm_peak_gbs", &c.device.hbm_peak_gbs);
        get("device.l2_bytes_per_xcd", &c.device.l2_bytes_per_xcd);
        get("device.mall_bytes", &c.device.mall_bytes);
    }
    c.loaded = true;
    *out = c;
    return true;
}

}  // namespace credit
