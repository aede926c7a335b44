// C ABI of libcredit.so (declared in include/credit.h): argument validation,
// planning, the per-(device, stream) split-row scratch, and kernel launches.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>
#include <utility>
#include <vector>

#include "api_internal.hpp"
#include "args.hpp"
#include "credit.h"
#include "planner.hpp"
#include "registry.hpp"

namespace credit {
namespace {

// ---------------------------------------------------------------------------
// kernel registry
// ---------------------------------------------------------------------------
const std::vector<KernelEntry> &registry()
{
    static const std::vector<KernelEntry> table = [] {
        std::vector<KernelEntry> r;
        register_softmax_kernels(r);
        register_layernorm_kernels(r);
        register_rmsnorm_kernels(r);
        register_softmax_bwd_kernels(r);
        register_layernorm_bwd_kernels(r);
        register_quantize_kernels(r);
        register_misc_kernels(r);
        return r;
    }();
    return table;
}

const KernelEntry *find_kernel(int kind, int op, int dt, int vb, int block, int items, int part = 0, int lds = 0)
{
    for (const KernelEntry &e : registry())
        if (e.kind == kind && e.op == op && e.dt == dt && e.vb == vb && e.block == block && e.items == items &&
            e.part == part && e.lds == lds)
            return &e;
    return nullptr;
}

const KernelEntry *find_misc(int id)
{
    for (const KernelEntry &e : registry())
        if (e.kind == 0 && e.op == id)
            return &e;
    return nullptr;
}

// ---------------------------------------------------------------------------
// calibration and device description
// ---------------------------------------------------------------------------
std::mutex g_mu;
Calibration g_cal;
std::map<int, DeviceModel> g_devices;

credit_status_t load_calibration_file(const char *json_path, Calibration *out);

// The calibration named by CREDIT_CALIB, loaded once before the first plan.
// Caller holds g_mu.
void load_env_calibration_locked()
{
    static bool done = false;
    if (done)
        return;
    done = true;
    const char *path = std::getenv("CREDIT_CALIB");
    if (path == nullptr || path[0] == '\0' || g_cal.loaded)
        return;
    Calibration c;
    if (load_calibration_file(path, &c) == CREDIT_OK)
        g_cal = c;
}

DeviceModel device_model_locked()
{
    load_env_calibration_locked();
    if (g_cal.has_device)
        return g_cal.device;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return DeviceModel{};
    }
    auto it = g_devices.find(dev);
    if (it != g_devices.end())
        return it->second;
    DeviceModel d;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
        d.cus = cus;
    else
        (void)hipGetLastError();
    g_devices[dev] = d;
    return d;
}

credit_status_t occupancy(const KernelEntry *k, int *out);

// Resident workgroups per CU of the compiled kernel `key` names, from the HIP
// runtime; 0 when there is no such kernel or no device to ask.
int kernel_occupancy(const OccKey &key)
{
    const KernelEntry *k = find_kernel(key.kind, key.op, key.dt, key.vb, key.block, key.items, key.part, key.lds);
    int occ = 0;
    if (k == nullptr || occupancy(k, &occ) != CREDIT_OK)
        return 0;
    return occ;
}

// The calibration in force with the device description and the compiled
// kernels' occupancy filled in.  Caller holds g_mu.
Calibration calibration_locked()
{
    load_env_calibration_locked();
    Calibration cal = g_cal;
    cal.device = device_model_locked();
    cal.occ_query = kernel_occupancy;
    return cal;
}

bool log_enabled()
{
    static const bool on = [] {
        const char *v = std::getenv("CREDIT_LOG");
        return v != nullptr && v[0] != '\0' && v[0] != '0';
    }();
    return on;
}

// ---------------------------------------------------------------------------
// split-row scratch, one per (device, stream)
//
// A control block (SplitCtl) and the exchange words.  The protocol's state
// (ticket counter, tags issued) lives in the control block and is advanced
// by the kernels themselves (see split_kernel), so the host keeps no
// counters: a launch enqueued by the host and one replayed from a graph see
// the same state.  A zero-filled scratch is the initial state.
// ---------------------------------------------------------------------------
constexpr int64_t kDefaultSpinLimit = INT64_C(1) << 20;

// Polls before a split-row wait gives up (credit_test_exchange).
std::atomic<int64_t> g_spin_limit{kDefaultSpinLimit};

struct Scratch {
    SplitCtl *ctl = nullptr;  // kScratchBytes: control block, then the exchange words
};
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

bool stream_capturing(hipStream_t s)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return st != hipStreamCaptureStatusNone;
}

// Returns the scratch of (current device, s), allocating it on first use;
// CREDIT_ERR_UNSUPPORTED if that first use is under stream capture (the
// allocation cannot be captured).  Caller holds g_mu.
credit_status_t get_scratch_locked(hipStream_t s, Scratch **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return CREDIT_ERR_HIP;
    auto key = std::make_pair(dev, s);
    auto it = g_scratch.find(key);
    if (it != g_scratch.end()) {
        *out = &it->second;
        return CREDIT_OK;
    }
    if (stream_capturing(s))
        return CREDIT_ERR_UNSUPPORTED;
    void *mem = nullptr;
    if (hipMalloc(&mem, kScratchBytes) != hipSuccess) {
        (void)hipGetLastError();
        return CREDIT_ERR_HIP;
    }
    if (hipMemset(mem, 0, kScratchBytes) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(mem);
        return CREDIT_ERR_HIP;
    }
    Scratch sc;
    sc.ctl = static_cast<SplitCtl *>(mem);
    *out = &(g_scratch[key] = sc);
    return CREDIT_OK;
}

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// CREDIT_ERR_INVALID_ARG for an operator or dtype outside the enums,
// CREDIT_ERR_UNSUPPORTED for a pair without kernels.
credit_status_t check_op_dt(int op, int dt)
{
    if (op < 0 || op >= kNumOps || (dt != CREDIT_F32 && dt != CREDIT_BF16))
        return CREDIT_ERR_INVALID_ARG;
    if (!op_supported(op, dt))
        return CREDIT_ERR_UNSUPPORTED;
    return CREDIT_OK;
}

// Which operands an operator reads or writes (credit_operands_t).
bool uses_dy(int op) { return op == CREDIT_OP_SOFTMAX_BACKWARD || op == CREDIT_OP_LAYERNORM_BACKWARD; }
bool uses_gamma(int op) { return n_params(op) >= 1; }
bool uses_beta(int op) { return n_params(op) >= 2; }
bool uses_row_out(int op) { return row_out_bytes(op) > 0; }
bool uses_eps(int op)
{
    return op == CREDIT_OP_LAYERNORM || op == CREDIT_OP_RMSNORM || op == CREDIT_OP_LAYERNORM_BACKWARD;
}

credit_status_t validate(int op, const credit_operands_t &t, int64_t rows, int64_t cols, float eps, int dt,
                         bool *noop)
{
    *noop = false;
    credit_status_t st = check_op_dt(op, dt);
    if (st != CREDIT_OK)
        return st;
    if (rows < 0 || cols < 1)
        return CREDIT_ERR_INVALID_ARG;
    if (uses_eps(op) && (!std::isfinite(eps) || eps < 0.0f))
        return CREDIT_ERR_INVALID_ARG;
    // element count and byte size must fit comfortably in int64
    const int64_t eb = elem_bytes(dt);
    if (rows > 0 && cols > (INT64_C(1) << 62) / eb / rows)
        return CREDIT_ERR_INVALID_ARG;
    if (rows == 0) {
        *noop = true;
        return CREDIT_OK;
    }
    if (t.x == nullptr || t.y == nullptr || (uses_dy(op) && t.dy == nullptr) ||
        (uses_gamma(op) && t.gamma == nullptr) || (uses_beta(op) && t.beta == nullptr) ||
        (uses_row_out(op) && t.row_out == nullptr))
        return CREDIT_ERR_INVALID_ARG;
    if (!aligned16(t.x) || !aligned16(t.y) || (uses_dy(op) && !aligned16(t.dy)) ||
        (uses_gamma(op) && !aligned16(t.gamma)) || (uses_beta(op) && !aligned16(t.beta)) ||
        (uses_row_out(op) && !aligned4(t.row_out)) ||
        (op == CREDIT_OP_LAYERNORM_BACKWARD && t.row_out != nullptr &&
         (reinterpret_cast<uintptr_t>(t.row_out) & 7u) != 0))
        return CREDIT_ERR_ALIGNMENT;
    return CREDIT_OK;
}

credit_status_t check_path_args(int path, int split_p)
{
    if (path < CREDIT_PATH_AUTO || path > CREDIT_PATH_REREAD)
        return CREDIT_ERR_INVALID_ARG;
    if (path == CREDIT_PATH_SPLIT_ROW) {
        if (split_p != 0 && split_p != 2 && split_p != 4 && split_p != 8)
            return CREDIT_ERR_INVALID_ARG;
    } else if (path == CREDIT_PATH_AUTO) {
        if (split_p != 0 && split_p != 1 && split_p != 2 && split_p != 4 && split_p != 8)
            return CREDIT_ERR_INVALID_ARG;
    } else if (split_p != 0 && split_p != 1) {
        return CREDIT_ERR_INVALID_ARG;
    }
    return CREDIT_OK;
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
constexpr int64_t kMaxGridWgs = INT64_C(1) << 30;

// Optional timing events: `start` takes the first kernel's begin timestamp and
// `stop` the last kernel's end timestamp (hipExtLaunchKernel records them from
// the dispatch itself, so the interval holds no queueing or dispatch latency).
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

credit_status_t launch_raw(const KernelEntry *k, uint32_t grid, uint32_t block, void *arg, hipStream_t s,
                           hipEvent_t ev_start, hipEvent_t ev_stop)
{
    void *args[] = {arg};
    // timed launches take the dispatch timestamps through hipExtLaunchKernel;
    // the others use the plain launch, which stream capture records as a
    // kernel node
    const hipError_t e = (ev_start != nullptr || ev_stop != nullptr)
                             ? hipExtLaunchKernel(k->fn, dim3(grid), dim3(block), args, 0, s, ev_start, ev_stop, 0)
                             : hipLaunchKernel(k->fn, dim3(grid), dim3(block), args, 0, s);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return CREDIT_ERR_HIP;
    }
    return CREDIT_OK;
}

// Workgroups of kernel `k` one CU holds at once; cached per kernel.
credit_status_t occupancy(const KernelEntry *k, int *out);

// The arguments for rows [r0, r0 + n) of `a` (null pointers stay null).
RowArgs rows_from(const RowArgs &a, int op, int dt, int64_t r0, int64_t n)
{
    auto at = [](const void *p, int64_t off) -> const char * {
        return p == nullptr ? nullptr : static_cast<const char *>(p) + off;
    };
    const int64_t in_off = r0 * a.cols * elem_bytes(dt);
    RowArgs r = a;
    r.x = at(a.x, in_off);
    r.dy = at(a.dy, in_off);
    r.y = const_cast<char *>(at(a.y, r0 * a.cols * out_bytes(op, dt)));
    r.row_out = const_cast<char *>(at(a.row_out, r0 * row_out_bytes(op)));
    r.rows = n;
    return r;
}

// Paths 1 and 3.  Path 1 kernels loop over rows: with wgs_per_cu == 0 the grid
// is as many workgroups as the device holds at once (each owner then takes
// every G-th row, loading the next row while it writes the current one), with
// k > 0 at most k workgroups per CU, and with -1 one workgroup per row (or per
// four rows for wave-per-row).  The reread kernel always takes one row per
// workgroup.
credit_status_t launch_rowwise(const KernelEntry *k, const RowArgs &a0, int wgs_per_cu, hipStream_t s,
                               const LaunchEvents &ev)
{
    const int64_t rows_per_wg = k->kind == kKindWave ? kWaveRowsPerWg : 1;
    const int block = k->kind == kKindWave ? 64 * kWaveRowsPerWg : k->block;
    int64_t grid_cap = kMaxGridWgs;
    if (k->kind != kKindReread && wgs_per_cu >= 0) {
        int occ = 0;
        const credit_status_t st = occupancy(k, &occ);
        if (st != CREDIT_OK)
            return st;
        DeviceModel d;
        {
            std::lock_guard<std::mutex> lk(g_mu);
            d = device_model_locked();
        }
        const int per_cu = wgs_per_cu == 0 ? occ : std::min(occ, wgs_per_cu);
        grid_cap = std::max<int64_t>(1, static_cast<int64_t>(per_cu) * d.cus);
    }
    const int64_t chunk_rows = kMaxGridWgs * rows_per_wg;
    for (int64_t r0 = 0; r0 < a0.rows; r0 += chunk_rows) {
        const int64_t n = std::min(chunk_rows, a0.rows - r0);
        RowArgs a = rows_from(a0, k->op, k->dt, r0, n);
        const int64_t grid = std::min(grid_cap, (n + rows_per_wg - 1) / rows_per_wg);
        const credit_status_t st = launch_raw(k, static_cast<uint32_t>(grid), block, &a, s,
                                              r0 == 0 ? ev.start : nullptr,
                                              r0 + n >= a0.rows ? ev.stop : nullptr);
        if (st != CREDIT_OK)
            return st;
    }
    return CREDIT_OK;
}

// Workgroups of kernel `k` one CU holds at once; cached, failures too (a
// process without a usable device asks once).  Its own lock: the planner
// asks while g_mu is held.
credit_status_t occupancy(const KernelEntry *k, int *out)
{
    static std::mutex mu;
    static std::map<const void *, int> cache;  // 0: the query failed
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(k->fn);
        if (it != cache.end()) {
            *out = it->second;
            return it->second > 0 ? CREDIT_OK : CREDIT_ERR_HIP;
        }
    }
    int occ = 0;
    const int block = k->kind == kKindWave ? 64 * kWaveRowsPerWg : k->block;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k->fn, block, 0) != hipSuccess || occ < 1) {
        (void)hipGetLastError();
        occ = 0;
    }
    std::lock_guard<std::mutex> lk(mu);
    cache[k->fn] = occ;
    *out = occ;
    return occ > 0 ? CREDIT_OK : CREDIT_ERR_HIP;
}

// Split-row launches of kernel `k` for the rows of a0 on the scratch `ctl`
// (kScratchBytes): persistent clusters, as many as `allowed` workgroups hold
// and the exchange words cover, never more than there are rows; a launch
// takes at most kMaxSplitIters row iterations per cluster.
credit_status_t launch_split_on(const KernelEntry *k, const RowArgs &a0, int p, int q, int64_t allowed,
                                SplitCtl *ctl, hipStream_t s, const LaunchEvents &ev)
{
    const int64_t clusters =
        std::min({std::max<int64_t>(1, allowed / p), kSlotWords / (INT64_C(2) * p * q), a0.rows});
    const int64_t rows_per_launch = clusters * static_cast<int64_t>(kMaxSplitIters);
    const uint32_t spin = static_cast<uint32_t>(g_spin_limit.load());
    for (int64_t r0 = 0; r0 < a0.rows; r0 += rows_per_launch) {
        const int64_t n = std::min(rows_per_launch, a0.rows - r0);
        const int64_t c = std::min(clusters, n);
        SplitArgs sa;
        sa.r = rows_from(a0, k->op, k->dt, r0, n);
        sa.ctl = ctl;
        sa.p = p;
        sa.clusters = static_cast<int32_t>(c);
        sa.spin_limit = spin;
        const uint32_t grid = static_cast<uint32_t>(c * p);
        const credit_status_t st = launch_raw(k, grid, k->block, &sa, s, r0 == 0 ? ev.start : nullptr,
                                              r0 + n >= a0.rows ? ev.stop : nullptr);
        if (st != CREDIT_OK)
            return st;
    }
    return CREDIT_OK;
}

// `fixed`: a scratch to use instead of the stream's own (null: the stream's).
credit_status_t launch_split(const KernelEntry *k, const RowArgs &a0, int p, int q, int wgs_per_cu,
                             hipStream_t s, const LaunchEvents &ev, SplitCtl *fixed)
{
    int occ = 0;
    credit_status_t st = occupancy(k, &occ);
    if (st != CREDIT_OK)
        return st;
    std::lock_guard<std::mutex> lk(g_mu);
    const DeviceModel d = device_model_locked();
    const int64_t resident = static_cast<int64_t>(occ) * d.cus;
    // wgs_per_cu > 0 caps the clusters (never above what the device holds)
    const int64_t allowed = wgs_per_cu > 0 ? std::min<int64_t>(resident, int64_t(wgs_per_cu) * d.cus) : resident;
    if (resident < p)
        return CREDIT_ERR_NOT_CORESIDENT;
    SplitCtl *ctl = fixed;
    if (ctl == nullptr) {
        Scratch *sc = nullptr;
        st = get_scratch_locked(s, &sc);
        if (st != CREDIT_OK)
            return st;
        ctl = sc->ctl;
    }
    return launch_split_on(k, a0, p, q, allowed, ctl, s, ev);
}

// Does `plan`'s tile exist and hold the row (or slice)?
credit_status_t resolve_plan(int op, int dt, int64_t cols, const credit_plan_t &plan, const KernelEntry **out,
                             int *kind_out)
{
    if (plan.path < CREDIT_PATH_SINGLE_WG || plan.path > CREDIT_PATH_REREAD)
        return CREDIT_ERR_INVALID_ARG;
    // a partial row (byte length a multiple of 4, not of 16) of an operator
    // with parameters, and a row of the others that is not a multiple of 64
    // bytes, are held as 16-byte vectors (held_row_kind) and reread by element
    // the LDS tier holds rows of whole 16-byte vectors as they are
    if (plan.lds_items < 0)
        return CREDIT_ERR_INVALID_ARG;
    const int part = plan_row_kind(op, dt, cols, plan.path, plan.lds_items);
    const int vb = path_vec_bytes(op, dt, cols, plan.path);
    if (plan.vec_bytes != 0 && plan.vec_bytes != vb)
        return CREDIT_ERR_ILLEGAL_PATH;
    const int64_t nv = plan.lds_items > 0 ? lds_row_vectors(dt, cols)
                       : plan.path != CREDIT_PATH_REREAD ? held_vectors(op, dt, cols, plan.path)
                                                         : (cols * elem_bytes(dt) + vb - 1) / vb;
    int kind = 0;
    int64_t need = nv;
    switch (plan.path) {
    case CREDIT_PATH_SINGLE_WG:
        kind = plan.block_threads == 64 ? kKindWave : kKindWg;
        break;
    case CREDIT_PATH_SPLIT_ROW:
        kind = kKindSplit;
        if (plan.split_p != 2 && plan.split_p != 4 && plan.split_p != 8)
            return CREDIT_ERR_ILLEGAL_PATH;
        need = slice_vectors(nv, plan.split_p, vb);
        if (need * (plan.split_p - 1) >= nv)
            return CREDIT_ERR_ILLEGAL_PATH;
        break;
    case CREDIT_PATH_REREAD:
        kind = kKindReread;
        need = 0;
        break;
    default:
        return CREDIT_ERR_INVALID_ARG;
    }
    // the LDS tier: workgroup tiles of paths 1 and 2, rows of whole 16-byte vectors
    if (plan.lds_items > 0 && (kind == kKindWave || kind == kKindReread || nv == 0 || vb != 16))
        return CREDIT_ERR_ILLEGAL_PATH;
    const KernelEntry *k = find_kernel(kind, op, dt, vb, plan.block_threads, plan.items, part, plan.lds_items);
    if (k == nullptr)
        return CREDIT_ERR_UNSUPPORTED;
    if (need > static_cast<int64_t>(plan.block_threads) * (plan.items + plan.lds_items))
        return CREDIT_ERR_ILLEGAL_PATH;
    // a row or slice is one buffer descriptor: its byte length must fit 32 bits
    if (kind != kKindReread && need * vb > INT64_C(0xFFFFFFFF))
        return CREDIT_ERR_UNSUPPORTED;
    *out = k;
    *kind_out = kind;
    return CREDIT_OK;
}

void to_c_plan(const Plan &p, credit_plan_t *out)
{
    std::memset(out, 0, sizeof(*out));
    out->path = p.path;
    out->split_p = p.split_p;
    out->block_threads = p.tile.block;
    out->items = p.tile.items;
    out->vec_bytes = p.tile.vb;
    out->wgs_per_cu = p.wgs_per_cu;
    out->lds_items = p.tile.lds;
    for (int i = 0; i < 3; ++i)
        out->predicted_us[i] = p.est[i].legal ? p.est[i].us : -1.0;
}

credit_status_t run_plan_checked(int op, const credit_operands_t &t, int64_t rows, int64_t cols, float eps, int dt,
                                 const credit_plan_t &plan, hipStream_t s, bool control,
                                 const LaunchEvents &ev = LaunchEvents{}, SplitCtl *fixed = nullptr)
{
    const KernelEntry *k = nullptr;
    int kind = 0;
    credit_status_t st = resolve_plan(op, dt, cols, plan, &k, &kind);
    if (st != CREDIT_OK)
        return st;
    if (control) {
        if (kind != kKindSplit)
            return CREDIT_ERR_INVALID_ARG;
        if (k->lds != 0)
            return CREDIT_ERR_UNSUPPORTED;  // the control twins are register tiles
        k = find_kernel(kKindControl, op, dt, k->vb, k->block, k->items);
        if (k == nullptr)
            return CREDIT_ERR_UNSUPPORTED;
    }
    RowArgs a;
    a.x = t.x;
    a.dy = uses_dy(op) ? t.dy : nullptr;
    a.gamma = uses_gamma(op) ? t.gamma : nullptr;
    a.beta = uses_beta(op) ? t.beta : nullptr;
    a.y = t.y;
    // LayerNorm backward writes each row's mean and rstd when given row_out
    a.row_out = (uses_row_out(op) || op == CREDIT_OP_LAYERNORM_BACKWARD) ? t.row_out : nullptr;
    a.rows = rows;
    a.cols = cols;
    a.eps = eps;
    if (log_enabled())
        std::fprintf(stderr, "[credit] op=%d dt=%d rows=%lld cols=%lld path=%d p=%d block=%d items=%d lds=%d vb=%d%s%s\n",
                     op, dt, static_cast<long long>(rows), static_cast<long long>(cols), plan.path, plan.split_p,
                     plan.block_threads, plan.items, plan.lds_items, k->vb,
                     k->part == 1 ? " (partial last vector)" : (k->part == 2 ? " (shifted row)" : ""),
                     control ? " (control)" : "");
    if (kind == kKindSplit)
        return launch_split(k, a, plan.split_p, stats_per_partial(op), plan.wgs_per_cu, s, ev, fixed);
    return launch_rowwise(k, a, plan.wgs_per_cu, s, ev);
}

credit_status_t run_op(int op, const credit_operands_t &t, int64_t rows, int64_t cols, float eps, int dt, int path,
                       int split_p, void *stream)
{
    bool noop = false;
    credit_status_t st = validate(op, t, rows, cols, eps, dt, &noop);
    if (st != CREDIT_OK)
        return st;
    st = check_path_args(path, split_p);
    if (st != CREDIT_OK)
        return st;
    if (noop)
        return CREDIT_OK;
    Plan p;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        const Calibration cal = calibration_locked();
        PlanRequest req;
        req.op = op;
        req.dt = dt;
        req.rows = rows;
        req.cols = cols;
        const int fp = split_p <= 1 ? 0 : split_p;
        if (!make_plan(req, cal, path, fp, &p))
            return CREDIT_ERR_ILLEGAL_PATH;
    }
    credit_plan_t cp;
    to_c_plan(p, &cp);
    return run_plan_checked(op, t, rows, cols, eps, dt, cp, static_cast<hipStream_t>(stream), false);
}

credit_operands_t operands(const void *x, const void *dy, const void *gamma, const void *beta, void *y,
                           void *row_out)
{
    credit_operands_t t;
    t.x = x;
    t.dy = dy;
    t.gamma = gamma;
    t.beta = beta;
    t.y = y;
    t.row_out = row_out;
    return t;
}

}  // namespace

credit_status_t validate_operands(credit_op_t op, const credit_operands_t &ops, int64_t rows, int64_t cols,
                                  float eps, credit_dtype_t dt, bool *noop)
{
    return validate(op, ops, rows, cols, eps, dt, noop);
}

credit_status_t run_plan_on_scratch(credit_op_t op, const credit_operands_t &ops, int64_t rows, int64_t cols,
                                    float eps, credit_dtype_t dt, const credit_plan_t &plan, void *stream,
                                    SplitCtl *ctl)
{
    bool noop = false;
    const credit_status_t st = validate(op, ops, rows, cols, eps, dt, &noop);
    if (st != CREDIT_OK || noop)
        return st;
    return run_plan_checked(op, ops, rows, cols, eps, dt, plan, static_cast<hipStream_t>(stream), false,
                            LaunchEvents{}, ctl);
}

}  // namespace credit

namespace credit {
namespace {

credit_status_t load_calibration_file(const char *json_path, Calibration *out)
{
    std::ifstream f(json_path);
    if (!f)
        return CREDIT_ERR_NO_CALIBRATION;
    std::stringstream ss;
    ss << f.rdbuf();
    if (!parse_calibration(ss.str(), out))
        return CREDIT_ERR_NO_CALIBRATION;
    return CREDIT_OK;
}

}  // namespace
}  // namespace credit

using namespace credit;

extern "C" {

credit_status_t credit_softmax(const void *x, void *y, int64_t rows, int64_t cols, credit_dtype_t dt,
                               credit_path_t path, int32_t split_p, void *stream)
{
    return run_op(CREDIT_OP_SOFTMAX, operands(x, nullptr, nullptr, nullptr, y, nullptr), rows, cols, 0.0f, dt, path,
                  split_p, stream);
}

credit_status_t credit_layernorm(const void *x, const void *gamma, const void *beta, void *y, int64_t rows,
                                 int64_t cols, float eps, credit_dtype_t dt, credit_path_t path,
                                 int32_t split_p, void *stream)
{
    return run_op(CREDIT_OP_LAYERNORM, operands(x, nullptr, gamma, beta, y, nullptr), rows, cols, eps, dt, path,
                  split_p, stream);
}

credit_status_t credit_rmsnorm(const void *x, const void *gamma, void *y, int64_t rows, int64_t cols, float eps,
                               credit_dtype_t dt, credit_path_t path, int32_t split_p, void *stream)
{
    return run_op(CREDIT_OP_RMSNORM, operands(x, nullptr, gamma, nullptr, y, nullptr), rows, cols, eps, dt, path,
                  split_p, stream);
}

credit_status_t credit_softmax_backward(const void *x, const void *dy, void *dx, int64_t rows, int64_t cols,
                                        credit_dtype_t dt, credit_path_t path, int32_t split_p, void *stream)
{
    return run_op(CREDIT_OP_SOFTMAX_BACKWARD, operands(x, dy, nullptr, nullptr, dx, nullptr), rows, cols, 0.0f, dt,
                  path, split_p, stream);
}

credit_status_t credit_layernorm_backward(const void *x, const void *dy, const void *gamma, void *dx,
                                          int64_t rows, int64_t cols, float eps, credit_dtype_t dt,
                                          credit_path_t path, int32_t split_p, void *stream)
{
    return run_op(CREDIT_OP_LAYERNORM_BACKWARD, operands(x, dy, gamma, nullptr, dx, nullptr), rows, cols, eps, dt,
                  path, split_p, stream);
}

credit_status_t credit_layernorm_backward_stats(const void *x, const void *dy, const void *gamma, void *dx,
                                                float *row_stats, int64_t rows, int64_t cols, float eps,
                                                credit_dtype_t dt, credit_path_t path, int32_t split_p, void *stream)
{
    if (row_stats == nullptr && rows > 0)
        return CREDIT_ERR_INVALID_ARG;
    return run_op(CREDIT_OP_LAYERNORM_BACKWARD, operands(x, dy, gamma, nullptr, dx, row_stats), rows, cols, eps, dt,
                  path, split_p, stream);
}

credit_status_t credit_quantize_int8(const void *x, int8_t *q, float *scale, int64_t rows, int64_t cols,
                                     credit_dtype_t dt, credit_path_t path, int32_t split_p, void *stream)
{
    return run_op(CREDIT_OP_QUANTIZE_INT8, operands(x, nullptr, nullptr, nullptr, q, scale), rows, cols, 0.0f, dt,
                  path, split_p, stream);
}

credit_status_t credit_select_path(credit_op_t op, credit_dtype_t dt, int64_t rows, int64_t cols,
                                   credit_plan_t *out)
{
    if (out == nullptr || rows < 0 || cols < 1)
        return CREDIT_ERR_INVALID_ARG;
    credit_status_t st = check_op_dt(op, dt);
    if (st != CREDIT_OK)
        return st;
    std::lock_guard<std::mutex> lk(g_mu);
    const Calibration cal = calibration_locked();
    PlanRequest req;
    req.op = op;
    req.dt = dt;
    req.rows = rows;
    req.cols = cols;
    Plan p;
    if (!make_plan(req, cal, 0, 0, &p))
        return CREDIT_ERR_ILLEGAL_PATH;
    to_c_plan(p, out);
    return CREDIT_OK;
}

credit_status_t credit_make_plan(credit_op_t op, credit_dtype_t dt, int64_t rows, int64_t cols, credit_path_t path,
                                 int32_t split_p, credit_plan_t *out)
{
    if (out == nullptr || rows < 0 || cols < 1)
        return CREDIT_ERR_INVALID_ARG;
    credit_status_t st = check_op_dt(op, dt);
    if (st != CREDIT_OK)
        return st;
    st = check_path_args(path, split_p);
    if (st != CREDIT_OK)
        return st;
    std::lock_guard<std::mutex> lk(g_mu);
    const Calibration cal = calibration_locked();
    PlanRequest req;
    req.op = op;
    req.dt = dt;
    req.rows = rows;
    req.cols = cols;
    Plan p;
    if (!make_plan(req, cal, path, split_p <= 1 ? 0 : split_p, &p))
        return CREDIT_ERR_ILLEGAL_PATH;
    to_c_plan(p, out);
    return CREDIT_OK;
}

credit_status_t credit_model_terms(credit_op_t op, credit_dtype_t dt, int64_t rows, int64_t cols, int32_t split_p,
                                   credit_model_terms_t *out)
{
    if (out == nullptr || rows < 1 || cols < 1 || (split_p != 2 && split_p != 4 && split_p != 8))
        return CREDIT_ERR_INVALID_ARG;
    const credit_status_t st = check_op_dt(op, dt);
    if (st != CREDIT_OK)
        return st;
    std::lock_guard<std::mutex> lk(g_mu);
    const Calibration cal = calibration_locked();
    PlanRequest req;
    req.op = op;
    req.dt = dt;
    req.rows = rows;
    req.cols = cols;
    TileSpec t;
    if (!split_tile(op, dt, cols, split_p, &t))
        return CREDIT_ERR_ILLEGAL_PATH;
    int base_path = 0;
    TileSpec base_tile;
    double base_us = 0.0;
    if (!analytic_baseline(req, cal, &base_path, &base_tile, &base_us))
        return CREDIT_ERR_ILLEGAL_PATH;
    const SplitTerms r = split_terms(req, cal, split_p, t, base_path, base_tile, base_us);
    std::memset(out, 0, sizeof(*out));
    out->baseline_path = base_path;
    out->split_block = t.block;
    out->split_items = t.items;
    out->split_resident = static_cast<int32_t>(r.resident);
    out->t_base_us = r.t_base_us;
    out->b_base = r.b_base;
    out->b_reread = r.b_reread;
    out->t_save_us = r.t_save_us;
    out->t_occ_us = r.t_occ_us;
    out->waves = r.waves;
    out->t_ctrl_us = r.t_ctrl_us;
    out->t_dsm_us = r.t_dsm_us;
    out->delta_us = r.delta_us;
    out->t_split_us = r.t_split_us;
    return CREDIT_OK;
}

credit_status_t credit_enumerate_plans(credit_op_t op, credit_dtype_t dt, int64_t rows, int64_t cols,
                                       credit_plan_t *out, int32_t capacity, int32_t *count)
{
    if (count == nullptr || capacity < 0 || (out == nullptr && capacity > 0) || rows < 0 || cols < 1)
        return CREDIT_ERR_INVALID_ARG;
    const credit_status_t st = check_op_dt(op, dt);
    if (st != CREDIT_OK)
        return st;
    std::vector<Candidate> cands;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        const Calibration cal = calibration_locked();
        PlanRequest req;
        req.op = op;
        req.dt = dt;
        req.rows = rows;
        req.cols = cols;
        enumerate_candidates(req, cal, &cands);
    }
    *count = static_cast<int32_t>(cands.size());
    for (int32_t i = 0; i < capacity && i < *count; ++i) {
        credit_plan_t &c = out[i];
        std::memset(&c, 0, sizeof(c));
        c.path = cands[i].path;
        c.split_p = cands[i].split_p;
        c.block_threads = cands[i].est.tile.block;
        c.items = cands[i].est.tile.items;
        c.vec_bytes = cands[i].est.tile.vb;
        c.wgs_per_cu = cands[i].wgs_per_cu;
        c.lds_items = cands[i].est.tile.lds;
        for (int j = 0; j < 3; ++j)
            c.predicted_us[j] = j == cands[i].path - 1 ? cands[i].est.us : -1.0;
    }
    return CREDIT_OK;
}

credit_status_t credit_occupancy(credit_op_t op, credit_dtype_t dt, int64_t cols, const credit_plan_t *plan,
                                 int32_t *wgs_per_cu)
{
    if (plan == nullptr || wgs_per_cu == nullptr || cols < 1)
        return CREDIT_ERR_INVALID_ARG;
    credit_status_t st = check_op_dt(op, dt);
    if (st != CREDIT_OK)
        return st;
    const KernelEntry *k = nullptr;
    int kind = 0;
    st = resolve_plan(op, dt, cols, *plan, &k, &kind);
    if (st != CREDIT_OK)
        return st;
    int occ = 0;
    st = occupancy(k, &occ);
    if (st != CREDIT_OK)
        return st;
    *wgs_per_cu = occ;
    return CREDIT_OK;
}

credit_status_t credit_run_plan(credit_op_t op, const credit_operands_t *ops, int64_t rows, int64_t cols,
                                float eps, credit_dtype_t dt, const credit_plan_t *plan, void *stream)
{
    if (plan == nullptr || ops == nullptr)
        return CREDIT_ERR_INVALID_ARG;
    bool noop = false;
    credit_status_t st = validate(op, *ops, rows, cols, eps, dt, &noop);
    if (st != CREDIT_OK || noop)
        return st;
    return run_plan_checked(op, *ops, rows, cols, eps, dt, *plan, static_cast<hipStream_t>(stream), false);
}

credit_status_t credit_run_plan_timed(credit_op_t op, const credit_operands_t *ops, int64_t rows, int64_t cols,
                                      float eps, credit_dtype_t dt, const credit_plan_t *plan, void *start_event,
                                      void *stop_event, void *stream)
{
    if (plan == nullptr || ops == nullptr || start_event == nullptr || stop_event == nullptr)
        return CREDIT_ERR_INVALID_ARG;
    bool noop = false;
    credit_status_t st = validate(op, *ops, rows, cols, eps, dt, &noop);
    if (st != CREDIT_OK)
        return st;
    if (noop)
        return CREDIT_ERR_INVALID_ARG;  // nothing would be launched, so nothing could be timed
    LaunchEvents ev;
    ev.start = static_cast<hipEvent_t>(start_event);
    ev.stop = static_cast<hipEvent_t>(stop_event);
    return run_plan_checked(op, *ops, rows, cols, eps, dt, *plan, static_cast<hipStream_t>(stream), false, ev);
}

credit_status_t credit_control(credit_op_t op, int64_t rows, int64_t cols, credit_dtype_t dt,
                               const credit_plan_t *plan, void *start_event, void *stop_event, void *stream)
{
    if (plan == nullptr || rows < 0 || cols < 1)
        return CREDIT_ERR_INVALID_ARG;
    const credit_status_t st = check_op_dt(op, dt);
    if (st != CREDIT_OK)
        return st;
    if (plan->path != CREDIT_PATH_SPLIT_ROW)
        return CREDIT_ERR_INVALID_ARG;
    if (rows == 0)
        return CREDIT_OK;
    LaunchEvents ev;
    ev.start = static_cast<hipEvent_t>(start_event);
    ev.stop = static_cast<hipEvent_t>(stop_event);
    return run_plan_checked(op, operands(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), rows, cols, 0.0f, dt,
                            *plan, static_cast<hipStream_t>(stream), true, ev);
}

credit_status_t credit_copy(const void *src, void *dst, int64_t bytes, void *start_event, void *stop_event,
                            void *stream)
{
    if (src == nullptr || dst == nullptr || bytes < 0 || bytes % 16 != 0)
        return CREDIT_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(dst))
        return CREDIT_ERR_ALIGNMENT;
    if (bytes == 0)
        return CREDIT_OK;
    const KernelEntry *k = find_misc(-1);
    int64_t n16 = bytes / 16;
    const int64_t grid = std::min<int64_t>((n16 + 255) / 256, INT64_C(1) << 22);
    struct {
        const void *s;
        void *d;
        int64_t n;
    } a{src, dst, n16};
    void *args[] = {&a.s, &a.d, &a.n};
    if (hipExtLaunchKernel(k->fn, dim3(static_cast<uint32_t>(grid)), dim3(256), args, 0,
                           static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                           static_cast<hipEvent_t>(stop_event), 0) != hipSuccess) {
        (void)hipGetLastError();
        return CREDIT_ERR_HIP;
    }
    return CREDIT_OK;
}

credit_status_t credit_flush(void *buf, int64_t bytes, void *stream)
{
    if (buf == nullptr || bytes < 0 || bytes % 16 != 0)
        return CREDIT_ERR_INVALID_ARG;
    if (!aligned16(buf))
        return CREDIT_ERR_ALIGNMENT;
    if (bytes == 0)
        return CREDIT_OK;
    const KernelEntry *k = find_misc(-2);
    int64_t n16 = bytes / 16;
    const int64_t grid = std::min<int64_t>((n16 + 255) / 256, INT64_C(1) << 20);
    void *b = buf;
    void *args[] = {&b, &n16};
    if (hipLaunchKernel(k->fn, dim3(static_cast<uint32_t>(grid)), dim3(256), args, 0,
                        static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return CREDIT_ERR_HIP;
    }
    return CREDIT_OK;
}

credit_status_t credit_load_calibration(const char *json_path)
{
    if (json_path == nullptr) {
        std::lock_guard<std::mutex> lk(g_mu);
        g_cal = Calibration{};
        return CREDIT_OK;
    }
    Calibration c;
    const credit_status_t st = load_calibration_file(json_path, &c);
    if (st != CREDIT_OK)
        return st;
    std::lock_guard<std::mutex> lk(g_mu);
    g_cal = c;
    return CREDIT_OK;
}

credit_status_t credit_check_errors(void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess) {
        (void)hipGetLastError();
        return CREDIT_ERR_HIP;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return CREDIT_ERR_HIP;
    SplitCtl *ctls[2] = {nullptr, static_scratch_if_set_up()};
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_scratch.find(std::make_pair(dev, s));
        if (it != g_scratch.end())
            ctls[0] = it->second.ctl;
    }
    bool timed_out = false;
    for (SplitCtl *ctl : ctls) {
        if (ctl == nullptr)
            continue;
        uint32_t err = 0;
        if (hipMemcpy(&err, &ctl->error, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) {
            (void)hipGetLastError();
            return CREDIT_ERR_HIP;
        }
        if (err != 0) {
            const uint32_t zero = 0;
            if (hipMemcpy(&ctl->error, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) {
                (void)hipGetLastError();
                return CREDIT_ERR_HIP;
            }
            timed_out = true;
        }
    }
    return timed_out ? CREDIT_ERR_DEVICE_TIMEOUT : CREDIT_OK;
}

credit_status_t credit_test_exchange(int64_t spin_limit)
{
    if (spin_limit > INT64_C(0xFFFFFFFF))
        return CREDIT_ERR_INVALID_ARG;
    g_spin_limit.store(spin_limit < 0 ? kDefaultSpinLimit : spin_limit);
    return CREDIT_OK;
}

credit_status_t credit_test_scratch(int64_t tags_used, int32_t unmatched_tags, void *stream)
{
    if (tags_used >= static_cast<int64_t>(kTagResetAt))
        return CREDIT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    SplitCtl *ctl = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        Scratch *sc = nullptr;
        const credit_status_t st = get_scratch_locked(s, &sc);
        if (st != CREDIT_OK)
            return st;
        ctl = sc->ctl;
    }
    const uint32_t used = static_cast<uint32_t>(tags_used);
    const uint32_t unmatched = unmatched_tags != 0 ? kTagResetAt : 0u;
    if (hipStreamSynchronize(s) != hipSuccess ||
        (tags_used >= 0 && hipMemcpy(&ctl->tags_used, &used, sizeof(used), hipMemcpyHostToDevice) != hipSuccess) ||
        hipMemcpy(&ctl->unmatched, &unmatched, sizeof(unmatched), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipGetLastError();
        return CREDIT_ERR_HIP;
    }
    return CREDIT_OK;
}

const char *credit_status_str(credit_status_t status)
{
    switch (status) {
    case CREDIT_OK:
        return "ok";
    case CREDIT_ERR_INVALID_ARG:
        return "invalid argument";
    case CREDIT_ERR_UNSUPPORTED:
        return "unsupported shape or option";
    case CREDIT_ERR_ALIGNMENT:
        return "pointer not 16-byte aligned";
    case CREDIT_ERR_ILLEGAL_PATH:
        return "path or split cannot hold the row";
    case CREDIT_ERR_NOT_CORESIDENT:
        return "split workgroups cannot be co-resident";
    case CREDIT_ERR_NO_CALIBRATION:
        return "calibration missing or malformed";
    case CREDIT_ERR_HIP:
        return "HIP runtime error";
    case CREDIT_ERR_DEVICE_TIMEOUT:
        return "split-row exchange wait timed out";
    }
    return "unknown status";
}

int32_t credit_version(void) { return 100; }

}  // extern "C"
