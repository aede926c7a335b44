/*
 * credit.h -- C ABI of libcredit.so: row-wise reduction-reuse operators
 * (softmax, LayerNorm, RMSNorm; softmax-logits backward, LayerNorm backward,
 * int8 quantization) for AMD Instinct MI355X (gfx950).
 *
 * The operators are the "wide reduction-reuse" workload class of the CREDIT
 * paper ("CREDIT: Cost-guided Reduction-reuse with Efficient DSMEM Inter-CTA
 * Tiling", Sec. I and Sec. III-B, Eq. 1): each row of width N is reduced to a
 * few statistics and every element is then reused to write a full-size output.
 * The library reads each row from HBM once whenever the row, or a 1/P slice of
 * it, fits on chip.
 *
 * Problem statement (Sec. III-B): M rows ("rows"), N elements per row ("cols"),
 * a statistic set per operator, and, for the split-row path, P workgroups per
 * row ("split_p", P in {2, 4, 8}; Sec. IV-A sweeps the same set).
 *
 * Conventions shared by every entry point:
 *   - x, dy, gamma, beta, y (dx, q) and scale are caller-owned DEVICE pointers;
 *     the library never frees or retains them.  Layout is dense row-major
 *     [rows][cols]; gamma and beta are [cols]; scale is [rows].  Every pointer
 *     must be 16-byte aligned, except scale (4-byte).  gamma, beta, dy and a
 *     floating-point output have the same dtype as x.  In-place operation
 *     (output == x, or dx == dy) is allowed; any other overlap is undefined.
 *     Shifted bf16 rows of odd length (see credit_plan_t.vec_bytes) are read
 *     in whole 4-byte words: when rows * cols is odd, the 2 bytes after the
 *     last element of x (and dy) are read, never written, and never affect
 *     the result (they lie in the same aligned 4-byte word as that element).
 *   - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t;
 *     NULL means the default stream).  A successful return means the work was
 *     enqueued; device faults surface at the caller's next synchronization.
 *   - Argument errors return a status before anything is enqueued, and y is
 *     left untouched.  rows == 0 is a successful no-op.
 *   - The library owns only a small exchange scratch per (device, stream) for
 *     the split-row path, allocated on first use of that path on that stream.
 *     Two streams never share a scratch; calls on one stream are ordered by
 *     the stream.  The state of the split-row protocol (ticket counter, tags)
 *     lives in that scratch and is advanced by the kernels themselves, so a
 *     split-row launch may be captured into a graph and replayed any number
 *     of times, provided the stream's scratch already exists when the capture
 *     starts (a first split-row call on a stream under capture returns
 *     CREDIT_ERR_UNSUPPORTED before enqueueing anything) and replays do not
 *     overlap other split-row work that uses the same scratch (e.g. by
 *     replaying on the capture stream).
 *   - If a split-row workgroup's wait for its peers' partials gives up (see
 *     credit_check_errors), that row's output is NaN (for the int8 quantizer:
 *     its scale is NaN), never a result from stale statistics.
 *
 * Arithmetic: fp32 inputs compute in fp32; bf16 inputs are widened exactly to
 * fp32, computed in fp32 and rounded to nearest-even bf16 on output (the int8
 * quantizer's codes are integers decided in fp32).
 */
#ifndef CREDIT_H
#define CREDIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CREDIT_OK = 0,
    CREDIT_ERR_INVALID_ARG = 1,    /* null pointer, cols < 1, rows < 0, bad enum, eps < 0 or not finite */
    CREDIT_ERR_UNSUPPORTED = 2,    /* shape or option this build has no kernel for */
    CREDIT_ERR_ALIGNMENT = 3,      /* a pointer is not 16-byte aligned */
    CREDIT_ERR_ILLEGAL_PATH = 4,   /* a forced path / split_p / plan cannot hold the row */
    CREDIT_ERR_NOT_CORESIDENT = 5, /* the device cannot hold split_p workgroups of this kernel at once */
    CREDIT_ERR_NO_CALIBRATION = 6, /* calibration file missing or malformed */
    CREDIT_ERR_HIP = 7,            /* a HIP runtime call failed */
    CREDIT_ERR_DEVICE_TIMEOUT = 8  /* a split-row spin-wait gave up (reported by credit_check_errors) */
} credit_status_t;

typedef enum { CREDIT_F32 = 0, CREDIT_BF16 = 1 } credit_dtype_t;

typedef enum {
    CREDIT_OP_SOFTMAX = 0,
    CREDIT_OP_LAYERNORM = 1,
    CREDIT_OP_RMSNORM = 2,
    CREDIT_OP_SOFTMAX_BACKWARD = 3,   /* softmax-logits backward */
    CREDIT_OP_LAYERNORM_BACKWARD = 4, /* LayerNorm backward, row part */
    CREDIT_OP_QUANTIZE_INT8 = 5       /* row-wise symmetric int8 quantization */
} credit_op_t;

/*
 * Operands of one operator call, for the explicit-plan entry points.  Each
 * operator reads the fields it needs and requires them non-NULL:
 *   softmax              x, y
 *   LayerNorm            x, gamma, beta, y
 *   RMSNorm              x, gamma, y
 *   softmax backward     x (logits), dy, y (= dx)
 *   LayerNorm backward   x, dy, gamma, y (= dx)
 *   int8 quantization    x, y (= int8 codes q), row_out (= fp32 scale per row)
 * Fields an operator does not use are ignored.
 */
typedef struct {
    const void *x;
    const void *dy;
    const void *gamma;
    const void *beta;
    void *y;
    void *row_out;
} credit_operands_t;

typedef enum {
    CREDIT_PATH_AUTO = 0,      /* the selector decides (credit_select_path) */
    CREDIT_PATH_SINGLE_WG = 1, /* path 1: one wavefront or workgroup per row, row held on chip */
    CREDIT_PATH_SPLIT_ROW = 2, /* path 2: split_p workgroups per row, slices held on chip */
    CREDIT_PATH_REREAD = 3     /* path 3: reduce pass + output pass, the row is read twice */
} credit_path_t;

/* A launch plan.  predicted_us[i] is the selector's estimate for path i+1
 * (at its best split_p for path 2); a negative value means illegal. */
typedef struct {
    int32_t path;          /* credit_path_t, never AUTO in a returned plan */
    int32_t split_p;       /* workgroups per row: 1 for paths 1 and 3 */
    int32_t block_threads; /* threads per row owner: 64 = one wavefront per row */
    int32_t items;         /* vectors per thread held (paths 1, 2) or streamed per step (path 3) */
    int32_t vec_bytes;     /* bytes per global access (0 in a plan passed in = the row's own): 16 for
                              rows of whole 16-byte vectors; for other rows one element on path 3,
                              and on paths 1 and 2 16 where the operator holds such rows as
                              16-byte vectors: from the 64-byte line at or below each row's start
                              (softmax, softmax backward, the quantizer, RMSNorm, odd-length bf16
                              LayerNorm rows, and on path 1 LayerNorm backward's fp32 rows of whole
                              16-byte vectors and bf16 rows that are not; the neighbouring rows'
                              elements masked, the words shared with them written byte-exactly),
                              or from the row's first byte with a partial last vector (LayerNorm's
                              and fp32 LayerNorm backward's other rows whose byte length is a
                              multiple of 4); one element otherwise */
    int32_t wgs_per_cu;    /* paths 1, 2: 0 = as many workgroups as the device holds at once, each
                              owner looping over rows (and loading the next row while writing the
                              current one); k > 0 = at most k per CU; path 1 only: -1 = one
                              workgroup per row (four rows for block_threads 64), no looping */
    int32_t lds_items;     /* paths 1 and 2, workgroup tiles of rows of whole 16-byte vectors: vectors
                              per thread held in LDS beside the `items` in registers (the LDS tier; the
                              row or slice is then at most block_threads * (items + lds_items) vectors);
                              0 = registers only */
    double predicted_us[3];
} credit_plan_t;

/*
 * Row-wise softmax over the last dimension (the two-stage reduction-reuse form
 * of Sec. III-B, Eq. 1: max, then sum of exp(x - max); output
 * exp(x_i - max) / sum).
 *   x, y     : [rows][cols] of dtype `dt`.
 *   path     : CREDIT_PATH_AUTO or a forced path.
 *   split_p  : 0 = library chooses; else 2, 4 or 8 (path 2 only; must be 0 or 1 otherwise).
 */
credit_status_t credit_softmax(const void *x, void *y, int64_t rows, int64_t cols, credit_dtype_t dt,
                               credit_path_t path, int32_t split_p, void *stream);

/*
 * Row-wise LayerNorm (Ba et al., cited by the paper for its LayerNorm
 * workload, Sec. IV-A): y = (x - mean) / sqrt(var + eps) * gamma + beta with the
 * biased (1/N) variance.  eps must be finite and >= 0.
 */
credit_status_t credit_layernorm(const void *x, const void *gamma, const void *beta, void *y, int64_t rows,
                                 int64_t cols, float eps, credit_dtype_t dt, credit_path_t path,
                                 int32_t split_p, void *stream);

/*
 * Row-wise RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma.  eps finite, >= 0.
 */
credit_status_t credit_rmsnorm(const void *x, const void *gamma, void *y, int64_t rows, int64_t cols,
                               float eps, credit_dtype_t dt, credit_path_t path, int32_t split_p,
                               void *stream);

/*
 * Softmax-logits backward, one of the reduction-reuse workloads of the
 * paper's evaluation (Sec. IV-A; its traffic in Sec. IV-D): the gradient of
 * row-wise softmax with respect to its logits x given the gradient dy of the
 * softmax output, with the probabilities recomputed from x:
 *   p = softmax(x),  dx_i = p_i (dy_i - sum_j dy_j p_j).
 * Reads x and dy once, writes dx once.
 *   x, dy, dx : [rows][cols] of dtype `dt` (fp32 or bf16).
 */
credit_status_t credit_softmax_backward(const void *x, const void *dy, void *dx, int64_t rows, int64_t cols,
                                        credit_dtype_t dt, credit_path_t path, int32_t split_p, void *stream);

/*
 * LayerNorm backward, row part (the LayerNorm workload of Sec. IV-A, in its
 * backward form): the gradient with respect to x of the LayerNorm above,
 * given dy, with mean and variance recomputed from x.  With
 * rstd = 1/sqrt(var + eps), xhat = (x - mean) rstd and g = gamma dy:
 *   dx_i = rstd (g_i - mean_j g_j - xhat_i mean_j (g_j xhat_j)).
 * The gradients of gamma and beta are the parameter part
 * (credit_layernorm_backward_params).
 *   x, dy, dx : [rows][cols]; gamma : [cols]; fp32 or bf16 (bf16 rows are held
 *   as loaded and gamma * dy is formed in fp32 at each use, never rounded to
 *   bf16).  eps finite, >= 0.
 * Through credit_run_plan, a non-NULL row_out (8-byte aligned) receives the
 * rows' statistics as credit_layernorm_backward_stats writes them.
 */
credit_status_t credit_layernorm_backward(const void *x, const void *dy, const void *gamma, void *dx,
                                          int64_t rows, int64_t cols, float eps, credit_dtype_t dt,
                                          credit_path_t path, int32_t split_p, void *stream);

/*
 * credit_layernorm_backward that also writes each row's statistics for the
 * parameter part: row_stats[2 i] = mean of row i, row_stats[2 i + 1] =
 * 1 / sqrt(var_i + eps), in fp32, as the row kernel computed them (8 bytes
 * per row: no other traffic).  row_stats : [rows][2] fp32, 8-byte aligned,
 * caller-owned; NULL (with rows > 0) is CREDIT_ERR_INVALID_ARG.
 */
credit_status_t credit_layernorm_backward_stats(const void *x, const void *dy, const void *gamma, void *dx,
                                                float *row_stats, int64_t rows, int64_t cols, float eps,
                                                credit_dtype_t dt, credit_path_t path, int32_t split_p,
                                                void *stream);

/*
 * LayerNorm backward, parameter part (the rest of the LayerNorm workload of
 * Sec. IV-A): with xhat_ij = (x_ij - mean_i) rstd_i from row_stats,
 *   dgamma_j = sum_i dy_ij xhat_ij,   dbeta_j = sum_i dy_ij.
 * Two kernels on `stream`: workgroups sum groups of rows of a block of
 * columns into `workspace`, then one thread per column adds the groups in
 * order (fp32 throughout; the same result on every run).  Reads x and dy
 * once (the row part has read them already: its registers hold the rows,
 * with no room for per-column sums).
 *   x, dy : [rows][cols] of dtype `dt` (fp32 or bf16; 16-byte aligned when a
 *     row is a whole number of 16-byte vectors, else element-aligned);
 *   row_stats : [rows][2] fp32 (credit_layernorm_backward_stats);
 *   dgamma, dbeta : [cols] fp32, caller-owned, 4-byte aligned;
 *   workspace : at least credit_layernorm_backward_params_workspace bytes of
 *     device memory, 16-byte aligned, caller-owned.
 * For rows = 0 the gradients are set to zero and x, dy, row_stats and
 * workspace may be NULL.
 * Errors: CREDIT_ERR_INVALID_ARG (NULL pointers, bad shape or dtype, too small
 * a workspace), CREDIT_ERR_ALIGNMENT, CREDIT_ERR_HIP.
 */
credit_status_t credit_layernorm_backward_params(const void *x, const void *dy, const float *row_stats,
                                                 float *dgamma, float *dbeta, int64_t rows, int64_t cols,
                                                 credit_dtype_t dt, void *workspace, size_t workspace_bytes,
                                                 void *stream);

/* Bytes of workspace credit_layernorm_backward_params needs for a shape. */
credit_status_t credit_layernorm_backward_params_workspace(int64_t rows, int64_t cols, credit_dtype_t dt,
                                                           size_t *bytes);

/*
 * Row-wise symmetric int8 quantization (the quantization workload of
 * Sec. IV-A; 9 -> 5 bytes per element in Sec. IV-D), in fp32 arithmetic:
 *   a = max_i |x_i|;  inv = min(127 / a, FLT_MAX) (0 when a = 0);
 *   q_i = clamp(round_half_even(x_i * inv), -127, 127);  scale = a / 127,
 * each division and product correctly rounded, so the codes are fully
 * determined by x.  Inputs must be finite (non-finite values give
 * unspecified codes).
 *   x : [rows][cols] of dtype `dt` (fp32 or bf16); q : [rows][cols] int8;
 *   scale : [rows] fp32 (4-byte aligned).
 */
credit_status_t credit_quantize_int8(const void *x, int8_t *q, float *scale, int64_t rows, int64_t cols,
                                     credit_dtype_t dt, credit_path_t path, int32_t split_p, void *stream);

/*
 * The selector (Sec. III-D, Eq. 3 and 7-9, adapted): legality of each path
 * from the on-chip capacity of the compiled kernels, then the predicted time of
 * each legal candidate; writes the fastest into *out.  Host-only: it queries
 * device properties once per device unless a calibration with a device
 * description is loaded.  Returns CREDIT_ERR_INVALID_ARG for a null `out` or
 * bad shape, CREDIT_ERR_UNSUPPORTED for an (op, dtype) pair with no kernels
 * (every operator has both dtypes in this build).
 */
credit_status_t credit_select_path(credit_op_t op, credit_dtype_t dt, int64_t rows, int64_t cols,
                                   credit_plan_t *out);

/*
 * The terms of the selector's analytic cost model (Sec. III-D) for splitting
 * the rows of a shape over split_p workgroups (2, 4 or 8), priced against the
 * non-split baseline: path 1 when one owner holds the row, else path 3.
 * Evaluated with the model constants of the calibration in force (its table
 * of measured plans is not used).  Times in microseconds.
 */
typedef struct {
    int32_t baseline_path;  /* 1 or 3 */
    int32_t split_block;    /* the split tile the terms are for: threads, */
    int32_t split_items;    /* and vectors per thread */
    int32_t split_resident; /* S: split workgroups the device holds at once */
    double t_base_us;       /* T_B: the baseline's predicted time */
    double b_base;          /* bytes per element the baseline moves (Eq. 4) */
    double b_reread;        /* of which its reread: the row inputs' bytes on path 3, else 0 */
    double t_save_us;       /* Eq. 7: (b_reread / b_base) * t_base_us */
    double t_occ_us;        /* the time a baseline that leaves CUs idle gives back:
                               (t_base_us - t_save_us) * (1 - u_base / u_split), u = the
                               fraction of the CUs given work */
    double waves;           /* Eq. 8: W = ceil(rows / floor(S / split_p)), S = split
                               workgroups the device holds at once */
    double t_ctrl_us;       /* W exchanges plus the split launch's control cost */
    double t_dsm_us;        /* s * W * (split_p - 1) * q / B_w: exchange words, not
                               multiplied by split_p */
    double delta_us;        /* Eq. 9: t_save + t_occ - t_ctrl - t_dsm (T_replay = T_deposit = 0:
                               slices are held in registers) */
    double t_split_us;      /* t_base_us - delta_us */
} credit_model_terms_t;

/*
 * Fill *out with the model terms above.  CREDIT_ERR_ILLEGAL_PATH if no split
 * tile holds a 1/split_p slice of the row, CREDIT_ERR_INVALID_ARG for a null
 * out, split_p outside {2, 4, 8} or a bad shape, CREDIT_ERR_UNSUPPORTED for an
 * (op, dtype) without kernels.  Host-only.
 */
credit_status_t credit_model_terms(credit_op_t op, credit_dtype_t dt, int64_t rows, int64_t cols, int32_t split_p,
                                   credit_model_terms_t *out);

/*
 * The plan the operator entry points use for `path` and `split_p` (the same
 * arguments and rules as credit_softmax & co.; CREDIT_PATH_AUTO with
 * split_p = 0 equals credit_select_path).  Returns CREDIT_ERR_ILLEGAL_PATH if
 * the forced path or split cannot hold the row, CREDIT_ERR_INVALID_ARG for bad
 * arguments.  Host-only, like credit_select_path.
 */
credit_status_t credit_make_plan(credit_op_t op, credit_dtype_t dt, int64_t rows, int64_t cols,
                                 credit_path_t path, int32_t split_p, credit_plan_t *out);

/*
 * Every worthwhile legal plan for a shape: each path 1 tile that holds the
 * row, each path 3 tile, and each (P, tile) of path 2 whose slice fits, in
 * that order; a held tile is listed when at least half of it is used or when
 * it is the smallest tile that holds the row (or slice).  Each plan carries
 * the model's estimate in predicted_us[path - 1] (the other two entries are
 * -1).  Writes min(capacity, *count) plans to `out` and the total number
 * to *count (call with capacity 0 to size the array).  For exhaustive timing,
 * the final search among legal candidates that the selector's screen narrows.
 * Host-only.
 */
credit_status_t credit_enumerate_plans(credit_op_t op, credit_dtype_t dt, int64_t rows, int64_t cols,
                                       credit_plan_t *out, int32_t capacity, int32_t *count);

/*
 * Workgroups of the kernel that `plan` selects for rows of `cols` elements
 * that one CU holds at once (from the compiled kernel's registers and LDS, via
 * the HIP occupancy calculator); the wave-per-row kernel's workgroups hold
 * four rows each.  Queries the current device.  Errors as credit_run_plan
 * (CREDIT_ERR_ILLEGAL_PATH, CREDIT_ERR_UNSUPPORTED), CREDIT_ERR_HIP if the
 * query fails.
 */
credit_status_t credit_occupancy(credit_op_t op, credit_dtype_t dt, int64_t cols, const credit_plan_t *plan,
                                 int32_t *wgs_per_cu);

/*
 * Run one operator with an explicit plan (as returned by credit_select_path,
 * or hand-built for exhaustive timing) on the operands `ops` (see
 * credit_operands_t for which fields each operator needs).  eps is used by
 * the normalizations and ignored otherwise.  Returns CREDIT_ERR_ILLEGAL_PATH
 * if the plan's tile cannot hold the row or slice, CREDIT_ERR_UNSUPPORTED if
 * no kernel with that tile exists, and the argument errors of the operator's
 * own entry point.
 */
credit_status_t credit_run_plan(credit_op_t op, const credit_operands_t *ops, int64_t rows, int64_t cols,
                                float eps, credit_dtype_t dt, const credit_plan_t *plan, void *stream);

/*
 * credit_run_plan with timing: start_event receives the begin timestamp of the
 * first kernel the plan launches and stop_event the end timestamp of the last
 * (both are hipEvent_t created by the caller; the timestamps come from the
 * kernel dispatches, so hipEventElapsedTime(start, stop) is device execution
 * time without queueing or launch latency).  Both events are required;
 * rows == 0 returns CREDIT_ERR_INVALID_ARG because nothing would be timed.
 * Otherwise identical to credit_run_plan.
 */
credit_status_t credit_run_plan_timed(credit_op_t op, const credit_operands_t *ops, int64_t rows, int64_t cols,
                                      float eps, credit_dtype_t dt, const credit_plan_t *plan, void *start_event,
                                      void *stop_event, void *stream);

/*
 * credit_run_plan for callers that cannot allocate device memory: code under
 * stream (graph) capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, validation, errors and results as
 * credit_run_plan; it allocates no device memory.  The split-row exchange
 * uses the library's static scratch, one array of 1 MiB + 640 bytes per GPU
 * (a control block and 2^17 exchange words), reserved when the library is
 * loaded and held until the process ends; its address on a device is looked
 * up on the first call there.  No shape needs more than that: a launch's
 * clusters are capped to the words, and further rows loop.  Nothing in it
 * needs clearing between calls: the kernels keep the control block consistent
 * from one launch to the next (a first call may be captured, and a captured
 * call replays correctly).  Paths 1 and 3 use no scratch at all.  Every call
 * on one GPU shares that scratch, so calls whose split-row launches overlap
 * on one GPU (from two streams without synchronization between them, or
 * concurrent with their own graph replays) race and must not be made; calls
 * on one stream are ordered by it.  credit_check_errors on any stream of the
 * device also reads (and clears) the static scratch's error word.
 */
credit_status_t credit_run_plan_static(credit_op_t op, const credit_operands_t *ops, int64_t rows, int64_t cols,
                                       float eps, credit_dtype_t dt, const credit_plan_t *plan, void *stream);

/*
 * Work-free control kernel (Sec. III-D, the control that isolates launch,
 * scheduling, occupancy and synchronization costs): the split-row kernel of
 * `plan` with the same grid, tickets and exchange but no row loads or output
 * stores.  plan->path must be CREDIT_PATH_SPLIT_ROW.  start_event and
 * stop_event (hipEvent_t, each may be NULL) receive the dispatch timestamps
 * as in credit_run_plan_timed.  Its time at M rows minus its time at one row
 * per cluster is the control overhead T_ctrl of Sec. III-D, Eq. 8.
 */
credit_status_t credit_control(credit_op_t op, int64_t rows, int64_t cols, credit_dtype_t dt,
                               const credit_plan_t *plan, void *start_event, void *stop_event, void *stream);

/*
 * Measurement helpers.  credit_copy: 128-bit streaming copy of `bytes` bytes
 * (a multiple of 16), the achievable read+write ceiling; start_event and
 * stop_event (hipEvent_t, each may be NULL) receive the copy kernel's begin and
 * end timestamps.  credit_flush: a read-modify-write pass over `bytes` bytes of
 * `buf` to evict L2 and the Infinity Cache between timed runs.  Both are
 * asynchronous on `stream`.
 */
credit_status_t credit_copy(const void *src, void *dst, int64_t bytes, void *start_event, void *stop_event,
                            void *stream);
credit_status_t credit_flush(void *buf, int64_t bytes, void *stream);

/*
 * Load selector calibration from a JSON file written by the calibration
 * script (wide_reduction_reuse_amd/calibrate.py): device constants for the
 * analytic model and a table of measured candidates, each a plan for one
 * (op, dtype, cols) with its median kernel time at several row counts.  A shape
 * whose (op, dtype, cols) the table measured is planned from it (each
 * candidate's time interpolated piecewise linearly in log rows / log time,
 * the fastest chosen).  At another width each legal plan is priced from the
 * same plan's measurements at the nearest measured widths below and above
 * (read at the row count that moves the same bytes, interpolated in log
 * width); only where the table measured none of the legal plans does the
 * analytic model decide.  NULL clears it (back to the analytic model alone).  Returns CREDIT_ERR_NO_CALIBRATION if the
 * file is missing or malformed, in which case the previous calibration stays
 * in force.  If the environment variable CREDIT_CALIB names a file, it is
 * loaded before the first plan unless a calibration was loaded explicitly.
 */
credit_status_t credit_load_calibration(const char *json_path);

/*
 * Synchronize `stream` and read (then clear) the device error word of that
 * stream's split-row scratch, and of the current device's static scratch if
 * credit_run_plan_static has used it: CREDIT_ERR_DEVICE_TIMEOUT if a
 * spin-wait gave up since the last check (the rows concerned were written as
 * NaN), CREDIT_ERR_HIP if synchronization failed, else CREDIT_OK.
 */
credit_status_t credit_check_errors(void *stream);

/*
 * Test hooks for the failure handling of the split-row exchange; normal use
 * needs neither.
 *
 * credit_test_exchange: for split-row launches enqueued after the call (in any
 * thread), a workgroup polls a peer's exchange word at most `spin_limit`
 * times before it gives up (spin_limit < 0 restores the default, 2^20; 0
 * gives up after the first poll).  Host-only; CREDIT_ERR_INVALID_ARG for a
 * spin_limit above 2^32 - 1.
 *
 * credit_test_scratch: after synchronizing `stream`, set two fields of the
 * control block of its split-row scratch (allocating the scratch if needed):
 * the count of exchange tags issued (0 <= tags_used < 2^31; a test can make
 * the next launches cross the point, 2^31, where the kernels clear the
 * exchange words and restart the tags; tags_used < 0 leaves the count as it
 * is), and, with unmatched_tags != 0, make every
 * reader wait for a tag no workgroup writes (while fewer than 2^30 tags have
 * been issued), so that every wait gives up: every kernel still runs to its
 * end, the rows come out NaN (a quantizer's scales NaN) and
 * credit_check_errors reports CREDIT_ERR_DEVICE_TIMEOUT.  unmatched_tags = 0
 * restores normal exchanges.  CREDIT_ERR_INVALID_ARG for tags_used >= 2^31,
 * CREDIT_ERR_HIP if a HIP call fails.
 */
credit_status_t credit_test_exchange(int64_t spin_limit);
credit_status_t credit_test_scratch(int64_t tags_used, int32_t unmatched_tags, void *stream);

/* Static, human-readable name of a status code. */
const char *credit_status_str(credit_status_t status);

/* Library version, as MAJOR * 10000 + MINOR * 100 + PATCH. */
int32_t credit_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CREDIT_H */
