// gfx950 kernels for the row-wise reduction-reuse operators.
//
//   path 1  single_wave_kernel / single_wg_kernel: one wavefront or one
//           workgroup owns a row, reads it from HBM once into VGPRs, reduces it
//           (DPP inside a wave, LDS across waves) and writes the output from the
//           registers.  This is the "local staging when the row fits in one
//           CTA" case of the CREDIT paper (Sec. IV-A), held in VGPRs.
//   path 2  split_kernel: P workgroups own disjoint slices of a row (Sec. III-B,
//           Eq. 2), each keeps its slice in VGPRs, and the P partials are
//           exchanged through a small global scratch (the replicated all-gather
//           of Sec. III-C, Eq. 5, with global words in place of peer shared
//           memory).  Every workgroup combines all P partials itself, in the
//           order c = 0..P-1.
//   path 3  reread_kernel: the conventional schedule of Fig. 2(a): one
//           workgroup streams its row to reduce it, then streams it again to
//           write the output.
//
// Co-residency of the P workgroups of a split row: workgroups take a ticket
// from a device counter when they start, and ticket t owns slice t mod P of row
// t / P.  Tickets are handed out in start order, so every complete group of P
// tickets belongs to workgroups that are running or finished; only the newest
// group can be incomplete, and its missing members are the next workgroups to
// start.  As long as the device can hold P workgroups at once, every waiting
// workgroup's peers are resident or will be dispatched, so no launch-wide
// guarantee (cooperative launch) is needed.
//
// Exchange words are 64-bit {value bits, epoch}; a reader polls each word until
// it carries the current launch's epoch, so no fence is needed between the data
// and its flag.  The last workgroup to finish resets the ticket counter and
// advances the epoch, which makes the scratch reusable by the next launch on the
// same stream (and by replays of a captured graph) with no host-side clearing.
#pragma once

#include "args.hpp"
#include "common.hpp"
#include "ops.hpp"

namespace credit {


template <class Partial>
__device__ __forceinline__ float comp(const Partial &p, int j)
{
    return j == 0 ? p.a : (j == 1 ? p.b : p.c);
}
template <class Partial>
__device__ __forceinline__ void set_comp(Partial &p, int j, float v)
{
    if (j == 0)
        p.a = v;
    else if (j == 1)
        p.b = v;
    else
        p.c = v;
}

// Number of k in [0, IT) with pos + k*G < n (a prefix).
template <int IT, int G>
__device__ __forceinline__ int count_valid(int64_t n, int pos)
{
    if (n <= pos)
        return 0;
    const int64_t c = (n - pos + G - 1) / G;
    return c < IT ? static_cast<int>(c) : IT;
}

template <class T, int VB, int IT, int G>
__device__ __forceinline__ void load_tile(Tile<T, VB, IT> &t, const char *row_base, int64_t first,
                                          int pos, int kvalid)
{
#pragma unroll
    for (int k = 0; k < IT; ++k)
        if (k < kvalid)
            t.v[k] = load_vec<VB>(row_base + (first + pos + static_cast<int64_t>(k) * G) * VB);
}

// Apply h to the held tile and write it out.  Parameter vectors are indexed by
// column, i.e. by the same vector index as x within the row.
template <OpKind OP, class T, int VB, int IT, int G, bool STREAM>
__device__ __forceinline__ void store_vec_out(const RawVec<VB> &in, char *yrow, const char *grow,
                                              const char *brow, int64_t vidx, const Coef &c)
{
    using Op = OpTraits<OP>;
    constexpr int E = VB / StorageTraits<T>::kBytes;
    float out[E];
    RawVec<VB> g, b;
    if constexpr (Op::kParams >= 1)
        g = load_vec_cached<VB>(grow + vidx * VB);
    if constexpr (Op::kParams >= 2)
        b = load_vec_cached<VB>(brow + vidx * VB);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float gv = Op::kParams >= 1 ? elem<T, VB>(g, e) : 1.0f;
        const float bv = Op::kParams >= 2 ? elem<T, VB>(b, e) : 0.0f;
        if constexpr (STREAM)
            out[e] = Op::template apply_stream<T>(elem<T, VB>(in, e), c, gv, bv);
        else
            out[e] = Op::template apply<T>(elem<T, VB>(in, e), c, gv, bv);
    }
    store_vec<VB>(yrow + vidx * VB, pack<T, VB, E>(out));
}

template <OpKind OP, class T, int VB, int IT, int G>
__device__ __forceinline__ void store_tile(Tile<T, VB, IT> &t, char *yrow, const char *grow,
                                           const char *brow, int64_t first, int pos, int kvalid,
                                           const Coef &c)
{
    fence_tile(t);
#pragma unroll
    for (int k = 0; k < IT; ++k)
        if (k < kvalid)
            store_vec_out<OP, T, VB, IT, G, false>(t.v[k], yrow, grow, brow,
                                                   first + pos + static_cast<int64_t>(k) * G, c);
}

// Combine the wave partials of a workgroup through LDS; every thread returns
// the same workgroup partial (fixed order w = 0..NW-1).
template <OpKind OP, int NW>
__device__ __forceinline__ Partial block_combine(const Partial &wp, Partial *sh)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (lane == 0)
        sh[wave] = wp;
    __syncthreads();
    Partial loc[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i)
        loc[i] = sh[i];
    return OpTraits<OP>::template merge<NW>(loc, NW);
}

// ---------------------------------------------------------------------------
// Path 1a: one wavefront per row, four rows per 256-thread workgroup.  No LDS
// and no barrier: the wave reduction is the row reduction.
// ---------------------------------------------------------------------------
template <OpKind OP, class T, int VB, int IT>
__global__ __launch_bounds__(kWave *kWaveRowsPerWg) void single_wave_kernel(RowArgs a)
{
    using Op = OpTraits<OP>;
    constexpr int E = VB / StorageTraits<T>::kBytes;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaveRowsPerWg + threadIdx.x / kWave;
    if (row >= a.rows)
        return;  // wave-uniform
    const int64_t nv = a.cols / E;
    const int64_t row_off = row * nv * VB;
    const char *xrow = static_cast<const char *>(a.x) + row_off;
    char *yrow = static_cast<char *>(a.y) + row_off;
    Tile<T, VB, IT> t;
    const int kv = count_valid<IT, kWave>(nv, lane);
    load_tile<T, VB, IT, kWave>(t, xrow, 0, lane, kv);
    const Partial wp = Op::template wave_partial<T, VB, IT>(t, kv);
    const Coef c = Op::template finalize<T>(wp, wp, a.cols, a.eps);
    store_tile<OP, T, VB, IT, kWave>(t, yrow, static_cast<const char *>(a.gamma),
                                     static_cast<const char *>(a.beta), 0, lane, kv, c);
}

// ---------------------------------------------------------------------------
// Path 1b: one workgroup of BLOCK threads per row.
// ---------------------------------------------------------------------------
template <OpKind OP, class T, int VB, int BLOCK, int IT>
__global__ __launch_bounds__(BLOCK) void single_wg_kernel(RowArgs a)
{
    using Op = OpTraits<OP>;
    constexpr int E = VB / StorageTraits<T>::kBytes;
    constexpr int NW = BLOCK / kWave;
    __shared__ Partial sh[NW];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t nv = a.cols / E;
    const int64_t row_off = row * nv * VB;
    const char *xrow = static_cast<const char *>(a.x) + row_off;
    char *yrow = static_cast<char *>(a.y) + row_off;
    Tile<T, VB, IT> t;
    const int kv = count_valid<IT, BLOCK>(nv, tid);
    load_tile<T, VB, IT, BLOCK>(t, xrow, 0, tid, kv);
    const Partial wp = Op::template wave_partial<T, VB, IT>(t, kv);
    const Partial rp = block_combine<OP, NW>(wp, sh);
    const Coef c = Op::template finalize<T>(rp, wp, a.cols, a.eps);
    store_tile<OP, T, VB, IT, BLOCK>(t, yrow, static_cast<const char *>(a.gamma),
                                     static_cast<const char *>(a.beta), 0, tid, kv, c);
}

// ---------------------------------------------------------------------------
// Path 2: P workgroups per row (see the header comment).  CONTROL = true is the
// work-free control kernel: identical launch shape, tickets, exchange and
// reductions, but no row loads and no output stores.
// ---------------------------------------------------------------------------
template <OpKind OP, class T, int VB, int BLOCK, int IT, bool CONTROL>
__global__ __launch_bounds__(BLOCK) void split_kernel(SplitArgs a)
{
    using Op = OpTraits<OP>;
    constexpr int E = VB / StorageTraits<T>::kBytes;
    constexpr int NW = BLOCK / kWave;
    constexpr int Q = Op::kQ;
    __shared__ Partial sh[NW];
    __shared__ Partial peer[kMaxSplit];
    __shared__ uint32_t sh_ticket, sh_epoch;
    const int tid = threadIdx.x;
    if (tid == 0) {
        sh_ticket = fetch_add_u32_agent(&a.ctl->ticket, 1u);
        sh_epoch = load_u32_agent(&a.ctl->epoch);
    }
    __syncthreads();
    // the counter starts each launch at 0; the modulo keeps indices inside this
    // launch's rows and slots even if it did not (tickets stay a permutation)
    const uint32_t ticket = sh_ticket % gridDim.x;
    const uint32_t epoch = sh_epoch;
    const int P = a.p;
    const int64_t rl = ticket / static_cast<uint32_t>(P);
    const int c = static_cast<int>(ticket % static_cast<uint32_t>(P));
    const int64_t row = a.row0 + rl;

    const int64_t nv = a.r.cols / E;
    const int64_t per = (nv + P - 1) / P;
    const int64_t v0 = min(nv, per * c);
    const int64_t v1 = min(nv, v0 + per);
    const int64_t row_off = row * nv * VB;
    const char *xrow = static_cast<const char *>(a.r.x) + row_off;
    char *yrow = static_cast<char *>(a.r.y) + row_off;

    Tile<T, VB, IT> t;
    const int kv = count_valid<IT, BLOCK>(v1 - v0, tid);
    if constexpr (CONTROL) {
#pragma unroll
        for (int k = 0; k < IT; ++k)
#pragma unroll
            for (int w = 0; w < RawVec<VB>::kWords; ++w)
                set_word<VB>(t.v[k], w, 0u);
    } else {
        load_tile<T, VB, IT, BLOCK>(t, xrow, v0, tid, kv);
    }
    const Partial wp = Op::template wave_partial<T, VB, IT>(t, kv);
    const Partial sp = block_combine<OP, NW>(wp, sh);

    // publish this slice's partial, then gather all P partials of the row
    uint64_t *row_slots = a.slots + rl * P * Q;
    if (tid < Q)
        store_u64_agent(row_slots + c * Q + tid,
                        (static_cast<uint64_t>(epoch) << 32) | __float_as_uint(comp(sp, tid)));
    if (tid < P * Q) {
        uint64_t w = load_u64_agent(row_slots + tid);
        uint32_t polls = 0;
        while (static_cast<uint32_t>(w >> 32) != epoch) {
            if (++polls > a.spin_limit) {
                fetch_or_u32_agent(&a.ctl->error, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
            w = load_u64_agent(row_slots + tid);
        }
        set_comp(peer[tid / Q], tid % Q, __uint_as_float(static_cast<uint32_t>(w)));
    }
    __syncthreads();
    if (tid == 0) {
        // every workgroup has taken its ticket and read the epoch before it
        // counts itself done, so the last one can recycle both
        const uint32_t d = fetch_add_u32_agent(&a.ctl->done, 1u);
        if (d == gridDim.x - 1) {
            store_u32_agent(&a.ctl->ticket, 0u);
            store_u32_agent(&a.ctl->done, 0u);
            store_u32_agent(&a.ctl->epoch, epoch + 1u == 0u ? 1u : epoch + 1u);
        }
    }
    Partial parts[kMaxSplit];
#pragma unroll
    for (int i = 0; i < kMaxSplit; ++i)
        parts[i] = peer[i];
    const Partial rp = Op::template merge<kMaxSplit>(parts, P);
    const Coef cf = Op::template finalize<T>(rp, wp, a.r.cols, a.r.eps);
    if constexpr (!CONTROL)
        store_tile<OP, T, VB, IT, BLOCK>(t, yrow, static_cast<const char *>(a.r.gamma),
                                         static_cast<const char *>(a.r.beta), v0, tid, kv, cf);
}

// ---------------------------------------------------------------------------
// Path 3: the reread baseline.  Pass 1 streams the row with ordinary cached
// loads (so a reread that can hit L2 or the Infinity Cache does), keeping a
// running partial per thread; pass 2 streams it again and writes the output.
// ---------------------------------------------------------------------------
template <OpKind OP, class T, int VB, int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void reread_kernel(RowArgs a)
{
    using Op = OpTraits<OP>;
    constexpr int E = VB / StorageTraits<T>::kBytes;
    constexpr int NW = BLOCK / kWave;
    constexpr int64_t CH = static_cast<int64_t>(BLOCK) * U;
    __shared__ Partial sh[NW];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t nv = a.cols / E;
    const int64_t row_off = row * nv * VB;
    const char *xrow = static_cast<const char *>(a.x) + row_off;
    char *yrow = static_cast<char *>(a.y) + row_off;

    Partial r = Op::stream_init();
    for (int64_t base = 0; base < nv; base += CH) {
        RawVec<VB> v[U];
        const int kv = count_valid<U, BLOCK>(nv - base, tid);
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kv)
                v[k] = load_vec_cached<VB>(xrow + (base + tid + static_cast<int64_t>(k) * BLOCK) * VB);
        Op::template stream_update<T, VB, U>(r, v, kv);
    }
    const Partial wp = Op::wave_from_thread(r);
    const Partial rp = block_combine<OP, NW>(wp, sh);
    const Coef c = Op::template finalize_stream<T>(rp, a.cols, a.eps);
    for (int64_t base = 0; base < nv; base += CH) {
        RawVec<VB> v[U];
        const int kv = count_valid<U, BLOCK>(nv - base, tid);
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kv)
                v[k] = load_vec<VB>(xrow + (base + tid + static_cast<int64_t>(k) * BLOCK) * VB);
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kv)
                store_vec_out<OP, T, VB, U, BLOCK, true>(v[k], yrow, static_cast<const char *>(a.gamma),
                                                         static_cast<const char *>(a.beta),
                                                         base + tid + static_cast<int64_t>(k) * BLOCK, c);
    }
}

}  // namespace credit
