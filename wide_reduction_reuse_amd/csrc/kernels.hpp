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
// Memory access: every row (or slice, or streamed chunk) is one buffer
// descriptor sized to its length.  Each wave of an owner holds one contiguous
// run of 64 * IT vectors: wave w's lane l holds vectors w*64*IT + l + 64k,
// k < IT (a streaming probe on MI355X favoured contiguous runs per wave over
// vectors strided by the workgroup width; in these kernels the two layouts
// measured within a few percent either way).  The IT loads issue back to
// back with no branch, and the ones past the end return zero and are excluded
// from the reduction by the valid count `kv`, while the matching stores are
// dropped by the range check.
//
// Split-row launches are persistent: the grid is C clusters of P workgroups,
// no larger than the device holds at once, and cluster k handles rows k, k+C,
// k+2C, ...  A workgroup takes a ticket from a device counter when it starts
// and ticket t is slice t mod P of cluster t / P.  Tickets are handed out in
// start order, so every complete group of P tickets belongs to workgroups that
// are running or finished; only the newest group can be incomplete, and its
// missing members are the next workgroups to start.  As long as the device can
// hold P workgroups at once, every waiting workgroup's peers are resident or
// will be dispatched, so no launch-wide co-residency guarantee is needed.
//
// Exchange words are 64-bit {value bits, tag}.  A cluster's words are double
// buffered by the parity of the row iteration, and iteration i of a launch
// writes tag tags_used + 1 + i, where tags_used is read from the control block
// (SplitCtl) at the start; a reader polls a word until it carries the tag it
// expects, so no fence is needed between the data and its flag.  A peer can
// only overwrite a buffer two iterations later, after every member has passed
// the exchange of the iteration in between, i.e. after every member has read
// this buffer.  The last workgroup of a launch to finish (counted on
// ctl->done) resets the ticket counter and advances tags_used past every tag
// the launch used, so the next launch on the scratch starts from a consistent
// state whether it was enqueued by the host or replayed from a graph; it reads
// that state only after this launch has ended (launches on one stream run in
// order).
#pragma once

#include <type_traits>

#include "args.hpp"
#include "common.hpp"
#include "ops.hpp"

namespace credit {

// Component j < Q of a partial, j a run-time index, as one explicit if/else
// chain on j.  (Written as a loop of conditional moves, or as a recursive
// template, the split kernel's exchange compiled to up to 19 more VGPRs.)
template <int Q>
__device__ __forceinline__ float comp(const Part<Q> &p, int j)
{
    static_assert(Q >= 1 && Q <= 5, "partials hold 1 to 5 scalars");
    if constexpr (Q <= 3)
        return j == 0 ? p.v[0] : (j == 1 ? p.v[1 % Q] : p.v[2 % Q]);
    else
        return j == 0 ? p.v[0] : (j == 1 ? p.v[1] : (j == 2 ? p.v[2] : (j == 3 ? p.v[3] : p.v[4 % Q])));
}
template <int Q>
__device__ __forceinline__ void set_comp(Part<Q> &p, int j, float v)
{
    static_assert(Q >= 1 && Q <= 5, "partials hold 1 to 5 scalars");
    if (j == 0)
        p.v[0] = v;
    else if (j == 1)
        p.v[1 % Q] = v;
    else if (Q <= 3 || j == 2)
        p.v[2 % Q] = v;
    else if (j == 3)
        p.v[3 % Q] = v;
    else
        p.v[4 % Q] = v;
}

// Output storage type and bytes per output vector for input vectors of VB bytes.
template <OpKind OP, class T>
using OutT = typename OpTraits<OP>::template Out<T>;
template <OpKind OP, class T, int VB>
constexpr int out_vb()
{
    return VB / StorageTraits<T>::kBytes * StorageTraits<OutT<OP, T>>::kBytes;
}

// Parameter vectors the output function reads on a held row (none when the
// parameters were folded into the tile before the reduction).
template <OpKind OP>
constexpr int out_params()
{
    return OpTraits<OP>::kParamsInReduce ? 0 : OpTraits<OP>::kParams;
}

// Held tiles that keep their inputs as loaded and use the operator's
// streaming form (stream_update on the held vectors, apply_stream with the
// parameters fetched at use) instead of folding the parameters into the tile:
// bf16 LayerNorm backward, whose dy tile cannot hold g = gamma * dy in fp32
// (rounding g to bf16 would lose what the fp32 path keeps).
template <OpKind OP, class T>
constexpr bool holds_raw()
{
    return OP == kLayerNormBwd && StorageTraits<T>::kBytes != 4;
}

// Parameter vectors a held tile's output pass applies.
template <OpKind OP, class T>
constexpr int held_out_params()
{
    return holds_raw<OP, T>() ? OpTraits<OP>::kParams : out_params<OP>();
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

// The row inputs of one owner: x, and dy for the backward operators; all of
// them cover the same columns.
template <int NI>
struct Srcs {
    rsrc_t r[NI];
};

// Scheduling-barrier mask that lets every instruction class cross except
// vector-memory reads: ALU 0x1, VALU 0x2, SALU 0x4, MFMA 0x8, VMEM write 0x40,
// DS 0x80, DS read 0x100, DS write 0x200, transcendental 0x400.
constexpr int kLoadOrderBarrier = 0x7CF;

// One-input tiles are loaded in the order the reduction consumes them
// (vector k = 0, 1, ...): with one in-order counter for all of a wave's memory
// operations, a vector issued early can be waited for while later ones are
// still in flight.  The scheduling barriers keep the compiler from reordering
// the loads (it otherwise issued them in nearly reverse order).  Two-input
// tiles (x, dy) are left to the compiler, input by input: pinning their order
// (either interleaved by vector or input by input) measured 1-3% slower on
// MI355X for softmax and LayerNorm backward.
template <class T, int VB, int IT, int G, int NI>
__device__ __forceinline__ void load_tile(Tile<T, VB, IT> (&t)[NI], const Srcs<NI> &src, int pos)
{
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            t[i].v[k] = buf_load<VB, kStream>(src.r[i], static_cast<uint32_t>(pos + k * G) * VB);
            if constexpr (NI == 1)
                __builtin_amdgcn_sched_barrier(kLoadOrderBarrier);
        }
}

// h for one vector: in[i] are the held (or reread) input vectors, g and b the
// parameter vectors of the same columns.
template <OpKind OP, class T, int VB, bool STREAM>
__device__ __forceinline__ RawVec<out_vb<OP, T, VB>()> apply_vec(const RawVec<VB> (&in)[OpTraits<OP>::kIn],
                                                                 const RawVec<VB> &g, const RawVec<VB> &b,
                                                                 const Coef &c)
{
    using Op = OpTraits<OP>;
    constexpr int E = VB / StorageTraits<T>::kBytes;
    constexpr int NP = STREAM ? Op::kParams : out_params<OP>();
    float out[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float gv = NP >= 1 ? elem<T, VB>(g, e) : 1.0f;
        const float bv = NP >= 2 ? elem<T, VB>(b, e) : 0.0f;
        float xin[Op::kIn];
#pragma unroll
        for (int i = 0; i < Op::kIn; ++i)
            xin[i] = elem<T, VB>(in[i], e);
        if constexpr (STREAM)
            out[e] = Op::template apply_stream<T>(xin, c, gv, bv);
        else
            out[e] = Op::template apply<T>(xin, c, gv, bv);
    }
    return pack<OutT<OP, T>, out_vb<OP, T, VB>(), E>(out);
}

// Parameter vectors fetched per group of the output loop when they are
// re-read for every row: four while the held tile is small; when it already
// takes 64 VGPRs, two (one pair for LayerNorm's two parameters).
template <int IT, int VB, int NP>
constexpr int param_group()
{
    return IT * VB / 4 >= 64 ? (NP >= 2 ? 1 : (IT < 2 ? IT : 2)) : (IT < 4 ? IT : 4);
}


// ---------------------------------------------------------------------------
// Parameter vectors (gamma, beta) of the columns a thread holds.  They are the
// same for every row, so a persistent owner fetches them once:
//   kParamNone   the operator has none (softmax);
//   kParamReg    held in VGPRs next to the tile, when both fit in 64 VGPRs;
//   kParamLds    staged in LDS once per workgroup, when that takes <= 64 KiB;
//   kParamDirect re-read from L2 for every row, a few vectors ahead of use.
// With the first three the output loop also loads the next row (below): its
// parameter reads do not queue behind HBM loads.  kParamDirect cannot do that
// (vector-memory loads complete in issue order, so a parameter load issued
// after the next row's loads would wait for them) and loads the next row
// after the output loop instead.
// ---------------------------------------------------------------------------
enum ParamMode { kParamNone = 0, kParamReg = 1, kParamLds = 2, kParamDirect = 3 };

// Which mode a kernel uses.  G: threads that together hold one row's (or
// slice's) columns.  Measured on MI355X: a workgroup-per-row kernel runs one
// row per workgroup, where an LDS or register copy only lowers occupancy, so
// it re-reads (kOwnerRow); the four waves of a wave-per-row workgroup share
// one LDS copy (kOwnerWaves); a split-row workgroup keeps its slice's columns
// for every row of its cluster (kOwnerSlice).
enum OwnerKind { kOwnerRow = 0, kOwnerWaves = 1, kOwnerSlice = 2 };

template <OpKind OP, int VB, int IT, int G, int OWNER>
constexpr int param_mode()
{
    constexpr int np = OpTraits<OP>::kParams;
    constexpr int ni = OpTraits<OP>::kIn;
    // tile + parameter VGPRs allowed: 64, but 32 for two parameter vectors or
    // two inputs at 1024 threads, whose 128-VGPR cap leaves less room beside
    // the statistics
    constexpr int reg_budget = (G >= 1024 && (np >= 2 || ni >= 2)) ? 32 : 64;
    if (np == 0)
        return kParamNone;
    if (OWNER == kOwnerRow)
        return kParamDirect;
    if (OWNER == kOwnerSlice && (np + ni) * IT * VB / 4 <= reg_budget)
        return kParamReg;
    if (np * G * IT * VB <= 64 * 1024)
        return kParamLds;
    return kParamDirect;
}

template <OpKind OP, int VB, int IT, int G, int OWNER>
constexpr int param_lds_vectors()
{
    return param_mode<OP, VB, IT, G, OWNER>() == kParamLds ? OpTraits<OP>::kParams * G * IT : 1;
}

// W: threads that together hold the columns (they share one LDS copy of
// W * IT vectors per parameter).  A thread's vector k is vector pos + 64 k of
// the row or slice (pos includes its wave's run offset).
//
// SH: the row is held shifted (SHIFT kernels), so held vector v covers
// columns v * E - s of a row that begins s elements into its held span, s
// changing from row to row: the parameters are re-read for every row from
// descriptors over the whole parameter arrays, at byte offset v * VB - s * b,
// each vector assembled from the two aligned vectors it straddles
// (load_shifted): where they are used (kParamDirect), or, for a raw tile that
// uses them in both of its passes, once per row into registers (kShiftReg,
// in shift()).
template <OpKind OP, class T, int VB, int IT, int W, int OWNER, bool SH = false>
struct ParamCache {
    // SH with a raw tile (which applies the parameters in both of its passes)
    // and room for them: realigned once per row into registers
    static constexpr bool kShiftReg = SH && holds_raw<OP, T>() && OpTraits<OP>::kParams == 1 && IT <= 8;
    static constexpr int kMode = SH && OpTraits<OP>::kParams > 0 ? (kShiftReg ? kParamReg : kParamDirect)
                                                                 : param_mode<OP, VB, IT, W, OWNER>();
    static constexpr int kNp = OpTraits<OP>::kParams;
    static constexpr int kRegs = kMode == kParamReg ? IT : 1;
    rsrc_t gam, bet;         // kParamDirect
    RawVec<VB> g[kRegs], b[kRegs];  // kParamReg
    const RawVec<VB> *lds;   // kParamLds: [kNp][W * IT], indexed by vector
    int32_t adj = 0;         // SH: byte offset of the slice's first held vector in the parameter arrays
    int pos0 = 0;            // kShiftReg: the thread's first held vector

    // SH: the row's shift (s elements of the previous row in front, held
    // vectors from v0 on); adj may be negative (the first vectors of a row
    // that starts mid-line cover columns before 0, which are never used).
    __device__ __forceinline__ void shift(int s, int64_t v0)
    {
        adj = static_cast<int32_t>(v0 * VB) - s * static_cast<int32_t>(StorageTraits<T>::kBytes);
        if constexpr (kShiftReg) {
            const int rb = __builtin_amdgcn_readfirstlane(adj) & 15;
#pragma unroll
            for (int k = 0; k < IT; ++k)
                g[k] = load_shifted(gam, static_cast<int32_t>((pos0 + k * kWave) * VB) + adj, rb);
        }
    }

    // SH: the parameter vector at byte offset o (o = held offset + adj) of
    // descriptor r: the aligned vectors A (at o rounded down to 16) and B (the
    // next), and the 16 bytes from o.  Offsets below 0 wrap past the end of
    // the descriptor and load zeros.
    __device__ __forceinline__ static RawVec<VB> load_shifted(rsrc_t r, int32_t o, int rb)
    {
        static_assert(VB == 16, "shifted parameter vectors: 16 bytes");
        const int32_t q = o & ~15;
        const RawVec<16> A = buf_load<16, kKeep>(r, static_cast<uint32_t>(q));
        if (rb == 0)
            return A;
        const RawVec<16> B = buf_load<16, kKeep>(r, static_cast<uint32_t>(q + 16));
        const uint32_t c[8] = {A.w[0], A.w[1], A.w[2], A.w[3], B.w[0], B.w[1], B.w[2], B.w[3]};
        const uint32_t sh = static_cast<uint32_t>(rb & 3) * 8u;
        RawVec<16> out;
        switch (rb >> 2) {
#define CREDIT_FUNNEL(W0)                                                                               \
    case W0:                                                                                            \
        out.w = u32x4{static_cast<uint32_t>((((uint64_t)c[W0 + 1] << 32) | c[W0]) >> sh),               \
                      static_cast<uint32_t>((((uint64_t)c[W0 + 2] << 32) | c[W0 + 1]) >> sh),           \
                      static_cast<uint32_t>((((uint64_t)c[W0 + 3] << 32) | c[W0 + 2]) >> sh),           \
                      static_cast<uint32_t>((((uint64_t)c[W0 + 4] << 32) | c[W0 + 3]) >> sh)};          \
        break;
            CREDIT_FUNNEL(0)
            CREDIT_FUNNEL(1)
            CREDIT_FUNNEL(2)
        default:
            out.w = u32x4{static_cast<uint32_t>((((uint64_t)c[4] << 32) | c[3]) >> sh),
                          static_cast<uint32_t>((((uint64_t)c[5] << 32) | c[4]) >> sh),
                          static_cast<uint32_t>((((uint64_t)c[6] << 32) | c[5]) >> sh),
                          static_cast<uint32_t>((((uint64_t)c[7] << 32) | c[6]) >> sh)};
            break;
#undef CREDIT_FUNNEL
        }
        return out;
    }

    // kParamDirect: the parameter vectors at held byte offset `off` of the slice.
    __device__ __forceinline__ void direct(uint32_t off, RawVec<VB> &gk, RawVec<VB> &bk) const
    {
        if constexpr (SH) {
            // off is a multiple of 16, so o's offset in its 16-byte vector is
            // adj's, the same in every lane
            const int32_t o = static_cast<int32_t>(off) + adj;
            const int rb = __builtin_amdgcn_readfirstlane(adj) & 15;
            if constexpr (kNp >= 1)
                gk = load_shifted(gam, o, rb);
            if constexpr (kNp >= 2)
                bk = load_shifted(bet, o, rb);
        } else {
            if constexpr (kNp >= 1)
                gk = buf_load<VB, kKeep>(gam, off);
            if constexpr (kNp >= 2)
                bk = buf_load<VB, kKeep>(bet, off);
        }
    }

    // Call once per owner, before the row loop.  `nthreads` threads with ids
    // `tid` fill the LDS copy (kParamLds); the caller puts a barrier between
    // this and the first get().
    __device__ __forceinline__ void init(rsrc_t gam_, rsrc_t bet_, int pos, RawVec<VB> *lds_buf, int tid,
                                         int nthreads)
    {
        gam = gam_;
        bet = bet_;
        lds = lds_buf;
        pos0 = pos;
        if constexpr (kMode == kParamReg && !kShiftReg) {
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                const uint32_t off = static_cast<uint32_t>(pos + k * kWave) * VB;
                g[k] = buf_load<VB, kKeep>(gam, off);
                if constexpr (kNp >= 2)
                    b[k] = buf_load<VB, kKeep>(bet, off);
            }
        } else if constexpr (kMode == kParamLds) {
            for (int i = tid; i < W * IT; i += nthreads) {
                lds_buf[i] = buf_load<VB, kKeep>(gam, static_cast<uint32_t>(i) * VB);
                if constexpr (kNp >= 2)
                    lds_buf[W * IT + i] = buf_load<VB, kKeep>(bet, static_cast<uint32_t>(i) * VB);
            }
        }
    }

    __device__ __forceinline__ void get(int k, int pos, RawVec<VB> &gk, RawVec<VB> &bk) const
    {
        if constexpr (kMode == kParamReg) {
            gk = g[k];
            if constexpr (kNp >= 2)
                bk = b[k];
        } else if constexpr (kMode == kParamLds) {
            gk = lds[pos + k * kWave];
            if constexpr (kNp >= 2)
                bk = lds[W * IT + pos + k * kWave];
        }
    }

    // As get(), and in kParamDirect mode a load from L2 (used where the
    // parameters enter the reduction).
    __device__ __forceinline__ void fetch(int k, int pos, RawVec<VB> &gk, RawVec<VB> &bk) const
    {
        if constexpr (kMode == kParamDirect) {
            direct(static_cast<uint32_t>(pos + k * kWave) * VB, gk, bk);
        } else {
            get(k, pos, gk, bk);
        }
    }
};

// The wave partial of a held tile, after folding the parameters into it when
// the operator reduces over them.  (A second, unmasked copy for full waves
// behind a wave-uniform branch was measured to raise register use by a third
// with no gain: the masks are register selects.)
template <OpKind OP, class T, int VB, int IT, int W, int OWNER, class L, bool SH = false>
__device__ __forceinline__ typename OpTraits<OP>::Partial tile_partial(
    Tile<T, VB, IT> (&t)[OpTraits<OP>::kIn], int kv, const ParamCache<OP, T, VB, IT, W, OWNER, SH> &pc, int pos,
    L &loc)
{
    using Op = OpTraits<OP>;
    if constexpr (holds_raw<OP, T>()) {
        // the streaming form over the held vectors, kLdsStep at a time, with
        // the parameters fetched per step (SHIFT rows: masked to the row)
        constexpr int U = IT < 4 ? IT : 4;
        static_assert(IT % U == 0, "held vectors per thread: a multiple of the step");
        static_assert(!L::kPartial || L::kHead, "raw tiles hold whole or shifted rows");
        typename Op::Partial r = Op::stream_init();
#pragma unroll
        for (int kb = 0; kb < IT; kb += U) {
            RawVec<VB> v[Op::kIn][U];
            RawVec<VB> g[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                RawVec<VB> b;
                pc.fetch(kb + u, pos, g[u], b);
#pragma unroll
                for (int i = 0; i < Op::kIn; ++i)
                    v[i][u] = t[i].v[kb + u];
            }
            const int kvb = kv - kb;
            if constexpr (L::kHead)
                Op::template stream_update_masked<T, VB, U>(r, v, g, kvb < 0 ? 0 : (kvb > U ? U : kvb), loc, kb);
            else
                Op::template stream_update<T, VB, U>(r, v, g, kvb < 0 ? 0 : (kvb > U ? U : kvb));
        }
        return Op::wave_from_thread(r);
    } else {
        if constexpr (Op::kParamsInReduce) {
#pragma unroll
            for (int k = 0; k < IT; ++k) {
                RawVec<VB> g, b;
                pc.fetch(k, pos, g, b);
                Op::template prepare<T, VB, IT>(t, k, g);
            }
        }
        return Op::template wave_partial<T, VB, IT>(t, kv, loc);
    }
}

// Whether the output loop loads the next row into the registers it frees
// ("rolling").  A wave has one in-order counter for its loads and stores, so
// when the next row's loads are issued after all of this row's stores, even
// its first vector can only be used once every store has drained.  Rolling
// issues load k right after store k, so the grouped reductions of the next row
// start while the stores still drain.  Measured on MI355X with the ordered
// loads and grouped softmax-family partials, the split kernel's best plan for
// 256 x 262144 fp32 softmax gained 6% and a 4096 x 65536 int8 quantization
// plan 4%; the two-input operators (softmax and LayerNorm backward) lost 3-5%
// at P = 4 and 8 and gained nothing at P = 2, and path 1 gained nothing (its
// owners mostly handle one row each).  So only one-input split slices roll.
// kParamDirect needs the freed registers for parameters.
template <int MODE, int OWNER, int NI>
constexpr bool rolls()
{
    return OWNER == kOwnerSlice && NI == 1 && MODE != kParamDirect;
}

// The output side of a SHIFT row (see shift_geom) for one thread: its
// vector 0 may begin with hb output bytes of the previous row, and its vector
// kpart (-1: none) holds the row's last element, the row's part of it being
// its first tb output bytes.  Those two vectors are written byte-exactly (the
// bytes outside the row belong to the neighbouring rows' owners): the last
// one through `whole`, the output span without a last word it shares with
// the next row (so one vector store writes its whole words), and that word's
// part separately.
struct ShiftOut {
    int hb;
    int kpart;
    int tb;
    rsrc_t whole;
};

// One output vector, k-th of the thread's: SHIFT rows write the vectors at the
// row's ends exactly (see ShiftOut), every other vector is one store.
template <int VBO, bool SHIFT>
__device__ __forceinline__ void store_out_vec(const RawVec<VBO> &ov, rsrc_t dst, uint32_t ooff, int k,
                                              const ShiftOut &so)
{
    if constexpr (SHIFT) {
        const bool head = k == 0 && so.hb > 0;
        if (head && k == so.kpart) {
            buf_store_bytes<VBO>(ov, dst, ooff, so.hb, so.tb);  // a row inside one vector
        } else if (head) {
            buf_store_from<VBO>(ov, dst, ooff, so.hb);
        } else if (k == so.kpart) {
            buf_store<VBO, kStreamStore>(ov, so.whole, ooff);
            if (so.tb & 3)
                buf_store_word_part(vec_word<VBO>(ov, so.tb >> 2), dst, ooff + static_cast<uint32_t>(so.tb & ~3), 0,
                                    so.tb & 3);
        } else {
            buf_store<VBO, kStreamStore>(ov, dst, ooff);
        }
    } else {
        buf_store<VBO, kStreamStore>(ov, dst, ooff);
    }
}

// Apply h to the held tile and write it out; dst, and the parameter
// descriptors, cover the same columns (the row or slice).  When rolling,
// vector k of the next row (`next`, a zero-length descriptor when there is
// none: its loads return zero without touching memory) is loaded into the
// register that vector k of this row leaves free.  SHIFT: the vectors at the
// row's ends are written byte-exactly (see ShiftOut).
template <OpKind OP, class T, int VB, int IT, int W, int OWNER, bool SHIFT = false>
__device__ __forceinline__ void store_tile(Tile<T, VB, IT> (&t)[OpTraits<OP>::kIn], rsrc_t dst,
                                           const ParamCache<OP, T, VB, IT, W, OWNER, SHIFT> &pc, int pos, const Coef &c,
                                           const Srcs<OpTraits<OP>::kIn> &next, const ShiftOut so = ShiftOut{})
{
    using Op = OpTraits<OP>;
    constexpr int NI = Op::kIn;
    constexpr int NP = held_out_params<OP, T>();
    constexpr bool RAW = holds_raw<OP, T>();
    constexpr int MODE = ParamCache<OP, T, VB, IT, W, OWNER, SHIFT>::kMode;
    constexpr int VBO = out_vb<OP, T, VB>();
    constexpr int G = kWave;  // vector stride between a thread's vectors
#pragma unroll
    for (int i = 0; i < NI; ++i)
        fence_tile(t[i]);
    // recompute the offsets here (one add each) instead of keeping the load
    // phase's offset registers alive across the reduction
    uint32_t base = static_cast<uint32_t>(pos) * VB;
    asm volatile("" : "+v"(base));
    (void)next;
    // output offsets: the input offsets when input and output vectors have
    // the same size, else their own
    uint32_t obase = base;
    if constexpr (VBO != VB) {
        obase = static_cast<uint32_t>(pos) * VBO;
        asm volatile("" : "+v"(obase));
    }
    if constexpr (MODE != kParamDirect || NP == 0) {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
            const uint32_t off = base + static_cast<uint32_t>(k * G * VB);
            const uint32_t ooff = VBO == VB ? off : obase + static_cast<uint32_t>(k * G * VBO);
            RawVec<VB> g, b;
            if constexpr (NP > 0)
                pc.get(k, pos, g, b);
            RawVec<VB> in[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i)
                in[i] = t[i].v[k];
            const RawVec<VBO> ov = apply_vec<OP, T, VB, RAW>(in, g, b, vec_coef<OP, T, IT>(c, k));
            store_out_vec<VBO, SHIFT>(ov, dst, ooff, k, so);
            if constexpr (rolls<MODE, OWNER, NI>())
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    t[i].v[k] = buf_load<VB, kStream>(next.r[i], off);
                    __builtin_amdgcn_sched_barrier(kLoadOrderBarrier);  // keeps the loads in order
                }
        }
    } else {
        // Unshifted rows: the next group's parameter loads are issued before
        // this group's stores (vector-memory operations complete in issue
        // order, so a load issued after a store could only be used once that
        // store had completed; measured 1-5% faster on wide LayerNorm and
        // RMSNorm rows on MI355X).  Shifted parameter vectors take two loads
        // each and a funnel shift: one vector at a time, not prefetched,
        // keeps their registers few.
        constexpr int GP = SHIFT ? 1 : param_group<IT, VB, NP>();
        constexpr bool kAhead = !SHIFT;
        RawVec<VB> g[GP], b[GP];
        if constexpr (kAhead)
#pragma unroll
            for (int j = 0; j < GP; ++j)
                pc.direct(base + static_cast<uint32_t>(j * G * VB), g[j], b[j]);
#pragma unroll
        for (int kb = 0; kb < IT; kb += GP) {
            RawVec<VB> gn[GP], bn[GP];
            if constexpr (kAhead) {
                if (kb + GP < IT)
#pragma unroll
                    for (int j = 0; j < GP; ++j)
                        pc.direct(base + static_cast<uint32_t>((kb + GP + j) * G * VB), gn[j], bn[j]);
            } else {
#pragma unroll
                for (int j = 0; j < GP; ++j)
                    pc.direct(base + static_cast<uint32_t>((kb + j) * G * VB), g[j], b[j]);
            }
#pragma unroll
            for (int j = 0; j < GP; ++j) {
                const uint32_t off = base + static_cast<uint32_t>((kb + j) * G * VB);
                const uint32_t ooff = VBO == VB ? off : obase + static_cast<uint32_t>((kb + j) * G * VBO);
                RawVec<VB> in[NI];
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    in[i] = t[i].v[kb + j];
                store_out_vec<VBO, SHIFT>(apply_vec<OP, T, VB, RAW>(in, g[j], b[j], vec_coef<OP, T, IT>(c, kb + j)),
                                          dst, ooff, kb + j, so);
            }
            if constexpr (kAhead)
                if (kb + GP < IT)
#pragma unroll
                    for (int j = 0; j < GP; ++j) {
                        g[j] = gn[j];
                        b[j] = bn[j];
                    }
        }
    }
}

// After store_tile: load the next row unless store_tile already did.
template <OpKind OP, class T, int VB, int IT, int W, int OWNER, bool SH = false>
__device__ __forceinline__ void load_next(Tile<T, VB, IT> (&t)[OpTraits<OP>::kIn],
                                          const Srcs<OpTraits<OP>::kIn> &next, int pos)
{
    if constexpr (!rolls<ParamCache<OP, T, VB, IT, W, OWNER, SH>::kMode, OWNER, OpTraits<OP>::kIn>())
        load_tile<T, VB, IT, kWave>(t, next, pos);
}

// Combine the wave partials of a workgroup through LDS; every thread returns
// the same workgroup partial (fixed order w = 0..NW-1).  The caller must not
// rewrite `sh` before every thread has passed a later barrier.
template <OpKind OP, int NW>
__device__ __forceinline__ typename OpTraits<OP>::Partial block_combine(const typename OpTraits<OP>::Partial &wp,
                                                                        typename OpTraits<OP>::Partial *sh)
{
    using Partial = typename OpTraits<OP>::Partial;
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

// Descriptor of `nvec` vectors starting at vector `first` of array `base`.
// (Integer arithmetic on the address: the parameter pointers are null for
// operators without parameters, whose descriptors are never used.)
template <int VB>
__device__ __forceinline__ rsrc_t span(const void *base, int64_t first, int64_t nvec)
{
    const uintptr_t p = reinterpret_cast<uintptr_t>(base) + static_cast<uintptr_t>(first * VB);
    return make_rsrc(reinterpret_cast<const void *>(p), static_cast<uint32_t>(nvec * VB));
}

// Vectors [first, first + nvec) of row `row`.  PEB = 0: rows of nv whole
// vectors.  PEB = element bytes (a PART kernel): rows of `cols` elements, the
// last vector partial, and the descriptor ends at the row's last byte.  On
// MI355X a descriptor's range check acts per dword (a straddling 16-byte load
// returns its in-row dwords and zeros, a straddling store writes only its
// in-row dwords) and 16-byte accesses at 4-byte alignment are served, so such
// rows keep 16-byte vectors when their byte length is a multiple of 4.
template <int VB, int PEB>
__device__ __forceinline__ rsrc_t row_span(const void *base, int64_t row, int64_t cols, int64_t nv,
                                           int64_t first, int64_t nvec)
{
    if constexpr (PEB == 0) {
        return span<VB>(base, row * nv + first, nvec);
    } else {
        constexpr int E = VB / PEB;
        const int64_t e0 = first * E;
        int64_t ne = cols - e0;
        ne = ne < nvec * E ? ne : nvec * E;
        ne = ne > 0 ? ne : 0;
        const uintptr_t p = reinterpret_cast<uintptr_t>(base) + static_cast<uintptr_t>((row * cols + e0) * PEB);
        return make_rsrc(reinterpret_cast<const void *>(p), static_cast<uint32_t>(ne * PEB));
    }
}

// SHIFT rows: a row whose start is not 64-byte aligned is held from the
// 64-byte boundary below its first byte, so that every wave's run of 16-byte
// vectors covers whole 64-byte lines (on MI355X, rows that start inside a
// line streamed 10-30% slower, in loads and stores alike, short rows too).
// Row r begins s elements into its held span, the last s elements of row
// r - 1 (masked in the reduction, never written); s is taken from x's
// address, and dy and y, whose bases are 16-byte aligned too, use the same s
// (their held spans then start 16-byte aligned, and line-aligned when their
// bases are congruent to x's modulo 64; the int8 codes' spans start 4- or
// 8-byte aligned, as their vectors need).  A row that starts less than 64
// bytes into the tensor is held from the tensor's start instead (s = its
// offset in elements), so no access precedes the tensor.  The held span ends
// with the 4-byte word that holds the row's last element (its other bytes,
// when it has any, are the next row's: read, masked, never written; after
// the tensor's last row they lie inside the same word).
struct ShiftRow {
    int s;        // elements of the previous row in front of the row
    int64_t nv;   // 16-byte vectors of the held span
    int ntail;    // elements of its last vector up to the row's end (1..E)
};

template <int EB, int E>
__device__ __forceinline__ ShiftRow shift_geom(const RowArgs &a, int64_t row)
{
    const int64_t cols = a.cols;
    const int64_t first = row * cols;
    const uintptr_t at = reinterpret_cast<uintptr_t>(a.x) + static_cast<uintptr_t>(first * EB);
    int64_t s = static_cast<int64_t>(at & 63u) / EB;
    s = s < first ? s : first;
    ShiftRow g;
    g.s = static_cast<int>(s);
    const int64_t n = s + cols;
    g.nv = (n + E - 1) / E;
    g.ntail = static_cast<int>(n - E * (g.nv - 1));
    return g;
}

// Vectors [first, first + nvec) of row `row`'s held span in a tensor of
// EBT-byte elements and VBT-byte vectors;
// whole = true: the span without a last word that the next row shares.
template <int VBT, int EBT>
__device__ __forceinline__ rsrc_t shift_span(const void *base, int64_t row, int64_t cols, int s, int64_t first,
                                             int64_t nvec, bool whole = false)
{
    const int64_t lo = (row * cols - s) * EBT;
    const int64_t len = whole ? ((s + cols) * EBT) & ~INT64_C(3) : ((s + cols) * EBT + 3) & ~INT64_C(3);
    int64_t n = len - first * VBT;
    n = n < nvec * VBT ? n : nvec * VBT;
    n = n > 0 ? n : 0;
    const uintptr_t p = reinterpret_cast<uintptr_t>(base) + static_cast<uintptr_t>(lo + first * VBT);
    return make_rsrc(reinterpret_cast<const void *>(p), static_cast<uint32_t>(n));
}

// The parameter vectors of held vectors [first, first + nvec) (row_span of
// row 0); SHIFT rows: the whole parameter array, up to the 4-byte word that
// holds its last element (ParamCache shifts the offsets row by row).
template <int VB, int PEB, bool SHIFT>
__device__ __forceinline__ rsrc_t param_span(const void *base, int64_t cols, int64_t nv, int64_t first, int64_t nvec)
{
    if constexpr (SHIFT)
        return make_rsrc(base, static_cast<uint32_t>((cols * PEB + 3) & ~INT64_C(3)));
    else
        return row_span<VB, PEB>(base, 0, cols, nv, first, nvec);
}

// The row inputs (x, and dy for two-input operators): `nvec` vectors from
// vector `first` of row `row` (nv vectors per row; PEB as for row_span; SHIFT
// rows as for shift_span, `sh` elements of the previous row in front).
template <OpKind OP, int VB, int PEB = 0, bool SHIFT = false>
__device__ __forceinline__ Srcs<OpTraits<OP>::kIn> row_srcs(const RowArgs &a, int64_t row, int64_t nv,
                                                            int64_t first, int64_t nvec, int sh = 0)
{
    Srcs<OpTraits<OP>::kIn> s;
    if constexpr (SHIFT) {
        static_assert(PEB > 0, "SHIFT rows are PART rows");
        s.r[0] = shift_span<VB, PEB>(a.x, row, a.cols, sh, first, nvec);
        if constexpr (OpTraits<OP>::kIn >= 2)
            s.r[1] = shift_span<VB, PEB>(a.dy, row, a.cols, sh, first, nvec);
    } else {
        s.r[0] = row_span<VB, PEB>(a.x, row, a.cols, nv, first, nvec);
        if constexpr (OpTraits<OP>::kIn >= 2)
            s.r[1] = row_span<VB, PEB>(a.dy, row, a.cols, nv, first, nvec);
    }
    return s;
}

// The thread's index (among its vectors k, at slice positions pos + k * G) of
// the slice's last vector, when that vector is the row's partial last one
// (`last` = the slice ends the row); -1 otherwise.
template <int IT, int G>
__device__ __forceinline__ int partial_index(int64_t ns, int pos, bool last)
{
    const int64_t d = ns - 1 - pos;
    if (!last || d < 0 || d % G != 0 || d / G >= IT)
        return -1;
    return static_cast<int>(d / G);
}

// Per-row state of a SHIFT row for the thread at slice position `pos` of a
// slice that starts at held vector v0 and holds ns of the row's held
// vectors: the masks of its first and last vectors (LocalShift) and their
// output bytes (ShiftOut, OEB output bytes per element).
template <int IT, int E, int OEB>
__device__ __forceinline__ ShiftOut shift_row(LocalShift &loc, const ShiftRow &g, int64_t v0, int64_t ns, int pos)
{
    loc.ntail = g.ntail;
    loc.kpart = partial_index<IT, kWave>(ns, pos, v0 + ns == g.nv);
    const int64_t h = g.s - (v0 + pos) * E;
    loc.hcount = h <= 0 ? 0 : (h >= E ? E : static_cast<int>(h));
    ShiftOut so;
    so.hb = loc.hcount * OEB;
    so.kpart = loc.kpart;
    so.tb = loc.ntail * OEB;
    return so;
}

// The per-row output of `row` (the quantization scale; LayerNorm backward's
// mean and rstd when row_out is given), written by one lane.
template <OpKind OP>
__device__ __forceinline__ void store_row_value(const RowArgs &a, int64_t row, const Coef &c, bool writer)
{
    using Op = OpTraits<OP>;
    if constexpr (Op::kRowOut) {
        if (writer && a.row_out != nullptr) {
            if constexpr (Op::kRowWords == 1) {
                RawVec<4> v;
                v.w = __float_as_uint(Op::row_value(c, 0));
                buf_store<4, kStreamStore>(v, span<4>(a.row_out, row, 1), 0u);
            } else {
                RawVec<8> v;
                v.w = u32x2{__float_as_uint(Op::row_value(c, 0)), __float_as_uint(Op::row_value(c, 1))};
                buf_store<8, kStreamStore>(v, span<8>(a.row_out, row, 1), 0u);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The LDS tier of a held tile.  The on-chip budget of a row owner is its
// registers and its share of the CU's LDS (CREDIT paper, Sec. III-B, Eq. 3);
// a tile with LT > 0 holds the first BLOCK * IT vectors of its row or slice in
// registers, as every tile does, and up to BLOCK * LT more in LDS: thread tid
// holds vectors BLOCK * IT + tid + j * BLOCK (j < LT) in LDS slot [j][tid].
// Consecutive threads use consecutive 16-byte slots (no bank conflicts), and
// a thread reads back only the slots it wrote, so the LDS part needs no
// barrier of its own.  It is reduced with the operator's streaming partial as
// its vectors arrive (kLdsStep at a time) and merged with the register part's
// wave partial; its output pass reads it back from LDS and applies the
// streaming form of the operator (apply_stream, from the same row partial).
// ---------------------------------------------------------------------------
constexpr int kLdsStep = 4;  // LDS-part vectors per input loaded and reduced at a time

template <OpKind OP, int VB, int BLOCK, int LT>
using LdsRow = RawVec<VB>[OpTraits<OP>::kIn][LT][BLOCK];

// Load the LDS part (nl vectors from `src`, parameters `gam` of the same
// columns) into `buf` and return its wave partial.
template <OpKind OP, class T, int VB, int BLOCK, int LT>
__device__ __forceinline__ typename OpTraits<OP>::Partial lds_load_reduce(LdsRow<OP, VB, BLOCK, LT> &buf,
                                                                          const Srcs<OpTraits<OP>::kIn> &src,
                                                                          rsrc_t gam, int64_t nl, int tid)
{
    using Op = OpTraits<OP>;
    constexpr int NI = Op::kIn;
    constexpr int U = kLdsStep;
    static_assert(LT % U == 0, "LDS vectors per thread: a multiple of the step");
    typename Op::Partial r = Op::stream_init();
#pragma unroll
    for (int j0 = 0; j0 < LT; j0 += U) {
        RawVec<VB> v[NI][U];
        RawVec<VB> g[U];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[i][u] = buf_load<VB, kStream>(src.r[i], static_cast<uint32_t>(tid + (j0 + u) * BLOCK) * VB);
        if constexpr (Op::kParamsInReduce)
#pragma unroll
            for (int u = 0; u < U; ++u)
                g[u] = buf_load<VB, kKeep>(gam, static_cast<uint32_t>(tid + (j0 + u) * BLOCK) * VB);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int u = 0; u < U; ++u)
                buf[i][j0 + u][tid] = v[i][u];
        Op::template stream_update<T, VB, U>(r, v, g, count_valid<U, BLOCK>(nl, tid + j0 * BLOCK));
    }
    return Op::wave_from_thread(r);
}

// Write the LDS part's output (nl vectors to `dst`; parameters `gam`, `bet`
// of the same columns) with the streaming coefficients c.
template <OpKind OP, class T, int VB, int BLOCK, int LT>
__device__ __forceinline__ void lds_store(const LdsRow<OP, VB, BLOCK, LT> &buf, rsrc_t dst, rsrc_t gam, rsrc_t bet,
                                          int tid, const Coef &c)
{
    using Op = OpTraits<OP>;
    constexpr int NI = Op::kIn;
    constexpr int VBO = out_vb<OP, T, VB>();
#pragma unroll
    for (int j = 0; j < LT; ++j) {
        const uint32_t idx = static_cast<uint32_t>(tid + j * BLOCK);
        RawVec<VB> in[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i)
            in[i] = buf[i][j][tid];
        RawVec<VB> g, b;
        if constexpr (Op::kParams >= 1)
            g = buf_load<VB, kKeep>(gam, idx * VB);
        if constexpr (Op::kParams >= 2)
            b = buf_load<VB, kKeep>(bet, idx * VB);
        buf_store<VBO, kStreamStore>(apply_vec<OP, T, VB, true>(in, g, b, c), dst, idx * VBO);
    }
}

// The wave partial of a tile's register part merged with its LDS part's.
template <OpKind OP>
__device__ __forceinline__ typename OpTraits<OP>::Partial merge_tiers(const typename OpTraits<OP>::Partial &reg,
                                                                      const typename OpTraits<OP>::Partial &lds)
{
    const typename OpTraits<OP>::Partial p[2] = {reg, lds};
    return OpTraits<OP>::template merge<2>(p, 2);
}

// ---------------------------------------------------------------------------
// Path 1a: one wavefront per row, four waves per 256-thread workgroup; wave w
// of the grid handles rows w, w + W, w + 2W, ... (W waves in the grid).  No
// barrier on the row: the wave reduction is the row reduction.
// ---------------------------------------------------------------------------
// PART: rows whose last vector is partial (see row_span).  SHIFT (with
// PART): rows held from the 64-byte boundary below their start (see
// shift_geom), whose held vector count varies from row to row.
template <OpKind OP, class T, int VB, int IT, bool PART = false, bool SHIFT = false>
__global__ __launch_bounds__(kWave *kWaveRowsPerWg) void single_wave_kernel(RowArgs a)
{
    using Op = OpTraits<OP>;
    using PC = ParamCache<OP, T, VB, IT, kWave, kOwnerWaves, SHIFT>;
    using Loc = std::conditional_t<SHIFT, LocalShift, std::conditional_t<PART, LocalPart, Local>>;
    constexpr int EB = StorageTraits<T>::kBytes;
    constexpr int E = VB / EB;
    constexpr int VBO = out_vb<OP, T, VB>();
    constexpr int OEB = StorageTraits<OutT<OP, T>>::kBytes;
    constexpr int PEB = PART ? EB : 0;
    static_assert(!PART || SHIFT || VBO == VB, "PART rows need outputs of the input's element size");
    static_assert(!SHIFT || (PART && VB == 16), "SHIFT rows: 16-byte vectors");
    __shared__ RawVec<VB> lds_params[param_lds_vectors<OP, VB, IT, kWave, kOwnerWaves>()];
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nv = PART ? (a.cols + E - 1) / E : a.cols / E;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * kWaveRowsPerWg;
    int64_t row = uniform(static_cast<int64_t>(blockIdx.x) * kWaveRowsPerWg + threadIdx.x / kWave);
    ShiftRow g{};
    if constexpr (SHIFT)
        g = shift_geom<EB, E>(a, row);
    Tile<T, VB, IT> t[Op::kIn];
    load_tile<T, VB, IT, kWave>(t, row_srcs<OP, VB, PEB, SHIFT>(a, row, nv, 0, row < a.rows ? (SHIFT ? g.nv : nv) : 0,
                                                                g.s), lane);
    PC pc;
    pc.init(param_span<VB, PEB, SHIFT>(a.gamma, a.cols, nv, 0, nv), param_span<VB, PEB, SHIFT>(a.beta, a.cols, nv, 0, nv),
            lane, lds_params, threadIdx.x, kWave * kWaveRowsPerWg);
    if constexpr (PC::kMode == kParamLds)
        __syncthreads();
    int kv = count_valid<IT, kWave>(nv, lane);
    Loc loc0;
    if constexpr (PART && !SHIFT) {
        loc0.ntail = static_cast<int>(a.cols % E);
        loc0.kpart = partial_index<IT, kWave>(nv, lane, loc0.ntail != 0);
    }
    for (; row < a.rows; row += waves) {
        const int64_t next = row + waves;
        Loc loc = loc0;
        ShiftOut so{};
        ShiftRow gn{};
        if constexpr (SHIFT) {
            so = shift_row<IT, E, OEB>(loc, g, 0, g.nv, lane);
            kv = count_valid<IT, kWave>(g.nv, lane);
            gn = shift_geom<EB, E>(a, next);
            pc.shift(g.s, 0);
        }
        const auto wp = tile_partial<OP, T, VB, IT, kWave, kOwnerWaves>(t, kv, pc, lane, loc);
        const Coef c = Op::template finalize<T>(wp, loc, a.cols, a.eps);
        store_row_value<OP>(a, row, c, lane == 0);
        const auto nsrc =
            row_srcs<OP, VB, PEB, SHIFT>(a, next, nv, 0, next < a.rows ? (SHIFT ? gn.nv : nv) : 0, gn.s);
        const rsrc_t dst = SHIFT ? shift_span<VBO, OEB>(a.y, row, a.cols, g.s, 0, g.nv)
                                 : row_span<VBO, PEB>(a.y, row, a.cols, nv, 0, nv);
        if constexpr (SHIFT)
            so.whole = shift_span<VBO, OEB>(a.y, row, a.cols, g.s, 0, g.nv, true);
        store_tile<OP, T, VB, IT, kWave, kOwnerWaves, SHIFT>(t, dst, pc, lane, c, nsrc, so);
        load_next<OP, T, VB, IT, kWave, kOwnerWaves, SHIFT>(t, nsrc, lane);
        g = gn;
    }
}

// ---------------------------------------------------------------------------
// Path 1b: one workgroup of BLOCK threads per row; workgroup g handles rows
// g, g + G, g + 2G, ... (G workgroups in the grid).
// ---------------------------------------------------------------------------
// LT > 0: the LDS tier (lds_load_reduce); rows of whole 16-byte vectors,
// at most BLOCK * (IT + LT) of them (the host checks).
template <OpKind OP, class T, int VB, int BLOCK, int IT, bool PART = false, bool SHIFT = false, int LT = 0>
__global__ __launch_bounds__(BLOCK) void single_wg_kernel(RowArgs a)
{
    using Op = OpTraits<OP>;
    using PC = ParamCache<OP, T, VB, IT, BLOCK, kOwnerRow, SHIFT>;
    using Loc = std::conditional_t<SHIFT, LocalShift, std::conditional_t<PART, LocalPart, Local>>;
    constexpr int EB = StorageTraits<T>::kBytes;
    constexpr int E = VB / EB;
    constexpr int PEB = PART ? EB : 0;
    constexpr int NW = BLOCK / kWave;
    constexpr int VBO = out_vb<OP, T, VB>();
    constexpr int OEB = StorageTraits<OutT<OP, T>>::kBytes;
    constexpr bool kLds = LT > 0;
    static_assert(!SHIFT || (PART && VB == 16), "SHIFT rows: 16-byte vectors");
    static_assert(!kLds || (!PART && VB == 16), "the LDS tier holds rows of whole 16-byte vectors");
    __shared__ typename Op::Partial sh[NW];
    __shared__ RawVec<VB> lds_params[param_lds_vectors<OP, VB, IT, BLOCK, kOwnerRow>()];
    __shared__ LdsRow<OP, VB, kLds ? BLOCK : 1, kLds ? LT : kLdsStep> lds_row;
    const int tid = threadIdx.x;
    const int pos = (tid / kWave) * kWave * IT + (tid & (kWave - 1));  // this wave's run + lane
    const int64_t nv = PART ? (a.cols + E - 1) / E : a.cols / E;
    // vectors held in registers, and in LDS (kLds)
    const int64_t nreg = kLds ? min(nv, static_cast<int64_t>(BLOCK) * IT) : nv;
    const int64_t nl = nv - nreg;
    int64_t row = blockIdx.x;
    ShiftRow g{};
    if constexpr (SHIFT)
        g = shift_geom<EB, E>(a, row);
    Tile<T, VB, IT> t[Op::kIn];
    load_tile<T, VB, IT, kWave>(t, row_srcs<OP, VB, PEB, SHIFT>(a, row, nv, 0, SHIFT ? g.nv : nreg, g.s), pos);
    PC pc;
    pc.init(param_span<VB, PEB, SHIFT>(a.gamma, a.cols, nv, 0, nreg),
            param_span<VB, PEB, SHIFT>(a.beta, a.cols, nv, 0, nreg), pos, lds_params, tid, BLOCK);
    if constexpr (PC::kMode == kParamLds)
        __syncthreads();
    int kv = count_valid<IT, kWave>(nreg, pos);
    Loc loc0;
    if constexpr (PART && !SHIFT) {
        loc0.ntail = static_cast<int>(a.cols % E);
        loc0.kpart = partial_index<IT, kWave>(nv, pos, loc0.ntail != 0);
    }
    for (; row < a.rows; row += gridDim.x) {
        const int64_t next = row + gridDim.x;
        Loc loc = loc0;
        ShiftOut so{};
        ShiftRow gn{};
        if constexpr (SHIFT) {
            so = shift_row<IT, E, OEB>(loc, g, 0, g.nv, pos);
            kv = count_valid<IT, kWave>(g.nv, pos);
            gn = shift_geom<EB, E>(a, next);
            pc.shift(g.s, 0);
        }
        typename Op::Partial lp;
        if constexpr (kLds)
            lp = lds_load_reduce<OP, T, VB, BLOCK, LT>(lds_row, row_srcs<OP, VB>(a, row, nv, nreg, nl),
                                                       span<VB>(a.gamma, nreg, nl), nl, tid);
        auto wp = tile_partial<OP, T, VB, IT, BLOCK, kOwnerRow>(t, kv, pc, pos, loc);
        if constexpr (kLds)
            wp = merge_tiers<OP>(wp, lp);
        const auto rp = block_combine<OP, NW>(wp, sh);
        const Coef c = Op::template finalize<T>(rp, loc, a.cols, a.eps);
        store_row_value<OP>(a, row, c, tid == 0);
        const auto nsrc =
            row_srcs<OP, VB, PEB, SHIFT>(a, next, nv, 0, next < a.rows ? (SHIFT ? gn.nv : nreg) : 0, gn.s);
        const rsrc_t dst = SHIFT ? shift_span<VBO, OEB>(a.y, row, a.cols, g.s, 0, g.nv)
                                 : row_span<VBO, PEB>(a.y, row, a.cols, nv, 0, nreg);
        if constexpr (SHIFT)
            so.whole = shift_span<VBO, OEB>(a.y, row, a.cols, g.s, 0, g.nv, true);
        store_tile<OP, T, VB, IT, BLOCK, kOwnerRow, SHIFT>(t, dst, pc, pos, c, nsrc, so);
        if constexpr (kLds)
            lds_store<OP, T, VB, BLOCK, LT>(lds_row, span<VBO>(a.y, row * nv + nreg, nl), span<VB>(a.gamma, nreg, nl),
                                            span<VB>(a.beta, nreg, nl), tid,
                                            Op::template finalize_stream<T>(rp, a.cols, a.eps));
        load_next<OP, T, VB, IT, BLOCK, kOwnerRow, SHIFT>(t, nsrc, pos);
        g = gn;
        // the next block_combine rewrites sh: every wave must have read it
        __syncthreads();
    }
}

// The end of every split-row workgroup, in its thread 0: count the
// workgroup on ctl->done, and in the launch's last workgroup reset the ticket
// counter and advance the tags past this launch's (clearing every exchange
// word first when they reach kTagResetAt; one thread, once per 2^31 row
// iterations).  Every workgroup reaches this only after its last exchange,
// so when the last one arrives no word is read or written any more.
__device__ __forceinline__ void finish_split_launch(const SplitArgs &a, uint32_t tag0)
{
    if (fetch_add_u32_agent(&a.ctl->done, 1u) != static_cast<uint32_t>(a.clusters * a.p) - 1u)
        return;
    const int64_t iters = (a.r.rows + a.clusters - 1) / a.clusters;
    const uint32_t used = tag0 - 1u + static_cast<uint32_t>(iters);
    const bool reset = used >= kTagResetAt;
    if (reset) {
        uint64_t *slots = scratch_slots(a.ctl);
        for (int64_t i = 0; i < kSlotWords; ++i)
            store_u64_agent(slots + i, 0);
    }
    store_u32_agent(&a.ctl->ticket, 0u);
    store_u32_agent(&a.ctl->done, 0u);
    store_u32_agent(&a.ctl->tags_used, reset ? 0u : used);
}

// ---------------------------------------------------------------------------
// Path 2: P workgroups per row (see the header comment).  CONTROL = true is the
// work-free control kernel: identical launch shape, tickets, exchange and
// reductions (over zero tiles), but no access to rows, parameters or outputs
// at all (the control launch passes null pointers for them).
// ---------------------------------------------------------------------------
// LT > 0: the LDS tier, as in single_wg_kernel (slices of whole 16-byte
// vectors, at most BLOCK * (IT + LT) of them).
template <OpKind OP, class T, int VB, int BLOCK, int IT, bool CONTROL, bool PART = false, bool SHIFT = false,
          int LT = 0>
__global__ __launch_bounds__(BLOCK) void split_kernel(SplitArgs a)
{
    using Op = OpTraits<OP>;
    using Partial = typename Op::Partial;
    using PC = ParamCache<OP, T, VB, IT, BLOCK, kOwnerSlice, SHIFT>;
    using Loc = std::conditional_t<SHIFT, LocalShift, std::conditional_t<PART, LocalPart, Local>>;
    constexpr int EB = StorageTraits<T>::kBytes;
    constexpr int E = VB / EB;
    constexpr int PEB = PART ? EB : 0;
    constexpr int OEB = StorageTraits<OutT<OP, T>>::kBytes;
    static_assert(!(PART && CONTROL), "the control twin touches no row");
    static_assert(!SHIFT || (PART && VB == 16), "SHIFT rows: 16-byte vectors");
    constexpr bool kLds = LT > 0;
    static_assert(!kLds || (!PART && !CONTROL && VB == 16), "the LDS tier holds slices of whole 16-byte vectors");
    constexpr int NW = BLOCK / kWave;
    constexpr int Q = Op::kQ;
    constexpr int VBO = out_vb<OP, T, VB>();
    __shared__ Partial sh[NW];
    __shared__ Partial peer[kMaxSplit];
    __shared__ uint32_t sh_ticket, sh_tag0, sh_unmatched;
    __shared__ RawVec<VB> lds_params[param_lds_vectors<OP, VB, IT, BLOCK, kOwnerSlice>()];
    __shared__ LdsRow<OP, VB, kLds ? BLOCK : 1, kLds ? LT : kLdsStep> lds_row;
    const int tid = threadIdx.x;
    if (tid == 0) {
        sh_ticket = fetch_add_u32_agent(&a.ctl->ticket, 1u);
        sh_tag0 = load_u32_agent(&a.ctl->tags_used) + 1u;
        sh_unmatched = load_u32_agent(&a.ctl->unmatched);
    }
    __syncthreads();
    // the modulo only guards against a control block left inconsistent (it
    // cannot be by a launch that ran to its end); it keeps every index inside
    // this launch's clusters and slots
    const uint32_t ticket = sh_ticket % gridDim.x;
    const uint32_t tag0 = __builtin_amdgcn_readfirstlane(sh_tag0);  // uniform: keep the tags in SGPRs
    const int P = a.p;
    const int64_t k = ticket / static_cast<uint32_t>(P);
    const int c = static_cast<int>(ticket % static_cast<uint32_t>(P));

    // vectors per row (SHIFT: the most any row's held span covers; each row's
    // own count, and so its last slices' lengths, come from shift_geom)
    const int64_t nv = SHIFT ? shift_held_vectors(a.r.cols, EB) : (PART ? (a.r.cols + E - 1) / E : a.r.cols / E);
    const int64_t per = slice_vectors(nv, P, VB);
    const int64_t v0 = min(nv, per * c);
    const int64_t ns = min(nv, v0 + per) - v0;  // vectors in this slice
    // of which held in registers, and in LDS (kLds)
    const int64_t nreg = kLds ? min(ns, static_cast<int64_t>(BLOCK) * IT) : ns;
    const int64_t nl = ns - nreg;
    const int pos = (tid / kWave) * kWave * IT + (tid & (kWave - 1));  // this wave's run + lane
    int kv = count_valid<IT, kWave>(nreg, pos);
    uint64_t *cslots = scratch_slots(a.ctl) + k * 2 * P * Q;
    // a SHIFT row's vectors in this slice
    auto shift_ns = [&](const ShiftRow &gr) __attribute__((always_inline)) {
        const int64_t n = gr.nv - v0;
        return n < 0 ? INT64_C(0) : (n < per ? n : per);
    };
    ShiftRow g{};
    if constexpr (SHIFT)
        g = shift_geom<EB, E>(a.r, k);

    Tile<T, VB, IT> t[Op::kIn];
    PC pc;
    if constexpr (CONTROL) {
#pragma unroll
        for (int i = 0; i < Op::kIn; ++i)
#pragma unroll
            for (int j = 0; j < IT; ++j)
                t[i].v[j] = RawVec<VB>{};
    } else {
        load_tile<T, VB, IT, kWave>(
            t, row_srcs<OP, VB, PEB, SHIFT>(a.r, k, nv, v0, k < a.r.rows ? (SHIFT ? shift_ns(g) : nreg) : 0, g.s),
            pos);
        pc.init(param_span<VB, PEB, SHIFT>(a.r.gamma, a.r.cols, nv, v0, nreg),
                param_span<VB, PEB, SHIFT>(a.r.beta, a.r.cols, nv, v0, nreg), pos, lds_params, tid, BLOCK);
        if constexpr (PC::kMode == kParamLds)
            __syncthreads();
    }

    // One row of this slice: reduce, exchange, write (and, rolling, load the
    // next row).  When the slice rolls, the first row is peeled off the loop
    // so that every path into the loop ends in the same interleaved store/load
    // sequence, which lets the compiler wait for each held vector precisely
    // instead of conservatively (measured: 3% on RMSNorm bf16 split plans; the
    // kernels that do not roll gain nothing from it and are not peeled).
    Loc loc0;
    if constexpr (PART && !SHIFT) {
        loc0.ntail = static_cast<int>(a.r.cols % E);
        loc0.kpart = partial_index<IT, kWave>(ns, pos, loc0.ntail != 0 && v0 + ns == nv);
    }
    auto step = [&](int64_t row, uint32_t it) __attribute__((always_inline)) {
        const int64_t next = row + a.clusters;
        Partial wp;
        Loc loc = loc0;
        ShiftOut so{};
        ShiftRow gn{};
        if constexpr (SHIFT) {
            const int64_t nsr = shift_ns(g);
            so = shift_row<IT, E, OEB>(loc, g, v0, nsr, pos);
            kv = count_valid<IT, kWave>(nsr, pos);
            gn = shift_geom<EB, E>(a.r, next);
            pc.shift(g.s, v0);
        }
        Partial lp;
        if constexpr (kLds)
            lp = lds_load_reduce<OP, T, VB, BLOCK, LT>(lds_row, row_srcs<OP, VB>(a.r, row, nv, v0 + nreg, nl),
                                                       span<VB>(a.r.gamma, v0 + nreg, nl), nl, tid);
        if constexpr (CONTROL)
            wp = Op::template wave_partial<T, VB, IT>(t, kv, loc);
        else
            wp = tile_partial<OP, T, VB, IT, BLOCK, kOwnerSlice>(t, kv, pc, pos, loc);
        if constexpr (kLds)
            wp = merge_tiers<OP>(wp, lp);
        const Partial sp = block_combine<OP, NW>(wp, sh);

        // publish this slice's partial, then gather all P partials of the row.
        // A wait that gives up flags the error word and takes NaN for the
        // scalar it waited for: every operator's merge carries a NaN into the
        // row's coefficients, so the slice's output is NaN (a quantizer's
        // scale NaN) rather than computed from a stale word.
        const uint32_t tag = tag0 + it;
        uint64_t *slots = cslots + (it & 1u) * P * Q;
        if (tid < Q)
            store_u64_agent(slots + c * Q + tid, (static_cast<uint64_t>(tag) << 32) | __float_as_uint(comp(sp, tid)));
        if (tid < P * Q) {
            const uint32_t want = tag + sh_unmatched;
            uint64_t w = load_u64_agent(slots + tid);
            uint32_t polls = 0;
            while (static_cast<uint32_t>(w >> 32) != want) {
                if (polls++ >= a.spin_limit) {
                    fetch_or_u32_agent(&a.ctl->error, 1u);
                    w = 0x7FC00000u;  // NaN
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                w = load_u64_agent(slots + tid);
            }
            set_comp(peer[tid / Q], tid % Q, __uint_as_float(static_cast<uint32_t>(w)));
        }
        __syncthreads();
        Partial parts[kMaxSplit];
#pragma unroll
        for (int i = 0; i < kMaxSplit; ++i)
            parts[i] = peer[i];
        const Partial rp = ExchangeMerge<OP>::template apply<kMaxSplit>(parts, P);
        const Coef cf = Op::template finalize<T>(rp, loc, a.r.cols, a.r.eps);
        if constexpr (CONTROL) {
            (void)cf;
            (void)next;
        } else {
            store_row_value<OP>(a.r, row, cf, c == 0 && tid == 0);
            const auto nsrc = row_srcs<OP, VB, PEB, SHIFT>(
                a.r, next, nv, v0, next < a.r.rows ? (SHIFT ? shift_ns(gn) : nreg) : 0, gn.s);
            const rsrc_t dst = SHIFT ? shift_span<VBO, OEB>(a.r.y, row, a.r.cols, g.s, v0, shift_ns(g))
                                     : row_span<VBO, PEB>(a.r.y, row, a.r.cols, nv, v0, nreg);
            if constexpr (SHIFT)
                so.whole = shift_span<VBO, OEB>(a.r.y, row, a.r.cols, g.s, v0, shift_ns(g), true);
            store_tile<OP, T, VB, IT, BLOCK, kOwnerSlice, SHIFT>(t, dst, pc, pos, cf, nsrc, so);
            if constexpr (kLds)
                lds_store<OP, T, VB, BLOCK, LT>(lds_row, span<VBO>(a.r.y, row * nv + v0 + nreg, nl),
                                                span<VB>(a.r.gamma, v0 + nreg, nl), span<VB>(a.r.beta, v0 + nreg, nl),
                                                tid, Op::template finalize_stream<T>(rp, a.r.cols, a.r.eps));
            load_next<OP, T, VB, IT, BLOCK, kOwnerSlice, SHIFT>(t, nsrc, pos);
        }
        g = gn;
        // (no barrier needed before the next row rewrites sh or peer: every
        // wave has read sh before the exchange barrier above and reads peer
        // before it reaches the next block_combine barrier)
    };
    if constexpr (rolls<PC::kMode, kOwnerSlice, Op::kIn>()) {
        if (k < a.r.rows) {
            step(k, 0u);
            uint32_t it = 1;
            for (int64_t row = k + a.clusters; row < a.r.rows; row += a.clusters, ++it)
                step(row, it);
        }
    } else {
        uint32_t it = 0;
        for (int64_t row = k; row < a.r.rows; row += a.clusters, ++it)
            step(row, it);
    }
    // every thread of the workgroup is past its last exchange once thread 0
    // is: each row's exchange ends in a barrier
    if (tid == 0)
        finish_split_launch(a, tag0);
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
    using Partial = typename Op::Partial;
    constexpr int NI = Op::kIn;
    constexpr int E = VB / StorageTraits<T>::kBytes;
    constexpr int NW = BLOCK / kWave;
    constexpr int GP = U < 4 ? U : 4;
    constexpr int VBO = out_vb<OP, T, VB>();
    constexpr int64_t CH = static_cast<int64_t>(BLOCK) * U;
    __shared__ Partial sh[NW];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t nv = a.cols / E;
    Partial r = Op::stream_init();
    for (int64_t base = 0; base < nv; base += CH) {
        const int64_t n = min(CH, nv - base);
        const auto src = row_srcs<OP, VB>(a, row, nv, base, n);
        RawVec<VB> v[NI][U];
        RawVec<VB> g[U];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int k = 0; k < U; ++k)
                v[i][k] = buf_load<VB, kKeep>(src.r[i], static_cast<uint32_t>(tid + k * BLOCK) * VB);
        if constexpr (Op::kParamsInReduce) {
            const rsrc_t gam = span<VB>(a.gamma, base, n);
#pragma unroll
            for (int k = 0; k < U; ++k)
                g[k] = buf_load<VB, kKeep>(gam, static_cast<uint32_t>(tid + k * BLOCK) * VB);
        }
        Op::template stream_update<T, VB, U>(r, v, g, count_valid<U, BLOCK>(n, tid));
    }
    const Partial wp = Op::wave_from_thread(r);
    const Partial rp = block_combine<OP, NW>(wp, sh);
    const Coef c = Op::template finalize_stream<T>(rp, a.cols, a.eps);
    store_row_value<OP>(a, row, c, tid == 0);
    for (int64_t base = 0; base < nv; base += CH) {
        const int64_t n = min(CH, nv - base);
        const auto src = row_srcs<OP, VB>(a, row, nv, base, n);
        const rsrc_t dst = span<VBO>(a.y, row * nv + base, n);
        const rsrc_t gam = span<VB>(a.gamma, base, n);
        const rsrc_t bet = span<VB>(a.beta, base, n);
        RawVec<VB> v[U][NI];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int k = 0; k < U; ++k)
                v[k][i] = buf_load<VB, kStream>(src.r[i], static_cast<uint32_t>(tid + k * BLOCK) * VB);
#pragma unroll
        for (int kb = 0; kb < U; kb += GP) {
            RawVec<VB> g[GP], b[GP];
#pragma unroll
            for (int j = 0; j < GP; ++j) {
                const uint32_t off = static_cast<uint32_t>(tid + (kb + j) * BLOCK) * VB;
                if constexpr (Op::kParams >= 1)
                    g[j] = buf_load<VB, kKeep>(gam, off);
                if constexpr (Op::kParams >= 2)
                    b[j] = buf_load<VB, kKeep>(bet, off);
            }
#pragma unroll
            for (int j = 0; j < GP; ++j) {
                const uint32_t ooff = static_cast<uint32_t>(tid + (kb + j) * BLOCK) * VBO;
                buf_store<VBO, kStreamStore>(apply_vec<OP, T, VB, true>(v[kb + j], g[j], b[j], c), dst, ooff);
            }
        }
    }
}

}  // namespace credit
