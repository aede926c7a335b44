// The reduction-reuse operators as (statistic, merge, output) triples.
//
// CREDIT paper, Sec. III-B, Eq. 1: per-row statistics r are reduced from
// per-element contributions, then an elementwise h(x_i, r) writes the output.
// Eq. 2: a row split into disjoint pieces reduces each piece to a partial and
// combines the partials.  Here every level of the hierarchy (wave, workgroup,
// the P workgroups of a split row) produces a partial of the same form and
// combines partials with the same rule, in a fixed order, so that every thread
// that finishes a row holds bit-identical statistics.
//
// Partials:
//   softmax   (m, s): m = max x, s = sum exp(x - m).   Two stages of Eq. 1
//             collapsed into one mergeable pair: (m_a,s_a)+(m_b,s_b) =
//             (m, s_a e^(m_a-m) + s_b e^(m_b-m)), m = max(m_a, m_b).
//   LayerNorm (n, mean, M2): count, mean and sum of squared deviations; the
//             two stages (mean, then variance) collapse into one partial and
//             are combined by the Chan-Golub-LeVeque pairwise rule.
//   RMSNorm   (ss): sum of squares; combined by addition.
// and for three further workloads of the paper's evaluation (Sec. IV-A):
//   softmax-logits backward (m, s, u): u = sum dy exp(x - m) rides along with
//             the softmax pair and is rescaled with s; dx = p (dy - u/s).
//   LayerNorm backward (n, mean, M2, a, b): with g = gamma dy, a = sum g and
//             b = sum g (x - mean) around the partial's own mean; b is
//             re-centred on the merged mean, b + a (mean_part - mean).
//   int8 quantization (amax): max |x|; combined by max.
//
// Interface of OpTraits<OP> (what the kernels call):
//   kQ       scalars per partial (exchanged between split workgroups)
//   kIn      row inputs held per element: 1 (x) or 2 (x, dy)
//   kParams  per-column parameter vectors (gamma, beta)
//   kParamsInReduce  the parameters enter the statistics (LayerNorm backward)
//            rather than only the output; `prepare` folds them into the
//            held tile before the reduction
//   kRowOut  kRowWords fp32 values per row are written besides the row, by
//            row_value(c, i): the quantization scale (always), LayerNorm
//            backward's mean and rstd (when the caller passes row_out)
//   Out<T>   storage type of the output row
//   wave_partial, merge, finalize, apply            held rows (paths 1, 2)
//   stream_init, stream_update, wave_from_thread,
//   finalize_stream, apply_stream                   streamed rows (path 3)
#pragma once

#include <float.h>

#include "common.hpp"

namespace credit {

enum OpKind { kSoftmax = 0, kLayerNorm = 1, kRmsNorm = 2, kSoftmaxBwd = 3, kLayerNormBwd = 4, kQuantInt8 = 5 };

// A partial of Q scalars.  The storage holds at least three (the unused ones
// stay zero and are never exchanged): with a one-scalar partial the compiler
// allocated up to 10 more VGPRs in the split kernel than with three.
template <int Q>
struct Part {
    float v[Q < 3 ? 3 : Q];
};

// Coefficients of the output function h, their meaning given per operator.
// k is the same in every thread of a row (bar the softmax family's k0, see
// vec_coef); f holds per-thread scales of the vector groups of a held tile.
struct Coef {
    float k[4];
    float f[4];
};

// Per-thread state that a held tile's partial leaves for the output: the
// softmax family keeps the maximum of each group of the thread's vectors
// (ref_groups of them), to which the fp32 tile's exponentials are relative.
struct Local {
    static constexpr bool kPartial = false;
    static constexpr bool kHead = false;
    float m[4];
};

// The same, for rows that are not whole vectors (see the kernels' PART mode):
// the row's last vector holds only ntail valid elements (the rest were loaded
// as zeros from past the row's end); kpart is its index among this thread's
// vectors, -1 when the thread does not hold it.
struct LocalPart : Local {
    static constexpr bool kPartial = true;
    int kpart = -1;
    int ntail = 0;
};

// The same, for rows held from the 64-byte boundary at or below their first
// byte (the kernels' SHIFT mode): the thread's vector 0 begins with `hcount`
// elements of the previous row (nonzero only in the few threads that hold the
// row's first vectors), and the last vector's ntail valid elements count from
// the start of the held span.
struct LocalShift : LocalPart {
    static constexpr bool kHead = true;
    int hcount = 0;
};

// Whether element e of the thread's vector k is part of the row (only the
// partial last vector of a PART or SHIFT row, and a SHIFT row's first
// vectors, have elements that are not).
template <class L>
__device__ __forceinline__ bool elem_in_row(const L &loc, int k, int e)
{
    if constexpr (L::kHead)
        return (k != loc.kpart || e < loc.ntail) && (k != 0 || e >= loc.hcount);
    else if constexpr (L::kPartial)
        return k != loc.kpart || e < loc.ntail;
    else
        return true;
}

// Whether a reduction must test element e of vector k before using it:
// PART rows mask their partial last vector element by element; a SHIFT row's
// elements outside the row are overwritten with the reduction's neutral value
// instead (fill_outside), so its reductions test nothing.
template <class L>
__device__ __forceinline__ bool counts(const L &loc, int k, int e)
{
    if constexpr (L::kHead)
        return true;
    else
        return elem_in_row(loc, k, e);
}

// Element e of a raw vector set to v (bf16: its upper 16 bits, which is exact
// for the values used here: -inf and 0).
template <class T, int VB>
__device__ __forceinline__ void set_elem(RawVec<VB> &r, int e, float v)
{
    if constexpr (StorageTraits<T>::kBytes == 4) {
        set_word<VB>(r, e, __float_as_uint(v));
    } else {
        const uint32_t b = __float_as_uint(v) >> 16;
        const uint32_t w = word<VB>(r, e >> 1);
        set_word<VB>(r, e >> 1, (e & 1) ? ((w & 0xffffu) | (b << 16)) : ((w & 0xffff0000u) | b));
    }
}

// SHIFT rows: vector k's elements outside the row (the thread's vector 0 when
// it starts before the row, its vector kpart when the row ends inside it)
// replaced by `fill`.  Called right before the vector's first use, inside a
// branch that only the lanes holding such a vector take, so the reductions
// pay one test per vector instead of per element.  Other rows: nothing.
template <class T, int VB, class L>
__device__ __forceinline__ void fill_outside(RawVec<VB> &v, const L &loc, int k, float fill)
{
    if constexpr (L::kHead) {
        constexpr int E = VB / StorageTraits<T>::kBytes;
        if ((k == 0 && loc.hcount > 0) || k == loc.kpart) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (!elem_in_row(loc, k, e))
                    set_elem<T, VB>(v, e, fill);
        }
    }
}

// Vector groups of a held tile of IT vectors reduced one after another (see
// softmax_groups).
template <int IT>
constexpr int ref_groups()
{
    return IT < 4 ? IT : 4;
}

// A register tile: IT vectors of VB bytes per thread.  Vector k of a thread at
// position `pos` in a group of G threads is vector (first + pos + k*G) of the
// row; `kvalid` of them (a prefix in k) lie inside the row or slice.
template <class T, int VB, int IT>
struct Tile {
    static constexpr int kEpv = VB / StorageTraits<T>::kBytes;  // elements per vector
    RawVec<VB> v[IT];
};

// Opaque no-op on every register of the tile.  Placed between passes over a
// held tile so the compiler re-derives fp32 values from the packed storage in
// each pass instead of keeping an unpacked copy live (which would double the
// VGPRs a bf16 row needs).
template <class T, int VB, int IT>
__device__ __forceinline__ void fence_tile(Tile<T, VB, IT> &t)
{
#pragma unroll
    for (int k = 0; k < IT; ++k)
        asm volatile("" : "+v"(t.v[k].w));
}

template <class T>
constexpr bool is_f32()
{
    return StorageTraits<T>::kBytes == 4;
}

template <OpKind OP>
struct OpTraits;

// Softmax exponential for the storage type: ~2 ulp for fp32 outputs, the bare
// hardware exp2 where the result is rounded to bf16.
template <class T>
__device__ __forceinline__ float exp_for(float d)
{
    if constexpr (is_f32<T>())
        return exp_acc(d);
    else
        return exp_fast(d);
}

// Opaque no-op on one vector of a tile (see fence_tile).
template <int VB>
__device__ __forceinline__ void fence_vec(RawVec<VB> &v)
{
    asm volatile("" : "+v"(v.w));
}

// The exponential sums of a held softmax-family tile: x in t[0] and, with DY,
// dy in t[1]; fp32 tiles are overwritten with the exponentials, so the output
// needs no second exponential.  Returns the wave partial (m, s[, u]).
//
// Grouped (fp32 softmax): the thread's IT vectors form ref_groups<IT>() groups
// of consecutive vectors; each group takes its own maximum gm and sums
// e = exp(x - gm), so its work starts as soon as its own loads have landed
// instead of after the whole tile and a wave-wide maximum, and each group is
// rescaled to the wave maximum at the end.  Ungrouped (the others, where
// grouping measured 1-2% slower on MI355X): every exponential is taken
// against the wave maximum.  Either way loc.m holds the reference maximum of
// each group's exponentials (the wave maximum for all of them, ungrouped).
template <bool DY, class T, int VB, int IT, int NI, class L>
__device__ __forceinline__ Part<DY ? 3 : 2> softmax_groups(Tile<T, VB, IT> (&t)[NI], int kvalid, L &loc)
{
    constexpr int E = Tile<T, VB, IT>::kEpv;
    constexpr bool kGrouped = !DY && is_f32<T>();
    constexpr int NG = kGrouped ? ref_groups<IT>() : 1;
    constexpr int GS = IT / NG;
    float sg[NG], ug[NG], gref[NG];
    float mw = -INFINITY;
    if constexpr (!kGrouped) {
        float mt = -INFINITY;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid) {
                fill_outside<T, VB>(t[0].v[k], loc, k, -INFINITY);
                if constexpr (DY)
                    fill_outside<T, VB>(t[1].v[k], loc, k, 0.0f);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    mt = fmaxf(mt, counts(loc, k, e) ? elem<T, VB>(t[0].v[k], e) : -INFINITY);
            }
        mw = wave_max(mt);
        fence_tile(t[0]);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float gm = mw;
        if constexpr (kGrouped) {
            gm = -INFINITY;
#pragma unroll
            for (int j = 0; j < GS; ++j)
                if (g * GS + j < kvalid) {
                    fill_outside<T, VB>(t[0].v[g * GS + j], loc, g * GS + j, -INFINITY);
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        gm = fmaxf(gm, counts(loc, g * GS + j, e) ? elem<T, VB>(t[0].v[g * GS + j], e)
                                                                  : -INFINITY);
                }
#pragma unroll
            for (int j = 0; j < GS; ++j)
                fence_vec(t[0].v[g * GS + j]);
        }
        // the reference of the exponentials: a group (or wave) whose valid
        // elements were all filled with -inf has gm = -inf, whose exp(x - gm)
        // would be NaN; any finite reference gives its elements exp = 0
        const float gx = gm == -INFINITY ? 0.0f : gm;
        float sv = 0.0f, uv = 0.0f;
#pragma unroll
        for (int j = 0; j < GS; ++j) {
            const int k = g * GS + j;
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float ex = counts(loc, k, e) ? exp_for<T>(elem<T, VB>(t[0].v[k], e) - gx) : 0.0f;
                    if constexpr (is_f32<T>())
                        set_word<VB>(t[0].v[k], e, __float_as_uint(ex));
                    sv += ex;
                    // (a SHIFT row's dy outside the row, the neighbouring
                    // rows' data, was filled with 0 and adds nothing to u)
                    if constexpr (DY)
                        uv = __builtin_fmaf(ex, elem<T, VB>(t[1].v[k], e), uv);
                }
        }
        gref[g] = gm;
        sg[g] = sv;
        ug[g] = uv;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
        loc.m[g] = kGrouped ? (g < NG ? gref[g] : -INFINITY) : mw;
    float st = sg[0], ut = ug[0];
    if constexpr (kGrouped) {
        float mt = gref[0];
#pragma unroll
        for (int g = 1; g < NG; ++g)
            mt = fmaxf(mt, gref[g]);
        mw = wave_max(mt);
        // a group with no valid vector has s = 0 (a valid one has s >= 1)
        st = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g)
            if (sg[g] != 0.0f)
                st += sg[g] * exp_acc(gref[g] - mw);
    }
    if constexpr (DY)
        return Part<3>{{mw, wave_sum(st), wave_sum(ut)}};
    else
        return Part<2>{{mw, wave_sum(st)}};
}

// fp32 output scales of the groups: e^(gm - m) / s, zero for a group with no
// valid vector.
__device__ __forceinline__ void group_scales(Coef &c, const Local &loc, float m, float inv_s)
{
#pragma unroll
    for (int g = 0; g < 4; ++g)
        c.f[g] = loc.m[g] != -INFINITY ? exp_acc(loc.m[g] - m) * inv_s : 0.0f;
}

// ---------------------------------------------------------------------------
// softmax.  Coef: k0 = 1 / s (held fp32 tiles: per vector, the group scale
// e^(gm - m) / s, because the tile holds e^(x - gm)), k1 = row max m.
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kSoftmax> {
    static constexpr int kQ = 2;
    static constexpr int kIn = 1;
    static constexpr int kParams = 0;
    static constexpr bool kParamsInReduce = false;
    static constexpr bool kRowOut = false;
    template <class T> using Out = T;
    using Partial = Part<kQ>;

    template <class T, int VB, int IT, class L>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> (&t)[kIn], int kvalid, L &loc)
    {
        return softmax_groups<false, T, VB, IT>(t, kvalid, loc);
    }

    // Combine partials p[0..n-1] (n <= N) in index order.
    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n)
                m = fmaxf(m, p[i].v[0]);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n && p[i].v[1] != 0.0f)
                s += p[i].v[1] * exp_acc(p[i].v[0] - m);
        return Partial{{m, s}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Local &loc, int64_t, float)
    {
        const float inv_s = 1.0f / row.v[1];
        Coef c{{inv_s, row.v[0], 0.0f, 0.0f}};
        if constexpr (is_f32<T>())
            group_scales(c, loc, row.v[0], inv_s);
        return c;
    }

    template <class T>
    __device__ __forceinline__ static float apply(const float (&in)[kIn], const Coef &c, float, float)
    {
        if constexpr (is_f32<T>())
            return in[0] * c.k[0];  // in[0] holds exp(x - gm), k0 the group's scale
        else
            return exp_fast(in[0] - c.k[1]) * c.k[0];
    }

    // ---- streaming form (the reread path): the row is not held, so each
    // thread keeps a running partial over the chunks it streams, and the
    // output pass recomputes the exponential from the reread input.
    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[kIn][U],
                                                         const RawVec<VB> (&)[U], int kvalid)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
        float cm = -INFINITY;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    cm = fmaxf(cm, elem<T, VB>(v[0][k], e));
        if (cm > r.v[0]) {
            r.v[1] = r.v[1] != 0.0f ? r.v[1] * exp_acc(r.v[0] - cm) : 0.0f;
            r.v[0] = cm;
        }
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    s += exp_for<T>(elem<T, VB>(v[0][k], e) - r.v[0]);
        r.v[1] += s;
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{{-INFINITY, 0.0f}}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r)
    {
        const float mw = wave_max(r.v[0]);
        const float s = r.v[1] != 0.0f ? r.v[1] * exp_acc(r.v[0] - mw) : 0.0f;
        return Partial{{mw, wave_sum(s)}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t, float)
    {
        return Coef{{1.0f / row.v[1], row.v[0], 0.0f, 0.0f}};
    }

    template <class T>
    __device__ __forceinline__ static float apply_stream(const float (&in)[kIn], const Coef &c, float, float)
    {
        return exp_for<T>(in[0] - c.k[1]) * c.k[0];
    }
};

// ---------------------------------------------------------------------------
// LayerNorm.  Coef: k0 = mean, k1 = 1/sqrt(var + eps).
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kLayerNorm> {
    static constexpr int kQ = 3;  // (n, mean, M2); n travels so empty slices merge correctly
    static constexpr int kIn = 1;
    static constexpr int kParams = 2;
    static constexpr bool kParamsInReduce = false;
    static constexpr bool kRowOut = false;
    template <class T> using Out = T;
    using Partial = Part<kQ>;

    template <class T, int VB, int IT, class L>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> (&tt)[kIn], int kvalid, L &loc)
    {
        Tile<T, VB, IT> &t = tt[0];
        constexpr int E = Tile<T, VB, IT>::kEpv;
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid) {
                fill_outside<T, VB>(t.v[k], loc, k, 0.0f);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    sum += elem<T, VB>(t.v[k], e);
            }
        int nvalid = kvalid * E;
        if constexpr (L::kPartial)
            if (loc.kpart >= 0 && loc.kpart < kvalid)
                nvalid -= E - loc.ntail;  // the partial vector's zeros are no elements
        if constexpr (L::kHead)
            if (kvalid > 0)
                nvalid -= loc.hcount;  // nor are a shifted row's leading elements
        const float nw = wave_sum(static_cast<float>(nvalid));
        const float sw = wave_sum(sum);
        const float mean = nw > 0.0f ? sw / nw : 0.0f;
        fence_tile(t);
        float m2 = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float d = elem_in_row(loc, k, e) ? elem<T, VB>(t.v[k], e) - mean : 0.0f;
                    m2 = __builtin_fmaf(d, d, m2);
                }
        return Partial{{nw, mean, wave_sum(m2)}};
    }

    // mean = sum n_i mean_i / n;  M2 = sum (M2_i + n_i (mean_i - mean)^2).
    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float nt = 0.0f, acc = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) {
                nt += p[i].v[0];
                acc = __builtin_fmaf(p[i].v[0], p[i].v[1], acc);
            }
        const float mean = nt > 0.0f ? acc / nt : 0.0f;
        float m2 = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) {
                float d = p[i].v[1] - mean;
                m2 += p[i].v[2] + p[i].v[0] * d * d;
            }
        return Partial{{nt, mean, m2}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Local &, int64_t cols, float eps)
    {
        const float var = row.v[2] / static_cast<float>(cols);
        return Coef{{row.v[1], 1.0f / sqrtf(var + eps), 0.0f, 0.0f}};
    }

    template <class T>
    __device__ __forceinline__ static float apply(const float (&in)[kIn], const Coef &c, float g, float b)
    {
        return __builtin_fmaf((in[0] - c.k[0]) * c.k[1], g, b);
    }

    // ---- streaming form: each chunk is reduced two-pass in registers to
    // (n_c, mean_c, M2_c) and folded into the running partial pairwise.
    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[kIn][U],
                                                         const RawVec<VB> (&)[U], int kvalid)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
        if (kvalid <= 0)
            return;
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    sum += elem<T, VB>(v[0][k], e);
        const float nc = static_cast<float>(kvalid * E);
        const float mc = sum / nc;
        float m2c = 0.0f;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float d = elem<T, VB>(v[0][k], e) - mc;
                    m2c = __builtin_fmaf(d, d, m2c);
                }
        const float n2 = r.v[0] + nc;
        const float d = mc - r.v[1];
        r.v[1] = __builtin_fmaf(d, nc / n2, r.v[1]);
        r.v[2] += m2c + d * d * (r.v[0] * nc / n2);
        r.v[0] = n2;
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{{0.0f, 0.0f, 0.0f}}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r)
    {
        const float nw = wave_sum(r.v[0]);
        const float mean = nw > 0.0f ? wave_sum(r.v[0] * r.v[1]) / nw : 0.0f;
        const float d = r.v[1] - mean;
        return Partial{{nw, mean, wave_sum(r.v[2] + r.v[0] * d * d)}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t cols, float eps)
    {
        return finalize<T>(row, Local{}, cols, eps);
    }

    template <class T>
    __device__ __forceinline__ static float apply_stream(const float (&in)[kIn], const Coef &c, float g, float b)
    {
        return apply<T>(in, c, g, b);
    }
};

// ---------------------------------------------------------------------------
// RMSNorm.  Coef: k0 = 1/sqrt(mean(x^2) + eps).
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kRmsNorm> {
    static constexpr int kQ = 1;
    static constexpr int kIn = 1;
    static constexpr int kParams = 1;
    static constexpr bool kParamsInReduce = false;
    static constexpr bool kRowOut = false;
    template <class T> using Out = T;
    using Partial = Part<kQ>;

    template <class T, int VB, int IT, class L>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> (&tt)[kIn], int kvalid, L &loc)
    {
        Tile<T, VB, IT> &t = tt[0];
        constexpr int E = Tile<T, VB, IT>::kEpv;
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid) {
                fill_outside<T, VB>(t.v[k], loc, k, 0.0f);  // (a PART row's tail loaded as zeros)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float x = elem<T, VB>(t.v[k], e);
                    ss = __builtin_fmaf(x, x, ss);
                }
            }
        return Partial{{wave_sum(ss)}};
    }

    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n)
                ss += p[i].v[0];
        return Partial{{ss}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Local &, int64_t cols, float eps)
    {
        return Coef{{1.0f / sqrtf(row.v[0] / static_cast<float>(cols) + eps), 0.0f, 0.0f, 0.0f}};
    }

    template <class T>
    __device__ __forceinline__ static float apply(const float (&in)[kIn], const Coef &c, float g, float)
    {
        return in[0] * c.k[0] * g;
    }

    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[kIn][U],
                                                         const RawVec<VB> (&)[U], int kvalid)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float x = elem<T, VB>(v[0][k], e);
                    r.v[0] = __builtin_fmaf(x, x, r.v[0]);
                }
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{{0.0f}}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r)
    {
        return Partial{{wave_sum(r.v[0])}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t cols, float eps)
    {
        return finalize<T>(row, Local{}, cols, eps);
    }

    template <class T>
    __device__ __forceinline__ static float apply_stream(const float (&in)[kIn], const Coef &c, float g, float b)
    {
        return apply<T>(in, c, g, b);
    }
};

// ---------------------------------------------------------------------------
// Softmax-logits backward: inputs x (logits) and dy; dx = p (dy - sum dy p)
// with p = softmax(x) recomputed from x.  Coef: k0 = 1 / s (held fp32 tiles:
// e^(m_wave - m) / s, the tile holding e^(x - m_wave)),
// k1 = u / s (the dot product of dy with p), k2 = row max m.
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kSoftmaxBwd> {
    static constexpr int kQ = 3;  // (m, s, u)
    static constexpr int kIn = 2;
    static constexpr int kParams = 0;
    static constexpr bool kParamsInReduce = false;
    static constexpr bool kRowOut = false;
    template <class T> using Out = T;
    using Partial = Part<kQ>;

    template <class T, int VB, int IT, class L>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> (&t)[kIn], int kvalid, L &loc)
    {
        return softmax_groups<true, T, VB, IT>(t, kvalid, loc);
    }

    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n)
                m = fmaxf(m, p[i].v[0]);
        float s = 0.0f, u = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n && p[i].v[1] != 0.0f) {
                const float f = exp_acc(p[i].v[0] - m);
                s += p[i].v[1] * f;
                u += p[i].v[2] * f;
            }
        return Partial{{m, s, u}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Local &loc, int64_t, float)
    {
        const float inv_s = 1.0f / row.v[1];
        Coef c{{inv_s, row.v[2] / row.v[1], row.v[0], 0.0f}};
        if constexpr (is_f32<T>())
            group_scales(c, loc, row.v[0], inv_s);
        return c;
    }

    template <class T>
    __device__ __forceinline__ static float apply(const float (&in)[kIn], const Coef &c, float, float)
    {
        float p;
        if constexpr (is_f32<T>())
            p = in[0] * c.k[0];  // in[0] holds exp(x - gm), k0 the group's scale
        else
            p = exp_fast(in[0] - c.k[2]) * c.k[0];
        return p * (in[1] - c.k[1]);
    }

    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[kIn][U],
                                                         const RawVec<VB> (&)[U], int kvalid)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
        float cm = -INFINITY;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    cm = fmaxf(cm, elem<T, VB>(v[0][k], e));
        if (cm > r.v[0]) {
            const float f = r.v[1] != 0.0f ? exp_acc(r.v[0] - cm) : 0.0f;
            r.v[1] *= f;
            r.v[2] *= f;
            r.v[0] = cm;
        }
        float s = 0.0f, u = 0.0f;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float ex = exp_for<T>(elem<T, VB>(v[0][k], e) - r.v[0]);
                    s += ex;
                    u = __builtin_fmaf(ex, elem<T, VB>(v[1][k], e), u);
                }
        r.v[1] += s;
        r.v[2] += u;
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{{-INFINITY, 0.0f, 0.0f}}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r)
    {
        const float mw = wave_max(r.v[0]);
        const float f = r.v[1] != 0.0f ? exp_acc(r.v[0] - mw) : 0.0f;
        return Partial{{mw, wave_sum(r.v[1] * f), wave_sum(r.v[2] * f)}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t, float)
    {
        return Coef{{1.0f / row.v[1], row.v[2] / row.v[1], row.v[0], 0.0f}};
    }

    template <class T>
    __device__ __forceinline__ static float apply_stream(const float (&in)[kIn], const Coef &c, float, float)
    {
        return exp_for<T>(in[0] - c.k[2]) * c.k[0] * (in[1] - c.k[1]);
    }
};

// ---------------------------------------------------------------------------
// LayerNorm backward, row part: inputs x and dy, parameter gamma; with
// g = gamma dy, rstd = 1/sqrt(var + eps) and xhat = (x - mean) rstd,
// dx = rstd (g - mean(g) - xhat mean(g xhat)).  fp32 storage only: the held
// dy tile is overwritten with g by `prepare`.  Coef: k0 = mean, k1 = rstd,
// k2 = mean(g), k3 = rstd^2 sum(g (x - mean)) / N.
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kLayerNormBwd> {
    static constexpr int kQ = 5;  // (n, mean, M2, a, b)
    static constexpr int kIn = 2;
    static constexpr int kParams = 1;
    static constexpr bool kParamsInReduce = true;
    static constexpr bool kRowOut = true;  // mean and rstd, when row_out is given
    static constexpr int kRowWords = 2;
    template <class T> using Out = T;
    using Partial = Part<kQ>;

    // Vector k of the dy tile becomes g = gamma dy (fp32 bits), `gv` holding
    // the gamma vector of the same columns.
    template <class T, int VB, int IT>
    __device__ __forceinline__ static void prepare(Tile<T, VB, IT> (&t)[kIn], int k, const RawVec<VB> &gv)
    {
        static_assert(is_f32<T>(), "LayerNorm backward holds g = gamma * dy in fp32");
        constexpr int E = Tile<T, VB, IT>::kEpv;
#pragma unroll
        for (int e = 0; e < E; ++e)
            set_word<VB>(t[1].v[k], e, __float_as_uint(elem<T, VB>(gv, e) * elem<T, VB>(t[1].v[k], e)));
    }

    // (A PART row's missing elements load as zeros in x and g, and a SHIFT
    // row's elements outside the row are overwritten with zeros: neutral in
    // the sums and in b, masked out of the count and of M2.)
    template <class T, int VB, int IT, class L>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> (&t)[kIn], int kvalid, L &loc)
    {
        constexpr int E = Tile<T, VB, IT>::kEpv;
        float sx = 0.0f, sg = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid) {
                fill_outside<T, VB>(t[0].v[k], loc, k, 0.0f);
                fill_outside<T, VB>(t[1].v[k], loc, k, 0.0f);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    sx += elem<T, VB>(t[0].v[k], e);
                    sg += elem<T, VB>(t[1].v[k], e);
                }
            }
        int nvalid = kvalid * E;
        if constexpr (L::kPartial)
            if (loc.kpart >= 0 && loc.kpart < kvalid)
                nvalid -= E - loc.ntail;
        if constexpr (L::kHead)
            if (kvalid > 0)
                nvalid -= loc.hcount;  // a shifted row's leading elements
        const float nw = wave_sum(static_cast<float>(nvalid));
        const float sw = wave_sum(sx);
        const float mean = nw > 0.0f ? sw / nw : 0.0f;
        fence_tile(t[0]);
        fence_tile(t[1]);
        float m2 = 0.0f, b = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = elem_in_row(loc, k, e) ? elem<T, VB>(t[0].v[k], e) - mean : 0.0f;
                    m2 = __builtin_fmaf(d, d, m2);
                    b = __builtin_fmaf(elem<T, VB>(t[1].v[k], e), d, b);
                }
        return Partial{{nw, mean, wave_sum(m2), wave_sum(sg), wave_sum(b)}};
    }

    // n, mean, M2 as LayerNorm; a adds; b_i is re-centred on the merged mean.
    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float nt = 0.0f, acc = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) {
                nt += p[i].v[0];
                acc = __builtin_fmaf(p[i].v[0], p[i].v[1], acc);
            }
        const float mean = nt > 0.0f ? acc / nt : 0.0f;
        float m2 = 0.0f, a = 0.0f, b = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) {
                const float d = p[i].v[1] - mean;
                m2 += p[i].v[2] + p[i].v[0] * d * d;
                a += p[i].v[3];
                b += __builtin_fmaf(p[i].v[3], d, p[i].v[4]);
            }
        return Partial{{nt, mean, m2, a, b}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Local &, int64_t cols, float eps)
    {
        const float inv_n = 1.0f / static_cast<float>(cols);
        const float rstd = 1.0f / sqrtf(row.v[2] * inv_n + eps);
        return Coef{{row.v[1], rstd, row.v[3] * inv_n, rstd * rstd * (row.v[4] * inv_n)}};
    }

    // the row's mean and rstd, for the parameter part
    __device__ __forceinline__ static float row_value(const Coef &c, int i) { return i == 0 ? c.k[0] : c.k[1]; }

    // in[0] = x, in[1] = g
    template <class T>
    __device__ __forceinline__ static float apply(const float (&in)[kIn], const Coef &c, float, float)
    {
        return c.k[1] * __builtin_fmaf(-(in[0] - c.k[0]), c.k[3], in[1] - c.k[2]);
    }

    // ---- streaming form: each chunk reduced two-pass to (n_c, mean_c, M2_c,
    // a_c, b_c) and folded into the running partial by the merge rule.
    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[kIn][U],
                                                         const RawVec<VB> (&gam)[U], int kvalid)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
        if (kvalid <= 0)
            return;
        float sx = 0.0f, sg = 0.0f;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    sx += elem<T, VB>(v[0][k], e);
                    sg = __builtin_fmaf(elem<T, VB>(gam[k], e), elem<T, VB>(v[1][k], e), sg);
                }
        const float nc = static_cast<float>(kvalid * E);
        const float mc = sx / nc;
        float m2c = 0.0f, bc = 0.0f;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = elem<T, VB>(v[0][k], e) - mc;
                    m2c = __builtin_fmaf(d, d, m2c);
                    bc = __builtin_fmaf(elem<T, VB>(gam[k], e) * elem<T, VB>(v[1][k], e), d, bc);
                }
        const float n2 = r.v[0] + nc;
        const float d = mc - r.v[1];
        const float mean2 = __builtin_fmaf(d, nc / n2, r.v[1]);
        r.v[2] += m2c + d * d * (r.v[0] * nc / n2);
        r.v[4] = __builtin_fmaf(r.v[3], r.v[1] - mean2, r.v[4]) + __builtin_fmaf(sg, mc - mean2, bc);
        r.v[3] += sg;
        r.v[1] = mean2;
        r.v[0] = n2;
    }

    // The same over held vectors kb .. kb + U - 1 of a SHIFT row (a raw bf16
    // tile): the elements outside the row (the previous row's in front, the
    // next row's in the last word) are zeroed in x and dy first, left out of
    // the count and of the centred squares; a chunk with no element of the
    // row adds nothing.
    template <class T, int VB, int U, class L>
    __device__ __forceinline__ static void stream_update_masked(Partial &r, RawVec<VB> (&v)[kIn][U],
                                                                const RawVec<VB> (&gam)[U], int kvalid, const L &loc,
                                                                int kb)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
        if (kvalid <= 0)
            return;
        int nout = 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < kvalid) {
                fill_outside<T, VB>(v[0][u], loc, kb + u, 0.0f);
                fill_outside<T, VB>(v[1][u], loc, kb + u, 0.0f);
                if (kb + u == 0)
                    nout += loc.hcount;
                if (kb + u == loc.kpart)
                    nout += E - loc.ntail;
            }
        const int nin = kvalid * E - nout;
        if (nin <= 0)
            return;
        float sx = 0.0f, sg = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    sx += elem<T, VB>(v[0][u], e);
                    sg = __builtin_fmaf(elem<T, VB>(gam[u], e), elem<T, VB>(v[1][u], e), sg);
                }
        const float nc = static_cast<float>(nin);
        const float mc = sx / nc;
        float m2c = 0.0f, bc = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = elem_in_row(loc, kb + u, e) ? elem<T, VB>(v[0][u], e) - mc : 0.0f;
                    m2c = __builtin_fmaf(d, d, m2c);
                    bc = __builtin_fmaf(elem<T, VB>(gam[u], e) * elem<T, VB>(v[1][u], e), d, bc);
                }
        const float n2 = r.v[0] + nc;
        const float d = mc - r.v[1];
        const float mean2 = __builtin_fmaf(d, nc / n2, r.v[1]);
        r.v[2] += m2c + d * d * (r.v[0] * nc / n2);
        r.v[4] = __builtin_fmaf(r.v[3], r.v[1] - mean2, r.v[4]) + __builtin_fmaf(sg, mc - mean2, bc);
        r.v[3] += sg;
        r.v[1] = mean2;
        r.v[0] = n2;
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{{0.0f, 0.0f, 0.0f, 0.0f, 0.0f}}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r)
    {
        const float nw = wave_sum(r.v[0]);
        const float mean = nw > 0.0f ? wave_sum(r.v[0] * r.v[1]) / nw : 0.0f;
        const float d = r.v[1] - mean;
        return Partial{{nw, mean, wave_sum(r.v[2] + r.v[0] * d * d), wave_sum(r.v[3]),
                        wave_sum(__builtin_fmaf(r.v[3], d, r.v[4]))}};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t cols, float eps)
    {
        return finalize<T>(row, Local{}, cols, eps);
    }

    // in[0] = x, in[1] = dy (not yet multiplied by gamma)
    template <class T>
    __device__ __forceinline__ static float apply_stream(const float (&in)[kIn], const Coef &c, float g, float)
    {
        const float held[kIn] = {in[0], g * in[1]};
        return apply<T>(held, c, g, 0.0f);
    }
};

// ---------------------------------------------------------------------------
// Row-wise symmetric int8 quantization: a = max |x|, inv = min(127 / a,
// FLT_MAX) (0 for a = 0), q = clamp(rint(x * inv), -127, 127), and the row's
// scale a / 127 written to the per-row output.  Each / and * is one correctly
// rounded fp32 operation, so the codes are fixed by the inputs.
// Coef: k0 = inv, k1 = scale.
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kQuantInt8> {
    static constexpr int kQ = 1;
    static constexpr int kIn = 1;
    static constexpr int kParams = 0;
    static constexpr bool kParamsInReduce = false;
    static constexpr bool kRowOut = true;
    template <class T> using Out = i8_t;
    using Partial = Part<kQ>;

    template <class T, int VB, int IT, class L>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> (&t)[kIn], int kvalid, L &loc)
    {
        constexpr int E = Tile<T, VB, IT>::kEpv;
        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid) {
                fill_outside<T, VB>(t[0].v[k], loc, k, 0.0f);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    a = fmaxf(a, counts(loc, k, e) ? fabsf(elem<T, VB>(t[0].v[k], e)) : 0.0f);
            }
        return Partial{{wave_max(a)}};
    }

    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n)
                a = fmaxf(a, p[i].v[0]);
        return Partial{{a}};
    }

    // The merge of a split row's exchanged partials: as merge, but a NaN
    // partial (an exchange word a workgroup gave up waiting for) makes the
    // absmax NaN, which fmaxf alone would drop.
    template <int N>
    __device__ __forceinline__ static Partial merge_exchanged(const Partial (&p)[N], int n)
    {
        bool nan = false;
#pragma unroll
        for (int i = 0; i < N; ++i)
            nan |= i < n && p[i].v[0] != p[i].v[0];
        return nan ? Partial{{__builtin_nanf("")}} : merge<N>(p, n);
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Local &, int64_t, float)
    {
        const float a = row.v[0];
        const float inv = a > 0.0f ? fminf(127.0f / a, FLT_MAX) : 0.0f;
        return Coef{{inv, a / 127.0f, 0.0f, 0.0f}};
    }

    template <class T>
    __device__ __forceinline__ static float apply(const float (&in)[kIn], const Coef &c, float, float)
    {
        return fminf(fmaxf(__builtin_rintf(in[0] * c.k[0]), -127.0f), 127.0f);
    }

    static constexpr int kRowWords = 1;
    __device__ __forceinline__ static float row_value(const Coef &c, int) { return c.k[1]; }

    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[kIn][U],
                                                         const RawVec<VB> (&)[U], int kvalid)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    r.v[0] = fmaxf(r.v[0], fabsf(elem<T, VB>(v[0][k], e)));
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{{0.0f}}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r) { return Partial{{wave_max(r.v[0])}}; }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t cols, float eps)
    {
        return finalize<T>(row, Local{}, cols, eps);
    }

    template <class T>
    __device__ __forceinline__ static float apply_stream(const float (&in)[kIn], const Coef &c, float g, float b)
    {
        return apply<T>(in, c, g, b);
    }
};

// The merge of the P partials a split row's workgroups exchanged.  For every
// operator but the quantizer, merge itself carries a NaN partial (left by an
// exchange wait that gave up) into the statistics and so into every
// output: each folds the partials by sums, and softmax's maximum, which
// fmaxf computes past a NaN, only scales sums that the NaN already reached.
template <OpKind OP>
struct ExchangeMerge {
    template <int N>
    __device__ __forceinline__ static typename OpTraits<OP>::Partial apply(
        const typename OpTraits<OP>::Partial (&p)[N], int n)
    {
        if constexpr (OP == kQuantInt8)
            return OpTraits<OP>::template merge_exchanged<N>(p, n);
        else
            return OpTraits<OP>::template merge<N>(p, n);
    }
};

// The coefficients for vector k of a held tile of IT vectors: for the fp32
// softmax family, k0 becomes the scale of the vector's group (softmax_groups).
template <OpKind OP, class T, int IT>
__device__ __forceinline__ Coef vec_coef(const Coef &c, int k)
{
    if constexpr (OP == kSoftmax && is_f32<T>()) {
        Coef r = c;
        r.k[0] = c.f[k / (IT / ref_groups<IT>())];
        return r;
    } else if constexpr (OP == kSoftmaxBwd && is_f32<T>()) {
        Coef r = c;
        r.k[0] = c.f[0];  // one reference (the wave maximum) for the whole tile
        return r;
    } else {
        return c;
    }
}

}  // namespace credit
