// The three reduction-reuse operators as (statistic, merge, output) triples.
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
#pragma once

#include "common.hpp"

namespace credit {

enum OpKind { kSoftmax = 0, kLayerNorm = 1, kRmsNorm = 2 };

struct Partial {
    float a, b, c;  // softmax: (m, s, -); LN: (n, mean, M2); RMS: (ss, -, -)
};

// Coefficients of the output function h, identical in every thread of a row.
struct Coef {
    float mean;   // LN: row mean
    float scale;  // softmax: 1/s (bf16) or e^(m_wave - m)/s (fp32); LN/RMS: 1/sqrt(var + eps)
    float m;      // softmax: row max
};

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

template <OpKind OP>
struct OpTraits;

// ---------------------------------------------------------------------------
// softmax
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kSoftmax> {
    static constexpr int kQ = 2;      // scalars exchanged per partial
    static constexpr int kParams = 0; // parameter vectors

    // Wave partial over the wave's elements.  For fp32 storage the tile is
    // overwritten with e_i = exp(x_i - m_wave) so that the output needs no
    // second exponential.
    template <class T, int VB, int IT>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> &t, int kvalid)
    {
        constexpr int E = Tile<T, VB, IT>::kEpv;
        float mt = -INFINITY;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    mt = fmaxf(mt, elem<T, VB>(t.v[k], e));
        const float mw = wave_max(mt);
        fence_tile(t);
        float st = 0.0f;
        if constexpr (StorageTraits<T>::kBytes == 4) {
#pragma unroll
            for (int k = 0; k < IT; ++k)
                if (k < kvalid)
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        float ex = exp_acc(elem<T, VB>(t.v[k], e) - mw);
                        set_word<VB>(t.v[k], e, __float_as_uint(ex));
                        st += ex;
                    }
        } else {
#pragma unroll
            for (int k = 0; k < IT; ++k)
                if (k < kvalid)
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        st += exp_fast(elem<T, VB>(t.v[k], e) - mw);
        }
        return Partial{mw, wave_sum(st), 0.0f};
    }

    // Combine partials p[0..n-1] (n <= N) in index order.
    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n)
                m = fmaxf(m, p[i].a);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n && p[i].b != 0.0f)
                s += p[i].b * exp_acc(p[i].a - m);
        return Partial{m, s, 0.0f};
    }

    // `own` is the partial whose exponentials are stored in this thread's tile.
    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Partial &own, int64_t, float)
    {
        const float inv_s = 1.0f / row.b;
        if constexpr (StorageTraits<T>::kBytes == 4)
            return Coef{0.0f, own.b != 0.0f ? exp_acc(own.a - row.a) * inv_s : 0.0f, row.a};
        else
            return Coef{0.0f, inv_s, row.a};
    }

    template <class T>
    __device__ __forceinline__ static float apply(float x, const Coef &c, float, float)
    {
        if constexpr (StorageTraits<T>::kBytes == 4)
            return x * c.scale;  // x already holds exp(x - m_wave)
        else
            return exp_fast(x - c.m) * c.scale;
    }

    // ---- streaming form (the reread path): the row is not held, so each
    // thread keeps a running partial over the chunks it streams, and the
    // output pass recomputes the exponential from the reread input.
    template <class T>
    __device__ __forceinline__ static float expf_t(float d)
    {
        if constexpr (StorageTraits<T>::kBytes == 4)
            return exp_acc(d);
        else
            return exp_fast(d);
    }

    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[U], int kvalid)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
        float cm = -INFINITY;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    cm = fmaxf(cm, elem<T, VB>(v[k], e));
        if (cm > r.a) {
            r.b = r.b != 0.0f ? r.b * exp_acc(r.a - cm) : 0.0f;
            r.a = cm;
        }
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    s += expf_t<T>(elem<T, VB>(v[k], e) - r.a);
        r.b += s;
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{-INFINITY, 0.0f, 0.0f}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r)
    {
        const float mw = wave_max(r.a);
        const float s = r.b != 0.0f ? r.b * exp_acc(r.a - mw) : 0.0f;
        return Partial{mw, wave_sum(s), 0.0f};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t, float)
    {
        return Coef{0.0f, 1.0f / row.b, row.a};
    }

    template <class T>
    __device__ __forceinline__ static float apply_stream(float x, const Coef &c, float, float)
    {
        return expf_t<T>(x - c.m) * c.scale;
    }
};

// ---------------------------------------------------------------------------
// LayerNorm
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kLayerNorm> {
    static constexpr int kQ = 3;  // (n, mean, M2); n travels so empty slices merge correctly
    static constexpr int kParams = 2;

    template <class T, int VB, int IT>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> &t, int kvalid)
    {
        constexpr int E = Tile<T, VB, IT>::kEpv;
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    sum += elem<T, VB>(t.v[k], e);
        const float nw = wave_sum(static_cast<float>(kvalid * E));
        const float sw = wave_sum(sum);
        const float mean = nw > 0.0f ? sw / nw : 0.0f;
        fence_tile(t);
        float m2 = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float d = elem<T, VB>(t.v[k], e) - mean;
                    m2 = __builtin_fmaf(d, d, m2);
                }
        return Partial{nw, mean, wave_sum(m2)};
    }

    // mean = sum n_i mean_i / n;  M2 = sum (M2_i + n_i (mean_i - mean)^2).
    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float nt = 0.0f, acc = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) {
                nt += p[i].a;
                acc = __builtin_fmaf(p[i].a, p[i].b, acc);
            }
        const float mean = nt > 0.0f ? acc / nt : 0.0f;
        float m2 = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) {
                float d = p[i].b - mean;
                m2 += p[i].c + p[i].a * d * d;
            }
        return Partial{nt, mean, m2};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Partial &, int64_t cols, float eps)
    {
        const float var = row.c / static_cast<float>(cols);
        return Coef{row.b, 1.0f / sqrtf(var + eps), 0.0f};
    }

    template <class T>
    __device__ __forceinline__ static float apply(float x, const Coef &c, float g, float b)
    {
        return __builtin_fmaf((x - c.mean) * c.scale, g, b);
    }

    // ---- streaming form: each chunk is reduced two-pass in registers to
    // (n_c, mean_c, M2_c) and folded into the running partial pairwise.
    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[U], int kvalid)
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
                    sum += elem<T, VB>(v[k], e);
        const float nc = static_cast<float>(kvalid * E);
        const float mc = sum / nc;
        float m2c = 0.0f;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float d = elem<T, VB>(v[k], e) - mc;
                    m2c = __builtin_fmaf(d, d, m2c);
                }
        const float n2 = r.a + nc;
        const float d = mc - r.b;
        r.b = __builtin_fmaf(d, nc / n2, r.b);
        r.c += m2c + d * d * (r.a * nc / n2);
        r.a = n2;
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{0.0f, 0.0f, 0.0f}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r)
    {
        const float nw = wave_sum(r.a);
        const float mean = nw > 0.0f ? wave_sum(r.a * r.b) / nw : 0.0f;
        const float d = r.b - mean;
        return Partial{nw, mean, wave_sum(r.c + r.a * d * d)};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t cols, float eps)
    {
        return finalize<T>(row, row, cols, eps);
    }

    template <class T>
    __device__ __forceinline__ static float apply_stream(float x, const Coef &c, float g, float b)
    {
        return apply<T>(x, c, g, b);
    }
};

// ---------------------------------------------------------------------------
// RMSNorm
// ---------------------------------------------------------------------------
template <>
struct OpTraits<kRmsNorm> {
    static constexpr int kQ = 1;
    static constexpr int kParams = 1;

    template <class T, int VB, int IT>
    __device__ __forceinline__ static Partial wave_partial(Tile<T, VB, IT> &t, int kvalid)
    {
        constexpr int E = Tile<T, VB, IT>::kEpv;
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < IT; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float x = elem<T, VB>(t.v[k], e);
                    ss = __builtin_fmaf(x, x, ss);
                }
        return Partial{wave_sum(ss), 0.0f, 0.0f};
    }

    template <int N>
    __device__ __forceinline__ static Partial merge(const Partial (&p)[N], int n)
    {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n)
                ss += p[i].a;
        return Partial{ss, 0.0f, 0.0f};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize(const Partial &row, const Partial &, int64_t cols, float eps)
    {
        return Coef{0.0f, 1.0f / sqrtf(row.a / static_cast<float>(cols) + eps), 0.0f};
    }

    template <class T>
    __device__ __forceinline__ static float apply(float x, const Coef &c, float g, float)
    {
        return x * c.scale * g;
    }

    template <class T, int VB, int U>
    __device__ __forceinline__ static void stream_update(Partial &r, const RawVec<VB> (&v)[U], int kvalid)
    {
        constexpr int E = VB / StorageTraits<T>::kBytes;
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (k < kvalid)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float x = elem<T, VB>(v[k], e);
                    r.a = __builtin_fmaf(x, x, r.a);
                }
    }

    __device__ __forceinline__ static Partial stream_init() { return Partial{0.0f, 0.0f, 0.0f}; }

    __device__ __forceinline__ static Partial wave_from_thread(const Partial &r)
    {
        return Partial{wave_sum(r.a), 0.0f, 0.0f};
    }

    template <class T>
    __device__ __forceinline__ static Coef finalize_stream(const Partial &row, int64_t cols, float eps)
    {
        return finalize<T>(row, row, cols, eps);
    }

    template <class T>
    __device__ __forceinline__ static float apply_stream(float x, const Coef &c, float g, float b)
    {
        return apply<T>(x, c, g, b);
    }
};

}  // namespace credit
