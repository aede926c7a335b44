// Device-side building blocks for the gfx950 reduction-reuse kernels:
// 128-bit row tiles held in VGPRs, bf16 conversion, wave64 DPP reductions and
// the fp32 exponential used by softmax.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace credit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Storage types.  `bf16_t` is the raw 16-bit pattern; arithmetic is in fp32.
// ---------------------------------------------------------------------------
struct bf16_t {
    uint16_t bits;
};

template <class T> struct StorageTraits;
template <> struct StorageTraits<float> {
    static constexpr int kBytes = 4;
};
template <> struct StorageTraits<bf16_t> {
    static constexpr int kBytes = 2;
};
// int8 output codes (quantization); never an input type.
struct i8_t {
    int8_t bits;
};
template <> struct StorageTraits<i8_t> {
    static constexpr int kBytes = 1;
};

// A vector of VB bytes moved by a single global access: 16 bytes, or one
// element; 8 and 1 bytes occur as the int8 output of a 16-byte bf16 or a
// one-element input vector.
template <int VB> struct RawVec;
template <> struct RawVec<16> {
    static constexpr int kWords = 4;
    u32x4 w;
};
template <> struct RawVec<8> {
    static constexpr int kWords = 2;
    u32x2 w;
};
template <> struct RawVec<4> {
    static constexpr int kWords = 1;
    uint32_t w;
};
template <> struct RawVec<2> {
    static constexpr int kWords = 1;  // low half used
    uint32_t w;
};
template <> struct RawVec<1> {
    static constexpr int kWords = 1;  // low byte used
    uint32_t w;
};

// ---------------------------------------------------------------------------
// Buffer accesses.  A row, slice or parameter vector is addressed through a
// buffer descriptor whose base is its first byte and whose size is its length:
// the lane offset is one VGPR, the per-vector step a scalar offset, and the
// hardware range check makes every access past the end harmless (loads return
// zero, stores are dropped), so tails need no branches.  The descriptor's
// third dword 0x00020000 is the raw 32-bit-element format of the gfx9 family.
// Cache policy: kStream marks row data non-temporal (it is touched once),
// kStreamStore additionally makes the output stores system-coherent (sc1),
// which measured 2-4% more write bandwidth on MI355X than nt alone; kKeep
// leaves the parameter vectors, shared by every row, cacheable.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kKeep = 0;
constexpr int kStream = 2;        // nt
constexpr int kStreamStore = 18;  // sc1 nt

// `bytes` must fit in 32 bits; callers keep one descriptor per row or slice.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// voff: the lane's whole byte offset into the buffer.  The scalar offset is
// always the constant 0, for two reasons: the range check covers the VGPR
// offset (plus the instruction's immediate) but not the scalar one, and on
// gfx950 a 16-byte buffer store whose scalar offset is an SGPR was observed to
// store data VGPRs that a VALU instruction right after it had already
// overwritten (the compiler inserts the store-data wait state only for a
// constant scalar offset).
template <int VB, int POLICY>
__device__ __forceinline__ RawVec<VB> buf_load(rsrc_t r, uint32_t voff)
{
    RawVec<VB> v;
    if constexpr (VB == 16) {
        v.w = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), 0, POLICY);
    } else if constexpr (VB == 4) {
        v.w = __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), 0, POLICY);
    } else {
        v.w = __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff), 0, POLICY);
    }
    return v;
}

template <int VB, int POLICY>
__device__ __forceinline__ void buf_store(const RawVec<VB> &v, rsrc_t r, uint32_t voff)
{
    if constexpr (VB == 16) {
        __builtin_amdgcn_raw_buffer_store_b128(v.w, r, static_cast<int>(voff), 0, POLICY);
    } else if constexpr (VB == 8) {
        __builtin_amdgcn_raw_buffer_store_b64(v.w, r, static_cast<int>(voff), 0, POLICY);
    } else if constexpr (VB == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(v.w, r, static_cast<int>(voff), 0, POLICY);
    } else if constexpr (VB == 2) {
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(v.w), r, static_cast<int>(voff), 0, POLICY);
    } else {
        __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(v.w), r, static_cast<int>(voff), 0, POLICY);
    }
}

// Bytes [lo, hi) (0 <= lo <= hi <= 4) of the 4-byte word w at byte offset
// voff: a 2-byte store for a half-word wholly inside, single bytes
// otherwise.  For the words at the ends of rows that share them with the
// neighbouring row, which writes the other bytes.
__device__ __forceinline__ void buf_store_word_part(uint32_t w, rsrc_t r, uint32_t voff, int lo, int hi)
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int b0 = 2 * h;
        if (lo <= b0 && b0 + 2 <= hi) {
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(w >> (16 * h)), r,
                                                  static_cast<int>(voff + b0), 0, kStreamStore);
        } else {
#pragma unroll
            for (int b = b0; b < b0 + 2; ++b)
                if (lo <= b && b < hi)
                    __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(w >> (8 * b)), r,
                                                         static_cast<int>(voff + b), 0, kStreamStore);
        }
    }
}

template <int VB>
__device__ __forceinline__ uint32_t vec_word(const RawVec<VB> &v, int j)
{
    if constexpr (VB >= 8)
        return v.w[j];
    else
        return v.w;
}

// Bytes [from, to) of a vector (0 <= from <= to <= VB, VB a multiple of 4),
// one at a time: for a row that lies inside one vector (rare; kept small).
template <int VB>
__device__ __forceinline__ void buf_store_bytes(const RawVec<VB> &v, rsrc_t r, uint32_t voff, int from, int to)
{
    static_assert(VB % 4 == 0, "vectors of whole words");
    for (int b = from; b < to; ++b) {
        uint32_t w = vec_word<VB>(v, 0);
#pragma unroll
        for (int j = 1; j < VB / 4; ++j)
            w = (b >> 2) == j ? vec_word<VB>(v, j) : w;
        __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(w >> (8 * (b & 3))), r,
                                             static_cast<int>(voff + static_cast<uint32_t>(b)), 0, kStreamStore);
    }
}

// Bytes [from, VB) of a vector (0 < from < VB): the part word, then the
// whole words after it as one store.
template <int VB>
__device__ __forceinline__ void buf_store_from(const RawVec<VB> &v, rsrc_t r, uint32_t voff, int from)
{
    static_assert(VB % 4 == 0, "vectors of whole words");
    const int w0 = (from + 3) >> 2;  // first whole word
    if (from & 3)
        buf_store_word_part(vec_word<VB>(v, w0 - 1), r, voff + 4u * static_cast<uint32_t>(w0 - 1), from & 3, 4);
    if constexpr (VB == 16) {
        typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
        if (w0 == 1) {
            const u32x3 w = {v.w[1], v.w[2], v.w[3]};
            __builtin_amdgcn_raw_buffer_store_b96(w, r, static_cast<int>(voff + 4u), 0, kStreamStore);
        } else if (w0 == 2) {
            const u32x2 w = {v.w[2], v.w[3]};
            __builtin_amdgcn_raw_buffer_store_b64(w, r, static_cast<int>(voff + 8u), 0, kStreamStore);
        } else if (w0 == 3) {
            __builtin_amdgcn_raw_buffer_store_b32(v.w[3], r, static_cast<int>(voff + 12u), 0, kStreamStore);
        }
    } else if constexpr (VB == 8) {
        if (w0 == 1)
            __builtin_amdgcn_raw_buffer_store_b32(v.w[1], r, static_cast<int>(voff + 4u), 0, kStreamStore);
    }
}

// Make a value the compiler treats as per-lane known to be wave-uniform.
__device__ __forceinline__ int64_t uniform(int64_t v)
{
    const uint64_t u = static_cast<uint64_t>(v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// True in every lane iff `pred` holds in every active lane of the wave.
__device__ __forceinline__ bool wave_all(bool pred)
{
    return __builtin_amdgcn_ballot_w64(!pred) == 0;
}

template <int VB> __device__ __forceinline__ uint32_t word(const RawVec<VB> &r, int i)
{
    if constexpr (VB >= 8)
        return r.w[i];
    else
        return r.w;
}
template <int VB> __device__ __forceinline__ void set_word(RawVec<VB> &r, int i, uint32_t v)
{
    if constexpr (VB >= 8)
        r.w[i] = v;
    else
        r.w = v;
}

// Element e (0 <= e < elements per vector) of a raw vector, as fp32.
template <class T, int VB>
__device__ __forceinline__ float elem(const RawVec<VB> &r, int e)
{
    if constexpr (StorageTraits<T>::kBytes == 4) {
        return __uint_as_float(word<VB>(r, e));
    } else {
        uint32_t w = word<VB>(r, e >> 1);
        return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
}

// Pack fp32 results into a raw vector of the storage type (bf16: round to
// nearest even with v_cvt_pk_bf16_f32; int8: the values are already integers
// in [-127, 127], converted exactly and packed little-endian).
template <class T, int VB, int EPV>
__device__ __forceinline__ RawVec<VB> pack(const float (&v)[EPV])
{
    RawVec<VB> r;
    if constexpr (StorageTraits<T>::kBytes == 1) {
#pragma unroll
        for (int w = 0; w < (EPV + 3) / 4; ++w) {
            uint32_t acc = 0;
#pragma unroll
            for (int e = 4 * w; e < EPV && e < 4 * w + 4; ++e)
                acc |= (static_cast<uint32_t>(static_cast<int32_t>(v[e])) & 0xffu) << (8 * (e - 4 * w));
            set_word<VB>(r, w, acc);
        }
    } else if constexpr (StorageTraits<T>::kBytes == 4) {
#pragma unroll
        for (int e = 0; e < EPV; ++e)
            set_word<VB>(r, e, __float_as_uint(v[e]));
    } else if constexpr (EPV == 1) {
        bf16x2 b = __builtin_convertvector((f32x2){v[0], 0.0f}, bf16x2);
        set_word<VB>(r, 0, __builtin_bit_cast(uint32_t, b) & 0xffffu);
    } else {
#pragma unroll
        for (int e = 0; e < EPV; e += 2) {
            bf16x2 b = __builtin_convertvector((f32x2){v[e], v[e + 1]}, bf16x2);
            set_word<VB>(r, e >> 1, __builtin_bit_cast(uint32_t, b));
        }
    }
    return r;
}

// ---------------------------------------------------------------------------
// Wave64 reductions.  Four DPP steps reduce each row of 16 lanes (quad swaps,
// half-row mirror, row mirror), leaving the row result in every lane of the
// row; the four row results are then read as uniform values with readlane and
// combined in a fixed order, so every lane gets the same bits.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppRowMirror = 0x140;   // row_mirror

__device__ __forceinline__ float lane_read(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppRowMirror>(v);
    return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp<kDppQuadXor1>(v));
    v = fmaxf(v, dpp<kDppQuadXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppRowMirror>(v));
    return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}

// ---------------------------------------------------------------------------
// Exponentials.
//
// exp_acc: exp(d) to about 2 ulp for the fp32 outputs.  exp(d) = 2^(d log2 e);
// the product is split as t + c, t = fl(d * L) with L = fl(log2 e), and
// c = (d * L - t) + d * (log2 e - L) (the first term exact by FMA), so
// exp(d) = 2^t * 2^c with |c| < 2^-20 and 2^c = 1 + c ln 2 to within 1e-13.
// 2^t uses the hardware v_exp_f32; where d * L overflows to -inf the result
// is 0.
//
// exp_fast: 2^(d * L) only; used where the output is bf16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_acc(float d)
{
    const float L = 1.44269502162933349609375f;       // fl(log2 e)
    const float Llo = 1.925963033500011e-08f;          // log2 e - L
    const float Ln2 = 0.693147180559945309f;
    float t = d * L;
    // |c| < 2^-20 wherever d * L is finite.  Below d = -FLT_MAX / log2 e (a
    // logit masked with a value near -FLT_MAX, minus the row maximum; every
    // caller passes d <= 0) t overflows to -inf and the exact product minus t
    // makes c = +inf (NaN for d = -inf): the clamp (minnum returns the number)
    // turns the result into 2^-inf * (1 + ln 2) = 0 there and changes nothing
    // elsewhere.  A NaN d still gives NaN through 2^t.
    float c = fminf(__builtin_fmaf(d, L, -t) + d * Llo, 1.0f);
    return __builtin_amdgcn_exp2f(t) * __builtin_fmaf(c, Ln2, 1.0f);
}

__device__ __forceinline__ float exp_fast(float d)
{
    return __builtin_amdgcn_exp2f(d * 1.44269502162933349609375f);
}

// ---------------------------------------------------------------------------
// Agent-scope atomics on 64-bit words, used for the split-row exchange.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_u64_agent(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_u64_agent(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_u32_agent(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_u32_agent(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_u32_agent(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fetch_or_u32_agent(uint32_t *p, uint32_t v)
{
    (void)__hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace credit
