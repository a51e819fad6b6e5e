// rope_device.hpp -- device-side building blocks of the kernels: vector types, fp32 <->
// storage conversions, the rotation of a pair, table lanes.
// Included once, by rope_kernels.hip (the one translation unit of the
// library): its kernels are instantiated there, next to the host code
// that selects and launches them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rope_fastdiv.hpp"
#include "rope_partial.h"
#include "rope_plan.hpp"

namespace rope {
namespace {


typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // one 16-byte vector
typedef uint32_t v2u __attribute__((ext_vector_type(2)));  // half of one

constexpr int kModeRH = ROPE_MODE_ROTATE_HALF;
constexpr int kModeIL = ROPE_MODE_INTERLEAVE;
// rotate_half schemes of the vector kernel (see there): each thread writes
// its own vector and takes its partner's from the lane that holds it (a
// row's threads in one wave), or loads the partner from memory (out of
// place, rows wider than a wave)
constexpr int kModeRHOwn = 2;
constexpr int kModeRHOwnLoad = 3;

// ---------------------------------------------------------------------------
// fp32 <-> storage conversions. A 32-bit word holds two adjacent 16-bit lanes
// (lower lane in the low half). Widening is exact; narrowing rounds to nearest
// even (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32), keeps fp16 subnormals and
// NaNs, and overflows to infinity.
// ---------------------------------------------------------------------------
template <int DT> struct Store;

template <> struct Store<ROPE_DTYPE_BF16> {
    static constexpr int kLanes = 8;  // per 16-byte vector
    __device__ static f32x2 widen(uint32_t w)
    {
        f32x2 r;
        r.x = __uint_as_float(w << 16);
        r.y = __uint_as_float(w & 0xffff0000u);
        return r;
    }
    __device__ static uint32_t narrow(f32x2 v)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
    __device__ static float load1(const void* p, int64_t i)
    {
        return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
    }
    __device__ static void store1(void* p, int64_t i, float v)
    {
        static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    }
};

template <> struct Store<ROPE_DTYPE_F16> {
    static constexpr int kLanes = 8;
    __device__ static f32x2 widen(uint32_t w)
    {
        return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
    }
    __device__ static uint32_t narrow(f32x2 v)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
    __device__ static float load1(const void* p, int64_t i)
    {
        return static_cast<float>(static_cast<const _Float16*>(p)[i]);
    }
    __device__ static void store1(void* p, int64_t i, float v)
    {
        static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
    }
};

template <> struct Store<ROPE_DTYPE_F32> {
    static constexpr int kLanes = 4;
    __device__ static float load1(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
    __device__ static void store1(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};

// A 16-byte vector of lanes as fp32 values.
template <int DT>
struct Lanes {
    float v[Store<DT>::kLanes];
    __device__ void unpack(const v4u& q)
    {
        if constexpr (DT == ROPE_DTYPE_F32) {
            v[0] = __uint_as_float(q[0]); v[1] = __uint_as_float(q[1]);
            v[2] = __uint_as_float(q[2]); v[3] = __uint_as_float(q[3]);
        } else {
            const uint32_t w[4] = {q[0], q[1], q[2], q[3]};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f32x2 f = Store<DT>::widen(w[k]);
                v[2 * k] = f.x;
                v[2 * k + 1] = f.y;
            }
        }
    }
    __device__ v4u pack() const
    {
        if constexpr (DT == ROPE_DTYPE_F32) {
            return v4u{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                       __float_as_uint(v[3])};
        } else {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f32x2 f;
                f.x = v[2 * k];
                f.y = v[2 * k + 1];
                w[k] = Store<DT>::narrow(f);
            }
            return v4u{w[0], w[1], w[2], w[3]};
        }
    }
};

// ---------------------------------------------------------------------------
// The rotation of one pair (a, b) = (x_j, x_p(j)) where j is the lane whose
// partner term is negated in the forward (even lane / first half):
//   forward : a' = a*c_a - b*s_a        b' = b*c_b + a*s_b
//   backward: a' = a*c_a + b*s_b        b' = b*c_b - a*s_a   (transpose)
// 16-bit x (UNFUSED): each product is rounded to fp32 and the sum is rounded
// once more, as the page's "cast to fp32, multiply-add in fp32" reads. With
// 16-bit tables both products are exact, so this is also the single
// rounding of the exact sum; with fp32 tables the product roundings are part
// of the definition. fp32 x: the compiler may fuse (the result is held to a
// tolerance, not to bits).
// ---------------------------------------------------------------------------
template <int DIR>
__device__ __forceinline__ void rotate_pair_unfused(float& a, float& b, float ca, float sa, float cb, float sb)
{
#pragma clang fp contract(off)
    // no fused multiply-add in this function: every product and sum rounds
    float na, nb;
    if constexpr (DIR == kFwd) {
        na = a * ca - b * sa;
        nb = b * cb + a * sb;
    } else {
        na = a * ca + b * sb;
        nb = b * cb - a * sa;
    }
    a = na;
    b = nb;
}

template <int DIR, bool UNFUSED>
__device__ __forceinline__ void rotate_pair(float& a, float& b, float ca, float sa, float cb, float sb)
{
    if constexpr (UNFUSED) {
        rotate_pair_unfused<DIR>(a, b, ca, sa, cb, sb);
    } else {
        float na, nb;
        if constexpr (DIR == kFwd) {
            na = a * ca - b * sa;
            nb = b * cb + a * sb;
        } else {
            na = a * ca + b * sb;
            nb = b * cb - a * sa;
        }
        a = na;
        b = nb;
    }
}

// One lane of rotate_half in the own-vector scheme: the lane's value x, its
// partner's value p, and y = x*c - p*s (neg) or x*c + p*s, with c the lane's
// cos and s the sine the direction takes (the lane's forward, the partner's
// backward). These are the same products and sum as rotate_pair forms for
// that lane, with the same roundings.
__device__ __forceinline__ float rotate_own_unfused(float x, float p, float c, float s, bool neg)
{
#pragma clang fp contract(off)
    const float t = p * s;
    return x * c + (neg ? -t : t);
}

template <bool UNFUSED>
__device__ __forceinline__ float rotate_own(float x, float p, float c, float s, bool neg)
{
    if constexpr (UNFUSED) {
        return rotate_own_unfused(x, p, c, s, neg);
    } else {
        const float t = p * s;
        return x * c + (neg ? -t : t);
    }
}

// The cos or sin values for the K lanes of one x vector, from a table of
// type TT. They take K * sizeof(TT) bytes, loaded as kVecs table units of
// type Vec: 8 bytes (half a vector) when fp32 x meets a 16-bit table, one
// 16-byte vector when the table is as wide as x, two when 16-bit x meets an
// fp32 table (the page's mixed bf16-x / fp32-table case).
template <int Bytes> struct TableUnit { using type = v4u; };
template <> struct TableUnit<8> { using type = v2u; };

template <int TT, int K>
struct TableLanes {
    static constexpr int kBytes = K * (TT == ROPE_DTYPE_F32 ? 4 : 2);
    static_assert(kBytes == 8 || kBytes == 16 || kBytes == 32, "table unit shape");
    using Vec = typename TableUnit<kBytes>::type;
    static constexpr int kVecs = kBytes == 32 ? 2 : 1;
    float v[K];
    __device__ void unpack(const Vec* q)
    {
        if constexpr (TT == ROPE_DTYPE_F32) {
#pragma unroll
            for (int t = 0; t < kVecs; ++t)
#pragma unroll
                for (int w = 0; w < 4; ++w) v[4 * t + w] = __uint_as_float(q[t][w]);
        } else {
#pragma unroll
            for (int w = 0; w < kBytes / 4; ++w) {
                f32x2 f = Store<TT>::widen(q[0][w]);
                v[2 * w] = f.x;
                v[2 * w + 1] = f.y;
            }
        }
    }
};

}  // namespace
}  // namespace rope
