// rac_device.h -- device-side building blocks shared by the gfx950 kernels:
// storage formats, the 32x32x16 MFMA wrappers and the one RoPE rotation
// routine that both the pre-rotation pass and the fused attention kernel use,
// so that both paths hand bit-identical rotated operands to the matrix cores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rac {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum { DT_BF16 = 0, DT_FP16 = 1 };

// Storage format traits: 16-bit element <-> fp32, packed 8-element operand
// vectors and the matching 32x32x16 MFMA (fp32 accumulate).
template <int DT> struct Fmt;

template <> struct Fmt<DT_BF16> {
    typedef bf16x8 vec8;
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    // two values, round to nearest even, one v_cvt_pk_bf16_f32 (a in the low half)
    static __device__ __forceinline__ uint32_t pack2(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Fmt<DT_FP16> {
    typedef f16x8 vec8;
    static __device__ __forceinline__ float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
    // two values, round to nearest even (the default mode), one v_cvt_pk_f16_f32
    static __device__ __forceinline__ uint32_t pack2(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    }
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <int DT>
__device__ __forceinline__ typename Fmt<DT>::vec8 as_vec8(u32x4 w) {
    return __builtin_bit_cast(typename Fmt<DT>::vec8, w);
}

// One RoPE turn of the pair (a, b) by the angle with cosine c and sine s,
// counter-clockwise, in fp32 with one fused multiply-add per output:
//   a' = a*c - b*s,  b' = a*s + b*c.
// Every rotation routine below is built from it, so all of them (and every
// kernel that uses them) produce the same bits for the same pair.
__device__ __forceinline__ void rope_turn(float a, float b, float c, float s, float& a2,
                                          float& b2) {
    a2 = __builtin_fmaf(a, c, -(b * s));
    b2 = __builtin_fmaf(a, s, b * c);
}

// RoPE on 8 consecutive elements (4 adjacent pairs) of one row.
// x: the 8 elements as 4 packed words; cs: the row's table entries for these
// pairs, (cos, sin) interleaved. Pair (x0, x1) turns counter-clockwise:
//   x0' = x0*c - x1*s,  x1' = x0*s + x1*c
// in fp32 with one fused multiply-add each, then rounds to the storage format.
// Every kernel rotates through this routine, so the rotated operands of the
// fused kernel and of the pre-rotation pass are bit-identical.
template <int DT>
__device__ __forceinline__ u32x4 rope_rotate8(u32x4 x, f32x4 cs_lo, f32x4 cs_hi) {
    typedef Fmt<DT> F;
    u32x4 y;
    const float c[4] = {cs_lo[0], cs_lo[2], cs_hi[0], cs_hi[2]};
    const float s[4] = {cs_lo[1], cs_lo[3], cs_hi[1], cs_hi[3]};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float a, b;
        rope_turn(F::lo(x[t]), F::hi(x[t]), c[t], s[t], a, b);
        y[t] = F::pack2(a, b);
    }
    return y;
}

// Half-split pairing ("rotate_half"): element d of the first half pairs with
// element d + D/2. lo, hi: the 8 elements d0 .. d0+7 (d0 < D/2) and their
// partners d0 + D/2 .. +7; cs: the table entries of frequencies d0 .. d0+7,
// (cos, sin) interleaved, 16 floats. Each pair (a, b) = (lo[j], hi[j]) turns
// counter-clockwise exactly as in rope_rotate8:
//   a' = a*c - b*s,  b' = a*s + b*c
// in fp32 with one fused multiply-add each, then rounds to the storage format.
template <int DT>
__device__ __forceinline__ void rope_rotate_half8(u32x4 lo, u32x4 hi, const f32x4 (&cs)[4],
                                                  u32x4& lo_out, u32x4& hi_out) {
    typedef Fmt<DT> F;
    float a[8], b[8], c[8], s[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        a[2 * t] = F::lo(lo[t]);
        a[2 * t + 1] = F::hi(lo[t]);
        b[2 * t] = F::lo(hi[t]);
        b[2 * t + 1] = F::hi(hi[t]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        c[j] = cs[j >> 1][2 * (j & 1)];
        s[j] = cs[j >> 1][2 * (j & 1) + 1];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float a0, b0, a1, b1;
        rope_turn(a[2 * t], b[2 * t], c[2 * t], s[2 * t], a0, b0);
        rope_turn(a[2 * t + 1], b[2 * t + 1], c[2 * t + 1], s[2 * t + 1], a1, b1);
        lo_out[t] = F::pack2(a0, a1);
        hi_out[t] = F::pack2(b0, b1);
    }
}

// Half of rope_rotate_half8: 4 elements d0 .. d0+3 of the first half (lo)
// and their partners d0 + D/2 .. +3 (hi), with the table entries of those 4
// frequencies, (cos, sin) interleaved in cs_lo, cs_hi; rotated in place.
template <int DT>
__device__ __forceinline__ void rope_rotate_half4(u32x2& lo, u32x2& hi, f32x4 cs_lo,
                                                  f32x4 cs_hi) {
    typedef Fmt<DT> F;
    const float c[4] = {cs_lo[0], cs_lo[2], cs_hi[0], cs_hi[2]};
    const float s[4] = {cs_lo[1], cs_lo[3], cs_hi[1], cs_hi[3]};
    u32x2 a_out, b_out;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float a0, b0, a1, b1;
        rope_turn(F::lo(lo[t]), F::lo(hi[t]), c[2 * t], s[2 * t], a0, b0);
        rope_turn(F::hi(lo[t]), F::hi(hi[t]), c[2 * t + 1], s[2 * t + 1], a1, b1);
        a_out[t] = F::pack2(a0, a1);
        b_out[t] = F::pack2(b0, b1);
    }
    lo = a_out;
    hi = b_out;
}

}  // namespace rac
