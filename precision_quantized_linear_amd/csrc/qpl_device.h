// Device-side helpers shared by the gfx950 kernels: bf16 conversion, the E4M3 and
// E2M1 encoders/decoders and the block-scale rules of the BFL fp8r / nvfp4 schemes
// (Diffusers guide "BFL (fp8r / nvfp4)", intro bullets).  Format readings: OCP FP8
// E4M3 (bias 7, max 448) and OCP MX FP4 E2M1; round to nearest even, saturate,
// keep the sign of zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qpl {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (finite input).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two floats to packed bf16, round to nearest even (V_CVT_PK_BF16_F32; checked
// against the bit-level rounding rule on 8M pairs including ties and subnormals).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// SVDQuant smoothing of a bf16 pair (Nunchaku post, "Background: SVDQuant and
// Nunchaku": activation outliers move into the weights, so input channel k is
// divided by its factor): bf16_rne(x / l) per half, with a correctly rounded fp32
// division (the library is compiled with -fhip-fp32-correctly-rounded-divide-sqrt).
// l0 divides the low half, l1 the high half.
__device__ __forceinline__ uint32_t smooth_pair(uint32_t pair, float l0, float l1) {
  return f32_to_bf16(bf16_lo(pair) / l0) | (f32_to_bf16(bf16_hi(pair) / l1) << 16);
}

// |v| (as raw fp32 bits without sign) -> E4M3 magnitude code.
//   below 2^-6: the subnormal grid of step 2^-9, code = rint(|v| * 2^9) (0..8);
//   otherwise: round the fp32 mantissa to 3 bits (ties to even) and rebias the
//   exponent from 127 to 7; anything that rounds past 448 saturates to 0x7E.
__device__ __forceinline__ uint32_t e4m3_mag(uint32_t a) {
  if (a < 0x3C800000u) return (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
  r -= (120u << 3);
  return r < 0x7Eu ? r : 0x7Eu;
}

__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t u = __float_as_uint(v);
  return e4m3_mag(u & 0x7FFFFFFFu) | ((u >> 24) & 0x80u);
}

// |v| bits -> E2M1 magnitude code 0..7 (values 0, .5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ uint32_t e2m1_mag(uint32_t a) {
  if (a < 0x3F800000u) return (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
  uint32_t r = (a + 0x1FFFFFu + ((a >> 22) & 1u)) >> 22;
  r -= (126u << 1);
  return r < 7u ? r : 7u;
}

__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  uint32_t u = __float_as_uint(v);
  return e2m1_mag(u & 0x7FFFFFFFu) | ((u >> 28) & 0x8u);
}

// E4M3 code (low byte of c) -> float, exact (hardware OCP E4M3 conversion).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// E2M1 code (0..15) -> float, exact.
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 stored as twice the value, one byte each
  uint32_t twice = (uint32_t)((0x0C08060403020100ull >> ((c & 7u) * 8u)) & 0xFFu);
  float v = (float)twice * 0.5f;
  return (c & 8u) ? -v : v;
}

// x / s from a precomputed r = RN(1 / s) with one Markstein correction step:
// q0 = x r, then q = q0 + r (x - s q0), the residual exact by fma.  It is formed as
// q = q0 - r ne with ne = RN(s q0 - x) = -(x - s q0): the same value (round to
// nearest is symmetric), and a zero x keeps its sign with no copysign (x = -0 gives
// ne = +0 and q = -0 - r (+0) = -0; x = +0 gives +0).  A quotient that overflows
// returns the infinity of x r (the correction would turn it into NaN).  Requires
// 2^-64 <= s <= 2^64 (r normal); the callers use the plain division outside that
// range.  q is the correctly rounded quotient unless the residual falls below the
// normal range, which takes x below about 2^-100; with s in that range such a
// quotient is below 2^-36, far under the smallest nonzero E4M3 or E2M1 code, so
// the codes are those of the correctly rounded quotient.  Checked on the GPU
// against IEEE division for every finite bf16 x over 8192 divisors spanning
// 2^-40..2^40 (including all-ones and zero mantissas): identical E4M3 and E2M1
// codes for every quotient below 2^126 (the quotient bits differ in 4% of the
// pairs, all with a tiny x), and bit for bit the same quotients as the q0 + r e
// form with a copysign.
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  const float q0 = x * r;
  const float ne = __builtin_fmaf(q0, s, -x);
  const float q = __builtin_fmaf(-ne, r, q0);
  return __builtin_isinf(q0) ? q0 : q;
}

// div_rn for quotients known to stay below 2^127 in magnitude (no overflow check).
__device__ __forceinline__ float div_rn_finite(float x, float s, float r) {
  const float q0 = x * r;
  const float ne = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-ne, r, q0);
}

// Whether s lies in the range where div_rn is exact.
__device__ __forceinline__ bool div_rn_ok(float s) { return s >= 0x1p-64f && s <= 0x1p64f; }

// E4M3 codes of two floats with the hardware OCP FP8 converter (round to nearest
// even).  The converter turns values above 464 into NaN instead of saturating, so
// magnitudes are clamped to 448 first; with that clamp it matched the bit-level
// encoder on 2^28 random values including every rounding midpoint +- 1 ulp.
// Returns the two codes in bits 7:0 and 15:8.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
}

// e4m3_pack2 for magnitudes below 464, which the converter rounds like the
// saturating encoder (nothing above 448 but below 464 is a different code).
__device__ __forceinline__ uint32_t e4m3_pack2_small(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// E2M1 codes of two floats with the hardware FP4 converter at scale 1 (round to
// nearest even, saturating at 6; matched the bit-level encoder on 2^28 random
// finite values including midpoints).  Inputs are clamped to +-6 first so that an
// infinite quotient also lands on the largest code.  Returns the codes in bits 3:0
// and 7:4.
__device__ __forceinline__ uint32_t e2m1_pack2(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, -6.0f, 6.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -6.0f, 6.0f);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, ca, cb, 1.0f, 0) & 0xFFu;
}

// e2m1_pack2 for finite inputs (the converter saturates them by itself).
__device__ __forceinline__ uint32_t e2m1_pack2_finite(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// div_rn without the sign fix: the quotient of a zero is +0 whatever the sign of x
// (for values whose sign of zero does not matter).  Same range conditions.
__device__ __forceinline__ float div_rn_nosign(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(e, r, q0);
}

// Running maximum of bf16 magnitudes kept as two 16-bit integers: non-negative
// floats order like their bit patterns, so an integer max of |x| bits is a float max.
__device__ __forceinline__ uint32_t absmax_acc(uint32_t m, uint32_t pair) {
  const u16x2 a = __builtin_bit_cast(u16x2, pair & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, m)));
}

// The float value of the larger half of an absmax_acc accumulator.
__device__ __forceinline__ float absmax_value(uint32_t m) {
  const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  return __uint_as_float((lo > hi ? lo : hi) << 16);
}

// Eight E2M1 codes (finite inputs, pairs in order) packed into one word with the
// converter's byte select: pair i lands in byte i, first value in the low nibble.
__device__ __forceinline__ uint32_t e2m1_pack8_finite(const float (&q)[8]) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
}

// Wave-wide max of a non-negative float (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace qpl
