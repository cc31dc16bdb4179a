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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (finite input).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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

// Wave-wide max of a non-negative float (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace qpl
