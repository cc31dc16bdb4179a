// The nvfp4 block rule on the device (Diffusers guide "BFL (fp8r / nvfp4)", intro
// bullet on nvfp4), used by the quantizers: per 16-element block
// sf = E4M3(bmax / (6 g)), d = dec(sf) * g, codes E2M1(x / d) equal to those of the
// correctly rounded divisions, and the exact bf16 expansion e2m1(code) * dec(sf).
#pragma once

#include "qpl_device.h"

namespace qpl {

struct Nvfp4Block {
  uint32_t sf;   // E4M3 block scale
  float d;       // dec(sf) * g
  float rd;      // RN(1 / d)
  float dsf;     // dec(sf)
  bool fast;     // d in div_rn's range and every |x / d| finite
};

// Block scale from the block's largest magnitude.  c6g = 6 g (fp32) and
// rc6g = RN(1 / c6g) come from the host, and so does the table of
// d = dec(sf) * g and RN(1 / d) for every block-scale code (tab_d, tab_rd in LDS).
__device__ __forceinline__ Nvfp4Block nvfp4_scale(float bmax, float c6g, float rc6g, const float* tab_d,
                                                  const float* tab_rd) {
  const float u = div_rn_ok(c6g) ? div_rn(bmax, c6g, rc6g) : bmax / c6g;
  Nvfp4Block b;
  b.sf = e4m3_pack2(u, 0.0f) & 0xFFu;
  b.dsf = e4m3_decode(b.sf);
  b.d = tab_d[b.sf];
  b.rd = tab_rd[b.sf];
  b.fast = div_rn_ok(b.d) && bmax * b.rd < 0x1p126f;
  return b;
}

// E2M1 codes of eight values (four bf16 pairs) under block scale s: byte i holds
// pair i, first value in the low nibble.  SIGNED_ZERO: a zero keeps its sign in
// the code (the codes are an output); otherwise the sign of a zero may be lost
// (the codes are only expanded to values, where +-0 are the same).
template <bool SIGNED_ZERO>
__device__ __forceinline__ uint32_t nvfp4_word(const uint32_t* p, const Nvfp4Block& s) {
  float q[8];
  if (s.fast) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = SIGNED_ZERO ? div_rn_finite(bf16_lo(p[i]), s.d, s.rd) : div_rn_nosign(bf16_lo(p[i]), s.d, s.rd);
      q[2 * i + 1] = SIGNED_ZERO ? div_rn_finite(bf16_hi(p[i]), s.d, s.rd) : div_rn_nosign(bf16_hi(p[i]), s.d, s.rd);
    }
    return e2m1_pack8_finite(q);
  }
  if (s.d > 0.0f) {
    // d outside div_rn's range or quotients that may overflow: IEEE division, clamped
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = __builtin_amdgcn_fmed3f(bf16_lo(p[i]) / s.d, -6.0f, 6.0f);
      q[2 * i + 1] = __builtin_amdgcn_fmed3f(bf16_hi(p[i]) / s.d, -6.0f, 6.0f);
    }
    return e2m1_pack8_finite(q);
  }
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) w |= (((p[i] >> 12) & 0x8u) | ((p[i] >> 24) & 0x80u)) << (8 * i);
  return w;
}

__device__ __forceinline__ float block_absmax(const uint32_t* p, int n) {
  uint32_t m = 0;
  for (int i = 0; i < n; ++i) m = absmax_acc(m, p[i]);
  return absmax_value(m);
}

// Eight packed E2M1 codes (one dword, element 2j in the low nibble of byte j) to
// eight bf16 values code * dsf: the FP4 converter at scale 1 gives the code values
// exactly, the product with an E4M3 value is exact (<= 6 significant bits), and
// the upper halves of the fp32 results are the bf16 values.
__device__ __forceinline__ uint32_t bf16_pair_of(f32x2 v, float m) {
  return (__float_as_uint(v[0] * m) >> 16) | (__float_as_uint(v[1] * m) & 0xFFFF0000u);
}

__device__ __forceinline__ void expand_word(uint32_t w, float dsf, uint32_t* o) {
  o[0] = bf16_pair_of(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), dsf);
  o[1] = bf16_pair_of(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), dsf);
  o[2] = bf16_pair_of(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), dsf);
  o[3] = bf16_pair_of(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), dsf);
}

}  // namespace qpl
