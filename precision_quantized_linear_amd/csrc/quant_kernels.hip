// Activation / weight quantizers, the amax reduction and the bf16 dequantizers for
// gfx950.  All of them are HBM-bound streaming kernels: 16-byte coalesced loads
// and stores, scales reduced within a lane (nvfp4 blocks) or across a wavefront
// (fp8r rows).
//
// Numerics follow the schemes of the Diffusers guide "BFL (fp8r / nvfp4)" (intro
// bullets) as read in qpl.h: fp8r s = amax / 448, codes E4M3(x / s); nvfp4
// sf = E4M3(bmax / (6 g)), d = dec(sf) * g, codes E2M1(x / d).  Divisions are
// IEEE correctly rounded (the library is built with correctly rounded fp32
// division and without contraction), so codes match an fp32 reference bit for bit.
#include "qpl_device.h"
#include "qpl_internal.h"

namespace qpl {

// ---------------------------------------------------------------------------
// fp8r: one wavefront per row, four rows per 256-thread workgroup.  VPT 16-byte
// vectors per lane stay in registers between the amax pass and the encode pass;
// VPT == 0 streams the row twice (rows longer than 64 * 8 * 24 elements).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float pair_absmax(uint32_t p, float m) {
  return fmaxf(m, fmaxf(bf16_lo(p & 0x7FFF7FFFu), bf16_hi(p & 0x7FFF7FFFu)));
}

// Codes of a bf16 pair in a row whose scale is 0 (every element is +-0): the sign only.
__device__ __forceinline__ uint32_t fp8_pair_zero(uint32_t p) { return ((p >> 8) & 0x80u) | ((p >> 16) & 0x8000u); }

// Row quantizer state: the scale s and r = RN(1/s) for the division.
struct RowDiv {
  float s, r;
  bool zero, tiny;
};

__device__ __forceinline__ RowDiv row_div(float amax) {
  RowDiv d;
  d.s = amax / 448.0f;
  d.zero = !(d.s > 0.0f);
  d.tiny = !div_rn_ok(d.s);
  d.r = 1.0f / d.s;
  return d;
}

__device__ __forceinline__ float qdiv(float x, const RowDiv& d) { return d.tiny ? x / d.s : div_rn(x, d.s, d.r); }

__device__ __forceinline__ uint32_t fp8_pair(uint32_t p, const RowDiv& d) {
  return e4m3_pack2(qdiv(bf16_lo(p), d), qdiv(bf16_hi(p), d));
}

__device__ __forceinline__ u32x2 fp8_vec(u32x4 v, const RowDiv& d) {
  u32x2 o;
  if (d.zero) {
    o.x = fp8_pair_zero(v.x) | (fp8_pair_zero(v.y) << 16);
    o.y = fp8_pair_zero(v.z) | (fp8_pair_zero(v.w) << 16);
    return o;
  }
  o.x = fp8_pair(v.x, d) | (fp8_pair(v.y, d) << 16);
  o.y = fp8_pair(v.z, d) | (fp8_pair(v.w, d) << 16);
  return o;
}

template <int VPT>
__global__ __launch_bounds__(256) void k_quant_fp8_row(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       uint8_t* __restrict__ xq, float* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int64_t nv = K >> 3;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * K);
  u32x2* qr = reinterpret_cast<u32x2*>(xq + row * K);
  float amax = 0.0f;
  if constexpr (VPT > 0) {
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t j = lane + 64 * i;
      if (j < nv) {
        v[i] = __builtin_nontemporal_load(xr + j);
        amax = pair_absmax(v[i].x, pair_absmax(v[i].y, pair_absmax(v[i].z, pair_absmax(v[i].w, amax))));
      }
    }
    amax = wave_max(amax);
    const RowDiv d = row_div(amax);
    if (lane == 0) xs[row] = d.s;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t j = lane + 64 * i;
      if (j < nv) qr[j] = fp8_vec(v[i], d);
    }
  } else {
    for (int64_t j = lane; j < nv; j += 64) {
      u32x4 v = xr[j];
      amax = pair_absmax(v.x, pair_absmax(v.y, pair_absmax(v.z, pair_absmax(v.w, amax))));
    }
    amax = wave_max(amax);
    const RowDiv d = row_div(amax);
    if (lane == 0) xs[row] = d.s;
    for (int64_t j = lane; j < nv; j += 64) qr[j] = fp8_vec(xr[j], d);
  }
}

hipError_t launch_quant_fp8_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* xq, float* xs,
                                hipStream_t stream) {
  const int64_t per_lane = (K / 8 + 63) / 64;
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
#define QPL_FP8_CASE(V) \
  if (per_lane <= V) { hipLaunchKernelGGL(k_quant_fp8_row<V>, grid, block, 0, stream, x, M, K, xq, xs); return hipGetLastError(); }
  QPL_FP8_CASE(1) QPL_FP8_CASE(2) QPL_FP8_CASE(4) QPL_FP8_CASE(6) QPL_FP8_CASE(8) QPL_FP8_CASE(12)
  QPL_FP8_CASE(16) QPL_FP8_CASE(24)
#undef QPL_FP8_CASE
  hipLaunchKernelGGL(k_quant_fp8_row<0>, grid, block, 0, stream, x, M, K, xq, xs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// nvfp4: one lane per 16-element block (32 bytes of bf16 in, 8 bytes of packed
// codes and one scale byte out).  Blocks never straddle rows (K % 16 == 0), so
// the tensor is processed as a flat array of blocks.
// ---------------------------------------------------------------------------
struct Nvfp4Block {
  uint32_t sf;   // E4M3 block scale
  float d;       // dec(sf) * g
  float rd;      // RN(1 / d)
  float dsf;     // dec(sf)
};

// g: global scale; c6g = 6 g (fp32) and rc6g = RN(1 / c6g), both from the host.
__device__ __forceinline__ Nvfp4Block nvfp4_block_scale(const uint32_t (&p)[8], float g, float c6g, float rc6g) {
  float bmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) bmax = pair_absmax(p[i], bmax);
  const float u = div_rn_ok(c6g) ? div_rn(bmax, c6g, rc6g) : bmax / c6g;
  Nvfp4Block b;
  b.sf = e4m3_pack2(u, 0.0f) & 0xFFu;
  b.dsf = e4m3_decode(b.sf);
  b.d = b.dsf * g;
  b.rd = 1.0f / b.d;
  return b;
}

// E2M1 codes of the 16 values; element 2j in the low nibble of byte j.
__device__ __forceinline__ u32x2 nvfp4_codes(const uint32_t (&p)[8], const Nvfp4Block& s) {
  uint32_t c[8];
  if (div_rn_ok(s.d)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = e2m1_pack2(div_rn(bf16_lo(p[i]), s.d, s.rd), div_rn(bf16_hi(p[i]), s.d, s.rd));
  } else if (s.d > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = e2m1_pack2(bf16_lo(p[i]) / s.d, bf16_hi(p[i]) / s.d);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = ((p[i] >> 12) & 0x8u) | ((p[i] >> 24) & 0x80u);
  }
  u32x2 o;
  o.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
  o.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
  return o;
}

__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int64_t b, uint32_t (&p)[8]) {
  const u32x4* src = reinterpret_cast<const u32x4*>(x + b * 16);
  const u32x4 v0 = __builtin_nontemporal_load(src), v1 = __builtin_nontemporal_load(src + 1);
  p[0] = v0.x; p[1] = v0.y; p[2] = v0.z; p[3] = v0.w;
  p[4] = v1.x; p[5] = v1.y; p[6] = v1.z; p[7] = v1.w;
}

__global__ __launch_bounds__(256) void k_quant_nvfp4(const uint16_t* __restrict__ x, int64_t nblocks, float g,
                                                     float c6g, float rc6g, uint8_t* __restrict__ xq,
                                                     uint8_t* __restrict__ xbs) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint32_t p[8];
  load_block(x, b, p);
  const Nvfp4Block s = nvfp4_block_scale(p, g, c6g, rc6g);
  reinterpret_cast<u32x2*>(xq)[b] = nvfp4_codes(p, s);
  xbs[b] = (uint8_t)s.sf;
}

// Same quantization; each quantized value e2m1(code) * dec(sf) is written as bf16.
// The product has at most 6 significant bits, so the bf16 value is exact.
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

__global__ __launch_bounds__(256) void k_quant_nvfp4_expand(const uint16_t* __restrict__ x, int64_t nblocks,
                                                            float g, float c6g, float rc6g,
                                                            uint16_t* __restrict__ xe) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint32_t p[8];
  load_block(x, b, p);
  const Nvfp4Block s = nvfp4_block_scale(p, g, c6g, rc6g);
  const u32x2 c = nvfp4_codes(p, s);
  uint32_t o[8];
  expand_word(c.x, s.dsf, o);
  expand_word(c.y, s.dsf, o + 4);
  u32x4* dst = reinterpret_cast<u32x4*>(xe + b * 16);
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t M, int64_t K, float g, uint8_t* xq, uint8_t* xbs,
                              hipStream_t stream) {
  const int64_t nb = M * (K / 16);
  const float c6g = 6.0f * g, rc6g = 1.0f / c6g;
  hipLaunchKernelGGL(k_quant_nvfp4, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream, x, nb, g, c6g, rc6g,
                     xq, xbs);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4_expand(const uint16_t* x, int64_t M, int64_t K, float g, uint16_t* xe,
                                     hipStream_t stream) {
  const int64_t nb = M * (K / 16);
  const float c6g = 6.0f * g, rc6g = 1.0f / c6g;
  hipLaunchKernelGGL(k_quant_nvfp4_expand, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream, x, nb, g,
                     c6g, rc6g, xe);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// amax: grid-stride over 16-byte vectors, wave max, one atomic per workgroup.
// Non-negative floats order like their bit patterns, so an unsigned atomic max
// on the bits is a float max.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_amax_bf16(const uint16_t* __restrict__ x, int64_t n,
                                                   float* __restrict__ amax) {
  __shared__ float part[4];
  const int64_t nv = n >> 3;
  float m = 0.0f;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nv; j += (int64_t)gridDim.x * 256) {
    const u32x4 v = xv[j];
    m = pair_absmax(v.x, pair_absmax(v.y, pair_absmax(v.z, pair_absmax(v.w, m))));
  }
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t i = nv * 8; i < n; ++i) m = fmaxf(m, bf16_lo(x[i] & 0x7FFFu));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(m));
  }
}

hipError_t launch_amax_bf16(const uint16_t* x, int64_t n, float* amax, hipStream_t stream) {
  int64_t blocks = (n / 8 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_amax_bf16, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, amax);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize to bf16 (the fallback of the guide's "Kernels" section).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant_fp8r(const uint8_t* __restrict__ w, const float* __restrict__ ws,
                                                      int64_t nchunks, int64_t chunks_per_row,
                                                      uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nchunks) return;
  const float s = ws[t / chunks_per_row];
  const u32x4 c = reinterpret_cast<const u32x4*>(w)[t];
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v0 = e4m3_decode(cw[i] & 0xFFu) * s, v1 = e4m3_decode((cw[i] >> 8) & 0xFFu) * s;
    const float v2 = e4m3_decode((cw[i] >> 16) & 0xFFu) * s, v3 = e4m3_decode(cw[i] >> 24) * s;
    o[2 * i] = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
    o[2 * i + 1] = f32_to_bf16(v2) | (f32_to_bf16(v3) << 16);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out) + 2 * t;
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

__global__ __launch_bounds__(256) void k_dequant_nvfp4(const uint8_t* __restrict__ w, const uint8_t* __restrict__ wbs,
                                                       float g2, int64_t nblocks, uint16_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const u32x2 c = reinterpret_cast<const u32x2*>(w)[b];
  const float dsf = e4m3_decode(wbs[b]);
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t byte = ((i < 4 ? c.x : c.y) >> (8 * (i & 3))) & 0xFFu;
    const float lo = (e2m1_decode(byte & 0xFu) * dsf) * g2;
    const float hi = (e2m1_decode(byte >> 4) * dsf) * g2;
    o[i] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + b * 16);
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

hipError_t launch_dequant_fp8r(const uint8_t* w, const float* ws, int64_t N, int64_t K, uint16_t* out,
                               hipStream_t stream) {
  const int64_t nch = N * K / 16;
  hipLaunchKernelGGL(k_dequant_fp8r, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, stream, w, ws, nch, K / 16,
                     out);
  return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t* w, const uint8_t* wbs, float g2, int64_t N, int64_t K, uint16_t* out,
                                hipStream_t stream) {
  const int64_t nb = N * K / 16;
  hipLaunchKernelGGL(k_dequant_nvfp4, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream, w, wbs, g2, nb, out);
  return hipGetLastError();
}

}  // namespace qpl
