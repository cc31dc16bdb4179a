// Activation / weight quantizers, the amax reduction and the bf16 dequantizers for
// gfx950.  All of them are HBM-bound streaming kernels: 16-byte coalesced loads
// and stores, scales reduced within a lane (nvfp4 blocks) or across a wavefront
// (fp8r rows).
//
// Numerics follow the schemes of the Diffusers guide "BFL (fp8r / nvfp4)" (intro
// bullets) as read in qpl.h: fp8r s = amax / 448, codes E4M3(x / s); nvfp4
// sf = E4M3(bmax / (6 g)), d = dec(sf) * g, codes E2M1(x / d).  Divisions give
// the codes of the correctly rounded quotient (a reciprocal with one fma
// correction, or IEEE division outside the range where that holds; see div_rn),
// so codes match an fp32 reference bit for bit.
#include <cmath>

#include "qpl_dma.h"
#include "qpl_internal.h"
#include "qpl_nvfp4.h"

namespace qpl {

// ---------------------------------------------------------------------------
// fp8r: one wavefront per row, four rows per 256-thread workgroup.  VPT 16-byte
// vectors per lane stay in registers between the amax pass and the encode pass;
// VPT == 0 streams the row twice (rows longer than 64 * 8 * 24 elements).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t vec_absmax(const u32x4& v, uint32_t m) {
  return absmax_acc(absmax_acc(absmax_acc(absmax_acc(m, v.x), v.y), v.z), v.w);
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

// |x| <= amax, so |x / s| stays at 448 up to rounding: no overflow, and no clamp
// needed before the converter.
__device__ __forceinline__ float qdiv(float x, const RowDiv& d) {
  return d.tiny ? x / d.s : div_rn_finite(x, d.s, d.r);
}

// E4M3 codes of two bf16 pairs: pair a in bits 15:0, pair b in bits 31:16 (the
// converter's word select fills the halves; no clamp, see qdiv).
__device__ __forceinline__ uint32_t fp8_word(uint32_t a, uint32_t b, const RowDiv& d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(qdiv(bf16_lo(a), d), qdiv(bf16_hi(a), d), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qdiv(bf16_lo(b), d), qdiv(bf16_hi(b), d), lo, true);
}

__device__ __forceinline__ u32x2 fp8_vec(u32x4 v, const RowDiv& d) {
  u32x2 o;
  if (d.zero) {
    o.x = fp8_pair_zero(v.x) | (fp8_pair_zero(v.y) << 16);
    o.y = fp8_pair_zero(v.z) | (fp8_pair_zero(v.w) << 16);
    return o;
  }
  o.x = fp8_word(v.x, v.y, d);
  o.y = fp8_word(v.z, v.w, d);
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
  uint32_t am = 0;
  float amax;
  if constexpr (VPT > 0) {
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t j = lane + 64 * i;
      if (j < nv) {
        v[i] = __builtin_nontemporal_load(xr + j);
        am = vec_absmax(v[i], am);
      }
    }
    amax = wave_max(absmax_value(am));
    const RowDiv d = row_div(amax);
    if (lane == 0) xs[row] = d.s;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t j = lane + 64 * i;
      if (j < nv) __builtin_nontemporal_store(fp8_vec(v[i], d), qr + j);
    }
  } else {
    for (int64_t j = lane; j < nv; j += 64) am = vec_absmax(xr[j], am);
    amax = wave_max(absmax_value(am));
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

// nvfp4_scale with d = dec(sf) g and RN(1 / d) formed in place, as the host forms
// its table (one fp32 product, one correctly rounded division; code 0x7F, which
// only a NaN block maximum reaches, gives d = 0), for kernels that do not stage
// the table in LDS.
__device__ __forceinline__ Nvfp4Block nvfp4_scale_g(float bmax, float c6g, float rc6g, float g) {
  const float u = div_rn_ok(c6g) ? div_rn(bmax, c6g, rc6g) : bmax / c6g;
  Nvfp4Block b;
  b.sf = e4m3_pack2(u, 0.0f) & 0xFFu;
  b.dsf = e4m3_decode(b.sf);
  b.d = b.sf == 0x7Fu ? 0.0f : b.dsf * g;
  b.rd = 1.0f / b.d;
  b.fast = div_rn_ok(b.d) && bmax * b.rd < 0x1p126f;
  return b;
}

// Copy the per-code table from the kernel arguments into LDS (whole workgroup).
__device__ __forceinline__ void load_scale_table(const Nvfp4ScaleTable& t, float* tab_d, float* tab_rd) {
  for (int i = threadIdx.x; i < 128; i += blockDim.x) {
    tab_d[i] = t.d[i];
    tab_rd[i] = t.rd[i];
  }
  __syncthreads();
}

__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int64_t b, uint32_t (&p)[8]) {
  const u32x4* src = reinterpret_cast<const u32x4*>(x + b * 16);
  const u32x4 v0 = __builtin_nontemporal_load(src), v1 = __builtin_nontemporal_load(src + 1);
  p[0] = v0.x; p[1] = v0.y; p[2] = v0.z; p[3] = v0.w;
  p[4] = v1.x; p[5] = v1.y; p[6] = v1.z; p[7] = v1.w;
}

// Smoothing of one 16-element block (b-th block of the tensor, kb blocks per row):
// element k of the row is divided by lam[k].  p[j] holds elements 2j and 2j + 1.
template <bool SMOOTH>
__device__ __forceinline__ void smooth_block(uint32_t (&p)[8], const float* __restrict__ lam, int64_t b,
                                             int64_t kb) {
  if constexpr (SMOOTH) {
    const f32x4* l = reinterpret_cast<const f32x4*>(lam + (b % kb) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = l[i];
      p[2 * i] = smooth_pair(p[2 * i], v[0], v[1]);
      p[2 * i + 1] = smooth_pair(p[2 * i + 1], v[2], v[3]);
    }
  }
}


// The scale work that every nvfp4 linear does before its GEMM, in whole workgroups
// (256 threads) numbered blk < wblocks + xblocks:
// * blk < wblocks: the weight's block scales [N, kb] (kb = K/16) into the GEMM's
//   slab-major layout [S, N, 8] (S = ceil(kb/8)), zeros past kb: one thread per
//   8-byte unit, slab index fastest so that a wavefront reads consecutive bytes;
// * the rest (only when kb % 8 != 0): zeros over the bytes past kb of every
//   activation row's last slab [S - 1, M, 8], so that the GEMM multiplies the codes
//   it reads as zeros there by a finite scale.  Only the pad bytes are written: the
//   quantizer may be writing the real blocks' bytes of the same slab at the same time.
struct Nvfp4Prep {
  const uint8_t* wbs;
  uint8_t* wsl;
  uint8_t* xs;
  int64_t N, M, kb, S;
  unsigned wblocks, xblocks;
};

__device__ __forceinline__ void nvfp4_prep_block(const Nvfp4Prep& a, unsigned blk) {
  if (blk < a.wblocks) {
    const int64_t u = (int64_t)blk * 256 + threadIdx.x;
    if (u >= a.N * a.S) return;
    const int64_t n = u / a.S, sl = u - n * a.S;
    const uint8_t* src = a.wbs + n * a.kb + 8 * sl;
    const int64_t left = a.kb - 8 * sl;  // >= 1
    u32x2 v;
    if (left >= 8 && (reinterpret_cast<uintptr_t>(src) & 7u) == 0) {
      v = *reinterpret_cast<const u32x2*>(src);  // a whole, aligned group of eight scales
    } else {
      v = u32x2{0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < left) v.x |= (uint32_t)src[i] << (8 * i);
        if (i + 4 < left) v.y |= (uint32_t)src[i + 4] << (8 * i);
      }
    }
    *reinterpret_cast<u32x2*>(a.wsl + (sl * a.N + n) * 8) = v;
  } else {
    const int64_t m = (int64_t)(blk - a.wblocks) * 256 + threadIdx.x;
    if (m >= a.M) return;
    uint8_t* row = a.xs + ((a.S - 1) * a.M + m) * 8;
    for (int j = (int)(a.kb & 7); j < 8; ++j) row[j] = 0;
  }
}

static Nvfp4Prep nvfp4_prep_args(const uint8_t* wbs, int64_t N, int64_t K, uint8_t* wsl, int64_t M, uint8_t* xs) {
  Nvfp4Prep a;
  a.wbs = wbs;
  a.wsl = wsl;
  a.xs = xs;
  a.N = N;
  a.M = M;
  a.kb = K / 16;
  a.S = (a.kb + 7) / 8;
  a.wblocks = (unsigned)((N * a.S + 255) / 256);
  a.xblocks = a.kb % 8 != 0 ? (unsigned)((M + 255) / 256) : 0u;
  return a;
}

// SMOOTH: the block is first smoothed by lam (kb = K / 16 blocks per row).  SLAB:
// the scales go slab-major [ceil(K/128), rows, 8] (the GEMM's operand layout;
// byte 8 s + i of a row's scales is block 8 s + i) instead of row-major [rows, kb].
// Each lane forms its block's d and RN(1 / d) from g itself: a division per block
// costs less than staging the 128-entry table per workgroup.  Workgroups past the
// qblocks that quantize do the linear's scale preparation (nvfp4_prep_block), so
// that it needs no launch of its own.
template <bool SMOOTH, bool SLAB>
__global__ __launch_bounds__(256) void k_quant_nvfp4(const uint16_t* __restrict__ x, int64_t nblocks,
                                                     float c6g, float rc6g, float g,
                                                     const float* __restrict__ lam, int64_t kb, int64_t rows,
                                                     uint8_t* __restrict__ xq, uint8_t* __restrict__ xbs,
                                                     unsigned qblocks, Nvfp4Prep prep) {
  if (blockIdx.x >= qblocks) {
    nvfp4_prep_block(prep, blockIdx.x - qblocks);
    return;
  }
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint32_t p[8];
  load_block(x, b, p);
  smooth_block<SMOOTH>(p, lam, b, kb);
  const Nvfp4Block s = nvfp4_scale_g(block_absmax(p, 8), c6g, rc6g, g);
  reinterpret_cast<u32x2*>(xq)[b] = u32x2{nvfp4_word<true>(p, s), nvfp4_word<true>(p + 4, s)};
  if constexpr (SLAB) {
    const int64_t row = b / kb, j = b - row * kb;
    xbs[((j >> 3) * rows + row) * 8 + (j & 7)] = (uint8_t)s.sf;
  } else {
    xbs[b] = (uint8_t)s.sf;
  }
}

// nvfp4 quantization fused with the SVDQuant low-rank down-projection
// T = x L1 (the pages fuse the down-projection into the quantization kernel so
// that the 16-bit branch does not read x a second time: "Bringing Nunchaku 4-bit
// Diffusion Inference to Diffusers", section "Background: SVDQuant and
// Nunchaku").  The branch takes the unquantized x.
//
// A workgroup (sixteen wavefronts) owns rpw <= 32 consecutive rows, rpw chosen so that
// there is about one workgroup per CU, and walks K in tiles of TK columns.  Each tile of x
// (32 x TK bf16) and of L1^T (rpad x TK) moves global -> LDS without register
// staging, S - 1 tiles ahead; a load instruction covers whole 512- or 256-byte row
// segments, so HBM sees full lines.  The sixteen wavefronts split the work by kind:
// wavefronts 0-3 issue every tile load and run the MFMAs, wavefronts 4-15
// quantize (wavefront i usually runs on SIMD i mod 4, so that each SIMD holds one
// loading and three quantizing wavefronts, and a tile's x slots, dealt out in
// turn, spread evenly over the SIMDs with at most one per wavefront for up to 24
// rows).
// A load instruction waits at issue while the memory pipeline is full; with the
// loads in wavefronts of their own, that wait overlaps the quantizer's arithmetic
// instead of adding to it.  Per tile,
//   1. quantizing wavefront 4 + q takes the x tile's 1 KB slots q, q + 12, ...
//      (lane l holds eight values, lanes l and l ^ 1 one 16-element block) and
//      stores the packed codes (4 bytes per lane) and, from the block's first
//      lane, its scale byte in the GEMM's slab-major layout [K/128][M][8], while
//      the loading wavefronts issue the loads of tile kt + S - 1;
//   2. the loading wavefronts run the bf16 MFMA 32x32x16 over their quarter of the
//      tile's k range, reading both operands from LDS, into per-wave partial sums
//      of T, while the quantizing ones work.
// The four partial sums meet in LDS at the end, in a fixed order; T is stored as
// [hi | lo] bf16 halves (row stride kl = 2 rpad) for the GEMM's low-rank pass.
//
// LDS layout: 16-byte chunk c of tile row r sits at chunk slot c ^ (r & 15) of
// the row, so the MFMA operand reads (16 rows, one chunk) hit 16 different bank
// groups; the load instructions fill slots in order and fetch the chunk each slot
// holds.
//
// SMOOTH (SVDQuant smoothing): each stage also holds the tile's TK smoothing
// factors (one dword load per loading wavefront: wave w moves factors
// 64 w .. 64 w + 63, zeros past TK or K).  Step 1 divides its values by them,
// quantizes the smoothed bf16 values and writes them back over the tile, and step
// 2 waits at a barrier for every wave's write-back, so that both branches read the
// same smoothed activation.
//
// INT4 (the INT4 variant of svdq_w4a4): step 1 quantizes 64-channel groups
// instead (s = amax / 7, q = clamp(rint(x / s), -8, 7)): a group is eight chunks of
// a row, held by an aligned block of eight lanes (the chunk swizzle only permutes
// within such blocks), whose maximum takes three DPP steps.  It stores the codes
// as the E4M3 bytes of their values (the INT4 GEMM's operand, 8 bytes per lane)
// and the group's scale from the block's first lane.
template <int NCT, bool SMOOTH, bool INT4>
struct LrTile {
  static constexpr int TK = NCT <= 2 ? 256 : 128;  // k per tile
  static constexpr int CPR = TK / 8;                // 16-byte chunks per tile row
  static constexpr int XB = 32 * TK * 2;            // x tile bytes
  static constexpr int LB = 32 * NCT * TK * 2;      // L1^T tile bytes
  static constexpr int FB = SMOOTH ? 4 * 256 : 0;  // smoothing factor bytes (one 256-byte slot per loading wave)
  static constexpr int SB = XB + LB + FB;           // stage bytes
  static constexpr int S = (NCT == 1 || NCT == 3) ? 4 : 3;  // stages in the ring (at most 147 KB)
  static constexpr int NW = 16;                     // wavefronts: 0-3 load, 4-15 quantize
  static constexpr int NQ = 12;                     // quantizing wavefronts
  static constexpr int NM = 4;                      // multiplying wavefronts (the loading ones)
  static constexpr int NSX = XB / 1024;             // 1 KB slots of the x tile
  static constexpr int NSL = LB / 1024;             // 1 KB slots of the L1^T tile
  static constexpr int DW = (NSX + NSL) / 4 + (SMOOTH ? 1 : 0);  // loads per loading wave per tile
  static constexpr int QS = (NSX + NQ - 1) / NQ;    // x slots per quantizing wave per tile (at most)
  static_assert(NSL % 4 == 0 && NSX % 4 == 0 && 64 * 4 >= TK && (TK / 16) % NM == 0, "even splits");
};

// xq: the packed E2M1 codes [M, K/2] (nvfp4) or the E4M3 code bytes [M, K] (INT4);
// xs: the nvfp4 block scales slab-major [ceil(K/128), M, 8] (bytes) or the INT4
// group scales group-major [K/64, M] (floats).
template <int NCT, bool SMOOTH, bool INT4>
__global__ __launch_bounds__(1024) void k_quant_act_lowrank(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                           float c6g, float rc6g, Nvfp4ScaleTable tab,
                                                           const uint16_t* __restrict__ l1t, int64_t kl,
                                                           const float* __restrict__ lam, int rpw,
                                                           uint8_t* __restrict__ xq, void* __restrict__ xs,
                                                           uint16_t* __restrict__ t_out) {
  using C = LrTile<NCT, SMOOTH, INT4>;
  constexpr int TK = C::TK, CPR = C::CPR, S = C::S, NW = C::NW;
  __shared__ __attribute__((aligned(16))) uint8_t lds[S * C::SB];
  __shared__ float tab_d[128], tab_rd[128];
  load_scale_table(tab, tab_d, tab_rd);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t m0 = (int64_t)blockIdx.x * rpw;
  const int64_t rows = M - m0 < rpw ? M - m0 : rpw;
  const uint32_t pitch = (uint32_t)(K * 2);
  const u32x4 dx = make_desc(x + m0 * K, rows * pitch);
  const u32x4 dl = make_desc(l1t, (int64_t)32 * NCT * pitch);
  const u32x4 df = make_desc(lam, SMOOTH ? K * 4 : 0);
  const int64_t qpitch = INT4 ? K : K / 2;  // bytes per row of xq
  const int64_t ng = K / 64;
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(xq + m0 * qpitch, (short)0,
                                                                      (int)(rows * qpitch), (int)kRawBufferWord3);
  // scales: INT4 group-major [K/64, M] floats, nvfp4 slab-major [ceil(K/128), M, 8]
  // bytes (the GEMMs' layouts); both below 2^31 bytes (checked by the host)
  const int64_t sc_bytes = INT4 ? M * ng * 4 : ((K + 127) / 128) * M * 8;
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(xs, (short)0, (int)sc_bytes,
                                                                       (int)kRawBufferWord3);
  const uint32_t lbase = lds_address(lds);
  const int ntiles = (int)((K + TK - 1) / TK);
  // 32-bit forms for the offsets (K <= 2^21 and every buffer below 2^31 bytes, checked
  // by the host)
  const int k32 = (int)K;
  const uint32_t m32 = (uint32_t)M, row0 = (uint32_t)m0;

  // Geometry of this lane's part of 1 KB slot sl of a tile (the same for every
  // tile): tile row and chunk held.
  auto slot_row = [&](int sl) { return (sl * 64 + lane) / CPR; };
  auto slot_chunk = [&](int sl) {
    const int sv = sl * 64 + lane;
    return (sv % CPR) ^ ((sv / CPR) & 15);
  };
  // Offsets valid for tile kt: chunks past K read zero (rows past M do through dx).
  auto voff = [&](int r, int c, int kt) -> uint32_t {
    return kt * TK + 8 * c < k32 ? (uint32_t)r * pitch + 16u * (uint32_t)c : kOutOfRange;
  };
  const bool loader = wv < 4;
  // The loads of tile kt (loading wavefronts): slots wv, wv + 4, ... of both tiles.
  auto issue = [&](int kt) {
    const uint32_t st = lbase + (uint32_t)((kt % S) * C::SB);
    const int soff = kt * TK * 2;
#pragma unroll
    for (int j = 0; j < C::NSX / 4; ++j) {
      const int sl = 4 * j + wv;
      dma16(st + (uint32_t)(sl * 1024), voff(slot_row(sl), slot_chunk(sl), kt), dx, soff);
    }
#pragma unroll
    for (int j = 0; j < C::NSL / 4; ++j) {
      const int sl = 4 * j + wv;
      dma16(st + C::XB + (uint32_t)(sl * 1024), voff(slot_row(sl), slot_chunk(sl), kt), dl, soff);
    }
    if constexpr (SMOOTH) {
      const int64_t k = (int64_t)kt * TK + wv * 64 + lane;
      dma4(st + C::XB + C::LB + (uint32_t)(wv * 256),
           wv * 64 < TK && k < K ? (uint32_t)(k * 4) : kOutOfRange, df, 0);
    }
  };

  f32x16 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x16{};

  if (loader) {
#pragma unroll
    for (int t = 0; t < S - 1; ++t) issue(t);
  }
  for (int kt = 0; kt < ntiles; ++kt) {
    // tile kt has landed: a loading wave's loads retire in order, and the ones it
    // issued after tile kt's are those of tiles kt + 1 .. kt + S - 2 (the
    // quantizing waves issue only stores, and never wait on them here)
    if (loader) QPL_WAIT_VMCNT((S - 2) * C::DW);
    QPL_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();  // every part of tile kt is in LDS; tile kt - 1's buffer is free
    uint8_t* xt = lds + (kt % S) * C::SB;
    const uint8_t* lt = xt + C::XB;

    if (loader) {
      issue(kt + S - 1);  // past the end: out-of-range offsets, zeros into an unused buffer
    } else {
      // 1. quantize and store this wave's slots of the x tile
#pragma unroll
      for (int j = 0; j < C::QS; ++j) {
        const int sl = C::NQ * j + (wv - 4);
        if (sl >= C::NSX || sl * 64 / CPR >= rows) continue;  // past the tile or the workgroup's rows (uniform)
        const int r = slot_row(sl), c = slot_chunk(sl);
        u32x4* slot = reinterpret_cast<u32x4*>(xt + (sl * 64 + lane) * 16);
        const u32x4 v = *slot;
        uint32_t p[4] = {v.x, v.y, v.z, v.w};
        if constexpr (SMOOTH) {
          if (kt * TK + 8 * c < k32) {  // chunks past K hold zeros and no factors
            const f32x4* f = reinterpret_cast<const f32x4*>(xt + C::XB + C::LB + 32 * c);
            const f32x4 f0 = f[0], f1 = f[1];
            p[0] = smooth_pair(p[0], f0[0], f0[1]);
            p[1] = smooth_pair(p[1], f0[2], f0[3]);
            p[2] = smooth_pair(p[2], f1[0], f1[1]);
            p[3] = smooth_pair(p[3], f1[2], f1[3]);
            *slot = u32x4{p[0], p[1], p[2], p[3]};
          }
        }
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = absmax_acc(m, p[i]);
        // the other half of the block is in lane l ^ 1 (chunk c ^ 1 of the same row)
        m = absmax_acc(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
        if constexpr (INT4) {
          // the rest of the 64-channel group: lanes l ^ 2 (quad_perm 2,3,0,1), then the
          // other quad of the 8-lane block (row_half_mirror)
          m = absmax_acc(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
          m = absmax_acc(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
          const float s = absmax_value(m) / 7.0f;
          uint32_t w0 = 0, w1 = 0;
          if (s > 0.0f) {
            const bool ok = div_rn_ok(s);
            const float rs = 1.0f / s;
            float q[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float a = bf16_lo(p[i]), b = bf16_hi(p[i]);
              q[2 * i] = __builtin_amdgcn_fmed3f(__builtin_rintf(ok ? div_rn_finite(a, s, rs) : a / s), -8.0f, 7.0f);
              q[2 * i + 1] =
                  __builtin_amdgcn_fmed3f(__builtin_rintf(ok ? div_rn_finite(b, s, rs) : b / s), -8.0f, 7.0f);
            }
            w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
            w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)w0, true);
            w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
            w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], (int)w1, true);
          }
          const uint32_t k0 = (uint32_t)(kt * TK + 8 * c);
          const bool in_k = k0 < (uint32_t)k32;
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, re, in_k ? (int)((uint32_t)r * (uint32_t)k32 + k0) : (int)kOutOfRange, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(
              __float_as_uint(s), rsc,
              in_k && (c & 7) == 0 && r < rows ? (int)(((k0 / 64) * m32 + row0 + (uint32_t)r) * 4) : (int)kOutOfRange, 0, 0);
        } else {
          const Nvfp4Block sc = nvfp4_scale(absmax_value(m), c6g, rc6g, tab_d, tab_rd);
          const uint32_t k0 = (uint32_t)(kt * TK + 8 * c);
          const bool in_k = k0 < (uint32_t)k32;
          __builtin_amdgcn_raw_buffer_store_b32(nvfp4_word<true>(p, sc), re,
                                                in_k ? (int)((uint32_t)r * (uint32_t)qpitch + k0 / 2) : (int)kOutOfRange,
                                                0, 0);
          // the block's scale, from the lane holding its first half (even chunk)
          const uint32_t jb = k0 / 16;
          __builtin_amdgcn_raw_buffer_store_b8(
              (uint8_t)sc.sf, rsc,
              in_k && (c & 1) == 0 && r < rows ? (int)(((jb >> 3) * m32 + row0 + (uint32_t)r) * 8 + (jb & 7))
                                               : (int)kOutOfRange,
              0, 0);
        }
      }
    }

    if constexpr (SMOOTH) {
      QPL_WAIT_LGKM0();
      __builtin_amdgcn_s_barrier();  // every wave's smoothed values are in the tile
    }

    // 2. T += x_tile L1t_tile^T over this wave's quarter of the k range (loading waves)
    if (loader) {
#pragma unroll
      for (int ks = 0; ks < TK / 16 / C::NM; ++ks) {
        const int ch = wv * (CPR / C::NM) + 2 * ks + (lane >> 5);  // chunk of the 32x32x16 operand
        const int r = lane & 31;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(xt + (r * CPR + (ch ^ (r & 15))) * 16);
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          const int rb = 32 * c + r;
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(lt + (rb * CPR + (ch ^ (rb & 15))) * 16);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        }
      }
    }
  }
  QPL_WAIT_VMCNT(0);
  __syncthreads();

  // partial sums of the four multiplying waves -> T = ((p0 + p1) + p2) + p3
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [4][c][4][64]
  if (loader) {
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        red[((wv * NCT + c) * 4 + q) * 64 + lane] =
            f32x4{acc[c][4 * q], acc[c][4 * q + 1], acc[c][4 * q + 2], acc[c][4 * q + 3]};
  }
  __syncthreads();
  // acc[c][r] is T[m0 + (r / 4) * 8 + (lane / 32) * 4 + r % 4][32 c + lane % 32]
  const int64_t rpad = kl / 2;
  for (int e = threadIdx.x; e < NCT * 4 * 64; e += 64 * NW) {
    const int c = e / 256, q = (e / 64) % 4, l = e % 64;
    f32x4 v = red[((0 * NCT + c) * 4 + q) * 64 + l];
#pragma unroll
    for (int w = 1; w < 4; ++w) v = v + red[((w * NCT + c) * 4 + q) * 64 + l];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mr = q * 8 + (l >> 5) * 4 + i;
      if (mr >= rows) continue;
      const int64_t m = m0 + mr;
      const float tv = v[i];
      const uint32_t hi = f32_to_bf16(tv);
      const uint32_t lo = f32_to_bf16(tv - __uint_as_float(hi << 16));
      t_out[m * kl + 32 * c + (l & 31)] = (uint16_t)hi;
      t_out[m * kl + rpad + 32 * c + (l & 31)] = (uint16_t)lo;
    }
  }
}

// ---------------------------------------------------------------------------
// INT4 (the INT4 variant of svdq_w4a4): one lane per group of 64 channels.
// s = amax / 7 (correctly rounded); q = clamp(rint(x / s), -8, 7), rint taken of
// the quotient div_rn forms inside its range (whose integer is that of the
// correctly rounded quotient) and of the IEEE quotient outside; an all-zero group
// gives s = 0 and codes 0.  F8: each code is
// written as the E4M3 byte of its integer value [rows, K] (the GEMM's operand:
// -8..7 are exact in E4M3) and the scales group-major [K/64, rows] (so that the
// GEMM reads one group's scales of consecutive rows contiguously); otherwise the
// codes are packed two per byte, the even channel in the low nibble, and the
// scales are row-major [rows, K/64].
// ---------------------------------------------------------------------------
template <bool SMOOTH, bool F8>
__global__ __launch_bounds__(256) void k_quant_int4(const uint16_t* __restrict__ x, int64_t ngroups, int64_t ng,
                                                    int64_t rows, const float* __restrict__ lam,
                                                    uint8_t* __restrict__ xq, float* __restrict__ xs) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= ngroups) return;
  uint32_t p[32];
  const u32x4* src = reinterpret_cast<const u32x4*>(x + gi * 64);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    p[4 * i] = v.x;
    p[4 * i + 1] = v.y;
    p[4 * i + 2] = v.z;
    p[4 * i + 3] = v.w;
  }
  if constexpr (SMOOTH) {
    const f32x4* l = reinterpret_cast<const f32x4*>(lam + (gi % ng) * 64);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const f32x4 v = l[i];
      p[2 * i] = smooth_pair(p[2 * i], v[0], v[1]);
      p[2 * i + 1] = smooth_pair(p[2 * i + 1], v[2], v[3]);
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = absmax_acc(m, p[i]);
  const float s = absmax_value(m) / 7.0f;
  uint32_t w[16];  // four codes per word, channel order: E4M3 bytes (F8) or int8
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = 0;
  if (s > 0.0f) {
    const bool ok = div_rn_ok(s);
    const float r = 1.0f / s;
    auto code = [&](float v) {
      return __builtin_amdgcn_fmed3f(__builtin_rintf(ok ? div_rn_finite(v, s, r) : v / s), -8.0f, 7.0f);
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float q0 = code(bf16_lo(p[2 * i])), q1 = code(bf16_hi(p[2 * i]));
      const float q2 = code(bf16_lo(p[2 * i + 1])), q3 = code(bf16_hi(p[2 * i + 1]));
      if constexpr (F8) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
        w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true);
      } else {
        w[i] = ((uint32_t)(int)q0 & 0xFFu) | (((uint32_t)(int)q1 & 0xFFu) << 8) |
               (((uint32_t)(int)q2 & 0xFFu) << 16) | (((uint32_t)(int)q3 & 0xFFu) << 24);
      }
    }
  }
  if constexpr (F8) {
    u32x4* dst = reinterpret_cast<u32x4*>(xq + gi * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  } else {
    // bytes (c0, c1, c2, c3) -> nibbles c0 | c1 << 4, c2 << 8 | c3 << 12
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = w[2 * i] & 0x0F0F0F0Fu, b = w[2 * i + 1] & 0x0F0F0F0Fu;
      const uint32_t pa = (a & 0xFu) | ((a >> 4) & 0xF0u) | ((a >> 8) & 0xF00u) | ((a >> 12) & 0xF000u);
      const uint32_t pb = (b & 0xFu) | ((b >> 4) & 0xF0u) | ((b >> 8) & 0xF00u) | ((b >> 12) & 0xF000u);
      o[i] = pa | (pb << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(xq + gi * 32);
    dst[0] = u32x4{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4{o[4], o[5], o[6], o[7]};
  }
  if constexpr (F8) xs[(gi % ng) * rows + gi / ng] = s;
  else xs[gi] = s;
}

// Packed INT4 codes [rows, K/2] -> E4M3 bytes of their values [rows, K]: one lane
// per 16 packed bytes.  Nibble t is the value (t ^ 8) - 8; the converter writes
// two values per operation (exact: small integers).  The lane holding the first
// half of a group also copies the group's scale into the group-major layout
// wst [K/64, rows] that the GEMM reads.
__global__ __launch_bounds__(256) void k_expand_int4(const uint8_t* __restrict__ wq, int64_t nvec, int64_t K,
                                                     int64_t rows, const float* __restrict__ ws,
                                                     uint8_t* __restrict__ w8, float* __restrict__ wst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nvec) return;
  {
    const int64_t rb = K / 2, n = (16 * i) / rb, bo = (16 * i) % rb;  // row, byte within the row
    if (bo % 32 == 0) {
      const int64_t ng = K / 64, g = bo / 32;
      wst[g * rows + n] = ws[n * ng + g];
    }
  }
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wq) + i);
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    auto val = [&](int byte, int shift) { return (float)((int)(((in[j] >> (8 * byte + shift)) & 0xFu) ^ 8u) - 8); };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(val(2 * h, 0), val(2 * h, 4), 0, false);
      o[2 * j + h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(val(2 * h + 1, 0), val(2 * h + 1, 4), lo, true);
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(w8) + 2 * i;
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

// Host side of the nvfp4 scale rule: d = dec(sf) * g and RN(1 / d) for every
// block-scale code, in fp32 as on the device (the host build does not contract or
// flush either).  Code 0x7F (NaN) is never produced.
static float e4m3_value_host(uint32_t c) {
  const int e = (int)((c >> 3) & 15u), m = (int)(c & 7u);
  return e ? std::ldexp(1.0f + (float)m / 8.0f, e - 7) : std::ldexp((float)m / 8.0f, -6);
}

Nvfp4ScaleTable nvfp4_scale_table(float g) {
  Nvfp4ScaleTable t;
  for (uint32_t c = 0; c < 128; ++c) {
    const float d = c == 0x7Fu ? 0.0f : e4m3_value_host(c) * g;
    t.d[c] = d;
    t.rd[c] = 1.0f / d;
  }
  return t;
}

template <bool SLAB>
static hipError_t launch_nvfp4_blocks(const uint16_t* x, int64_t M, int64_t K, float g, const float* lam, uint8_t* xq,
                                      uint8_t* xbs, const Nvfp4Prep& prep, hipStream_t stream) {
  const int64_t nb = M * (K / 16);
  const float c6g = 6.0f * g, rc6g = 1.0f / c6g;
  const unsigned qblocks = (unsigned)((nb + 255) / 256);
  const dim3 grid(qblocks + prep.wblocks + prep.xblocks), block(256);
  if (lam)
    hipLaunchKernelGGL((k_quant_nvfp4<true, SLAB>), grid, block, 0, stream, x, nb, c6g, rc6g, g, lam, K / 16, M,
                       xq, xbs, qblocks, prep);
  else
    hipLaunchKernelGGL((k_quant_nvfp4<false, SLAB>), grid, block, 0, stream, x, nb, c6g, rc6g, g, lam, K / 16, M,
                       xq, xbs, qblocks, prep);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t M, int64_t K, float g, const float* lam, uint8_t* xq,
                              uint8_t* xbs, hipStream_t stream) {
  Nvfp4Prep none{};
  none.wblocks = none.xblocks = 0u;
  return launch_nvfp4_blocks<false>(x, M, K, g, lam, xq, xbs, none, stream);
}

hipError_t launch_quant_nvfp4_linear(const uint16_t* x, int64_t M, int64_t K, float g, const float* lam,
                                     uint8_t* xq, uint8_t* xs, const uint8_t* wbs, int64_t N, uint8_t* wsl,
                                     hipStream_t stream) {
  return launch_nvfp4_blocks<true>(x, M, K, g, lam, xq, xs, nvfp4_prep_args(wbs, N, K, wsl, M, xs), stream);
}

template <int NCT, bool SMOOTH, bool INT4>
static void launch_act_lr(dim3 grid, hipStream_t stream, const uint16_t* x, int64_t M, int64_t K, float c6g,
                          float rc6g, const Nvfp4ScaleTable& tab, const uint16_t* l1t, int64_t kl, const float* lam,
                          int rpw, uint8_t* xq, void* xs, uint16_t* t) {
  hipLaunchKernelGGL((k_quant_act_lowrank<NCT, SMOOTH, INT4>), grid, dim3(64 * LrTile<NCT, SMOOTH, INT4>::NW), 0, stream, x, M, K, c6g, rc6g, tab,
                     l1t, kl, lam, rpw, xq, xs, t);
}

template <bool INT4>
static hipError_t launch_act_lowrank(const uint16_t* x, int64_t M, int64_t K, float c6g, float rc6g,
                                     const Nvfp4ScaleTable& tab, const float* lam, const uint16_t* l1t, int64_t kl,
                                     uint8_t* xq, void* xs, uint16_t* t, hipStream_t stream) {
  // buffer offsets are 32-bit: the L1^T tile rows (at most 128) times the pitch (the
  // host checks this and the scale buffer's size before anything is queued)
  if (K > (int64_t{1} << 21)) return hipErrorInvalidValue;
  // about one workgroup per CU (256 on MI355X), at most 32 rows each
  const int64_t rpw64 = (M + 255) / 256;
  const int rpw = (int)(rpw64 < 32 ? rpw64 : 32);
  const dim3 grid((unsigned)((M + rpw - 1) / rpw));
#define QPL_ACT_LR(NCT)                                                                                   \
  (lam ? launch_act_lr<NCT, true, INT4>(grid, stream, x, M, K, c6g, rc6g, tab, l1t, kl, lam, rpw, xq, xs, t) \
       : launch_act_lr<NCT, false, INT4>(grid, stream, x, M, K, c6g, rc6g, tab, l1t, kl, lam, rpw, xq, xs, t))
  switch (kl / 64) {  // rpad / 32
    case 1: QPL_ACT_LR(1); break;
    case 2: QPL_ACT_LR(2); break;
    case 3: QPL_ACT_LR(3); break;
    case 4: QPL_ACT_LR(4); break;
    default: return hipErrorInvalidValue;
  }
#undef QPL_ACT_LR
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4_lowrank(const uint16_t* x, int64_t M, int64_t K, float g, const float* lam,
                                      const uint16_t* l1t, int64_t kl, uint8_t* xq, uint8_t* xs, uint16_t* t,
                                      hipStream_t stream) {
  const float c6g = 6.0f * g, rc6g = 1.0f / c6g;
  return launch_act_lowrank<false>(x, M, K, c6g, rc6g, nvfp4_scale_table(g), lam, l1t, kl, xq, xs, t, stream);
}

hipError_t launch_quant_int4_lowrank(const uint16_t* x, int64_t M, int64_t K, const float* lam, const uint16_t* l1t,
                                     int64_t kl, uint8_t* xq, float* xs, uint16_t* t, hipStream_t stream) {
  if (M * (K / 64) * 4 >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  return launch_act_lowrank<true>(x, M, K, 0.0f, 0.0f, Nvfp4ScaleTable{}, lam, l1t, kl, xq, xs, t, stream);
}

hipError_t launch_quant_int4(const uint16_t* x, int64_t M, int64_t K, const float* lam, bool f8, uint8_t* xq,
                             float* xs, hipStream_t stream) {
  const int64_t ng = K / 64, n = M * ng;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (lam) {
    if (f8) hipLaunchKernelGGL((k_quant_int4<true, true>), grid, block, 0, stream, x, n, ng, M, lam, xq, xs);
    else hipLaunchKernelGGL((k_quant_int4<true, false>), grid, block, 0, stream, x, n, ng, M, lam, xq, xs);
  } else {
    if (f8) hipLaunchKernelGGL((k_quant_int4<false, true>), grid, block, 0, stream, x, n, ng, M, lam, xq, xs);
    else hipLaunchKernelGGL((k_quant_int4<false, false>), grid, block, 0, stream, x, n, ng, M, lam, xq, xs);
  }
  return hipGetLastError();
}

hipError_t launch_expand_int4(const uint8_t* wq, const float* ws, int64_t N, int64_t K, uint8_t* w8, float* wst,
                              hipStream_t stream) {
  const int64_t nvec = N * K / 32;
  hipLaunchKernelGGL(k_expand_int4, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, stream, wq, nvec, K, N, ws,
                     w8, wst);
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
  uint32_t am = 0;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nv; j += (int64_t)gridDim.x * 256)
    am = vec_absmax(xv[j], am);
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t i = nv * 8; i < n; ++i) am = absmax_acc(am, x[i]);
  float m = wave_max(absmax_value(am));
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

// nvfp4 weight to bf16.  Output vector j (eight bf16) is half j % 2 of block j / 2:
// one dword of packed codes in, one 16-byte vector out per lane and step, so loads
// and stores of a wavefront are consecutive; DEQUANT_U steps per lane, loads first.
// The hardware FP4 converter gives the code values exactly; each value is
// bf16_rne(fp32(e2m1 * dec(sf)) * g2).
constexpr int DEQUANT_U = 4;

__device__ __forceinline__ void dequant_half(uint32_t w, float dsf, float g2, uint32_t* o) {
  auto out2 = [&](f32x2 v) { return pack_bf16((v[0] * dsf) * g2, (v[1] * dsf) * g2); };
  o[0] = out2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0));
  o[1] = out2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1));
  o[2] = out2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2));
  o[3] = out2(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3));
}

// Factor layouts of the SVDQuant low-rank branch, one element per thread:
// l1t[r][k] = L1[k][r] (zero for r >= R) and l2t[n][c] = L2[c mod rpad][n] (zero
// past R): L1 transposed for the fused quantizer, [L2^T | L2^T] for the GEMM's
// second pass.
__device__ __forceinline__ void lowrank_layout(const LowRankPrep& q, int64_t i) {
  const int64_t n1 = q.rpad * q.K, n2 = q.N * q.kl;
  if (i < n1) {
    const int64_t r = i / q.K, k = i % q.K;
    q.l1t[i] = r < q.R ? q.l1[k * q.R + r] : (uint16_t)0;
  } else if (i < n1 + n2) {
    const int64_t j = i - n1, n = j / q.kl, c = (j % q.kl) % q.rpad;
    q.l2t[j] = c < q.R ? q.l2[c * q.N + n] : (uint16_t)0;
  }
}

__global__ __launch_bounds__(256) void k_lowrank_transpose(LowRankPrep q) {
  lowrank_layout(q, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

__global__ __launch_bounds__(256) void k_dequant_nvfp4(const uint8_t* __restrict__ w, const uint8_t* __restrict__ wbs,
                                                       float g2, int64_t nvec, uint16_t* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * 256 * DEQUANT_U + threadIdx.x;
  uint32_t c[DEQUANT_U], sc[DEQUANT_U];
#pragma unroll
  for (int u = 0; u < DEQUANT_U; ++u) {
    const int64_t j = base + 256 * u;
    c[u] = j < nvec ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(w) + j) : 0u;
    sc[u] = j < nvec ? wbs[j >> 1] : 0u;
  }
#pragma unroll
  for (int u = 0; u < DEQUANT_U; ++u) {
    const int64_t j = base + 256 * u;
    if (j < nvec) {
      uint32_t o[4];
      dequant_half(c[u], e4m3_decode(sc[u]), g2, o);
      reinterpret_cast<u32x4*>(out)[j] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

// Preparation of an nvfp4 linear with a low-rank branch (one launch): the scale
// work of nvfp4_prep_block, then the branch's factor layouts (lowrank_layout).
__global__ __launch_bounds__(256) void k_nvfp4_prep(Nvfp4Prep a, LowRankPrep q) {
  const unsigned blk = blockIdx.x;
  if (blk < a.wblocks + a.xblocks)
    nvfp4_prep_block(a, blk);
  else
    lowrank_layout(q, (int64_t)(blk - a.wblocks - a.xblocks) * 256 + threadIdx.x);
}

static unsigned lowrank_blocks(const LowRankPrep& q) {
  return (unsigned)((q.rpad * q.K + q.N * q.kl + 255) / 256);
}

hipError_t launch_lowrank_prep(const uint16_t* l1, const uint16_t* l2, int64_t K, int64_t N, int64_t R, int64_t kl,
                               uint16_t* l1t, uint16_t* l2t, hipStream_t stream) {
  const LowRankPrep q{l1, l2, K, N, R, kl / 2, kl, l1t, l2t};
  hipLaunchKernelGGL(k_lowrank_transpose, dim3(lowrank_blocks(q)), dim3(256), 0, stream, q);
  return hipGetLastError();
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
  const int64_t nvec = N * K / 8;
  const dim3 grid((unsigned)((nvec + 256 * DEQUANT_U - 1) / (256 * DEQUANT_U))), block(256);
  hipLaunchKernelGGL(k_dequant_nvfp4, grid, block, 0, stream, w, wbs, g2, nvec, out);
  return hipGetLastError();
}

hipError_t launch_nvfp4_prep(const uint8_t* wbs, int64_t N, int64_t K, uint8_t* wsl, int64_t M, uint8_t* xs,
                             const LowRankPrep& lr, hipStream_t stream) {
  const Nvfp4Prep a = nvfp4_prep_args(wbs, N, K, wsl, M, xs);
  const dim3 grid(a.wblocks + a.xblocks + lowrank_blocks(lr)), block(256);
  hipLaunchKernelGGL(k_nvfp4_prep, grid, block, 0, stream, a, lr);
  return hipGetLastError();
}

}  // namespace qpl
