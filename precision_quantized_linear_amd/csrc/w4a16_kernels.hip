// Weight-only 4-bit linear with bf16 activations for gfx950 (the awq_w4a16 layer
// of the Nunchaku post, "Introducing Nunchaku Lite": 4-bit weights, 16-bit
// activations, for the memory-bound adaptive-normalization and modulation
// projections).
//
// Format: codes q in 0..15 packed two per byte (even input channel in the low
// nibble), one bf16 scale s and one zero point z (a byte, 0..15) per group of G
// consecutive input channels; the weight value is (q - z) s.  That product has at
// most 12 significant bits, so it is exact in fp32, and so is its product with a
// bf16 activation: the only roundings are the fp32 accumulation and the final
// bf16 rounding.
//
// The layer runs at M = batch (one conditioning vector per image), so it is a
// GEMV over a weight read once: the kernel streams the codes at full width and
// keeps the activations in registers.
#include "qpl_device.h"
#include "qpl_dma.h"
#include "qpl_internal.h"

namespace qpl {

namespace {

// ---------------------------------------------------------------------------
// Quantizer: one lane per group.  hi = max(max w, 0), lo = min(min w, 0);
// s = bf16(fp32((hi - lo) / 15)); z = clamp(rint(-lo / s), 0, 15);
// q = clamp(rint(w / s) + z, 0, 15); a group whose s is 0 gets q = z = 0.
// Divisions are correctly rounded (build flag), rint is ties-to-even.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void k_quant_w4g(const uint16_t* __restrict__ w, int64_t ngroups,
                                                   uint8_t* __restrict__ wq, uint16_t* __restrict__ ws,
                                                   uint8_t* __restrict__ wz) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= ngroups) return;
  uint32_t p[G / 2];
  const u32x4* src = reinterpret_cast<const u32x4*>(w + gi * G);
#pragma unroll
  for (int i = 0; i < G / 8; ++i) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    p[4 * i] = v.x;
    p[4 * i + 1] = v.y;
    p[4 * i + 2] = v.z;
    p[4 * i + 3] = v.w;
  }
  float hi = 0.0f, lo = 0.0f;
#pragma unroll
  for (int i = 0; i < G / 2; ++i) {
    hi = fmaxf(hi, fmaxf(bf16_lo(p[i]), bf16_hi(p[i])));
    lo = fminf(lo, fminf(bf16_lo(p[i]), bf16_hi(p[i])));
  }
  const uint32_t sb = f32_to_bf16((hi - lo) / 15.0f);
  const float s = __uint_as_float(sb << 16);
  uint32_t codes[G / 8];
  uint32_t z = 0;
  if (s > 0.0f) {
    const float zf = __builtin_amdgcn_fmed3f(__builtin_rintf(-lo / s), 0.0f, 15.0f);
    z = (uint32_t)zf;
#pragma unroll
    for (int i = 0; i < G / 8; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t pr = p[4 * i + j];
        const uint32_t q0 = (uint32_t)__builtin_amdgcn_fmed3f(__builtin_rintf(bf16_lo(pr) / s) + zf, 0.0f, 15.0f);
        const uint32_t q1 = (uint32_t)__builtin_amdgcn_fmed3f(__builtin_rintf(bf16_hi(pr) / s) + zf, 0.0f, 15.0f);
        word |= (q0 | (q1 << 4)) << (8 * j);
      }
      codes[i] = word;
    }
  } else {
#pragma unroll
    for (int i = 0; i < G / 8; ++i) codes[i] = 0;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(wq + gi * (G / 2));
#pragma unroll
  for (int i = 0; i < G / 32; ++i)
    dst[i] = u32x4{codes[4 * i], codes[4 * i + 1], codes[4 * i + 2], codes[4 * i + 3]};
  ws[gi] = (uint16_t)sb;
  wz[gi] = (uint8_t)z;
}

// ---------------------------------------------------------------------------
// GEMV y[m, n] = sum_k x[m, k] (q[n, k] - z[n, k / G]) s[n, k / G].
//
// A wavefront owns RPW = 2 output rows at a time (grid-stride over the rows).
// The input channels are cut into chunks of 16 (8 bytes of codes); lane l takes
// chunks l, l + 64, ... of a K slice of 1024 CPL channels, so one load
// instruction moves 512 contiguous bytes of a weight row, and the lane's
// activations are the same for every row: they are loaded once into registers
// (MB rows of x, CPL chunks, 8 bf16 pairs each) and reused.  K beyond one slice
// is walked slice by slice, reloading the activations (only for K > 4096).
// Per chunk: nibbles -> floats (V_CVT_F32_UBYTE), w = q s - z s by one fma
// (exact), then one fma per activation row.  The lane sums are reduced across
// the wavefront in a fixed butterfly order.
// ---------------------------------------------------------------------------
constexpr int RPW = 2;

// The activations a lane keeps for its chunks (MB rows, CPL chunks of 16 channels):
// as floats when they fit in registers (MB CPL <= 6), so that no row pays for
// unpacking them again; otherwise as bf16 pairs unpacked at use.
template <int MB, int CPL>
struct XLane {
  static constexpr bool F = MB * CPL <= 6;
  float f[F ? MB : 1][F ? CPL : 1][16];
  uint32_t p[F ? 1 : MB][F ? 1 : CPL][8];
  __device__ __forceinline__ void set(int m, int i, const u32x4& a, const u32x4& b) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (F) {
        f[m][i][2 * e] = bf16_lo(w[e]);
        f[m][i][2 * e + 1] = bf16_hi(w[e]);
      } else {
        p[m][i][e] = w[e];
      }
    }
  }
  __device__ __forceinline__ float get(int m, int i, int e) const {
    if constexpr (F) return f[m][i][e];
    else return (e & 1) ? bf16_hi(p[m][i][e >> 1]) : bf16_lo(p[m][i][e >> 1]);
  }
};

// acc[m] += sum over the chunk's 16 channels of x[m][k] (q[k] - z) s, with
// w = q s - z s by one fma (exact) and one fma per row.  The masked code words go
// through an empty asm so that each code becomes a float by one byte conversion
// (V_CVT_F32_UBYTE0..3) rather than a bit-field extract and a conversion.
template <int MB, int CPL>
__device__ __forceinline__ void chunk_dot(const XLane<MB, CPL>& xl, int i, u32x2 cw, float s, float nzs,
                                          float (&acc)[MB]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t ev = cw[h] & 0x0F0F0F0Fu, od = (cw[h] >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(ev), "+v"(od));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float we = __builtin_fmaf((float)((ev >> (8 * b)) & 0xFFu), s, nzs);
      const float wo = __builtin_fmaf((float)((od >> (8 * b)) & 0xFFu), s, nzs);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        acc[m] = __builtin_fmaf(xl.get(m, i, 8 * h + 2 * b), we, acc[m]);
        acc[m] = __builtin_fmaf(xl.get(m, i, 8 * h + 2 * b + 1), wo, acc[m]);
      }
    }
  }
}

template <int MB, int CPL>
__global__ __launch_bounds__(256) void k_gemv_w4a16(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                    int64_t N, const uint8_t* __restrict__ wq,
                                                    const uint16_t* __restrict__ ws, const uint8_t* __restrict__ wz,
                                                    int gshift, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t m0 = (int64_t)blockIdx.y * MB;
  const int64_t nchunks = K >> 4;             // 16-channel chunks per row
  const int64_t ngroups = K >> gshift;
  constexpr int SLICE = 64 * CPL;             // chunks per slice
  const int nslices = (int)((nchunks + SLICE - 1) / SLICE);

  XLane<MB, CPL> xl;
  int xslice = -1;
  auto load_x = [&](int sl) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t c = (int64_t)sl * SLICE + i * 64 + lane;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        u32x4 a = u32x4{0u, 0u, 0u, 0u}, b = a;
        if (c < nchunks && m0 + m < M) {
          const u32x4* src = reinterpret_cast<const u32x4*>(x + (m0 + m) * K + 16 * c);
          a = src[0];
          b = src[1];
        }
        xl.set(m, i, a, b);
      }
    }
    xslice = sl;
  };

  for (int64_t n0 = wave * RPW; n0 < N; n0 += nwaves * RPW) {
    float acc[RPW][MB];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[r][m] = 0.0f;
    for (int sl = 0; sl < nslices; ++sl) {
      if (sl != xslice) load_x(sl);
      // this slice's codes, scales and zero points for both rows
      u32x2 cw[RPW][CPL];
      uint32_t sc[RPW][CPL], zp[RPW][CPL];
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int64_t n = n0 + r, c = (int64_t)sl * SLICE + i * 64 + lane;
          cw[r][i] = u32x2{0u, 0u};
          sc[r][i] = 0u;
          zp[r][i] = 0u;
          if (n < N && c < nchunks) {
            cw[r][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(wq + n * (K >> 1) + 8 * c));
            const int64_t g = n * ngroups + ((16 * c) >> gshift);
            sc[r][i] = ws[g];
            zp[r][i] = wz[g];
          }
        }
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const float s = __uint_as_float(sc[r][i] << 16);
          const float nzs = -(float)zp[r][i] * s;  // exact: at most 12 significant bits
          chunk_dot<MB, CPL>(xl, i, cw[r][i], s, nzs, acc[r]);
        }
    }
    // butterfly over the 64 lanes: every lane ends with the row sum
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        float v = acc[r][m];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        acc[r][m] = v;
      }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int m = 0; m < MB; ++m)
          if (n0 + r < N && m0 + m < M) y[(m0 + m) * N + n0 + r] = (uint16_t)f32_to_bf16(acc[r][m]);
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming GEMV for K <= 4096 with K / G a multiple of 4 (the modulation
// shapes): the same arithmetic and lane mapping as k_gemv_w4a16 (lane l takes
// chunks l, l + 64, ... of a row; its activations stay in registers), but every
// wavefront streams its rows (n = wave, wave + nwaves, ...) through a private
// ring of SS stages in LDS, one row per stage, moved by direct-to-LDS loads issued
// SS - 1 rows ahead, before the wait for the current row: per stage two 1 KB code
// loads, one 256-byte load of the row's scales and one of its zero points (loads
// past the row write zeros).  The multiply is VALU-bound (about three operations
// per weight: byte conversion, dequantizing fma, accumulating fma), so the ring
// only has to cover the memory latency.
// The wavefronts never share LDS, so there is no barrier; each wave counts its
// own loads and stores (vector memory operations retire in issue order).  The row
// sum is reduced with DPP within 16-lane rows and read out of lanes 0, 16, 32, 48
// in a fixed order; the stores are issued by every lane (lanes other than 0, and
// rows or activations past the end, with an out-of-range offset) so that each
// row costs exactly MB store operations.
// ---------------------------------------------------------------------------
constexpr int SS = 3;             // stages per wave
static_assert(SS == 3, "the wait-count switch of k_gemv_w4a16_stream is written for three stages");
constexpr int STG = 2560;         // stage bytes: codes 2048, scales 256, zero points 256
constexpr int SD = 4;             // loads per stage

__device__ __forceinline__ float row16_sum(float v) {
  // sums over each 16-lane row, left in every lane of the row
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

template <int MB, int CPL>
__global__ __launch_bounds__(256) void k_gemv_w4a16_stream(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                           int64_t N, const uint8_t* __restrict__ wq,
                                                           const uint16_t* __restrict__ ws,
                                                           const uint8_t* __restrict__ wz, int gshift,
                                                           uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * SS * STG];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t m0 = (int64_t)blockIdx.y * MB;
  const int64_t nchunks = K >> 4;
  const int64_t ng = K >> gshift;
  const int64_t nrows = wave < N ? (N - wave + nwaves - 1) / nwaves : 0;
  const uint32_t base = lds_address(lds) + (uint32_t)(wv * SS * STG);
  const uint8_t* mine = lds + wv * SS * STG;

  // activations of this lane's chunks, through buffer loads: an intrinsic that
  // reads memory stays ahead of the stream's load statements (so the stream's wait
  // counts hold), and nothing waits for these loads before their first use
  XLane<MB, CPL> xl;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0,
                                                                      (int)(M * K * 2), (int)kRawBufferWord3);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int64_t c = i * 64 + lane;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const bool ok = c < nchunks && m0 + m < M;
      const int off = ok ? (int)(((m0 + m) * K + 16 * c) * 2) : (int)kOutOfRange;
      const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
      const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? off + 16 : (int)kOutOfRange, 0, 0));
      xl.set(m, i, a, b);
    }
  }

  auto issue = [&](int64_t j) {
    const bool valid = j < nrows;
    const int64_t n = valid ? wave + j * nwaves : 0;
    const uint32_t st = base + (uint32_t)((j % SS) * STG);
    const u32x4 dc = make_desc(wq + n * (K >> 1), valid ? (K >> 1) : 0);
    const u32x4 dsc = make_desc(ws + n * ng, valid ? 2 * ng : 0);
    const u32x4 dz = make_desc(wz + n * ng, valid ? ng : 0);
    dma16(st, (uint32_t)(16 * lane), dc, 0);
    dma16(st + 1024, (uint32_t)(16 * lane + 1024), dc, 0);
    dma4(st + 2048, (uint32_t)(4 * lane), dsc, 0);
    dma4(st + 2304, (uint32_t)(4 * lane), dz, 0);
  };

  // y as a buffer of exactly M N bf16 (< 2^30 bytes), so that kOutOfRange drops a store
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(y, (short)0, (int)(M * N * 2),
                                                                      (int)kRawBufferWord3);
#pragma unroll
  for (int j = 0; j < SS - 1; ++j) issue(j);

  for (int64_t j = 0; j < nrows; ++j) {
    // row j + SS - 1 goes into the stage of row j - 1, whose LDS reads have completed;
    // then row j must have landed: issued after its loads are the loads of rows
    // j + 1 .. j + SS - 1 and the MB stores of each row since (at most SS - 1 rows)
    issue(j + SS - 1);
    switch (j < SS - 1 ? (int)j : SS - 1) {
      case 0: QPL_WAIT_VMCNT((SS - 1) * SD); break;
      case 1: QPL_WAIT_VMCNT((SS - 1) * SD + MB); break;
      default: QPL_WAIT_VMCNT((SS - 1) * SD + 2 * MB); break;
    }
    const uint8_t* st = mine + (j % SS) * STG;
    float acc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * 64 + lane;
      if (c < nchunks) {
        const u32x2 cw = *reinterpret_cast<const u32x2*>(st + 8 * c);
        const int g = (16 * c) >> gshift;
        const float s = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(st + 2048 + 2 * g) << 16);
        const float nzs = -(float)st[2304 + g] * s;  // exact: at most 12 significant bits
        chunk_dot<MB, CPL>(xl, i, cw, s, nzs, acc);
      }
    }
    const int64_t n = wave + j * nwaves;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float r = row16_sum(acc[m]);
      const float v = ((__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)) +
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16))) +
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 32))) +
                      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 48));
      const bool ok = lane == 0 && m0 + m < M;
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16(v), ry,
                                           ok ? (int)(((m0 + m) * N + n) * 2) : (int)kOutOfRange, 0, 0);
    }
  }
  QPL_WAIT_VMCNT(0);
}

template <int MB>
hipError_t launch_gemv_stream(int cpl, dim3 grid, hipStream_t stream, const uint16_t* x, int64_t M, int64_t K,
                              int64_t N, const uint8_t* wq, const uint16_t* ws, const uint8_t* wz, int gshift,
                              uint16_t* y) {
  switch (cpl) {
    case 1: hipLaunchKernelGGL((k_gemv_w4a16_stream<MB, 1>), grid, dim3(256), 0, stream, x, M, K, N, wq, ws, wz, gshift, y); break;
    case 2: hipLaunchKernelGGL((k_gemv_w4a16_stream<MB, 2>), grid, dim3(256), 0, stream, x, M, K, N, wq, ws, wz, gshift, y); break;
    case 3: hipLaunchKernelGGL((k_gemv_w4a16_stream<MB, 3>), grid, dim3(256), 0, stream, x, M, K, N, wq, ws, wz, gshift, y); break;
    default: hipLaunchKernelGGL((k_gemv_w4a16_stream<MB, 4>), grid, dim3(256), 0, stream, x, M, K, N, wq, ws, wz, gshift, y); break;
  }
  return hipGetLastError();
}

template <int MB>
hipError_t launch_gemv(int cpl, dim3 grid, hipStream_t stream, const uint16_t* x, int64_t M, int64_t K, int64_t N,
                       const uint8_t* wq, const uint16_t* ws, const uint8_t* wz, int gshift, uint16_t* y) {
  switch (cpl) {
    case 1: hipLaunchKernelGGL((k_gemv_w4a16<MB, 1>), grid, dim3(256), 0, stream, x, M, K, N, wq, ws, wz, gshift, y); break;
    case 2: hipLaunchKernelGGL((k_gemv_w4a16<MB, 2>), grid, dim3(256), 0, stream, x, M, K, N, wq, ws, wz, gshift, y); break;
    case 3: hipLaunchKernelGGL((k_gemv_w4a16<MB, 3>), grid, dim3(256), 0, stream, x, M, K, N, wq, ws, wz, gshift, y); break;
    default: hipLaunchKernelGGL((k_gemv_w4a16<MB, 4>), grid, dim3(256), 0, stream, x, M, K, N, wq, ws, wz, gshift, y); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_w4g(const uint16_t* w, int64_t N, int64_t K, int group, uint8_t* wq, uint16_t* ws,
                            uint8_t* wz, hipStream_t stream) {
  const int64_t ng = N * (K / group);
  const dim3 grid((unsigned)((ng + 255) / 256)), block(256);
  switch (group) {
    case 32: hipLaunchKernelGGL(k_quant_w4g<32>, grid, block, 0, stream, w, ng, wq, ws, wz); break;
    case 64: hipLaunchKernelGGL(k_quant_w4g<64>, grid, block, 0, stream, w, ng, wq, ws, wz); break;
    case 128: hipLaunchKernelGGL(k_quant_w4g<128>, grid, block, 0, stream, w, ng, wq, ws, wz); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_w4a16(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* wq,
                             const uint16_t* ws, const uint8_t* wz, int group, uint16_t* y, hipStream_t stream) {
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;
  const int64_t cpl64 = (K / 16 + 63) / 64;
  const int cpl = (int)(cpl64 < 4 ? cpl64 : 4);
  const int mb = M == 1 ? 1 : 2;
  if (K <= 4096 && (K >> gshift) % 4 == 0 && M * K * 2 < (int64_t{1} << 30) && M * N * 2 < (int64_t{1} << 30)) {
    // streaming kernel: enough waves for every row, at most 5 workgroups (20 waves,
    // 150 KB of rings) per CU
    const int64_t wgs = (N + 3) / 4;
    const dim3 grid((unsigned)(wgs < 1280 ? wgs : 1280), (unsigned)((M + mb - 1) / mb));
    if (mb == 1) return launch_gemv_stream<1>(cpl, grid, stream, x, M, K, N, wq, ws, wz, gshift, y);
    return launch_gemv_stream<2>(cpl, grid, stream, x, M, K, N, wq, ws, wz, gshift, y);
  }
  // enough workgroups to keep every CU streaming: up to 8 per CU, each wave at least one row pair
  const int64_t need = (N + 4 * RPW - 1) / (4 * RPW);
  const unsigned gx = (unsigned)(need < 2048 ? need : 2048);
  const dim3 grid(gx, (unsigned)((M + mb - 1) / mb));
  if (mb == 1) return launch_gemv<1>(cpl, grid, stream, x, M, K, N, wq, ws, wz, gshift, y);
  return launch_gemv<2>(cpl, grid, stream, x, M, K, N, wq, ws, wz, gshift, y);
}

}  // namespace qpl
