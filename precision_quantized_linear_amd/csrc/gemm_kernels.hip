// Quantized GEMMs for gfx950 (CDNA4): y[M,N] = x[M,K] * W[N,K]^T with fp32
// accumulation in the MFMA units and bf16 output rounded to nearest even.
//
// fp8r (Diffusers guide "BFL (fp8r / nvfp4)", "Kernels" table, fp8r row): E4M3 x
// E4M3 on the f8f6f4 MFMA (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with unit E8M0
// scales); output (acc * s_x[m]) * s_w[n].
//
// nvfp4 ("Kernels" table, nvfp4 row): the guide's kernel is a block-scaled FP4
// GEMM with one E4M3 scale per 16 elements.  gfx950's scaled MFMA applies one
// power-of-two (E8M0) scale per 32 elements, and a code times an E4M3 scale needs
// up to 6 significant bits, which no 8-, 6- or 4-bit operand format holds.  The
// exact route taken here: both operands are expanded to bf16 values
// e2m1(code) * dec(sf) (exact) -- activations by the quantize kernel, weights by
// one streaming pass over the packed weight -- and multiplied on the bf16 MFMA
// (V_MFMA_F32_32X32X16_BF16).  The global factor input_scale * weight_scale_2
// and the optional SVDQuant low-rank term (Nunchaku post, "Background: SVDQuant
// and Nunchaku": the up-projection fused into the GEMM) are applied to the fp32
// accumulators before the single bf16 rounding.
//
// Pipeline (both GEMMs):
// * a 256-thread workgroup (4 wavefronts, 2 x 2) owns a 256 x 256 output tile; a
//   wavefront owns 128 x 128 (16 MFMA tiles of 32 x 32, 256 fp32 accumulators
//   per lane in AGPRs, one wavefront per SIMD);
// * K is walked in 64-byte slabs (64 fp8 or 32 bf16 elements per row); each
//   stage holds the 256-row slab of both operands (32 KB) and four stages ring
//   through 128 KB of the 160 KB LDS;
// * slabs move global -> LDS with buffer_load_dwordx4 ... lds (no register
//   staging), issued four stages ahead and spread between the MFMAs; rows past
//   the matrix and bytes past K read as zero through the buffer range check;
// * the 16-byte chunks of each 64-byte row are XOR-swizzled with
//   (r ^ r >> 3) & 3, which makes the MFMA operand reads bank-conflict free;
// * operand fragments of the next slab are read into the registers of the
//   current slab's fragments as each one is used for the last time;
// * operands are swapped (the MFMA computes y^T), so each lane ends with four
//   consecutive output columns of a row and stores them as one 8-byte segment.
#include "qpl_dma.h"
#include "qpl_internal.h"

namespace qpl {

namespace {

constexpr int SROW = 64;            // bytes per slab row
constexpr int SLAB = 256 * SROW;    // 16 KB per operand per stage
constexpr int STAGE = 2 * SLAB;     // x slab then W slab
constexpr int NST = 4;              // stages in the ring
constexpr int DMA_PER_STAGE = 8;    // per wavefront: 4 x-slab and 4 W-slab instructions of 1 KB

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 3; }
__device__ __forceinline__ int soff(int r, int c) { return r * SROW + ((c ^ swz(r)) << 4); }

typedef f32x16 Acc[4][4];

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
}

// Buffer descriptor over the tile's rows of a row-major byte matrix: reads past
// the tile's last valid row return zero.
__device__ __forceinline__ u32x4 tile_desc(const void* base, int64_t rows_left, int64_t pitch) {
  const int64_t rows = rows_left < 256 ? rows_left : 256;
  return make_desc(base, rows * pitch);
}

// Operand fragments.  fp8: a 32x32x64 MFMA operand (32 K-bytes per lane, two
// chunks).  bf16: a 32x32x16 MFMA operand (8 K-values per lane, one chunk); a
// 64-byte slab holds two of them (sub-steps).
struct Fp8Mma {
  static constexpr int SUB = 1;
  typedef i32x8 Frag;
  static __device__ __forceinline__ Frag read(const uint8_t* slab, int row, int sub, int lane) {
    (void)sub;
    const int c = 2 * (lane >> 5);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(slab + soff(row, c));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(slab + soff(row, c + 1));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  static __device__ __forceinline__ f32x16 mma(const Frag& w, const Frag& x, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, c, 0, 0, 0, 127, 0, 127);
  }
};

struct Bf16Mma {
  static constexpr int SUB = 2;
  typedef bf16x8 Frag;
  static __device__ __forceinline__ Frag read(const uint8_t* slab, int row, int sub, int lane) {
    return *reinterpret_cast<const bf16x8*>(slab + soff(row, 2 * sub + (lane >> 5)));
  }
  static __device__ __forceinline__ f32x16 mma(const Frag& w, const Frag& x, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, x, c, 0, 0, 0);
  }
};

// One pass of the pipeline over K: acc += W_tile x_tile^T in the D^T layout
// (acc[i][j] row index = W row, column index = x row).  dx / dw are descriptors
// over the tile's x rows and W rows (same pitch, kbytes valid bytes per row).
// Ends with every load drained and all waves past a barrier, so LDS is free.
template <class T>
__device__ __forceinline__ void gemm_pass(Acc& acc, uint8_t* lds, uint32_t lbase, u32x4 dx, u32x4 dw, int pitch,
                                          int kbytes, int wv, int wm, int wn, int lane) {
  uint32_t vbase[4];
  int cb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // instruction q of this wave covers slab rows 16 (4 wv + q) .. + 15; lane l
    // fills physical chunk l % 4 of row ... + l / 4, i.e. logical chunk (l % 4) ^ swz
    const int row = 16 * (4 * wv + q) + (lane >> 2);
    cb[q] = ((lane & 3) ^ swz(row)) * 16;
    vbase[q] = (uint32_t)(row * pitch + cb[q]);
  }
  const int nk = (kbytes + SROW - 1) / SROW;
  auto voff = [&](int s, int q) -> uint32_t { return (s < nk && s * SROW + cb[q] < kbytes) ? vbase[q] : kOutOfRange; };
  auto dma = [&](int s, int q, bool w_slab) {
    const uint32_t dst = lbase + (s % NST) * STAGE + (w_slab ? SLAB : 0) + (4 * wv + q) * 1024;
    dma16(dst, voff(s, q), w_slab ? dw : dx, s * SROW);
  };
#pragma unroll
  for (int s = 0; s < NST; ++s)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dma(s, q, false);
      dma(s, q, true);
    }
  QPL_WAIT_VMCNT((NST - 1) * DMA_PER_STAGE);
  __builtin_amdgcn_s_barrier();
  typename T::Frag fw[T::SUB][4], fx[T::SUB][4];
#pragma unroll
  for (int u = 0; u < T::SUB; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fw[u][i] = T::read(lds + SLAB, wn * 128 + i * 32 + (lane & 31), u, lane);
      fx[u][i] = T::read(lds, wm * 128 + i * 32 + (lane & 31), u, lane);
    }
  constexpr int NMMA = 16 * T::SUB;
  for (int kt = 0; kt < nk; ++kt) {
    // slab kt + 1 has landed for every wave, and every wave is done with step kt - 1
    QPL_WAIT_LGKM0();
    QPL_WAIT_VMCNT((NST - 2) * DMA_PER_STAGE);
    __builtin_amdgcn_s_barrier();
    const uint8_t* nx = lds + ((kt + 1) % NST) * STAGE;
    const int sref = kt + NST;  // refill the buffer slab kt used with slab kt + NST
#pragma unroll
    for (int u = 0; u < T::SUB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = T::mma(fw[u][i], fx[u][j], acc[i][j]);
          const int k = 16 * u + 4 * i + j;
          if (i == 3) fx[u][j] = T::read(nx, wm * 128 + j * 32 + (lane & 31), u, lane);
          if (j == 3) fw[u][i] = T::read(nx + SLAB, wn * 128 + i * 32 + (lane & 31), u, lane);
          // spread this step's 8 refill loads over its MFMAs
          constexpr int every = NMMA / DMA_PER_STAGE;
          if (k % every == every - 1) {
            const int d = k / every;
            dma(sref, d & 3, d >= 4);
          }
        }
  }
  QPL_WAIT_VMCNT(0);
  QPL_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
}

// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs and each XCD
// has its own L2, so each XCD gets a contiguous run of the tile sequence; the
// sequence walks groups of GROUP_M tile-rows column by column, so the ~32 tiles an
// XCD runs at once form a 4 x 8 block that shares 4 activation slabs and 8 weight
// slabs in that XCD's L2.
constexpr int GROUP_M = 4;

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int64_t& m0, int64_t& n0) {
  const int T = tiles_m * tiles_n;
  int b = blockIdx.x;
  if ((T & 7) == 0) b = (b & 7) * (T >> 3) + (b >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int g = b / per_group;
  const int first_m = g * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int r = b - g * per_group;
  m0 = (int64_t)(first_m + r % gm) * 256;
  n0 = (int64_t)(r / gm) * 256;
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

// Store the tile: y[m][n .. n+3] = bf16((acc * rs(m)) * cs(n .. n+3)) as 8-byte
// segments.  Interior tiles (and N % 4 == 0) take a path without per-element
// checks; edge tiles check rows and columns and fall back to element stores.
template <class RowScale, class ColScale>
__device__ __forceinline__ void store_tile(const Acc& acc, int wm, int wn, int lane, int64_t m0, int64_t n0,
                                           int64_t M, int64_t N, uint16_t* __restrict__ y, const RowScale& rs,
                                           const ColScale& cs) {
  float fr[4];
  f32x4 fc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) fr[j] = rs(wm * 128 + j * 32 + (lane & 31));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) fc[i][g] = cs(wn * 128 + i * 32 + g * 8 + (lane >> 5) * 4);
  auto seg = [&](int i, int j, int g) {
    const f32x16& a = acc[i][j];
    u32x2 o;
    o.x = pack_bf16((a[g * 4 + 0] * fr[j]) * fc[i][g][0], (a[g * 4 + 1] * fr[j]) * fc[i][g][1]);
    o.y = pack_bf16((a[g * 4 + 2] * fr[j]) * fc[i][g][2], (a[g * 4 + 3] * fr[j]) * fc[i][g][3]);
    return o;
  };
  const int64_t mb = m0 + wm * 128 + (lane & 31), nb = n0 + wn * 128 + (lane >> 5) * 4;
  if (m0 + 256 <= M && n0 + 256 <= N && (N & 3) == 0) {
    uint16_t* yb = y + mb * N + nb;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<u32x2*>(yb + (int64_t)(j * 32) * N + i * 32 + g * 8) = seg(i, j, g);
    return;
  }
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = mb + j * 32;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = nb + i * 32 + g * 8;
        const u32x2 o = seg(i, j, g);
        if (vec && n < N) {
          *reinterpret_cast<u32x2*>(y + m * N + n) = o;
        } else {
          const uint32_t w[2] = {o.x, o.y};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) y[m * N + n + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_fp8r(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ B,
    const float* __restrict__ sb, int64_t M, int64_t K, int64_t N, uint16_t* __restrict__ Y, int tiles_m,
    int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE];
  __shared__ __attribute__((aligned(16))) float lscale[2][256];  // the tile's row scales and column scales
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  int64_t m0, n0;
  tile_coords(tiles_m, tiles_n, m0, n0);
  lscale[0][t] = m0 + t < M ? sa[m0 + t] : 0.0f;
  lscale[1][t] = n0 + t < N ? sb[n0 + t] : 0.0f;
  const uint32_t lbase = lds_address(lds);
  Acc acc;
  zero_acc(acc);
  gemm_pass<Fp8Mma>(acc, lds, lbase, tile_desc(A + m0 * K, M - m0, K), tile_desc(B + n0 * K, N - n0, K), (int)K,
                    (int)K, wv, wm, wn, lane);
  store_tile(acc, wm, wn, lane, m0, n0, M, N, Y, [&](int r) { return lscale[0][r]; },
             [&](int c) { return *reinterpret_cast<const f32x4*>(&lscale[1][c]); });
}

template <bool LOWRANK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_nvfp4(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, float gscale, int64_t M, int64_t K, int64_t N,
    const uint16_t* __restrict__ T, const uint16_t* __restrict__ L2t, int64_t KL, uint16_t* __restrict__ Y,
    int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  int64_t m0, n0;
  tile_coords(tiles_m, tiles_n, m0, n0);
  const uint32_t lbase = lds_address(lds);
  Acc acc;
  zero_acc(acc);
  const int kb = (int)(2 * K);
  gemm_pass<Bf16Mma>(acc, lds, lbase, tile_desc(A + m0 * K, M - m0, kb), tile_desc(W + n0 * K, N - n0, kb), kb, kb,
                     wv, wm, wn, lane);
  float oscale = gscale;
  if constexpr (LOWRANK) {
    // SVDQuant up-projection: acc = g * acc + [T_hi | T_lo] [L2^T | L2^T]^T, in fp32
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] *= gscale;
    const int lb = (int)(2 * KL);
    gemm_pass<Bf16Mma>(acc, lds, lbase, tile_desc(T + m0 * KL, M - m0, lb), tile_desc(L2t + n0 * KL, N - n0, lb), lb,
                       lb, wv, wm, wn, lane);
    oscale = 1.0f;
  }
  store_tile(acc, wm, wn, lane, m0, n0, M, N, Y, [&](int) { return oscale; },
             [&](int) { return f32x4{1.0f, 1.0f, 1.0f, 1.0f}; });
}

// l1t[r][k] = L1[k][r] (zero for r >= R); l2t[n][c] = L2[c mod rpad][n] (zero past R).
__global__ __launch_bounds__(256) void k_lowrank_transpose(const uint16_t* __restrict__ l1,
                                                           const uint16_t* __restrict__ l2, int64_t K, int64_t N,
                                                           int64_t R, int64_t rpad, int64_t kl,
                                                           uint16_t* __restrict__ l1t, uint16_t* __restrict__ l2t) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n1 = rpad * K, n2 = N * kl;
  if (i < n1) {
    const int64_t r = i / K, k = i % K;
    l1t[i] = r < R ? l1[k * R + r] : (uint16_t)0;
  } else if (i < n1 + n2) {
    const int64_t j = i - n1, n = j / kl, c = (j % kl) % rpad;
    l2t[j] = c < R ? l2[c * N + n] : (uint16_t)0;
  }
}

}  // namespace

hipError_t launch_gemm_fp8r(const uint8_t* xq, const float* xs, const uint8_t* w, const float* ws, int64_t M,
                            int64_t K, int64_t N, uint16_t* y, hipStream_t stream) {
  const int tm = (int)((M + 255) / 256), tn = (int)((N + 255) / 256);
  hipLaunchKernelGGL(k_gemm_fp8r, dim3((unsigned)(tm * tn)), dim3(256), 0, stream, xq, xs, w, ws, M, K, N, y, tm,
                     tn);
  return hipGetLastError();
}

hipError_t launch_gemm_nvfp4(const uint16_t* xe, const uint16_t* we, float gscale, int64_t M, int64_t K, int64_t N,
                             LowRank lr, uint16_t* y, hipStream_t stream) {
  const int tm = (int)((M + 255) / 256), tn = (int)((N + 255) / 256);
  const dim3 grid((unsigned)(tm * tn)), block(256);
  if (lr.kl > 0)
    hipLaunchKernelGGL(k_gemm_nvfp4<true>, grid, block, 0, stream, xe, we, gscale, M, K, N, lr.t, lr.l2t, lr.kl, y,
                       tm, tn);
  else
    hipLaunchKernelGGL(k_gemm_nvfp4<false>, grid, block, 0, stream, xe, we, gscale, M, K, N, lr.t, lr.l2t, lr.kl, y,
                       tm, tn);
  return hipGetLastError();
}

hipError_t launch_lowrank_prep(const uint16_t* l1, const uint16_t* l2, int64_t K, int64_t N, int64_t R, int64_t kl,
                               uint16_t* l1t, uint16_t* l2t, hipStream_t stream) {
  const int64_t rpad = kl / 2;
  const int64_t ntr = rpad * K + N * kl;
  hipLaunchKernelGGL(k_lowrank_transpose, dim3((unsigned)((ntr + 255) / 256)), dim3(256), 0, stream, l1, l2, K, N, R,
                     rpad, kl, l1t, l2t);
  return hipGetLastError();
}

}  // namespace qpl
