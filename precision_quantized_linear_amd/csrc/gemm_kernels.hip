// Quantized GEMMs for gfx950 (CDNA4): y[M,N] = x[M,K] * W[N,K]^T, fp32 accumulation
// in the MFMA units, bf16 output rounded to nearest even.
//
// fp8r (Diffusers guide "BFL (fp8r / nvfp4)", "Kernels" table, fp8r row): E4M3 x
// E4M3 on the f8f6f4 MFMA (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with unit E8M0 scales),
// epilogue (acc * s_x[m]) * s_w[n].
//
// nvfp4 ("Kernels" table, nvfp4 row): the guide's kernel is a block-scaled FP4
// GEMM with one E4M3 scale per 16 elements.  gfx950's scaled MFMA takes one
// power-of-two (E8M0) scale per 32 elements, and a code times an E4M3 scale needs
// up to 6 significant bits, which no 8-, 6- or 4-bit operand format holds.  The
// exact route taken here expands each value e2m1(code) * dec(sf) to bf16 (exact)
// and runs the bf16 MFMA (V_MFMA_F32_32X32X16_BF16): activations arrive already
// expanded from the quantize kernel, weight codes stay packed in HBM and are
// expanded once per workgroup tile while being staged into LDS.  The global
// factor input_scale * weight_scale_2 and the optional SVDQuant low-rank term
// (Nunchaku post, "Background: SVDQuant and Nunchaku": up-projection fused into
// the 4-bit GEMM) are applied in the fp32 accumulators before the bf16 rounding.
//
// Tiling: a 256-thread workgroup (4 wavefronts, 2 x 2) owns a 256 x 256 output
// tile; each wavefront owns 128 x 128 (16 MFMA tiles of 32 x 32, 256 fp32
// accumulators per lane, one wavefront per SIMD).  Each K-step stages a 256-row x
// 128-byte slab of both operands in LDS (fp8: 128 elements, bf16: 64 elements),
// double-buffered (128 KB of the 160 KB LDS), with the 16-byte chunks of a row
// XOR-swizzled so the MFMA operand reads are bank-conflict free.  The output tile
// is transposed through LDS so every global store is a 16-byte row segment.
#include "qpl_device.h"
#include "qpl_internal.h"

namespace qpl {

namespace {

constexpr int TM = 256;        // tile rows (M)
constexpr int TN = 256;        // tile columns (N)
constexpr int ROWB = 128;      // bytes per LDS slab row
constexpr int SLAB = TM * ROWB;  // 32 KB per operand per stage
constexpr int LDS_BYTES = 4 * SLAB;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int ch) { return r * ROWB + ((ch ^ swz(r)) << 4); }

// 256 rows x 128 bytes of a row-major byte matrix (pitch bytes per row), rows and
// bytes beyond the limits read as zero.  Thread t loads chunk t % 8 of rows
// t / 8 + 32 i, so eight consecutive threads read one 128-byte row segment.
struct Slab {
  u32x4 v[8];
};

__device__ __forceinline__ void load_slab(Slab& s, const uint8_t* __restrict__ base, int64_t pitch,
                                          int64_t rows_left, int64_t bytes_left, int t) {
  const int ch = t & 7;
  const bool kin = (int64_t)ch * 16 < bytes_left;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = i * 32 + (t >> 3);
    if (kin && r < rows_left)
      s.v[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)r * pitch + ch * 16);
    else
      s.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_slab(const Slab& s, uint8_t* lds, int t) {
  const int ch = t & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(lds + lds_off(i * 32 + (t >> 3), ch)) = s.v[i];
}

typedef f32x16 Acc[4][4];

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
}

// One 128-element fp8 K-step: two 32x32x64 sub-steps.  Lane l holds row (l % 32)
// of its 32-row fragment and the 32 K-values 64 s + 32 (l / 32) + [0, 32); the B
// operand holds the same K-values, so each MFMA sums a complete 64-wide K range.
__device__ __forceinline__ void mma_fp8(const uint8_t* lA, const uint8_t* lB, Acc& acc, int wm, int wn,
                                        int lane) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    i32x8 a[4], b[4];
    const int c0 = 4 * s + 2 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 128 + i * 32 + (lane & 31);
      const u32x4 lo = *reinterpret_cast<const u32x4*>(lA + lds_off(ra, c0));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(lA + lds_off(ra, c0 + 1));
      a[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int rb = wn * 128 + i * 32 + (lane & 31);
      const u32x4 lo2 = *reinterpret_cast<const u32x4*>(lB + lds_off(rb, c0));
      const u32x4 hi2 = *reinterpret_cast<const u32x4*>(lB + lds_off(rb, c0 + 1));
      b[i] = i32x8{(int)lo2.x, (int)lo2.y, (int)lo2.z, (int)lo2.w, (int)hi2.x, (int)hi2.y, (int)hi2.z, (int)hi2.w};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 127, 0, 127);
  }
}

// One 64-element bf16 K-step: four 32x32x16 sub-steps, lane l holding the 8
// K-values 16 s + 8 (l / 32) + [0, 8) of its row.
__device__ __forceinline__ void mma_bf16(const uint8_t* lA, const uint8_t* lB, Acc& acc, int wm, int wn,
                                         int lane) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 a[4], b[4];
    const int c = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *reinterpret_cast<const bf16x8*>(lA + lds_off(wm * 128 + i * 32 + (lane & 31), c));
      b[i] = *reinterpret_cast<const bf16x8*>(lB + lds_off(wn * 128 + i * 32 + (lane & 31), c));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Packed E2M1 weight slab for one K-step of 64 elements: thread t owns weight row
// n0 + t (32 bytes of codes and 4 block-scale bytes).
struct Fp4Slab {
  uint32_t c[8];
  uint32_t s;
};

template <bool ALIGNED>
__device__ __forceinline__ void load_fp4(Fp4Slab& f, const uint8_t* __restrict__ w, const uint8_t* __restrict__ wbs,
                                         int64_t K, int64_t n, int64_t N, int64_t k0) {
  if (n >= N) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f.c[i] = 0u;
    f.s = 0u;
    return;
  }
  if constexpr (ALIGNED) {  // K % 64 == 0: rows 32-byte aligned, K-steps always full
    const u32x4* src = reinterpret_cast<const u32x4*>(w + n * (K / 2) + k0 / 2);
    const u32x4 a = src[0], b = src[1];
    f.c[0] = a.x; f.c[1] = a.y; f.c[2] = a.z; f.c[3] = a.w;
    f.c[4] = b.x; f.c[5] = b.y; f.c[6] = b.z; f.c[7] = b.w;
    f.s = *reinterpret_cast<const uint32_t*>(wbs + n * (K / 16) + k0 / 16);
  } else {  // K % 16 == 0 only: byte loads, blocks past K read as zero
    const uint8_t* row = w + n * (K / 2);
    const uint8_t* srow = wbs + n * (K / 16);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t v = 0;
      if (k0 + 8 * q < K) {
#pragma unroll
        for (int b = 0; b < 4; ++b) v |= (uint32_t)row[(k0 + 8 * q) / 2 + b] << (8 * b);
      }
      f.c[q] = v;
    }
    uint32_t s = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (k0 + 16 * b < K) s |= (uint32_t)srow[k0 / 16 + b] << (8 * b);
    f.s = s;
  }
}

// Upper halves of two floats whose values are exact in bf16: (lo, hi) packed.
__device__ __forceinline__ uint32_t pack_bf16_hi(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Expand 64 packed codes of one weight row to bf16 e2m1(code) * dec(sf) (exact)
// and write them as 8 swizzled 16-byte chunks of LDS row t.  The hardware
// conversion applies only the exponent of its scale operand, so it runs with
// scale 1 and the E4M3 block scale is multiplied in fp32 (exact product); the
// upper halves of the fp32 results are then the bf16 values.
__device__ __forceinline__ void store_fp4_expanded(const Fp4Slab& f, uint8_t* lB, int t) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float sf = e4m3_decode((f.s >> (8 * (q >> 1))) & 0xFFu);
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f.c[q], 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f.c[q], 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f.c[q], 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(f.c[q], 1.0f, 3);
    const uint32_t o[4] = {pack_bf16_hi(v0[0] * sf, v0[1] * sf), pack_bf16_hi(v1[0] * sf, v1[1] * sf),
                           pack_bf16_hi(v2[0] * sf, v2[1] * sf), pack_bf16_hi(v3[0] * sf, v3[1] * sf)};
    *reinterpret_cast<u32x4*>(lB + lds_off(t, q)) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

// Write the 256 x 256 tile: scale in fp32, round to bf16, transpose through LDS,
// then store 16-byte row segments (element stores when N % 8 != 0).
template <class Scale>
__device__ __forceinline__ void epilogue(Acc& acc, uint8_t* lds, int wm, int wn, int lane, int t, int64_t m0,
                                         int64_t n0, int64_t M, int64_t N, uint16_t* __restrict__ y,
                                         const Scale& scale) {
  uint16_t* ly = reinterpret_cast<uint16_t*>(lds);
  __syncthreads();
  float fc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) fc[j] = scale.col(wn * 128 + j * 32 + (lane & 31));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const float fr = scale.row(row);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = wn * 128 + j * 32 + (lane & 31);
        ly[row * TN + col] = (uint16_t)f32_to_bf16((acc[i][j][r] * fr) * fc[j]);
      }
    }
  __syncthreads();
  const bool vec = (N % 8) == 0;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int c = it * 256 + t;
    const int row = c >> 5, ch = c & 31;
    const int64_t gm = m0 + row, gn = n0 + ch * 8;
    if (gm >= M || gn >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ly + row * TN + ch * 8);
    if (vec) {
      *reinterpret_cast<u32x4*>(y + gm * N + gn) = v;
    } else {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (gn + e < N) y[gm * N + gn + e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Tile order: workgroups are dispatched round-robin over the 8 XCDs, so give each
// XCD a contiguous run of tiles (row-major over the tile grid) to share its L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int64_t& m0, int64_t& n0) {
  const int T = tiles_m * tiles_n;
  int b = blockIdx.x;
  if ((T & 7) == 0) b = (b & 7) * (T >> 3) + (b >> 3);
  m0 = (int64_t)(b / tiles_n) * TM;
  n0 = (int64_t)(b % tiles_n) * TN;
}

// Output scaling y = (acc * row(m)) * col(n).
struct RowColScale {
  const float* sa;
  const float* sb;
  int64_t m0, n0, M, N;
  __device__ float row(int r) const { return m0 + r < M ? sa[m0 + r] : 0.0f; }
  __device__ float col(int c) const { return n0 + c < N ? sb[n0 + c] : 0.0f; }
};

struct UniformScale {
  float g;
  __device__ float row(int) const { return g; }
  __device__ float col(int) const { return 1.0f; }
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_fp8r(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ B,
    const float* __restrict__ sb, int64_t M, int64_t K, int64_t N, uint16_t* __restrict__ Y, int tiles_m,
    int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
  int64_t m0, n0;
  tile_coords(tiles_m, tiles_n, m0, n0);
  const uint8_t* Ab = A + m0 * K;
  const uint8_t* Bb = B + n0 * K;
  const int64_t nk = (K + ROWB - 1) / ROWB;
  Acc acc;
  zero_acc(acc);
  Slab ra, rb;
  load_slab(ra, Ab, K, M - m0, K, t);
  load_slab(rb, Bb, K, N - n0, K, t);
  store_slab(ra, lds, t);
  store_slab(rb, lds + SLAB, t);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * 2 * SLAB;
    uint8_t* nxt = lds + ((kt + 1) & 1) * 2 * SLAB;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t k1 = (kt + 1) * ROWB;
      load_slab(ra, Ab + k1, K, M - m0, K - k1, t);
      load_slab(rb, Bb + k1, K, N - n0, K - k1, t);
    }
    mma_fp8(cur, cur + SLAB, acc, wm, wn, lane);
    if (more) {
      store_slab(ra, nxt, t);
      store_slab(rb, nxt + SLAB, t);
    }
    __syncthreads();
  }
  epilogue(acc, lds, wm, wn, lane, t, m0, n0, M, N, Y, RowColScale{sa, sb, m0, n0, M, N});
}

template <bool ALIGNED, bool LOWRANK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_nvfp4(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ W, const uint8_t* __restrict__ Wbs, float gscale,
    int64_t M, int64_t K, int64_t N, const uint16_t* __restrict__ T, const uint16_t* __restrict__ L2t, int64_t KL,
    uint16_t* __restrict__ Y, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w >> 1, wn = w & 1;
  int64_t m0, n0;
  tile_coords(tiles_m, tiles_n, m0, n0);
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(A + m0 * K);
  const int64_t kb = 2 * K;  // bytes per activation row
  const int64_t nk = (K + 63) / 64;
  Acc acc;
  zero_acc(acc);
  Slab ra;
  Fp4Slab fw;
  load_slab(ra, Ab, kb, M - m0, kb, t);
  load_fp4<ALIGNED>(fw, W, Wbs, K, n0 + t, N, 0);
  store_slab(ra, lds, t);
  store_fp4_expanded(fw, lds + SLAB, t);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * 2 * SLAB;
    uint8_t* nxt = lds + ((kt + 1) & 1) * 2 * SLAB;
    const bool more = kt + 1 < nk;
    if (more) {
      load_slab(ra, Ab + (kt + 1) * ROWB, kb, M - m0, kb - (kt + 1) * ROWB, t);
      load_fp4<ALIGNED>(fw, W, Wbs, K, n0 + t, N, (kt + 1) * 64);
    }
    mma_bf16(cur, cur + SLAB, acc, wm, wn, lane);
    if (more) {
      store_slab(ra, nxt, t);
      store_fp4_expanded(fw, nxt + SLAB, t);
    }
    __syncthreads();
  }
  float oscale = gscale;
  if constexpr (LOWRANK) {
    // SVDQuant up-projection: acc = g * acc + [T_hi | T_lo] [L2^T | L2^T]^T, in fp32.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] *= gscale;
    const uint8_t* Tb = reinterpret_cast<const uint8_t*>(T + m0 * KL);
    const uint8_t* Lb = reinterpret_cast<const uint8_t*>(L2t + n0 * KL);
    const int64_t lb = 2 * KL;
    Slab rl;
    for (int64_t k1 = 0; k1 < lb; k1 += ROWB) {
      load_slab(ra, Tb + k1, lb, M - m0, lb - k1, t);
      load_slab(rl, Lb + k1, lb, N - n0, lb - k1, t);
      store_slab(ra, lds, t);
      store_slab(rl, lds + SLAB, t);
      __syncthreads();
      mma_bf16(lds, lds + SLAB, acc, wm, wn, lane);
      __syncthreads();
    }
    oscale = 1.0f;
  }
  epilogue(acc, lds, wm, wn, lane, t, m0, n0, M, N, Y, UniformScale{oscale});
}

// T = x L1 for the low-rank branch: one workgroup per 32 rows x 32 rank columns,
// the four wavefronts split K and their partial sums meet in LDS.  T is stored
// split into a bf16 high part and a bf16 remainder ([hi | lo], KL columns per row)
// so the GEMM epilogue can apply it on the bf16 MFMA while keeping ~16 bits.
__global__ __launch_bounds__(256) void k_lowrank_t(const uint16_t* __restrict__ x, const uint16_t* __restrict__ l1t,
                                                   int64_t M, int64_t K, int64_t rpad, int64_t kl,
                                                   uint16_t* __restrict__ t_out) {
  __shared__ float red[4][16 * 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 32, c0 = (int64_t)blockIdx.y * 32;
  const int64_t row = m0 + (lane & 31);
  f32x16 acc = {};
  const int64_t nsteps = K / 16;
  for (int64_t s = wv; s < nsteps; s += 4) {
    const int64_t k = s * 16 + g * 8;
    bf16x8 a = {};
    if (row < M) a = *reinterpret_cast<const bf16x8*>(x + row * K + k);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(l1t + (c0 + (lane & 31)) * K + k);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wv][r * 64 + lane] = acc[r];
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float v = ((red[0][r * 64 + lane] + red[1][r * 64 + lane]) + red[2][r * 64 + lane]) + red[3][r * 64 + lane];
    const int64_t m = m0 + (r >> 2) * 8 + g * 4 + (r & 3);
    if (m >= M) continue;
    const uint32_t hi = f32_to_bf16(v);
    const uint32_t lo = f32_to_bf16(v - __uint_as_float(hi << 16));
    t_out[m * kl + c0 + (lane & 31)] = (uint16_t)hi;
    t_out[m * kl + rpad + c0 + (lane & 31)] = (uint16_t)lo;
  }
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
  const int tm = (int)((M + TM - 1) / TM), tn = (int)((N + TN - 1) / TN);
  hipLaunchKernelGGL(k_gemm_fp8r, dim3((unsigned)(tm * tn)), dim3(256), 0, stream, xq, xs, w, ws, M, K, N, y, tm,
                     tn);
  return hipGetLastError();
}

hipError_t launch_gemm_nvfp4(const uint16_t* xe, const uint8_t* w, const uint8_t* wbs, float gscale, int64_t M,
                             int64_t K, int64_t N, LowRank lr, uint16_t* y, hipStream_t stream) {
  const int tm = (int)((M + TM - 1) / TM), tn = (int)((N + TN - 1) / TN);
  const dim3 grid((unsigned)(tm * tn)), block(256);
#define QPL_NVFP4_GEMM(AL, LR)                                                                                   \
  hipLaunchKernelGGL((k_gemm_nvfp4<AL, LR>), grid, block, 0, stream, xe, w, wbs, gscale, M, K, N, lr.t, lr.l2t, \
                     lr.kl, y, tm, tn)
  const bool aligned = K % 64 == 0, lowrank = lr.kl > 0;
  if (aligned && !lowrank) QPL_NVFP4_GEMM(true, false);
  else if (aligned) QPL_NVFP4_GEMM(true, true);
  else if (!lowrank) QPL_NVFP4_GEMM(false, false);
  else QPL_NVFP4_GEMM(false, true);
#undef QPL_NVFP4_GEMM
  return hipGetLastError();
}

hipError_t launch_lowrank_prep(const uint16_t* x, const uint16_t* l1, const uint16_t* l2, int64_t M, int64_t K,
                               int64_t N, int64_t R, int64_t kl, uint16_t* l1t, uint16_t* t, uint16_t* l2t,
                               hipStream_t stream) {
  const int64_t rpad = kl / 2;
  const int64_t ntr = rpad * K + N * kl;
  hipLaunchKernelGGL(k_lowrank_transpose, dim3((unsigned)((ntr + 255) / 256)), dim3(256), 0, stream, l1, l2, K, N, R,
                     rpad, kl, l1t, l2t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lowrank_t, dim3((unsigned)((M + 31) / 32), (unsigned)(rpad / 32)), dim3(256), 0, stream, x,
                     l1t, M, K, rpad, kl, t);
  return hipGetLastError();
}

}  // namespace qpl
