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
// exact route taken here: both operands travel packed (E2M1 codes and E4M3 block
// scales) into LDS, and each lane expands its own fragments in registers to f16
// values e2m1(code) * dec(sf) (exact) for the f16 MFMA
// (V_MFMA_F32_32X32X16_F16).  The global factor input_scale * weight_scale_2
// scales the fp32 accumulators; the optional SVDQuant low-rank term (Nunchaku
// post, "Background: SVDQuant and Nunchaku": the up-projection fused into the
// GEMM) then adds T L2 to them on the bf16 MFMA, before the single bf16 rounding.
//
// Common to the fp8r and nvfp4 GEMMs (the INT4 GEMM at the end of the file has a
// ring of its own, described there):
// * a 256-thread workgroup (4 wavefronts, 2 x 2) owns a 256 x 256 output tile; a
//   wavefront owns 128 x 128 (16 MFMA tiles of 32 x 32, 256 fp32 accumulators
//   per lane in AGPRs, one wavefront per SIMD);
// * workgroups are persistent and walk an XCD-grouped tile order; the tail tiles
//   of the last round are split into 128-row halves;
// * K is walked in pairs of slabs whose rows are whole 128-byte lines; two stages
//   ring through the LDS, and a pair's loads (buffer_load_dwordx4 ... lds, no
//   register staging) are issued one after an MFMA while the previous pair is
//   multiplied; rows past the matrix and bytes past K read as zero through the
//   buffer range check;
// * chunk c of a 128-byte stage row r sits at chunk c ^ (r % 8), which keeps the
//   16-byte operand reads of a wavefront on distinct banks;
// * operands are swapped (the MFMA computes y^T), so each lane ends with runs of
//   four consecutive output columns of a row; lanes l and l + 32 swap halves
//   (V_PERMLANE32_SWAP) and each stores eight consecutive columns as one 16-byte
//   segment.
#include <type_traits>

#include "qpl_dma.h"
#include "qpl_internal.h"

namespace qpl {

namespace {

constexpr int SROW = 64;            // bytes per slab row of the INT4 GEMM (one 64-channel group)
constexpr int NST = 4;              // slabs per tile from which workgroups are persistent

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 3; }
__device__ __forceinline__ int soff(int r, int c) { return r * SROW + ((c ^ swz(r)) << 4); }

typedef f32x16 Acc[4][4];

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
}

// Rows of a 256-row tile that lie inside the matrix (rows_left = rows from the
// tile's first row to the matrix end).
__device__ __forceinline__ int64_t M_rows(int64_t rows_left) { return rows_left < 256 ? rows_left : 256; }

// MFMA operands.  fp8: a 32x32x64 MFMA operand (32 K-bytes per lane).  bf16: a
// 32x32x16 MFMA operand (8 K-values per lane, one 16-byte chunk); a 64-byte slab
// holds two of them (sub-steps).
struct Fp8Mma {
  typedef i32x8 Frag;
  static __device__ __forceinline__ f32x16 mma(const Frag& w, const Frag& x, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, c, 0, 0, 0, 127, 0, 127);
  }
};

struct Bf16Mma {
  typedef bf16x8 Frag;
  static __device__ __forceinline__ Frag read(const uint8_t* slab, int row, int sub, int lane) {
    return *reinterpret_cast<const bf16x8*>(slab + soff(row, 2 * sub + (lane >> 5)));
  }
  static __device__ __forceinline__ f32x16 mma(const Frag& w, const Frag& x, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, x, c, 0, 0, 0);
  }
};

// Tile order.  The tile sequence walks groups of GROUP_M tile-rows column by column.
// Workgroups are dispatched round-robin over the 8 XCDs and each XCD has its own
// L2, so in every round of the persistent loop the 32 workgroups of one XCD take a
// contiguous run of 32 tiles of the sequence: a 4 x 8 block that shares 4
// activation slabs and 8 weight slabs in that XCD's L2.
constexpr int GROUP_M = 4;

// tm: rows of x per tile (256, or 128 for the INT4 GEMM); tiles are 256 columns wide.
__device__ __forceinline__ void tile_coords(int s, int tiles_m, int tiles_n, int64_t& m0, int64_t& n0,
                                            int tm = 256) {
  const int per_group = GROUP_M * tiles_n;
  const int g = s / per_group;
  const int first_m = g * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int r = s - g * per_group;
  m0 = (int64_t)(first_m + r % gm) * tm;
  n0 = (int64_t)(r / gm) * 256;
}

// Position in the tile sequence of workgroup b's i-th tile (nwg workgroups).
__device__ __forceinline__ int tile_seq(int i, int b, int nwg) {
  return (nwg & 7) == 0 ? i * nwg + (b & 7) * (nwg >> 3) + (b >> 3) : i * nwg + b;
}

// What the GEMM kernels multiply.  Pass 1: rows of x (a) and of W (w), pitch1
// bytes apart, kbytes1 valid bytes each.  Pass 2 (the low-rank up-projection):
// rows of [T_hi | T_lo] and [L2^T | L2^T].
// Tile sequence positions [0, nfull) are computed whole; each of the ntail tiles
// after them is computed as two 128-row halves by workgroups 2j and 2j + 1.
struct GemmArgs {
  const uint8_t* a;
  const uint8_t* w;
  const uint8_t* a2;
  const uint8_t* w2;
  int64_t M, N;
  int pitch1, kbytes1, pitch2, kbytes2;
  int tiles_m, tiles_n, ntiles, nwg, nfull, ntail;
};

constexpr int NSTORE = 32;           // 16-byte output stores per wave per tile (fast path)
constexpr int SCALE_BUF = 2048;      // per tile parity: s_x of the tile's 256 rows, then s_w of its 256 columns

// f(integral_constant<int, I>) for I = B .. E - 1, expanded at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Epilogue kinds (bit flags; the Nunchaku post, "Introducing Nunchaku Lite", names
// fused QKV projections and fused GELU/MLP kernels as the model-specific paths of
// its original engine):
// * EPI_GELU: the tanh form of GELU on each fp32 result before the bf16 rounding;
// * EPI_QKV: the output row's three parts (columns [0, d), [d, 2d), [2d, 3d)) go to
//   three tensors [heads, tokens, head_dim] at a token offset, the layout attention
//   reads, instead of the row-major y.
constexpr int EPI_GELU = 1, EPI_QKV = 2;

struct EpiArgs {
  uint16_t* qkv[3];  // EPI_QKV: q, k, v
  int64_t d;         // EPI_QKV: columns per part (heads * head_dim)
  int64_t tokens;    // EPI_QKV: tokens per head
  int64_t off;       // EPI_QKV: token of output row 0
  int lg_hd;         // EPI_QKV: log2(head_dim)
};
// GELU, tanh form: v sigma(2u) with u = sqrt(2/pi) (v + 0.044715 v^3), since
// (1 + tanh u) / 2 = 1 / (1 + exp(-2u)).  exp2 and the reciprocal run on the
// transcendental unit; the exponent is t = -2 u log2(e) = v (C1 + C3 v^2).  Large
// negative v gives t = +inf and a result of -0; large positive v gives v.
constexpr float GELU_C1 = -0x1.26aec2p+1f;  // -2 sqrt(2/pi) log2(e), -2.3022082
constexpr float GELU_C3 = -0x1.a5a7d0p-4f;  // GELU_C1 * 0.044715, -0.10294324
__device__ __forceinline__ float gelu_tanh(float v) {
  const float t = v * __builtin_fmaf(GELU_C3, v * v, GELU_C1);
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// Destination of output element (m, n): y[m, n], or under EPI_QKV element
// n mod head_dim of head (n mod d) / head_dim of part n / d at token off + m.
template <int EPI>
__device__ __forceinline__ uint16_t* out_ptr(uint16_t* __restrict__ y, int64_t m, int64_t n, int64_t N,
                                             const EpiArgs& e) {
  if constexpr ((EPI & EPI_QKV) != 0) {
    const int part = (n >= e.d) + (n >= 2 * e.d);
    const int64_t c = n - part * e.d;
    const int64_t h = c >> e.lg_hd;
    return e.qkv[part] + (((h * e.tokens + e.off + m) << e.lg_hd) + (c & ((int64_t{1} << e.lg_hd) - 1)));
  } else {
    return y + m * N + n;
  }
}

// Epilogue of one tile: y = bf16(act((acc * rs(m)) * cs(n))), then the EPI output
// transform.  acc[i][j] holds y^T: its
// element r at lane l is row m = m0 + 128 wm + 32 j + l % 32, column
// n = n0 + 128 wn + 32 i + 8 (r / 4) + 4 (l / 32) + r % 4.  Lanes l and l + 32
// exchange halves (V_PERMLANE32_SWAP) so that each lane holds eight consecutive
// columns of one row and stores them as one 16-byte segment.  NJ: 32-row blocks
// per wavefront (4 for a 256-row tile, 2 for a 128-row half tile, whose rows are
// m0 + 64 wm + 32 j + l % 32); NI: 32-column blocks per wavefront (4: columns
// n0 + 128 wn + ..., wn in 0..1; 2: n0 + 64 wn + ..., wn in 0..3).  Returns the
// number of store instructions left in flight: 2 NJ NI on the interior path, 0 on
// the edge path (which checks every element and drains its stores).
template <int NJ, int NI, int EPI, bool FAST, class RowScale, class ColScale>
__device__ __forceinline__ void store_tile_path(const Acc& acc, int wm, int wn, int lane, int64_t m0, int64_t n0,
                                                int64_t M, int64_t N, uint16_t* __restrict__ y, const RowScale& rs,
                                                const ColScale& cs, const EpiArgs& e) {
  // unrolled at compile time: with a heavy epilogue the body exceeds what the
  // unroll pragma accepts, and a rolled loop would index acc dynamically (scratch)
  static_for<0, NJ>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    const int mr = wm * 32 * NJ + j * 32 + (lane & 31);
    const float fr = rs(mr);
    const int64_t m = m0 + mr;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        uint32_t w[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int g = 2 * gp + h;
          const f32x4 fc = cs(wn * 32 * NI + i * 32 + g * 8 + (lane >> 5) * 4);
          const f32x16& a = acc[i][j];
          float o[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            o[c] = (a[g * 4 + c] * fr) * fc[c];
            if constexpr ((EPI & EPI_GELU) != 0) o[c] = gelu_tanh(o[c]);
          }
          w[h][0] = pack_bf16(o[0], o[1]);
          w[h][1] = pack_bf16(o[2], o[3]);
        }
        const auto r0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
        const u32x4 v = u32x4{r0[0], r1[0], r0[1], r1[1]};
        const int64_t n = n0 + wn * 32 * NI + i * 32 + (2 * gp + (lane >> 5)) * 8;
        // the segment's eight columns stay inside one head (head_dim >= 8, n % 8 == 0)
        uint16_t* dst = out_ptr<EPI>(y, m, n, N, e);
        if constexpr (FAST) {
          *reinterpret_cast<u32x4*>(dst) = v;
        } else if (m < M) {
          const uint32_t el[4] = {v.x, v.y, v.z, v.w};
          if ((N & 7) == 0 && n + 8 <= N) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int c = 0; c < 8; ++c)
              if (n + c < N) dst[c] = (uint16_t)(el[c >> 1] >> (16 * (c & 1)));
          }
        }
      }
  });
}

template <int NJ, int NI = 4, int EPI = 0, class RowScale, class ColScale>
__device__ __forceinline__ int store_tile(const Acc& acc, int wm, int wn, int lane, int64_t m0, int64_t n0,
                                          int64_t M, int64_t N, uint16_t* __restrict__ y, const RowScale& rs,
                                          const ColScale& cs, const EpiArgs& e = EpiArgs{}) {
  // interior: the wavefront's rows and columns all inside the matrix; the two paths
  // are separate code, so the interior one has no per-segment branches
  const bool fast = m0 + (wm + 1) * 32 * NJ <= M && n0 + (wn + 1) * 32 * NI <= N && (N & 7) == 0;
  if (fast) {
    store_tile_path<NJ, NI, EPI, true>(acc, wm, wn, lane, m0, n0, M, N, y, rs, cs, e);
    return 2 * NJ * NI;
  }
  store_tile_path<NJ, NI, EPI, false>(acc, wm, wn, lane, m0, n0, M, N, y, rs, cs, e);
  QPL_WAIT_VMCNT(0);
  return 0;
}

// Persistent GEMMs (fp8r and nvfp4 below): workgroup b walks its tiles (tile_seq)
// one after the other, and the slabs of all of them form one stream through the
// LDS ring: the loads for the next tile's first slabs are issued while the current
// tile's last slabs are multiplied, and the current tile's output stores drain
// while the next tile's MFMAs run.  A wavefront's vector memory operations retire
// in issue order (loads and stores alike), so a wait for a slab's loads names how
// many later operations (loads of later slabs, epilogue stores) may stay in flight.

// ---------------------------------------------------------------------------
// fp8r GEMM (guide "BFL (fp8r / nvfp4)", "Kernels" table, fp8r row: a row-wise
// scaled FP8 GEMM).  256 x 256 tiles of 4 wavefronts (2 x 2, 128 x 128 each,
// sixteen 32 x 32 accumulators in AGPRs), V_MFMA_SCALE_F32_32X32X64_F8F6F4 with unit
// scales on the E4M3 codes, output scale s_x[m] s_w[n] in the epilogue.  A load moves 8 rows x
// 128 bytes (whole 128-byte lines) instead of 16 rows x 64 bytes: a stage holds two
// 64-byte slabs of both operands (256 rows x 128 bytes each, 64 KB), and two stages
// ring through 128 KB of LDS.  Loading half lines made every line two requests,
// and the load path, not the MFMAs, set the pace.
//
// Pair P (slabs 2P, 2P + 1) of the stream, in stage P % 2:
// * top: wait for pair P's loads (issued during pair P - 1; only the epilogue
//   stores issued after them may stay in flight), barrier (pair P is in LDS for
//   every wave, and every wave is done with pair P - 1, whose stage is free);
// * slab 2P: read its fragments, multiply, and issue pair P + 1's 16 loads per wave
//   into the free stage, one after each MFMA; read slab 2P + 1's fragments as slab
//   2P's are used up;
// * slab 2P + 1: multiply, and issue the next unit's output scales when pair P + 1
//   starts a unit.
// Within a stage row r holds its two slabs as eight 16-byte chunks; chunk c of row
// r sits at chunk c ^ (r % 8), so the eight lanes of a 16-byte LDS read pass hit
// eight different chunk positions.
// ---------------------------------------------------------------------------
constexpr int PR_ROW = 128;                      // bytes per row per stage (two slabs)
constexpr int PR_OPER = 256 * PR_ROW;            // 32 KB per operand per stage
constexpr int PR_STAGE = 2 * PR_OPER;            // x rows then W rows
constexpr int PR_LOADS = 16;                     // 1 KB loads per wave per pair

__device__ __forceinline__ int proff(int r, int c) { return r * PR_ROW + ((c ^ (r & 7)) << 4); }

template <int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_fp8r(
    GemmArgs p, const float* __restrict__ sa, const float* __restrict__ sb, uint16_t* __restrict__ Y, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * PR_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lsc[3 * SCALE_BUF];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wv >> 1, wn = wv & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int b = blockIdx.x;
  const uint32_t lbase = lds_address(lds);
  const uint32_t sbase = lds_address(lsc);

  // units: whole tiles at tile sequence positions tile_seq(0..nt - 1), then
  // (has_half) half u of the tail: rows 128 (u % 2) .. + 127 of tile nfull + u / 2
  int nt = 0;
  while (tile_seq(nt, b, p.nwg) < p.nfull) ++nt;
  const int hu = tile_seq(nt, b, p.nwg) - p.nfull;
  const bool has_half = hu < 2 * p.ntail;
  const int nu = nt + (has_half ? 1 : 0);
  const int np = (p.kbytes1 + PR_ROW - 1) / PR_ROW;  // pairs per unit
  struct Unit {
    int64_t m0, n0;
    int rows;
  };
  auto unit = [&](int ti) {
    Unit r;
    if (ti < nt) {
      tile_coords(tile_seq(ti, b, p.nwg), p.tiles_m, p.tiles_n, r.m0, r.n0);
      r.rows = 256;
    } else {
      tile_coords(p.nfull + (hu >> 1), p.tiles_m, p.tiles_n, r.m0, r.n0);
      r.m0 += 128 * (hu & 1);
      r.rows = 128;
    }
    return r;
  };

  // load q (0..7) of an operand: rows 64 wv + 8 q .. + 7; lane l writes row + l / 8,
  // stage chunk l % 8, which holds the row's chunk (l % 8) ^ (l / 8)
  const int lc = (lane & 7) ^ (lane >> 3);
  uint32_t vrow[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) vrow[q] = (uint32_t)((64 * wv + 8 * q + (lane >> 3)) * p.pitch1 + 16 * lc);

  struct PairSrc {
    u32x4 dx, dw, ds;
    int kb, koff, stage, tpar;
    bool first, valid;
  };
  int s_ti = 0, s_kp = 0, s_stage = 0;
  Unit s_u{0, 0, 256};
  if (nu > 0) s_u = unit(0);
  auto next_src = [&]() {
    PairSrc r;
    r.valid = s_ti < nu;
    r.stage = s_stage;
    r.first = s_kp == 0;
    r.tpar = s_ti & 1;
    r.kb = r.valid ? p.kbytes1 : 0;
    r.koff = s_kp * PR_ROW;
    const int64_t left = p.M - s_u.m0;
    const int64_t rm = left < 0 ? 0 : (left < s_u.rows ? left : s_u.rows);
    const int64_t rn = M_rows(p.N - s_u.n0);
    r.dx = make_desc(p.a + s_u.m0 * p.pitch1, rm * p.pitch1);
    r.dw = make_desc(p.w + s_u.n0 * p.pitch1, rn * p.pitch1);
    const bool row = wv < 2;
    r.ds = make_desc(row ? sa + s_u.m0 : sb + s_u.n0, (row ? rm : rn) * 4);
    s_stage ^= 1;
    if (++s_kp == np) {
      s_kp = 0;
      ++s_ti;
      if (s_ti < nu) s_u = unit(s_ti);
    }
    return r;
  };
  // load d of a pair: 0..7 x rows, 8..15 W rows
  auto issue = [&](const PairSrc& s, int d) {
    const int q = d & 7;
    const bool wl = d >= 8;
    const uint32_t dst = lbase + s.stage * PR_STAGE + (wl ? PR_OPER : 0) + (8 * wv + q) * 1024;
    const uint32_t vo = s.koff + 16 * lc < s.kb ? vrow[q] : kOutOfRange;
    dma16(dst, vo, wl ? s.dw : s.dx, s.koff);
  };
  // the unit's output scales: wave w moves 128 floats of s_x (w = 0, 1) or s_w
  // (w = 2, 3), 64 per load.  Every pair issues the two loads (out of range into a
  // spare area unless the pair starts a unit): a branch here would let the compiler
  // move the MFMAs around it
  auto issue_scales = [&](const PairSrc& s, int hh) {
    const bool real = s.valid && s.first;
    const uint32_t dst = sbase + (real ? s.tpar * SCALE_BUF : 2 * SCALE_BUF) + wv * 512 + hh * 256;
    const uint32_t vo = real ? (uint32_t)(((wv & 1) * 128 + hh * 64 + lane) * 4) : kOutOfRange;
    dma4(dst, vo, s.ds, 0);
  };

  typedef Fp8Mma::Frag Frag;
  Frag fw[4], fx[4];
  auto frag = [&](const uint8_t* st, int row, int u) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(st + proff(row, 4 * u + 2 * h));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(st + proff(row, 4 * u + 2 * h + 1));
    return Frag{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  // prologue: pair 0 (and unit 0's scales)
  int st1 = 0;  // output stores in flight from the epilogue after the previous pair
  {
    const PairSrc src = next_src();
#pragma unroll
    for (int d = 0; d < PR_LOADS; ++d) issue(src, d);
    issue_scales(src, 0);
    issue_scales(src, 1);
  }
  int cur = 0;  // stage of the pair being multiplied

  // One pair of a unit with NJ x tile-rows per wave (4 whole, 2 half).
  auto pair = [&](Acc& acc, auto nj) {
    constexpr int NJ = decltype(nj)::value;
    if (st1 == NSTORE) {
      QPL_WAIT_VMCNT(NSTORE);
    } else {
      QPL_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    st1 = 0;
    const PairSrc src = next_src();
    const uint8_t* cs = lds + cur * PR_STAGE;
    cur ^= 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) fw[i] = frag(cs + PR_OPER, wn * 128 + i * 32 + r32, 0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fx[j] = frag(cs, wm * 32 * NJ + j * 32 + r32, 0);
    // slab 2P, with pair P + 1's loads and slab 2P + 1's fragment reads
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[i][j] = Fp8Mma::mma(fw[i], fx[j], acc[i][j]);
        const int k = NJ * i + j;
        if (i == 3) fx[j] = frag(cs, wm * 32 * NJ + j * 32 + r32, 1);
        if (j == NJ - 1) fw[i] = frag(cs + PR_OPER, wn * 128 + i * 32 + r32, 1);
        // one load after each MFMA (a half unit has 8 MFMAs per slab: two after each)
#pragma unroll
        for (int d = 0; d < PR_LOADS; ++d)
          if (k == (d * 4 * NJ) / PR_LOADS) issue(src, d);
        __builtin_amdgcn_sched_barrier(0);
      }
    // slab 2P + 1, x tile-rows outer: its first MFMAs need the fragments that slab
    // 2P freed first (all of W's, then x's in order)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i][j] = Fp8Mma::mma(fw[i], fx[j], acc[i][j]);
        if (i == 0 && j == 0) issue_scales(src, 0);
        if (i == 0 && j == 1) issue_scales(src, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  using Whole = std::integral_constant<int, 4>;
  using Half = std::integral_constant<int, 2>;
  auto run_unit = [&](int ti, auto nj) {
    constexpr int NJ = decltype(nj)::value;
    Acc acc;
    zero_acc(acc);
    for (int kp = 0; kp < np; ++kp) pair(acc, nj);
    const Unit un = unit(ti);
    const float* ls = reinterpret_cast<const float*>(lsc + (ti & 1) * SCALE_BUF);
    st1 = __builtin_amdgcn_readfirstlane(store_tile<NJ, 4, EPI>(
        acc, wm, wn, lane, un.m0, un.n0, p.M, p.N, Y, [&](int r) { return ls[r]; },
        [&](int c) { return *reinterpret_cast<const f32x4*>(&ls[256 + c]); }, e));
  };
  for (int ti = 0; ti < nt; ++ti) run_unit(ti, Whole{});
  if (has_half) run_unit(nt, Half{});
  QPL_WAIT_VMCNT(0);
  QPL_WAIT_LGKM0();
}

// ---------------------------------------------------------------------------
// nvfp4 GEMM on the packed operands (guide "BFL (fp8r / nvfp4)", "Kernels" table,
// nvfp4 row: the quantized tensors keep their storage format; Nunchaku post,
// "Background: SVDQuant and Nunchaku": the 4-bit GEMM carries the low-rank
// up-projection).  Both operands stay E2M1 codes (two per byte) with one E4M3
// scale per 16 elements all the way into LDS; each lane expands its own MFMA
// fragments in registers to f16 values e2m1(code) * dec(sf): the FP4 converter
// gives the code values and one packed f16 multiply applies the block scale.
// The product has at most 6 significant bits and lies in [2^-10, 2688], so the
// f16 value is exact, and so is each f16 x f16 product the MFMA forms
// (V_MFMA_F32_32X32X16_F16, fp32 accumulation).  input_scale * weight_scale_2
// scales the fp32 result.
//
// Tiling and schedule follow the fp8r GEMM (256 x 256 tiles, 4 wavefronts of
// 128 x 128, persistent workgroups, XCD-grouped tile order, half tiles in the
// last round, y^T epilogue, slab pairs moved as whole 128-byte lines), with these
// slabs and pairs:
// * a slab is 128 K elements: 64 code bytes per row and 8 block-scale bytes per row
//   (slab-major in global memory: [K/128][rows][8], zero past K/16, so one 1 KB
//   load moves 128 rows' scales of one slab); a stage holds a pair of slabs of both
//   operands (codes 256 rows x 128 bytes per operand, scales two planes of 256 rows
//   x 8 bytes per operand, 72 KB), and two stages ring through 144 KB of LDS;
// * lane half h of a fragment row takes blocks 4h .. 4h + 3 of a slab: code bytes
//   32h .. 32h + 31 (two 16-byte LDS reads, four MFMA steps each) and one scale
//   dword.  MFMA step s (0..7) multiplies nibbles 8 (s % 2) .. + 7 of block
//   4h + s / 2; both operands use this order, so the pairs of a product are the
//   same k;
// * each step expands the next step's eight fragments while its 16 MFMAs run,
//   one MFMA then a share of the expansion in turn, into the other of two fragment
//   sets; the codes of the next group of four steps are read during the current
//   group, and each slab's scales one slab ahead;
// * pair P (16 steps) issues pair P + 1's loads during its first six steps (16 of
//   codes and 2 of scales per wave) into the other stage; at step 12 every wave
//   waits for them and meets at a barrier, after which pair P + 1 is in LDS for
//   every wave and every wave is done reading pair P's stage, so steps 12 .. 15
//   read pair P + 1's first codes and scales and expand its first step;
// * blocks past K have scale 0 (they multiply to 0 whatever codes straddle the row
//   end), rows past M or N read zeros through the buffer range check.
// LOWRANK: after the packed pairs of a tile the accumulators are multiplied by
// gscale, then bf16 pairs of [T_hi | T_lo] and [L2^T | L2^T] (128 bytes per row, four
// 32 x 32 x 16 steps) continue the same accumulation on the bf16 MFMA, so
// y = bf16(gscale x_q w_q^T + T L2) with T unscaled.
// ---------------------------------------------------------------------------
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int PK_CODES = 256 * PR_ROW;              // code bytes per operand per stage (two slabs)
constexpr int PK_PLANE = 256 * 8;                   // one slab's block scales per operand
constexpr int PK_SC = 2 * PK_PLANE;                 // both slabs' block scales per operand
constexpr int PK_STAGE = 2 * PK_CODES + 2 * PK_SC;  // [x codes][w codes][x scales][w scales]
constexpr int PK_LOADS = 18;                        // loads per wave per pair: 16 of codes, 2 of scales

struct PackedArgs {
  const uint8_t* xq;   // activation codes [M, K/2]
  const uint8_t* wq;   // weight codes [N, K/2]
  const uint8_t* xs;   // activation block scales [S, M, 8], S = ceil(K/128)
  const uint8_t* wsc;  // weight block scales [S, N, 8]
  const uint8_t* a2;   // low-rank pass: [T_hi | T_lo] bf16 [M, kl]
  const uint8_t* w2;   // [L2^T | L2^T] bf16 [N, kl]
  int64_t M, N;
  int cpitch;          // code bytes per row (K/2)
  int nk1;             // packed slabs per tile (S)
  int pitch2, kbytes2; // low-rank rows: 2 kl bytes
  int tiles_m, tiles_n, ntiles, nwg, nfull, ntail;
};

// Eight E2M1 codes (a dword, element 2i in the low nibble of byte i) times the
// pair s: f16 values code * s in element order.
__device__ __forceinline__ f16x8 fp4_expand(uint32_t cw, f16x2 s) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * s;
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * s;
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * s;
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * s;
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <bool LOWRANK, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_nvfp4(
    PackedArgs p, float gscale, uint16_t* __restrict__ Y, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * PK_STAGE];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wv >> 1, wn = wv & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int b = blockIdx.x;
  const uint32_t lbase = lds_address(lds);

  // units of work: whole tiles, then (has_half) one 128-row half of a leftover tile.
  // With the low-rank pass a workgroup takes one tile (the host launches one per
  // tile): the pass's extra state leaves no registers for the persistent loop.
  int nt = 0;
  if constexpr (LOWRANK) {
    nt = 1;
  } else {
    while (tile_seq(nt, b, p.nwg) < p.nfull) ++nt;
  }
  const int hu = LOWRANK ? 0 : tile_seq(nt, b, p.nwg) - p.nfull;
  const bool has_half = !LOWRANK && hu < 2 * p.ntail;
  const int nu = nt + (has_half ? 1 : 0);
  const int np1 = (p.nk1 + 1) >> 1;                             // packed pairs per unit
  const int np2 = LOWRANK ? (p.kbytes2 + PR_ROW - 1) / PR_ROW : 0;  // low-rank pairs
  const int npu = np1 + np2;
  struct Unit {
    int64_t m0, n0;
    int rows;
  };
  auto unit = [&](int ti) {
    Unit r;
    if (ti < nt) {
      tile_coords(tile_seq(ti, b, p.nwg), p.tiles_m, p.tiles_n, r.m0, r.n0);
      r.rows = 256;
    } else {
      tile_coords(p.nfull + (hu >> 1), p.tiles_m, p.tiles_n, r.m0, r.n0);
      r.m0 += 128 * (hu & 1);
      r.rows = 128;
    }
    return r;
  };

  // code loads q (0..7) of an operand: rows 64 wv + 8 q .. + 7 of the pair; lane l
  // writes row + l / 8, stage chunk l % 8, which holds the row's chunk (l % 8) ^ (l / 8)
  const int lc = (lane & 7) ^ (lane >> 3);
  uint32_t vo1[8], vo2[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int lrow = 64 * wv + 8 * q + (lane >> 3);
    vo1[q] = (uint32_t)(lrow * p.cpitch + 16 * lc);
    vo2[q] = LOWRANK ? (uint32_t)(lrow * p.pitch2 + 16 * lc) : 0u;
  }
  // scale loads: wave wv moves rows 128 (wv % 2) .. + 127 of operand wv / 2 (x, W),
  // one load per slab of the pair
  const bool sc_x = wv < 2;
  const int sc_r0 = 128 * (wv & 1);

  // The pair stream.  Its sources change only where it enters a unit or the unit's
  // low-rank pass: the code descriptors and the scale rows are worked out there;
  // from pair to pair the scale address moves by two slabs of scales.
  struct PairSrc {
    u32x4 dx, dw, ds0, ds1;
    int kb, koff, stage;
    bool pass2;
  };
  int s_ti = 0, s_kp = 0, s_stage = 0;
  Unit s_u{0, 0, 256};
  u32x4 s_dx{}, s_dw{};
  const uint8_t* s_sc = nullptr;  // this wave's scale bytes of the next pair's first slab
  int64_t s_scb = 0;              // their count: 8 per row present, 0 in a low-rank pass
  int s_kb = 0;
  const int64_t sstride = 8 * (sc_x ? p.M : p.N);
  auto enter = [&](bool pass2) {
    const int pitch = pass2 ? p.pitch2 : p.cpitch;
    const int64_t left = p.M - s_u.m0;
    const int64_t rm = left < 0 ? 0 : (left < s_u.rows ? left : s_u.rows);
    const int64_t rn = M_rows(p.N - s_u.n0);
    s_dx = make_desc((pass2 ? p.a2 : p.xq) + s_u.m0 * pitch, rm * pitch);
    s_dw = make_desc((pass2 ? p.w2 : p.wq) + s_u.n0 * pitch, rn * pitch);
    s_kb = pass2 ? p.kbytes2 : p.cpitch;
    const int64_t lim = (sc_x ? rm : rn) - sc_r0;
    s_scb = pass2 ? 0 : 8 * (lim < 0 ? 0 : (lim < 128 ? lim : 128));
    s_sc = (sc_x ? p.xs : p.wsc) + ((sc_x ? s_u.m0 : s_u.n0) + sc_r0) * 8;
  };
  if (nu > 0) {
    s_u = unit(0);
    enter(false);
  }
  auto next_src = [&]() {
    PairSrc r;
    r.stage = s_stage;
    r.pass2 = LOWRANK && s_kp >= np1;
    r.kb = s_kb;
    r.koff = (r.pass2 ? s_kp - np1 : s_kp) * PR_ROW;
    r.dx = s_dx;
    r.dw = s_dw;
    // the pair's second slab exists unless the unit has an odd number of slabs
    const bool two = r.pass2 || 2 * s_kp + 1 < p.nk1;
    r.ds0 = make_desc(s_sc, s_scb);
    r.ds1 = make_desc(s_sc + sstride, two ? s_scb : 0);
    s_sc += 2 * sstride;
    s_stage ^= 1;
    if (++s_kp == npu) {
      s_kp = 0;
      if (++s_ti < nu) {
        s_u = unit(s_ti);
        enter(false);
      } else {
        s_kb = 0;  // past the last unit: every load reads zeros
        s_scb = 0;
      }
    } else if (LOWRANK && s_kp == np1) {
      enter(true);
    }
    return r;
  };
  auto issue = [&](const PairSrc& s, int d) {
    const uint32_t st = lbase + s.stage * PK_STAGE;
    if (d < 16) {
      const int q = d & 7;
      const bool wl = d >= 8;
      const uint32_t vo = s.koff + 16 * lc < s.kb ? (LOWRANK && s.pass2 ? vo2[q] : vo1[q]) : kOutOfRange;
      dma16(st + (wl ? PK_CODES : 0) + (8 * wv + q) * 1024, vo, wl ? s.dw : s.dx, s.koff);
    } else {
      // 1 KB of one slab's scales (128 rows x 8 bytes); rows past the unit read zero
      const int u = d - 16;
      dma16(st + 2 * PK_CODES + (sc_x ? 0 : PK_SC) + u * PK_PLANE + sc_r0 * 8, (uint32_t)lane * 16u,
            u ? s.ds1 : s.ds0, 0);
    }
  };

  // fragment rows of tile-row t of a unit with nj x tile-rows: t < 4 W, t >= 4 x
  auto frow = [&](int t, int nj) { return t < 4 ? wn * 128 + t * 32 + r32 : wm * 32 * nj + (t - 4) * 32 + r32; };
  // codes of group g (steps 4 g .. 4 g + 3) of slab u of the pair in stage st, for
  // tile-rows t0 .. t0 + 3: one 16-byte chunk 4 u + 2 h + g per row
  auto read_codes = [&](const uint8_t* st, int nj, int u, int g, int t0, int ntr, u32x4 (&dst)[8]) {
#pragma unroll
    for (int t = t0; t < t0 + 4; ++t)
      if (t < ntr)
        dst[t] = *reinterpret_cast<const u32x4*>(st + (t < 4 ? PK_CODES : 0) + proff(frow(t, nj), 4 * u + 2 * h + g));
  };
  // block-scale dword (blocks 4 h .. 4 h + 3) of slab u of every tile-row
  auto read_scales = [&](const uint8_t* st, int nj, int u, uint32_t (&dst)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      dst[t] = *reinterpret_cast<const uint32_t*>(st + 2 * PK_CODES + (t < 4 ? PK_SC : 0) + u * PK_PLANE +
                                                  frow(t, nj) * 8 + 4 * h);
  };
  // Fragment sets F[s % 2], code groups CW[g % 2] (group g of the pair: slab g / 2,
  // steps 4 (g % 2) ..), scale dwords SC[u] of the pair's slab u.
  f16x8 F[2][8];
  u32x4 CW[2][8];
  uint32_t SC[2][8];
  // expand step s (0..15) of the pair into dst: the scale of the step's block is
  // one half of an f16 pair converted from two scale bytes, broadcast to both halves
  auto expand_step = [&](int s, f16x8 (&dst)[8], int ntr) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (t < ntr) {
        const f16x2 two = ((s >> 2) & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SC[s >> 3][t], 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(SC[s >> 3][t], 1.0f, false);
        const _Float16 sv = two[(s >> 1) & 1];
        dst[t] = fp4_expand(CW[(s >> 2) & 1][t][s & 3], f16x2{sv, sv});
      }
  };
  // first step of the pair in stage st (a unit with nj x tile-rows), unpipelined
  auto prime = [&](const uint8_t* st, int nj) {
    read_codes(st, nj, 0, 0, 0, 8, CW[0]);
    read_codes(st, nj, 0, 0, 4, 8, CW[0]);
    read_scales(st, nj, 0, SC[0]);
    expand_step(0, F[0], 8);
  };
  // every wave's loads of the pair issued last have landed, and every wave is done
  // with the stage read before it
  auto sync = [&]() {
    QPL_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
  };

  // prologue: pair 0, then its first step
  {
    const PairSrc src = next_src();
#pragma unroll
    for (int d = 0; d < PK_LOADS; ++d) issue(src, d);
  }
  sync();
  prime(lds, nt > 0 ? 4 : 2);
  int cur = 0;  // stage of the pair being multiplied

  // A packed pair.  njn: x tile-rows of the unit the next pair belongs to, or 0 when
  // the next pair is not a packed one (its first step is then primed by whoever
  // starts it).  The next pair's first group and scales are read and expanded
  // whether or not it is packed (without branches, so the expansion stays among
  // this pair's MFMAs); when it is not, the values are not used.
  auto pair_packed = [&](Acc& acc, auto nj, int njn) {
    constexpr int NJ = decltype(nj)::value;
    const PairSrc src = next_src();
    const uint8_t* cs = lds + cur * PK_STAGE;
    cur ^= 1;
    const uint8_t* ns = lds + cur * PK_STAGE;
    const int njr = njn ? njn : NJ;
    static_for<0, 16>([&](auto sc_) __attribute__((always_inline)) {
      constexpr int s = decltype(sc_)::value;
      if constexpr (s == 12) sync();
      // the next group's codes: groups 1 .. 3 of this pair, then group 0 of the next
      if constexpr (s % 4 < 2 && s < 12) read_codes(cs, NJ, ((s >> 2) + 1) >> 1, ((s >> 2) + 1) & 1, 4 * (s % 4), 4 + NJ,
                                                   CW[((s >> 2) + 1) & 1]);
      if constexpr (s == 12 || s == 13) read_codes(ns, njr, 0, 0, 4 * (s - 12), 8, CW[0]);
      if constexpr (s == 5) read_scales(cs, NJ, 1, SC[1]);
      if constexpr (s == 13) read_scales(ns, njr, 0, SC[0]);
      // the next step's fragments
      if constexpr (s + 1 < 16) {
        expand_step(s + 1, F[(s + 1) & 1], 4 + NJ);
      } else {
        expand_step(0, F[0], 8);
      }
      // this step's MFMAs; pair P + 1's loads after some of them in steps 0 .. 5
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F[s & 1][i], F[s & 1][4 + j], acc[i][j], 0, 0, 0);
          const int k = s * 4 * NJ + i * NJ + j;
#pragma unroll
          for (int d = 0; d < PK_LOADS; ++d)
            if (k == d * (NJ == 4 ? 5 : 2) + 1) issue(src, d);
        }
      // one MFMA, then a share of the expansion, in turn
#pragma unroll
      for (int m = 0; m < 4 * NJ; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NJ == 4 ? 5 : 10, 0);
        if (m % 4 == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // A bf16 pair of the low-rank pass: four 32 x 32 x 16 steps, fragments read from
  // its stage; the next pair's loads after some MFMAs of steps 0 .. 1, the sync
  // before step 3, and the next unit's first step primed at the end.
  auto pair_lowrank = [&](Acc& acc, auto nj, int njn) {
    constexpr int NJ = decltype(nj)::value;
    const PairSrc src = next_src();
    const uint8_t* cs = lds + cur * PK_STAGE;
    cur ^= 1;
    const uint8_t* ns = lds + cur * PK_STAGE;
    static_for<0, 4>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u == 3) sync();
      bf16x8 fw[4], fx[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fw[i] = *reinterpret_cast<const bf16x8*>(cs + PK_CODES + proff(frow(i, NJ), 2 * u + h));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fx[j] = *reinterpret_cast<const bf16x8*>(cs + proff(frow(4 + j, NJ), 2 * u + h));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = Bf16Mma::mma(fw[i], fx[j], acc[i][j]);
          const int k = u * 4 * NJ + i * NJ + j;
#pragma unroll
          for (int d = 0; d < PK_LOADS; ++d)
            if (k == d) issue(src, d);
        }
      __builtin_amdgcn_sched_barrier(0);
    });
    if (njn) prime(ns, njn);
  };

  using Whole = std::integral_constant<int, 4>;
  using Half = std::integral_constant<int, 2>;
  const float escale = LOWRANK ? 1.0f : gscale;
  auto run_unit = [&](int ti, auto nj) {
    constexpr int NJ = decltype(nj)::value;
    // x tile-rows of the next unit (0: none)
    const int njn = ti + 1 < nt ? 4 : (ti + 1 < nu ? 2 : 0);
    Acc acc;
    zero_acc(acc);
    for (int kp = 0; kp < np1; ++kp) pair_packed(acc, nj, kp + 1 < np1 ? NJ : (np2 > 0 ? 0 : njn));
    if constexpr (LOWRANK) {
      // the 4-bit product in output units; each tile goes back to its accumulator
      // registers at once (the empty asm pins it there), so that the scaled values do
      // not wait in ordinary registers for the low-rank MFMAs
      static_for<0, 4 * NJ>([&](auto tc) __attribute__((always_inline)) {
        constexpr int q = decltype(tc)::value;
        acc[q / NJ][q % NJ] = acc[q / NJ][q % NJ] * gscale;
        asm volatile("" : "+a"(acc[q / NJ][q % NJ]));
      });
      for (int kp = 0; kp < np2; ++kp) pair_lowrank(acc, nj, kp + 1 < np2 ? 0 : njn);
    }
    const Unit un = unit(ti);
    store_tile<NJ, 4, EPI>(
        acc, wm, wn, lane, un.m0, un.n0, p.M, p.N, Y, [&](int) { return escale; },
        [&](int) { return f32x4{1.0f, 1.0f, 1.0f, 1.0f}; }, e);
  };
  for (int ti = 0; ti < nt; ++ti) run_unit(ti, Whole{});
  if (has_half) run_unit(nt, Half{});
  QPL_WAIT_VMCNT(0);
  QPL_WAIT_LGKM0();
}


// ---------------------------------------------------------------------------
// INT4 GEMM (the INT4 variant of svdq_w4a4).  The operands are the code values
// -8..7 as E4M3 bytes [rows, K] with fp32 group scales stored group-major, s_x
// [K/64, M] and s_w [K/64, N] (a slab's scales of consecutive rows are then
// contiguous); a 64-byte slab row is exactly one group.  Per slab and 32 x 32 tile,
// one V_MFMA_SCALE_F32_32X32X64_F8F6F4 from zero gives the group's dot products:
// the products are integers of magnitude <= 64 and the sums stay below 2^12, and
// the MFMA returns them exactly (checked against integer sums on 4M outputs with
// random and extreme codes).  They are folded into fp32 accumulators as
// acc += (P s_w[n]) s_x[m].
// The optional low-rank pass (bf16 [T_hi | T_lo] and [L2^T | L2^T], as in the
// nvfp4 GEMM) adds T L2 to the same accumulators on the bf16 MFMA.
//
// The fold runs on the VALU, so the accumulators live in VGPRs and the MFMA results
// must too.  A workgroup has eight wavefronts (two per SIMD, so that one wave's
// MFMAs overlap the other's fold) and owns TM rows of x by 256 rows of W; a
// wavefront owns 32 NJ rows of x by 32 NI rows of W (2 x 4 waves).  A lane's s_x
// is one value per x tile, while its s_w are 16 values per W tile (its 16 output
// columns): the waves are made tall in x (NJ = TM / 64) and narrow in W (NI = 2)
// so that the s_w reads from LDS stay few.  Without the low-rank pass TM = 256
// (128 accumulators per wave: the slab traffic per MAC of the other GEMMs); the
// low-rank pass needs more registers, so with it TM = 128.  Persistent, with the tile
// order of the other GEMMs.  The ring has NST4 = 4 stages; slab g + 3 is issued
// during slab g's step into the stage of slab g - 1, so the current slab's
// fragments and scales stay in LDS while it is multiplied and folded.  A slab's
// loads per wave: TM / 128 loads of 1 KB of x, two of W, and one dword load of 64
// scales (waves 0-3: s_w; then s_x; any other wave loads nothing into a spare area).
// ---------------------------------------------------------------------------
template <bool LOWRANK>
struct I4Cfg {
  static constexpr int TM = LOWRANK ? 128 : 256;  // rows of x per tile
  static constexpr int WM = 2, WN = 4;            // wavefronts along x rows, W rows
  static constexpr int NJ = TM / 64;              // 32-row x tiles per wavefront
  static constexpr int NI = 2;                    // 32-row W tiles per wavefront
  static constexpr int XI = TM / 128;             // x loads per wave per slab
  static constexpr int D = XI + 3;                // loads per wave per slab
  static constexpr int XB = TM * SROW;            // x slab bytes
  static constexpr int SC = XB + 256 * SROW;      // s_w (256 floats), then s_x (TM floats)
  static constexpr int STAGE = SC + 1024 + 4 * TM;
  static constexpr int NSTORE = 2 * NJ * NI;      // store_tile<NJ, NI> fast path
};
constexpr int NST4 = 4;

template <bool LOWRANK, int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_int4(
    GemmArgs p, const float* __restrict__ sxp, const float* __restrict__ swp, uint16_t* __restrict__ Y, EpiArgs e) {
  using C = I4Cfg<LOWRANK>;
  constexpr int TM = C::TM, WN = C::WN, NJ = C::NJ, NI = C::NI, XI = C::XI, D = C::D, XB = C::XB, SC = C::SC;
  constexpr int STAGE = C::STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST4 * STAGE + 256];  // + a spare area for dummy loads
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wv / WN, wn = wv % WN;
  const int b = blockIdx.x;
  const uint32_t lbase = lds_address(lds);
  const uint32_t spare = lbase + NST4 * STAGE;

  int nt = 0;
  while (tile_seq(nt, b, p.nwg) < p.ntiles) ++nt;
  const int nk1 = p.kbytes1 / SROW;  // groups of 64 channels (K % 64 == 0)
  const int nk2 = LOWRANK ? (p.kbytes2 + SROW - 1) / SROW : 0;
  const int nk = nk1 + nk2;

  // lane geometry of the slab loads (16-byte chunk l % 4 of slab row + l / 4,
  // swizzled): x instruction q fills rows 16 (XI wv + q) .., W instruction q rows
  // 16 (2 wv + q) ..
  int xrow[XI], xcb[XI], wrow[2], wcb[2];
#pragma unroll
  for (int q = 0; q < XI; ++q) {
    xrow[q] = 16 * (XI * wv + q) + (lane >> 2);
    xcb[q] = ((lane & 3) ^ swz(xrow[q])) * 16;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    wrow[q] = 16 * (2 * wv + q) + (lane >> 2);
    wcb[q] = ((lane & 3) ^ swz(wrow[q])) * 16;
  }
  // this wave's scale load: 64 of s_w (waves 0-3), 64 of s_x (waves 4 .. 4 + TM / 64 - 1)
  const bool sc_w = wv < 4, sc_real = wv < 4 + TM / 64;
  const int sc_first = 64 * (sc_w ? wv : wv - 4);
  const uint32_t sc_dst = SC + (sc_w ? 0 : 1024) + 256 * (sc_w ? wv : wv - 4);

  struct SlabSrc {
    u32x4 dx, dw, dsc;
    int pitch, kb, koff, stage;
    bool scales;
  };
  int s_ti = 0, s_ks = 0, s_stage = 0;
  int64_t s_m0 = 0, s_n0 = 0;
  if (nt > 0) tile_coords(tile_seq(0, b, p.nwg), p.tiles_m, p.tiles_n, s_m0, s_n0, TM);
  auto next_src = [&]() {
    SlabSrc r;
    const bool valid = s_ti < nt;
    const bool pass2 = LOWRANK && s_ks >= nk1;
    r.stage = s_stage;
    r.scales = valid && !pass2 && sc_real;
    r.pitch = pass2 ? p.pitch2 : p.pitch1;
    r.kb = valid ? (pass2 ? p.kbytes2 : p.kbytes1) : 0;
    r.koff = (pass2 ? s_ks - nk1 : s_ks) * SROW;
    const int64_t lm = p.M - s_m0, ln = p.N - s_n0;
    const int64_t rm = lm < TM ? lm : TM, rn = ln < 256 ? ln : 256;
    r.dx = make_desc((pass2 ? p.a2 : p.a) + s_m0 * r.pitch, rm * r.pitch);
    r.dw = make_desc((pass2 ? p.w2 : p.w) + s_n0 * r.pitch, rn * r.pitch);
    r.dsc = sc_w ? make_desc(swp + (int64_t)s_ks * p.N + s_n0, rn * 4)
                 : make_desc(sxp + (int64_t)s_ks * p.M + s_m0, rm * 4);
    s_stage = s_stage == NST4 - 1 ? 0 : s_stage + 1;
    if (++s_ks == nk) {
      s_ks = 0;
      ++s_ti;
      if (s_ti < nt) tile_coords(tile_seq(s_ti, b, p.nwg), p.tiles_m, p.tiles_n, s_m0, s_n0, TM);
    }
    return r;
  };
  auto issue = [&](const SlabSrc& s, int d) {
    const uint32_t st = lbase + s.stage * STAGE;
    if (d < XI) {
      const uint32_t vo = s.koff + xcb[d] < s.kb ? (uint32_t)(xrow[d] * s.pitch + xcb[d]) : kOutOfRange;
      dma16(st + (XI * wv + d) * 1024, vo, s.dx, s.koff);
    } else if (d < XI + 2) {
      const int q = d - XI;
      const uint32_t vo = s.koff + wcb[q] < s.kb ? (uint32_t)(wrow[q] * s.pitch + wcb[q]) : kOutOfRange;
      dma16(st + XB + (2 * wv + q) * 1024, vo, s.dw, s.koff);
    } else {
      const uint32_t vo = s.scales ? (uint32_t)((sc_first + lane) * 4) : kOutOfRange;
      dma4(s.scales ? st + sc_dst : spare, vo, s.dsc, 0);
    }
  };

  // prologue: slabs 0 .. NST4 - 2
#pragma unroll
  for (int s0 = 0; s0 < NST4 - 1; ++s0) {
    const SlabSrc src = next_src();
#pragma unroll
    for (int d = 0; d < D; ++d) issue(src, d);
  }
  // fragments: 32 bytes per lane, chunks 2 (lane / 32) and + 1 of the row, read as
  // two 16-byte halves u (which are also the two bf16 MFMA steps of a low-rank
  // slab) from the current slab's stage just before they are used; the other
  // wavefront on the SIMD covers the LDS latency
  auto frag = [&](const uint8_t* stage, bool wslab, int row, int u) {
    return *reinterpret_cast<const i32x4*>(stage + (wslab ? XB : 0) + soff(row, 2 * (lane >> 5) + u));
  };
  int cur = 0;                     // stage of the slab being multiplied
  int st1 = 0, st2 = 0, st3 = 0;  // stores left in flight after iterations g - 1, g - 2, g - 3
  auto step = [&](Acc& acc, auto pass2) {
    constexpr bool P2 = decltype(pass2)::value;
    QPL_WAIT_LGKM0();
    // slab g must have landed: issued after it (in step g - 3, or the prologue) are
    // slabs g + 1 and g + 2 and the stores of the epilogues after iterations g - 3
    // .. g - 1 (at most one epilogue: a tile is at least NST4 slabs)
    const int extra = st1 + st2 + st3;
    if (extra == 0) {
      QPL_WAIT_VMCNT((NST4 - 2) * D);
    } else if (extra == C::NSTORE) {
      QPL_WAIT_VMCNT((NST4 - 2) * D + C::NSTORE);
    } else {
      QPL_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();  // slab g is in LDS for every wave; slab g - 1's stage is free
    const SlabSrc src = next_src();  // slab g + NST4 - 1, into slab g - 1's stage
    const uint8_t* cs = lds + cur * STAGE;
    cur = cur == NST4 - 1 ? 0 : cur + 1;
    i32x4 fx[2][NJ];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < NJ; ++j) fx[u][j] = frag(cs, false, wm * 32 * NJ + j * 32 + (lane & 31), u);
    float sx[NJ];
    if constexpr (!P2) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        sx[j] = *reinterpret_cast<const float*>(cs + SC + 1024 + 4 * (wm * 32 * NJ + j * 32 + (lane & 31)));
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int wr = wn * 32 * NI + i * 32;  // first W row of the tile row
      i32x4 fw[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) fw[u] = frag(cs, true, wr + (lane & 31), u);
      // s_w of this lane's 16 output columns wr + 8 q + 4 (lane / 32) + 0..3
      f32x4 sw[4];
      if constexpr (!P2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) sw[q] = *reinterpret_cast<const f32x4*>(cs + SC + 4 * (wr + 8 * q + 4 * (lane >> 5)));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if constexpr (P2) {
          // bf16 low-rank slab in two 32x32x16 steps: step u takes chunk 2 (lane / 32) + u
          // of both operands' rows, so each step sums the same (permuted) k positions of
          // W and x, and the two steps cover the slab's four chunks once
#pragma unroll
          for (int u = 0; u < 2; ++u)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fw[u]),
                                                                __builtin_bit_cast(bf16x8, fx[u][j]), acc[i][j], 0, 0, 0);
        } else {
          const i32x8 a = __builtin_shufflevector(fw[0], fw[1], 0, 1, 2, 3, 4, 5, 6, 7);
          const i32x8 bx = __builtin_shufflevector(fx[0][j], fx[1][j], 0, 1, 2, 3, 4, 5, 6, 7);
          const f32x16 pr = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bx, f32x16{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[i][j][r] = __builtin_fmaf(pr[r] * sw[r >> 2][r & 3], sx[j], acc[i][j][r]);
        }
        // the slab's D loads spread over its NI NJ tiles
        const int t = NJ * i + j;
#pragma unroll
        for (int d = 0; d < D; ++d)
          if (t == (d * NI * NJ) / D) issue(src, d);
      }
    }
    st3 = st2;
    st2 = st1;
    st1 = 0;
  };

  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  for (int ti = 0; ti < nt; ++ti) {
    Acc acc;
    zero_acc(acc);
    for (int kt = 0; kt < nk1; ++kt) step(acc, No{});
    if constexpr (LOWRANK) {
      for (int kt = 0; kt < nk2; ++kt) step(acc, Yes{});
    }
    int64_t m0, n0;
    tile_coords(tile_seq(ti, b, p.nwg), p.tiles_m, p.tiles_n, m0, n0, TM);
    st1 = store_tile<NJ, NI, EPI>(acc, wm, wn, lane, m0, n0, p.M, p.N, Y, [](int) { return 1.0f; },
                                  [](int) { return f32x4{1.0f, 1.0f, 1.0f, 1.0f}; }, e);
    if (st1 == 0) st2 = st3 = 0;
  }
  QPL_WAIT_VMCNT(0);
  QPL_WAIT_LGKM0();
}

}  // namespace

// Persistent workgroups: one per CU while every slab stream is at least NST
// slabs per tile (the ring and the scale buffers assume it); one per tile otherwise.
static int gemm_workgroups(int ntiles, int nk) { return nk >= NST ? (ntiles < 256 ? ntiles : 256) : ntiles; }

// Workgroup count and the split of the last round.  With 256 persistent
// workgroups and ntiles % 256 <= 128 leftover tiles, the leftover tiles are
// computed as 2 (ntiles % 256) half tiles, one per workgroup, so the last round
// takes half a tile's time instead of a whole one.
static void gemm_plan(GemmArgs& p, int nk) {
  p.nwg = gemm_workgroups(p.ntiles, nk);
  const int tail = p.ntiles % 256;
  const bool split = p.nwg == 256 && p.ntiles > 256 && tail > 0 && tail <= 128;
  p.nfull = split ? p.ntiles - tail : p.ntiles;
  p.ntail = split ? tail : 0;
}

// Kernel-side epilogue arguments and kind (EPI flags) of a launch.
static int epi_kind(const Epilogue& ep, EpiArgs& e) {
  e = EpiArgs{};
  int k = ep.gelu ? EPI_GELU : 0;
  if (ep.qkv[0]) {
    k |= EPI_QKV;
    for (int i = 0; i < 3; ++i) e.qkv[i] = ep.qkv[i];
    e.d = ep.d;
    e.tokens = ep.tokens;
    e.off = ep.off;
    e.lg_hd = ep.lg_hd;
  }
  return k;
}

hipError_t launch_gemm_fp8r(const uint8_t* xq, const float* xs, const uint8_t* w, const float* ws, int64_t M,
                            int64_t K, int64_t N, const Epilogue& ep, uint16_t* y, hipStream_t stream) {
  GemmArgs p{};
  p.a = xq;
  p.w = w;
  p.M = M;
  p.N = N;
  p.pitch1 = (int)K;
  p.kbytes1 = (int)K;
  p.tiles_m = (int)((M + 255) / 256);
  p.tiles_n = (int)((N + 255) / 256);
  p.ntiles = p.tiles_m * p.tiles_n;
  gemm_plan(p, (p.kbytes1 + SROW - 1) / SROW);
  EpiArgs e;
  const dim3 grid((unsigned)p.nwg), block(256);
  switch (epi_kind(ep, e)) {
    case 0: hipLaunchKernelGGL(k_gemm_fp8r<0>, grid, block, 0, stream, p, xs, ws, y, e); break;
    case EPI_GELU: hipLaunchKernelGGL(k_gemm_fp8r<EPI_GELU>, grid, block, 0, stream, p, xs, ws, y, e); break;
    case EPI_QKV: hipLaunchKernelGGL(k_gemm_fp8r<EPI_QKV>, grid, block, 0, stream, p, xs, ws, y, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool LR>
static hipError_t launch_nvfp4_epi(int kind, dim3 grid, hipStream_t stream, const PackedArgs& p, float gscale,
                                   uint16_t* y, const EpiArgs& e) {
  switch (kind) {
    case 0: hipLaunchKernelGGL((k_gemm_nvfp4<LR, 0>), grid, dim3(256), 0, stream, p, gscale, y, e); break;
    case EPI_GELU: hipLaunchKernelGGL((k_gemm_nvfp4<LR, EPI_GELU>), grid, dim3(256), 0, stream, p, gscale, y, e); break;
    case EPI_QKV: hipLaunchKernelGGL((k_gemm_nvfp4<LR, EPI_QKV>), grid, dim3(256), 0, stream, p, gscale, y, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_nvfp4(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* wsc,
                             float gscale, int64_t M, int64_t K, int64_t N, LowRank lr, const Epilogue& ep, uint16_t* y,
                             hipStream_t stream) {
  PackedArgs p{};
  p.xq = xq;
  p.wq = wq;
  p.xs = xs;
  p.wsc = wsc;
  p.M = M;
  p.N = N;
  p.cpitch = (int)(K / 2);
  p.nk1 = (int)((K + 127) / 128);
  if (lr.kl > 0) {
    p.a2 = reinterpret_cast<const uint8_t*>(lr.t);
    p.w2 = reinterpret_cast<const uint8_t*>(lr.l2t);
    p.pitch2 = (int)(2 * lr.kl);
    p.kbytes2 = (int)(2 * lr.kl);
  }
  p.tiles_m = (int)((M + 255) / 256);
  p.tiles_n = (int)((N + 255) / 256);
  p.ntiles = p.tiles_m * p.tiles_n;
  // persistent (one workgroup per CU at most); leftover tiles of a last round of at
  // most 128 are split into half tiles.  With the low-rank pass: one tile per workgroup.
  p.nwg = lr.kl > 0 ? p.ntiles : (p.ntiles < 256 ? p.ntiles : 256);
  const int tail = p.ntiles % 256;
  const bool split = lr.kl == 0 && p.ntiles > 256 && tail > 0 && tail <= 128;
  p.nfull = split ? p.ntiles - tail : p.ntiles;
  p.ntail = split ? tail : 0;
  EpiArgs e;
  const int kind = epi_kind(ep, e);
  const dim3 grid((unsigned)p.nwg);
  return lr.kl > 0 ? launch_nvfp4_epi<true>(kind, grid, stream, p, gscale, y, e)
                   : launch_nvfp4_epi<false>(kind, grid, stream, p, gscale, y, e);
}

template <bool LR>
static hipError_t launch_int4_epi(int kind, dim3 grid, hipStream_t stream, const GemmArgs& p, const float* xs,
                                  const float* ws, uint16_t* y, const EpiArgs& e) {
  switch (kind) {
    case 0: hipLaunchKernelGGL((k_gemm_int4<LR, 0>), grid, dim3(512), 0, stream, p, xs, ws, y, e); break;
    case EPI_GELU: hipLaunchKernelGGL((k_gemm_int4<LR, EPI_GELU>), grid, dim3(512), 0, stream, p, xs, ws, y, e); break;
    case EPI_QKV: hipLaunchKernelGGL((k_gemm_int4<LR, EPI_QKV>), grid, dim3(512), 0, stream, p, xs, ws, y, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_int4(const uint8_t* x8, const float* xs, const uint8_t* w8, const float* ws, int64_t M,
                            int64_t K, int64_t N, LowRank lr, const Epilogue& ep, uint16_t* y, hipStream_t stream) {
  GemmArgs p{};
  p.a = x8;
  p.w = w8;
  p.M = M;
  p.N = N;
  p.pitch1 = (int)K;
  p.kbytes1 = (int)K;
  int nk = (int)(K / 64);
  if (lr.kl > 0) {
    p.a2 = reinterpret_cast<const uint8_t*>(lr.t);
    p.w2 = reinterpret_cast<const uint8_t*>(lr.l2t);
    p.pitch2 = (int)(2 * lr.kl);
    p.kbytes2 = (int)(2 * lr.kl);
    nk += (p.kbytes2 + SROW - 1) / SROW;
  }
  const int tm = lr.kl > 0 ? I4Cfg<true>::TM : I4Cfg<false>::TM;
  p.tiles_m = (int)((M + tm - 1) / tm);
  p.tiles_n = (int)((N + 255) / 256);
  p.ntiles = p.tiles_m * p.tiles_n;
  // persistent while every tile is at least NST4 slabs (one epilogue per wait window)
  p.nwg = nk >= NST4 ? (p.ntiles < 256 ? p.ntiles : 256) : p.ntiles;
  p.nfull = p.ntiles;
  p.ntail = 0;
  EpiArgs e;
  const int kind = epi_kind(ep, e);
  const dim3 grid((unsigned)p.nwg);
  return lr.kl > 0 ? launch_int4_epi<true>(kind, grid, stream, p, xs, ws, y, e)
                   : launch_int4_epi<false>(kind, grid, stream, p, xs, ws, y, e);
}

}  // namespace qpl
