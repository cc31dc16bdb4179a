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
// accumulators before the single bf16 rounding; the low-rank pass accumulates
// (T / gscale) L2 into the same accumulators, and the epilogue scales by gscale.
//
// Pipeline (both GEMMs):
// * a 256-thread workgroup (4 wavefronts, 2 x 2) owns a 256 x 256 output tile; a
//   wavefront owns 128 x 128 (16 MFMA tiles of 32 x 32, 256 fp32 accumulators
//   per lane in AGPRs, one wavefront per SIMD);
// * K is walked in 64-byte slabs (64 fp8 or 32 bf16 elements per row); each
//   stage holds the 256-row slab of both operands (32 KB) and four stages ring
//   through 128 KB of the 160 KB LDS;
// * slabs move global -> LDS with buffer_load_dwordx4 ... lds (no register
//   staging): slab g + 4 is issued while slab g is multiplied, three steps before
//   its fragments are first read, spread between the MFMAs; rows past the matrix
//   and bytes past K read as zero through the buffer range check;
// * the 16-byte chunks of each 64-byte row are XOR-swizzled with
//   (r ^ r >> 3) & 3, which makes the MFMA operand reads bank-conflict free;
// * operand fragments of the next slab are read into the registers of the
//   current slab's fragments as each one is used for the last time;
// * operands are swapped (the MFMA computes y^T), so each lane ends with runs of
//   four consecutive output columns of a row; lanes l and l + 32 swap halves
//   (V_PERMLANE32_SWAP) and each stores eight consecutive columns as one 16-byte
//   segment.
#include <type_traits>

#include "qpl_dma.h"
#include "qpl_internal.h"

namespace qpl {

namespace {

constexpr int SROW = 64;            // bytes per slab row
constexpr int SLAB = 256 * SROW;    // 16 KB per operand per stage
constexpr int STAGE = 2 * SLAB;     // x slab then W slab
constexpr int NST = 4;              // stages in the ring

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
template <int NJ, int NI = 4, int EPI = 0, class RowScale, class ColScale>
__device__ __forceinline__ int store_tile(const Acc& acc, int wm, int wn, int lane, int64_t m0, int64_t n0,
                                          int64_t M, int64_t N, uint16_t* __restrict__ y, const RowScale& rs,
                                          const ColScale& cs, const EpiArgs& e = EpiArgs{}) {
  // interior: the wavefront's rows and columns all inside the matrix
  const bool fast = m0 + (wm + 1) * 32 * NJ <= M && n0 + (wn + 1) * 32 * NI <= N && (N & 7) == 0;
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
        if (fast) {
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
  if (fast) return 2 * NJ * NI;
  QPL_WAIT_VMCNT(0);
  return 0;
}

// Persistent GEMM: workgroup b walks its tiles (tile_seq) one after the other,
// and the slabs of all of them form one stream through the LDS ring: the loads
// for the next tile's first slabs are issued while the current tile's last slabs
// are multiplied, and the current tile's output stores drain while the next
// tile's MFMAs run.
//
// Wait accounting (vector memory operations of a wave retire in issue order): at
// the top of iteration g, slab g + 1 must have landed; issued after its loads are
// the loads of slabs g + 2 and g + 3 (2 D) and the output stores of the
// epilogues that ran after iterations g - 3 .. g - 1.
//
// ROWCOL: fp8r output scales s_x[m] s_w[n], moved into LDS by two extra dword
// loads per wave per slab (real for a tile's first slab, out of range otherwise).
// Otherwise the output scale is gscale.  LOWRANK: pass 2 continues the same
// accumulation with T / gscale and L2 (the quantizer stores T divided by gscale),
// so y = bf16(gscale (x_q w_q^T + (T / gscale) L2)).
template <class T, bool ROWCOL, bool LOWRANK, int EPI>
__device__ __forceinline__ void gemm_persistent(const GemmArgs& p, const float* __restrict__ sa,
                                                const float* __restrict__ sb, float gscale,
                                                uint16_t* __restrict__ Y, const EpiArgs& e) {
  constexpr int D = ROWCOL ? 10 : 8;  // loads per wave per slab
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lsc[ROWCOL ? 3 * SCALE_BUF : 16];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wv >> 1, wn = wv & 1;
  const int b = blockIdx.x;
  const uint32_t lbase = lds_address(lds);
  const uint32_t sbase = lds_address(lsc);

  // Units of work: whole tiles at tile sequence positions tile_seq(0..nt - 1), then
  // (has_half) half u of the tail: rows 128 (u % 2) .. + 127 of tile nfull + u / 2.
  int nt = 0;
  while (tile_seq(nt, b, p.nwg) < p.nfull) ++nt;
  const int hu = tile_seq(nt, b, p.nwg) - p.nfull;
  const bool has_half = hu < 2 * p.ntail;
  const int nu = nt + (has_half ? 1 : 0);
  const int nk1 = (p.kbytes1 + SROW - 1) / SROW;
  const int nk2 = LOWRANK ? (p.kbytes2 + SROW - 1) / SROW : 0;
  const int nk = nk1 + nk2;
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

  // lane geometry of the slab loads: instruction q of this wave fills slab rows
  // 16 (4 wv + q) .. + 15; lane l writes physical chunk l % 4 of row + l / 4,
  // which holds logical chunk (l % 4) ^ swz(row)
  int lrow[4], cb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lrow[q] = 16 * (4 * wv + q) + (lane >> 2);
    cb[q] = ((lane & 3) ^ swz(lrow[q])) * 16;
  }

  // The load stream: slab ks of the workgroup's unit ti, advanced one slab per
  // call of next_src (unit coordinates recomputed at unit boundaries only).  A half
  // unit's x slab rows 128 .. 255 lie outside its descriptor and load zeros.
  struct SlabSrc {
    u32x4 dx, dw, ds;
    int pitch, kb, koff, stage, tpar;
    bool first, valid;
  };
  int s_ti = 0, s_ks = 0, s_stage = 0;
  Unit s_u{0, 0, 256};
  if (nu > 0) s_u = unit(0);
  auto next_src = [&]() {
    SlabSrc r;
    r.valid = s_ti < nu;
    r.stage = s_stage;
    r.first = s_ks == 0;
    r.tpar = s_ti & 1;
    const bool pass2 = LOWRANK && s_ks >= nk1;
    r.pitch = pass2 ? p.pitch2 : p.pitch1;
    r.kb = r.valid ? (pass2 ? p.kbytes2 : p.kbytes1) : 0;
    r.koff = (pass2 ? s_ks - nk1 : s_ks) * SROW;
    const int64_t left = p.M - s_u.m0;
    const int64_t rm = left < 0 ? 0 : (left < s_u.rows ? left : s_u.rows);
    const int64_t rn = M_rows(p.N - s_u.n0);
    r.dx = make_desc((pass2 ? p.a2 : p.a) + s_u.m0 * r.pitch, rm * r.pitch);
    r.dw = make_desc((pass2 ? p.w2 : p.w) + s_u.n0 * r.pitch, rn * r.pitch);
    if constexpr (ROWCOL) {
      const bool row = wv < 2;
      r.ds = make_desc(row ? sa + s_u.m0 : sb + s_u.n0, (row ? rm : rn) * 4);
    }
    s_stage = s_stage == NST - 1 ? 0 : s_stage + 1;
    if (++s_ks == nk) {
      s_ks = 0;
      ++s_ti;
      if (s_ti < nu) s_u = unit(s_ti);
    }
    return r;
  };
  auto issue = [&](const SlabSrc& s, int d) {
    if (d < 8) {
      const int q = d & 3;
      const bool wslab = d >= 4;
      const uint32_t dst = lbase + s.stage * STAGE + (wslab ? SLAB : 0) + (4 * wv + q) * 1024;
      const uint32_t vo = s.koff + cb[q] < s.kb ? (uint32_t)(lrow[q] * s.pitch + cb[q]) : kOutOfRange;
      dma16(dst, vo, wslab ? s.dw : s.dx, s.koff);
    } else {
      // scale vectors of a unit: wave w moves 128 floats of s_x (w = 0, 1) or s_w
      // (w = 2, 3), 64 per instruction; other slabs load nothing into a spare area
      const int h = d - 8;
      const bool real = s.valid && s.first;
      const uint32_t dst = sbase + (real ? s.tpar * SCALE_BUF : 2 * SCALE_BUF) + wv * 512 + h * 256;
      const uint32_t vo = real ? (uint32_t)(((wv & 1) * 128 + h * 64 + lane) * 4) : kOutOfRange;
      dma4(dst, vo, s.ds, 0);
    }
  };

  // prologue: the first NST slabs of the stream, then slab 0's fragments
#pragma unroll
  for (int s0 = 0; s0 < NST; ++s0) {
    const SlabSrc src = next_src();
#pragma unroll
    for (int d = 0; d < D; ++d) issue(src, d);
  }
  QPL_WAIT_VMCNT((NST - 1) * D);
  __builtin_amdgcn_s_barrier();
  typename T::Frag fw[T::SUB][4], fx[T::SUB][4];

  int st1 = 0, st2 = 0, st3 = 0;  // stores left in flight after iterations g - 1, g - 2, g - 3
  int cur = 0;                     // stage of the slab being multiplied
  // NJ: 32-row blocks of x per wavefront in the current unit (4 whole, 2 half).
  // One slab: wait for the next slab, multiply this one while reading the next
  // one's fragments (FRAGS) and issuing the loads of slab + NST.  Before the
  // epilogue (and the low-rank rescale) the next fragments are read afterwards
  // instead (read_frags), so that they do not occupy registers meanwhile.
  auto read_frags = [&](auto nj) {
    constexpr int NJ = decltype(nj)::value;
    const uint8_t* nx = lds + cur * STAGE;
#pragma unroll
    for (int u = 0; u < T::SUB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fw[u][i] = T::read(nx + SLAB, wn * 128 + i * 32 + (lane & 31), u, lane);
        if (i < NJ) fx[u][i] = T::read(nx, wm * 32 * NJ + i * 32 + (lane & 31), u, lane);
      }
  };
  auto step = [&](Acc& acc, auto frags, auto nj) {
    constexpr bool FRAGS = decltype(frags)::value;
    constexpr int NJ = decltype(nj)::value;
    constexpr int NMMA = 4 * NJ * T::SUB;
    QPL_WAIT_LGKM0();
    const int extra = st1 + st2 + st3;
    if (extra == 0) {
      QPL_WAIT_VMCNT((NST - 2) * D);
    } else if (extra == NSTORE) {
      QPL_WAIT_VMCNT((NST - 2) * D + NSTORE);
    } else {
      QPL_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();  // the next slab is in LDS for every wave; the previous slab's stage is free
    const SlabSrc src = next_src();
    cur = cur == NST - 1 ? 0 : cur + 1;
    const uint8_t* nx = lds + cur * STAGE;
#pragma unroll
    for (int u = 0; u < T::SUB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = T::mma(fw[u][i], fx[u][j], acc[i][j]);
          const int k = 4 * NJ * u + NJ * i + j;
          if (FRAGS && i == 3) fx[u][j] = T::read(nx, wm * 32 * NJ + j * 32 + (lane & 31), u, lane);
          if (FRAGS && j == NJ - 1) fw[u][i] = T::read(nx + SLAB, wn * 128 + i * 32 + (lane & 31), u, lane);
          // spread the D loads of slab + NST over this slab's MFMAs
#pragma unroll
          for (int d = 0; d < D; ++d)
            if (k == (d * NMMA) / D) issue(src, d);
        }
    st3 = st2;
    st2 = st1;
    st1 = 0;
  };

  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  using Whole = std::integral_constant<int, 4>;
  using Half = std::integral_constant<int, 2>;
  auto epilogue = [&](const Acc& acc, int ti, auto nj) {
    constexpr int NJ = decltype(nj)::value;
    const Unit un = unit(ti);
    if constexpr (ROWCOL) {
      const float* ls = reinterpret_cast<const float*>(lsc + (ti & 1) * SCALE_BUF);
      st1 = __builtin_amdgcn_readfirstlane(store_tile<NJ, 4, EPI>(
          acc, wm, wn, lane, un.m0, un.n0, p.M, p.N, Y, [&](int r) { return ls[r]; },
          [&](int c) { return *reinterpret_cast<const f32x4*>(&ls[256 + c]); }, e));
    } else {
      st1 = __builtin_amdgcn_readfirstlane(store_tile<NJ, 4, EPI>(
          acc, wm, wn, lane, un.m0, un.n0, p.M, p.N, Y, [&](int) { return gscale; },
          [&](int) { return f32x4{1.0f, 1.0f, 1.0f, 1.0f}; }, e));
    }
    if (st1 == 0) st2 = st3 = 0;
  };

  if (nt > 0)
    read_frags(Whole{});
  else
    read_frags(Half{});
  for (int ti = 0; ti < nt; ++ti) {
    Acc acc;
    zero_acc(acc);
    for (int kt = 0; kt < nk - 1; ++kt) step(acc, Yes{}, Whole{});
    step(acc, No{}, Whole{});
    epilogue(acc, ti, Whole{});
    if (ti + 1 < nt)
      read_frags(Whole{});
    else
      read_frags(Half{});
  }
  if (has_half) {
    Acc acc;
    zero_acc(acc);
    for (int kt = 0; kt < nk - 1; ++kt) step(acc, Yes{}, Half{});
    step(acc, No{}, Half{});
    epilogue(acc, nt, Half{});
  }
  QPL_WAIT_VMCNT(0);
  QPL_WAIT_LGKM0();
}

template <int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_fp8r(
    GemmArgs p, const float* __restrict__ sa, const float* __restrict__ sb, uint16_t* __restrict__ Y, EpiArgs e) {
  gemm_persistent<Fp8Mma, true, false, EPI>(p, sa, sb, 1.0f, Y, e);
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
// Tiling and schedule follow gemm_persistent (256 x 256 tiles, 4 wavefronts of
// 128 x 128, persistent workgroups, XCD-grouped tile order, half tiles in the
// last round, y^T epilogue), with these slabs:
// * a slab is 128 K elements: 64 code bytes per row (16 KB per operand) and 8
//   block-scale bytes per row (2 KB per operand, slab-major in global memory:
//   [K/128][rows][8], zero past K/16, so one 1 KB load moves 128 rows' scales);
//   a stage is 36 KB and four stages ring through 144 KB of LDS;
// * lane half h of a fragment row takes blocks 4h .. 4h + 3 of the slab: code
//   bytes 32h .. 32h + 31 (two 16-byte LDS reads) and one scale dword.  MFMA step
//   s (0..7) multiplies nibbles 8 (s % 2) .. + 7 of block 4h + s / 2; both
//   operands use this order, so the pairs of a product are the same k;
// * software pipeline across slabs: the second half of a slab's codes is read
//   from LDS when the slab starts, and once its steps 0-3 have used the first half,
//   the first half and the scales of the next slab are read into those registers.
//   The barrier at the top of slab g therefore waits for slab g + 1 and frees the
//   stage of slab g - 1, into which slab g + 3 is issued (9 loads per wave: 8 of
//   codes and 1 of scales, spread over the slab's 128 MFMAs);
// * blocks past K have scale 0 (they multiply to 0 whatever codes straddle the row
//   end), rows past M or N read zeros through the buffer range check.
// LOWRANK: after the packed slabs of a tile the accumulators are multiplied by
// gscale, then bf16 slabs of [T_hi | T_lo] and [L2^T | L2^T] (64 bytes per row)
// continue the same accumulation on the bf16 MFMA, so y = bf16(gscale x_q w_q^T
// + T L2) with T unscaled.
// ---------------------------------------------------------------------------
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int PK_CODES = 256 * SROW;                // code bytes per operand per stage
constexpr int PK_SC = 256 * 8;                      // block-scale bytes per operand per stage
constexpr int PK_STAGE = 2 * PK_CODES + 2 * PK_SC;  // [x codes][w codes][x scales][w scales]
constexpr int PK_NST = 4;
constexpr int PK_D = 9;                             // loads per wave per slab

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

// (s, s) as an f16 pair for the E4M3 scale in byte j of sc (exact).
__device__ __forceinline__ f16x2 e4m3_pair(uint32_t sc, uint32_t j) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(sc, sc, j * 0x01010101u), 1.0f, false);
}

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
  __shared__ __attribute__((aligned(16))) uint8_t lds[PK_NST * PK_STAGE];
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
  const int nk1 = p.nk1;
  const int nk2 = LOWRANK ? (p.kbytes2 + SROW - 1) / SROW : 0;
  const int nk = nk1 + nk2;
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

  // row loads: instruction q of this wave fills slab rows 16 (4 wv + q) .. + 15;
  // lane l writes physical chunk l % 4 of row + l / 4 (logical chunk (l % 4) ^ swz),
  // at byte offset vo1 (packed rows) or vo2 (low-rank rows) of the tile
  int cb[4];
  uint32_t vo1[4], vo2[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lrow = 16 * (4 * wv + q) + (lane >> 2);
    cb[q] = ((lane & 3) ^ swz(lrow)) * 16;
    vo1[q] = (uint32_t)(lrow * p.cpitch + cb[q]);
    vo2[q] = LOWRANK ? (uint32_t)(lrow * p.pitch2 + cb[q]) : 0u;
  }
  // scale loads: wave wv moves rows 128 (wv % 2) .. + 127 of operand wv / 2 (x, W)
  const bool sc_x = wv < 2;
  const int sc_r0 = 128 * (wv & 1);

  struct SlabSrc {
    u32x4 dx, dw, ds;
    int kb, koff, stage;
    bool pass2;
  };
  // The slab stream's sources change only where it enters a unit or the unit's
  // low-rank pass: then the code descriptors, the row count and the first slab's
  // scale address are worked out; from slab to slab only the scale address moves
  // (by one slab of scales) with the stage and the K offset.
  int s_ti = 0, s_ks = 0, s_stage = 0;
  Unit s_u{0, 0, 256};
  u32x4 s_dx{}, s_dw{};
  const uint8_t* s_sc = nullptr;  // scale bytes of the next slab (this wave's rows)
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
    SlabSrc r;
    r.stage = s_stage;
    r.pass2 = LOWRANK && s_ks >= nk1;
    r.kb = s_kb;
    r.koff = (r.pass2 ? s_ks - nk1 : s_ks) * SROW;
    r.dx = s_dx;
    r.dw = s_dw;
    r.ds = make_desc(s_sc, s_scb);
    s_sc += sstride;
    s_stage = s_stage == PK_NST - 1 ? 0 : s_stage + 1;
    if (++s_ks == nk) {
      s_ks = 0;
      if (++s_ti < nu) {
        s_u = unit(s_ti);
        enter(false);
      } else {
        s_kb = 0;  // past the last unit: every load reads zeros
        s_scb = 0;
      }
    } else if (LOWRANK && s_ks == nk1) {
      enter(true);
    }
    return r;
  };
  auto issue = [&](const SlabSrc& s, int d) {
    const uint32_t st = lbase + s.stage * PK_STAGE;
    if (d < 8) {
      const int q = d & 3;
      const bool wslab = d >= 4;
      const uint32_t vo = s.koff + cb[q] < s.kb ? (LOWRANK && s.pass2 ? vo2[q] : vo1[q]) : kOutOfRange;
      dma16(st + (wslab ? PK_CODES : 0) + (4 * wv + q) * 1024, vo, wslab ? s.dw : s.dx, s.koff);
    } else {
      // 1 KB of scales (128 rows x 8 bytes); rows past the unit read zero
      dma16(st + 2 * PK_CODES + (sc_x ? 0 : PK_SC) + sc_r0 * 8, (uint32_t)lane * 16u, s.ds, 0);
    }
  };

  // prologue: slabs 0 .. 2, then slab 0's first code half and scales
#pragma unroll
  for (int s0 = 0; s0 < PK_NST - 1; ++s0) {
    const SlabSrc src = next_src();
#pragma unroll
    for (int d = 0; d < PK_D; ++d) issue(src, d);
  }
  QPL_WAIT_VMCNT(2 * PK_D);
  __builtin_amdgcn_s_barrier();

  // fragment rows of tile-row t of a unit with nj x tile-rows: t < 4 W, t >= 4 x
  auto frow = [&](int t, int nj) { return t < 4 ? wn * 128 + t * 32 + r32 : wm * 32 * nj + (t - 4) * 32 + r32; };
  // Codes of step group g (steps 4 g .. 4 g + 3) of tile-rows t0 .. t0 + 3 of the slab
  // in stage st: one 16-byte chunk 2 h + g per row, dword s % 4 of it for step s
  auto read_codes = [&](const uint8_t* st, int nj, int g, int t0, int ntr, u32x4 (&dst)[8]) {
#pragma unroll
    for (int t = t0; t < t0 + 4; ++t)
      if (t < ntr) dst[t] = *reinterpret_cast<const u32x4*>(st + (t < 4 ? PK_CODES : 0) + soff(frow(t, nj), 2 * h + g));
  };
  // block-scale dword (blocks 4 h .. 4 h + 3) of every tile-row of the slab in stage st
  auto read_scales = [&](const uint8_t* st, int nj, uint32_t (&dst)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      dst[t] = *reinterpret_cast<const uint32_t*>(st + 2 * PK_CODES + (t < 4 ? PK_SC : 0) + frow(t, nj) * 8 + 4 * h);
  };
  // Two fragment sets alternate: while step s is multiplied from F[s % 2], step s + 1
  // is expanded into F[(s + 1) % 2], so no fragment is copied.  Codes come a group of
  // four steps at a time into CW[g % 2]; the next group's reads are issued during the
  // first two steps of the current one.  Across slabs, the second half of a slab
  // reads the next packed slab's first group and scales, and its last step expands
  // the next slab's first step.
  f16x8 F[2][8];
  u32x4 CW[2][8];
  uint32_t sc[8];
  auto expand_step = [&](int s, const uint32_t (&scd)[8], f16x8 (&dst)[8], int ntr) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (t < ntr) dst[t] = fp4_expand(CW[(s >> 2) & 1][t][s & 3], e4m3_pair(scd[t], (s >> 1) & 3));
  };
  // first step of the slab in stage st (a unit with nj x tile-rows), unpipelined
  auto prime = [&](const uint8_t* st, int nj) {
    read_codes(st, nj, 0, 0, 8, CW[0]);
    read_codes(st, nj, 0, 4, 8, CW[0]);
    read_scales(st, nj, sc);
    expand_step(0, sc, F[0], 8);
  };
  prime(lds, nt > 0 ? 4 : 2);

  int cur = 0;                // stage of the slab being multiplied
  int st1 = 0, st2 = 0;       // stores left in flight after iterations g - 1, g - 2
  // Top of a slab: slab g + 1 has landed (issued after it: slab g + 2's loads and
  // the stores of the epilogues after iterations g - 2 and g - 1), every wave is
  // done with slab g - 1, whose stage receives slab g + 3.
  auto top = [&]() {
    QPL_WAIT_LGKM0();
    const int extra = st1 + st2;
    if (extra == 0) {
      QPL_WAIT_VMCNT(PK_D);
    } else if (extra == NSTORE) {
      QPL_WAIT_VMCNT(PK_D + NSTORE);
    } else {
      QPL_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    st2 = st1;
    st1 = 0;
    return next_src();
  };

  // A packed slab.  njn: x tile-rows of the unit the next slab belongs to, or 0
  // when the next slab is not a packed one (its first step is then primed by
  // whoever starts it).
  auto step_packed = [&](Acc& acc, auto nj, int njn) {
    constexpr int NJ = decltype(nj)::value;
    constexpr int NMMA = 32 * NJ;  // 8 steps x 4 x NJ
    const SlabSrc src = top();
    const uint8_t* cs = lds + cur * PK_STAGE;
    cur = cur == PK_NST - 1 ? 0 : cur + 1;
    const uint8_t* ns = lds + cur * PK_STAGE;
    uint32_t scn[8];
    // The next slab's first group is read and expanded whether or not it is a packed
    // slab (without branches, so the expansion stays among this slab's MFMAs); when it
    // is not, the values are not used, and whoever starts that slab primes it.
    const int njr = njn ? njn : NJ;
    static_for<0, 8>([&](auto sc_) __attribute__((always_inline)) {
      constexpr int s = decltype(sc_)::value;
      // the next group's codes: this slab's second group, or the next slab's first
      if constexpr (s == 0 || s == 1) read_codes(cs, NJ, 1, 4 * s, 4 + NJ, CW[1]);
      if constexpr (s == 4 || s == 5) read_codes(ns, njr, 0, 4 * (s - 4), 8, CW[0]);
      if constexpr (s == 5) read_scales(ns, njr, scn);
      // the next step's fragments
      if constexpr (s + 1 < 8) {
        expand_step(s + 1, sc, F[(s + 1) & 1], 4 + NJ);
      } else {
        expand_step(0, scn, F[0], 8);
      }
      // this step's MFMAs, with the slab loads spread among them
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F[s & 1][i], F[s & 1][4 + j], acc[i][j], 0, 0, 0);
          const int k = s * 4 * NJ + i * NJ + j;
#pragma unroll
          for (int d = 0; d < PK_D; ++d)
            if (k == (d * NMMA) / PK_D) issue(src, d);
        }
      // one MFMA, then a share of the expansion, in turn: the expansion of the next
      // step hides under this step's MFMAs
#pragma unroll
      for (int m = 0; m < 4 * NJ; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NJ == 4 ? 5 : 10, 0);
        if (m % 4 == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int t = 0; t < 8; ++t) sc[t] = scn[t];
  };

  // A bf16 slab of the low-rank pass (fragments read from its stage at the top).
  auto step_lowrank = [&](Acc& acc, auto nj, int njn) {
    constexpr int NJ = decltype(nj)::value;
    constexpr int NMMA = 8 * NJ;
    const SlabSrc src = top();
    const uint8_t* cs = lds + cur * PK_STAGE;
    cur = cur == PK_NST - 1 ? 0 : cur + 1;
    const uint8_t* ns = lds + cur * PK_STAGE;
    static_for<0, 2>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      bf16x8 fw[4], fx[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i) fw[i] = Bf16Mma::read(cs + PK_CODES, frow(i, NJ), u, lane);
#pragma unroll
      for (int j = 0; j < NJ; ++j) fx[j] = Bf16Mma::read(cs, frow(4 + j, NJ), u, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = Bf16Mma::mma(fw[i], fx[j], acc[i][j]);
          const int k = u * 4 * NJ + i * NJ + j;
#pragma unroll
          for (int d = 0; d < PK_D; ++d)
            if (k == (d * NMMA) / PK_D) issue(src, d);
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
    for (int ks = 0; ks < nk1; ++ks) step_packed(acc, nj, ks + 1 < nk1 ? NJ : (nk2 > 0 ? 0 : njn));
    if constexpr (LOWRANK) {
      // the 4-bit product in output units; each tile goes back to its accumulator
      // registers at once (the empty asm pins it there), so that the scaled values do
      // not wait in ordinary registers for the low-rank MFMAs
      static_for<0, 4 * NJ>([&](auto tc) __attribute__((always_inline)) {
        constexpr int q = decltype(tc)::value;
        acc[q / NJ][q % NJ] = acc[q / NJ][q % NJ] * gscale;
        asm volatile("" : "+a"(acc[q / NJ][q % NJ]));
      });
      for (int ks = 0; ks < nk2; ++ks) step_lowrank(acc, nj, ks + 1 < nk2 ? 0 : njn);
    }
    const Unit un = unit(ti);
    // the store count is wave-uniform; keeping it in a scalar register keeps the wait
    // at the next slab's top a scalar branch
    st1 = __builtin_amdgcn_readfirstlane(store_tile<NJ, 4, EPI>(
        acc, wm, wn, lane, un.m0, un.n0, p.M, p.N, Y, [&](int) { return escale; },
        [&](int) { return f32x4{1.0f, 1.0f, 1.0f, 1.0f}; }, e));
    if (st1 == 0) st2 = 0;
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
