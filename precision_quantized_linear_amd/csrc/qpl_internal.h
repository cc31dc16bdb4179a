// Launchers of the gfx950 kernels, called by the C ABI in qpl_api.hip after the
// arguments have been checked.  Every launcher queues work on `stream` and returns
// the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qpl {

// Per block-scale code sf (E4M3, 0..127): d = dec(sf) * g and RN(1 / d) in fp32,
// computed on the host for one global scale g and passed by value to the nvfp4
// quantizers.
struct Nvfp4ScaleTable {
  float d[128];
  float rd[128];
};
Nvfp4ScaleTable nvfp4_scale_table(float g);

hipError_t launch_quant_fp8_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* xq, float* xs,
                                hipStream_t stream);
// lam: SVDQuant smoothing factors [K] (x is divided by them first) or nullptr.
hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t M, int64_t K, float g, const float* lam, uint8_t* xq,
                              uint8_t* xbs, hipStream_t stream);
// The nvfp4 quantizer of the linear layer without a low-rank branch: packed codes
// [M, K/2] (as quant_act_nvfp4) and block scales slab-major [ceil(K/128), M, 8]
// (the GEMM's layout, zeros past K/16), and in the same launch the weight's block
// scales wbs [N, K/16] relaid into wsl [ceil(K/128), N, 8] (zeros past K/16).
hipError_t launch_quant_nvfp4_linear(const uint16_t* x, int64_t M, int64_t K, float g, const float* lam,
                                     uint8_t* xq, uint8_t* xs, const uint8_t* wbs, int64_t N, uint8_t* wsl,
                                     hipStream_t stream);
// The same, fused with the low-rank down-projection: t [M, kl] bf16 receives
// T = x L1 (fp32) as [hi | lo] bf16 halves of kl / 2 columns each; l1t [kl / 2, K]
// is L1 transposed (zero past R); kl / 2 is a multiple of 32, at most 128.  With
// lam, both the codes and T are computed from the smoothed activation.
hipError_t launch_quant_nvfp4_lowrank(const uint16_t* x, int64_t M, int64_t K, float g, const float* lam,
                                      const uint16_t* l1t, int64_t kl, uint8_t* xq, uint8_t* xs, uint16_t* t,
                                      hipStream_t stream);
// INT4 (svdq_w4a4 INT4 variant): group-wise quantizer, writing packed codes and
// scales [M, K/64], or (f8, for the GEMM) the E4M3 bytes of the code values and
// scales group-major [K/64, M]; and the packed -> E4M3 byte expansion of a weight,
// which also copies its scales [N, K/64] into group-major wst [K/64, N].
hipError_t launch_quant_int4(const uint16_t* x, int64_t M, int64_t K, const float* lam, bool f8, uint8_t* xq,
                             float* xs, hipStream_t stream);
hipError_t launch_expand_int4(const uint8_t* wq, const float* ws, int64_t N, int64_t K, uint8_t* w8, float* wst,
                              hipStream_t stream);
// The INT4 quantizer (E4M3 code bytes, group-major scales) fused with T = x L1,
// stored as in launch_quant_nvfp4_lowrank.
hipError_t launch_quant_int4_lowrank(const uint16_t* x, int64_t M, int64_t K, const float* lam, const uint16_t* l1t,
                                     int64_t kl, uint8_t* xq, float* xs, uint16_t* t, hipStream_t stream);

// Weight-only 4-bit linear (group-wise codes, bf16 scales, byte zero points):
// the quantizer (one lane per group) and the GEMV y = x W_hat^T.
hipError_t launch_quant_w4g(const uint16_t* w, int64_t N, int64_t K, int group, uint8_t* wq, uint16_t* ws,
                            uint8_t* wz, hipStream_t stream);
hipError_t launch_gemv_w4a16(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* wq,
                             const uint16_t* ws, const uint8_t* wz, int group, uint16_t* y, hipStream_t stream);
hipError_t launch_amax_bf16(const uint16_t* x, int64_t n, float* amax, hipStream_t stream);
hipError_t launch_dequant_fp8r(const uint8_t* w, const float* ws, int64_t N, int64_t K, uint16_t* out,
                               hipStream_t stream);
// Factor layouts of the low-rank branch (see launch_lowrank_prep): L1 [K, R] and
// L2 [R, N] bf16 in; l1t [rpad, K] and l2t [N, kl] out, rpad = kl / 2.
struct LowRankPrep {
  const uint16_t* l1 = nullptr;
  const uint16_t* l2 = nullptr;
  int64_t K = 0, N = 0, R = 0, rpad = 0, kl = 0;
  uint16_t* l1t = nullptr;
  uint16_t* l2t = nullptr;
};
hipError_t launch_dequant_nvfp4(const uint8_t* w, const uint8_t* wbs, float g2, int64_t N, int64_t K,
                                uint16_t* out, hipStream_t stream);
// What an nvfp4 linear with a low-rank branch prepares before its quantizer, in
// one launch: the weight block scales [N, K/16] copied into the GEMM's slab-major
// layout wsl [ceil(K/128), N, 8] (zero past K/16), zeros over the bytes past K/16
// of the activation scales' last slab xs [ceil(K/128) - 1, M, 8], and the factor
// layouts of the low-rank branch.
hipError_t launch_nvfp4_prep(const uint8_t* wbs, int64_t N, int64_t K, uint8_t* wsl, int64_t M, uint8_t* xs,
                             const LowRankPrep& lr, hipStream_t stream);

// What a GEMM's epilogue writes (default: y = bf16 result, row-major [M, N]).
// gelu: the tanh form of GELU on the fp32 result before the bf16 rounding.
// qkv: (all three set) the result's column parts [0, d), [d, 2d), [2d, 3d) go to
// q, k, v, each [heads, tokens, 2^lg_hd] bf16, row m at token off + m; y unused.
struct Epilogue {
  bool gelu = false;
  uint16_t* qkv[3] = {nullptr, nullptr, nullptr};
  int64_t d = 0, tokens = 0, off = 0;
  int lg_hd = 0;
};

hipError_t launch_gemm_fp8r(const uint8_t* xq, const float* xs, const uint8_t* w, const float* ws,
                            int64_t M, int64_t K, int64_t N, const Epilogue& ep, uint16_t* y, hipStream_t stream);

// Low-rank operands of the GEMMs' second pass: t [M, KL] bf16 holds T = x L1 split
// into hi and lo bf16 halves, l2t [N, KL] bf16 holds L2^T twice; KL = 2 * ceil(R/32) * 32.
struct LowRank {
  const uint16_t* t = nullptr;
  const uint16_t* l2t = nullptr;
  int64_t kl = 0;
};

// The nvfp4 GEMM on packed operands: xq [M, K/2] and wq [N, K/2] E2M1 codes, xs
// [S, M, 8] and wsc [S, N, 8] E4M3 block scales (S = ceil(K/128), zero past K/16);
// y = bf16(gscale xq wq^T [+ T L2]).
hipError_t launch_gemm_nvfp4(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* wsc,
                             float gscale, int64_t M, int64_t K, int64_t N, LowRank lr, const Epilogue& ep, uint16_t* y,
                             hipStream_t stream);

// INT4 GEMM: x8 [M, K] and w8 [N, K] code values as E4M3 bytes, xs [K/64, M] and
// ws [K/64, N] fp32 group scales (group-major), K % 64 == 0; optional low-rank
// pass.
hipError_t launch_gemm_int4(const uint8_t* x8, const float* xs, const uint8_t* w8, const float* ws, int64_t M,
                            int64_t K, int64_t N, LowRank lr, const Epilogue& ep, uint16_t* y, hipStream_t stream);
// Factor layouts for the low-rank branch: l1t [kl / 2, K] = L1^T and l2t [N, kl] =
// [L2^T | L2^T], both zero past R.
hipError_t launch_lowrank_prep(const uint16_t* l1, const uint16_t* l2, int64_t K, int64_t N, int64_t R, int64_t kl,
                               uint16_t* l1t, uint16_t* l2t, hipStream_t stream);

}  // namespace qpl
