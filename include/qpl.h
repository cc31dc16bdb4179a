/*
 * qpl.h - C ABI of the MI355X (gfx950) quantized linear library (libqpl.so).
 *
 * The operations are those of the two checkpoint schemes in the Diffusers guide
 * "BFL (fp8r / nvfp4)" (intro bullets and the "Kernels" section), plus the
 * low-rank branch of SVDQuant ("Bringing Nunchaku 4-bit Diffusion Inference to
 * Diffusers", section "Background: SVDQuant and Nunchaku").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, row-major, in device memory owned by the caller.  The
 *   library allocates nothing and keeps no pointer after a call returns.
 * - bf16 values travel as their 16-bit patterns (uint16_t).
 * - E4M3 is the OCP FP8 E4M3 encoding (bias 7, largest finite 448, NaN only at
 *   S.1111.111, no infinity).  E2M1 is the OCP MX FP4 element type (magnitudes
 *   0, 0.5, 1, 1.5, 2, 3, 4, 6).  Encoders round to nearest even, saturate at the
 *   largest finite magnitude and keep the sign of zero.
 * - A linear is y[M,N] = x[M,K] * W[N,K]^T (the nn.Linear layout).
 * - Packed E2M1: byte j of a row holds element 2j in its low nibble and element
 *   2j+1 in its high nibble.  Block scales are row-major [rows, K/16].
 * - `stream` is a hipStream_t (NULL = the default stream).  Work is queued on it
 *   and the call returns without waiting; no entry point synchronizes the host.
 * - Arguments are checked on the host before anything is queued; a bad argument
 *   returns a non-zero status and touches no memory.  Checks: non-NULL pointers,
 *   16-byte aligned pointers, M, N >= 1, K >= 16 and K % 16 == 0, scalars finite
 *   and > 0, workspace large enough, and a current HIP device that is gfx950.
 * - Size limits of the linears (QPL_ERR_SHAPE beyond them): the GEMMs address a
 *   256-row tile of an operand with 32-bit offsets below 2^30, so K < 2^22 for
 *   fp8r and INT4 (K-byte rows) and K < 2^23 for nvfp4 (K/2-byte rows); with a
 *   low-rank branch (R > 0) K <= 2^21 and the activation's scales (8 M ceil(K/128)
 *   bytes for nvfp4, 4 M K/64 for INT4) below 2^31 bytes.
 * - Inputs must be finite: NaN or infinity in x or W is outside the contract.
 * - Faults inside a kernel surface at the caller's next synchronization.
 */
#ifndef QPL_H
#define QPL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QPL_OK = 0,
  QPL_ERR_NULL = 1,      /* a required pointer is NULL */
  QPL_ERR_SHAPE = 2,     /* M or N < 1, K < 16, K % 16 != 0, R outside [0, 128], or a size overflows */
  QPL_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  QPL_ERR_ARG = 4,       /* a scale is not finite and > 0, unknown scheme, or low-rank pointers inconsistent with R */
  QPL_ERR_WORKSPACE = 5, /* ws_bytes < qlinear_workspace_bytes(...) */
  QPL_ERR_DEVICE = 6,    /* no HIP device, or the current device is not gfx950 */
  QPL_ERR_LAUNCH = 7     /* the HIP runtime rejected a kernel launch */
} qpl_status;

typedef enum { QPL_FP8R = 0, QPL_NVFP4 = 1, QPL_INT4 = 2 } qpl_scheme;

/*
 * Row-wise FP8 quantization (guide "BFL (fp8r / nvfp4)", intro bullet on fp8r:
 * activations are quantized per row to E4M3 at run time).  The same routine
 * quantizes a weight [N,K] into `weight` / `weight_scale`.
 *   x        bf16 [M,K]            input
 *   x_q      uint8 E4M3 [M,K]      out: codes, E4M3(x / s[m]) with a correctly
 *                                  rounded fp32 division
 *   x_scale  float [M]             out: s[m] = max_k |x[m,k]| / 448 (fp32); an
 *                                  all-zero row gives s = 0 and signed-zero codes
 */
qpl_status quant_act_fp8_row(const uint16_t* x, int64_t M, int64_t K,
                             uint8_t* x_q, float* x_scale, void* stream);

/*
 * NVFP4 quantization under a global scale g (guide, intro bullet on nvfp4: packed
 * E2M1 values with an E4M3 scale per 16 elements and a calibrated fp32
 * `input_scale`).  With g = weight_scale_2 the same routine quantizes a weight.
 * Per 16-element block: sf = E4M3(bmax / (6 g)), d = dec(sf) * g (fp32),
 * codes E2M1(x / d) (signed zeros when d == 0).
 *   x              bf16 [M,K]                  input
 *   input_scale    g, finite and > 0, with 6 g finite in fp32 (else QPL_ERR_ARG)
 *   smooth         float [K] or NULL: SVDQuant smoothing factors (Nunchaku post,
 *                  "Background: SVDQuant and Nunchaku": activation outliers move
 *                  into the weights, whose column k carries smooth[k]).  When
 *                  given, the quantized activation is x_hat[m,k] =
 *                  bf16_rne(x[m,k] / smooth[k]) (correctly rounded fp32
 *                  division).  The factors are device data the call does not
 *                  check: they must be positive and finite and every x / smooth
 *                  finite in bf16; otherwise the codes are unspecified.
 *   x_q            uint8 [M,K/2]               out: packed E2M1 codes
 *   x_block_scale  uint8 E4M3 [M,K/16]         out: block scales
 * All pointers 16-byte aligned (smooth too when not NULL).
 */
qpl_status quant_act_nvfp4(const uint16_t* x, int64_t M, int64_t K, float input_scale,
                           const float* smooth, uint8_t* x_q, uint8_t* x_block_scale, void* stream);

/*
 * fp8r linear (guide, "Kernels" table, fp8r row: a row-wise scaled FP8 GEMM):
 *   y[m,n] = bf16_rne( sum_k dec(xq[m,k]) dec(w[n,k]) * s_x[m] * weight_scale[n] )
 * with xq, s_x from quant_act_fp8_row(x), fp32 accumulation.
 *   weight        uint8 E4M3 [N,K]
 *   weight_scale  float [N]
 *   y             bf16 [M,N]          out
 *   ws, ws_bytes  scratch of at least qlinear_workspace_bytes(QPL_FP8R, M, K, N, 0)
 */
qpl_status qlinear_fp8r(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                        const uint8_t* weight, const float* weight_scale,
                        uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * qlinear_fp8r without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, checks, kernels and
 * results as qlinear_fp8r; the workspace is instead a static device array of
 * QPL_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the first call
 * on that GPU (which looks up its address) until the process ends.
 *   Limit: the fp8r workspace, 256 ceil(M K / 256) + 256 ceil(4 M / 256) bytes, must
 *   fit in QPL_NOALLOC_SCRATCH_BYTES (32 MiB: M K up to about 33.5 M, e.g. 9216 x 3072),
 *   else QPL_ERR_WORKSPACE and nothing is queued.
 *   Sharing: every call on one GPU uses that GPU's one array, so calls that overlap on
 *   one GPU (different streams, or different threads without ordering) race and give
 *   undefined results; calls in one stream are ordered and safe.  Nothing in the array
 *   needs to start at zero; it keeps the last call's quantized activation.
 * No hipMalloc, hipFree, event or other allocating call is made; kernel timing
 * (qpl_timing_enable) does not cover this entry point.
 */
#define QPL_NOALLOC_SCRATCH_BYTES (32u << 20)
qpl_status qlinear_fp8r_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                                const uint8_t* weight, const float* weight_scale,
                                uint16_t* y, void* stream);

/*
 * nvfp4 linear (guide, "Kernels" table, nvfp4 row: an activation quantize followed
 * by a block-scaled FP4 GEMM), optionally with the SVDQuant low-rank branch:
 *   y = bf16_rne( input_scale * weight_scale_2 *
 *                 sum_b sx[m,b] sw[n,b] sum_{k in b} e2m1(xq) e2m1(w)  +  (x L1) L2 )
 * where xq, sx come from quant_act_nvfp4(x, input_scale, smooth) and the low-rank
 * term is accumulated in fp32 before the single rounding to bf16.  With smooth,
 * x in both terms is the smoothed x_hat that quant_act_nvfp4 defines (the
 * weight and L1 of such a layer were built for x_hat).
 *   weight          uint8 [N,K/2]        packed E2M1
 *   weight_scale    uint8 E4M3 [N,K/16]
 *   weight_scale_2  global weight scale, finite and > 0
 *   input_scale     calibrated activation scale, finite and > 0, 6 * input_scale finite;
 *                   the product input_scale * weight_scale_2 must be a normal fp32
 *                   number (else QPL_ERR_ARG); it scales the fp32 4-bit product
 *   smooth          float [K] smoothing factors or NULL (as in quant_act_nvfp4)
 *   lora_down       bf16 [K,R] (L1) or NULL when R == 0
 *   lora_up         bf16 [R,N] (L2) or NULL when R == 0
 *   R               rank, 0..128
 *   y               bf16 [M,N]          out
 *   ws, ws_bytes    scratch of at least qlinear_workspace_bytes(QPL_NVFP4, M, K, N, R);
 *                   after the call it holds the quantized activation the GEMM read:
 *                   its first M K/2 bytes are the packed codes (identical to
 *                   quant_act_nvfp4's x_q), and the 8 M S bytes from offset
 *                   256 ceil(M K/2 / 256) its block scales in the GEMM's slab-major
 *                   layout [S, M, 8], S = ceil(K/128): byte (s M + m) 8 + i is block
 *                   8 s + i of row m (quant_act_nvfp4's x_block_scale[m, 8 s + i]),
 *                   zero for 8 s + i >= K/16.
 * The GEMM multiplies the packed operands as they are: E2M1 codes and E4M3 block
 * scales are expanded in registers to exact f16 values and summed in fp32 on the
 * MFMA units.  With R > 0 the 4-bit product is scaled by input_scale *
 * weight_scale_2 before the low-rank term is added.
 */
qpl_status qlinear_nvfp4(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                         const uint8_t* weight, const uint8_t* weight_scale,
                         float weight_scale_2, float input_scale, const float* smooth,
                         const uint16_t* lora_down, const uint16_t* lora_up, int64_t R,
                         uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * INT4 variant of the SVDQuant W4A4 linear (Nunchaku post, "Introducing Nunchaku
 * Lite": svdq_w4a4 comes in INT4 and NVFP4 variants; the post gives no INT4
 * format, this library's):
 *   codes          signed 4-bit two's complement, channel 2j in the low nibble of
 *                  byte j: uint8 [rows, K/2]
 *   scales         float [rows, K/64], one per group of 64 channels
 *   rule           s = amax / 7 (fp32), q = clamp(rint(x / s), -8, 7) with a
 *                  correctly rounded division, ties to even; an all-zero group
 *                  has s = 0 and codes 0.  The same rule quantizes a weight.
 * quant_act_int4: x bf16 [M,K] (K % 64 == 0) -> x_q, x_scale; with smooth
 *   (float [K] or NULL, as in quant_act_nvfp4) the quantized activation is
 *   bf16_rne(x / smooth).
 * qlinear_int4:
 *   y = bf16_rne( sum_g sx[m,g] sw[n,g] sum_{k in g} qx qw  +  (x L1) L2 )
 *   with qx, sx from quant_act_int4(x, smooth), fp32 accumulation, and the
 *   low-rank term (x replaced by the smoothed x when smooth is given) added
 *   before the single rounding.  weight uint8 [N,K/2], weight_scale float
 *   [N,K/64], lora_down / lora_up / R as in qlinear_nvfp4; ws of at least
 *   qlinear_workspace_bytes(QPL_INT4, M, K, N, R).
 * All pointers 16-byte aligned.
 */
qpl_status quant_act_int4(const uint16_t* x, int64_t M, int64_t K, const float* smooth,
                          uint8_t* x_q, float* x_scale, void* stream);
qpl_status qlinear_int4(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                        const uint8_t* weight, const float* weight_scale, const float* smooth,
                        const uint16_t* lora_down, const uint16_t* lora_up, int64_t R,
                        uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Weight-only 4-bit linear with bf16 activations (Nunchaku post, "Introducing
 * Nunchaku Lite": the awq_w4a16 layer, 4-bit weights and 16-bit activations for
 * the memory-bound adaptive-normalization and modulation projections).  The post
 * gives no format; this library's:
 *   weight        uint8 [N,K/2]     codes q in 0..15, channel 2j in the low nibble of byte j
 *   weight_scale  bf16 [N,K/group]  one scale s per group of `group` input channels
 *   weight_zero   uint8 [N,K/group] one zero point z in 0..15 per group
 *   group         32, 64 or 128; K % group == 0 (else QPL_ERR_ARG / QPL_ERR_SHAPE)
 * The weight value is (q - z) * s, exact in fp32.
 *
 * quant_weight_awq: quantize a bf16 weight w [N,K] into that format.  Per group:
 *   hi = max(max w, 0), lo = min(min w, 0), s = bf16_rne(fp32((hi - lo) / 15)),
 *   z = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15)
 *   (fp32, correctly rounded divisions, ties to even); s == 0 gives q = z = 0.
 *   Activation-aware channel scaling, if any, is applied to w beforehand.
 *   The group spans (hi - lo) must be finite in fp32.
 *
 * qlinear_awq_w4a16: y[m,n] = bf16_rne( sum_k x[m,k] (q[n,k] - z[n,g]) s[n,g] ),
 *   g = k / group, fp32 accumulation.  x bf16 [M,K], y bf16 [M,N].  Built for
 *   small M (one row per image): the weight is streamed once per two rows of x.
 * All pointers 16-byte aligned.  No workspace.
 */
qpl_status quant_weight_awq(const uint16_t* w, int64_t N, int64_t K, int64_t group,
                            uint8_t* w_q, uint16_t* w_scale, uint8_t* w_zero, void* stream);
qpl_status qlinear_awq_w4a16(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                             const uint8_t* weight, const uint16_t* weight_scale,
                             const uint8_t* weight_zero, int64_t group, uint16_t* y, void* stream);

/*
 * Model-specific epilogues (Nunchaku post, "Introducing Nunchaku Lite", first
 * paragraph: the original engine's fused QKV projections and fused GELU/MLP
 * kernels).  The *_ex calls are qlinear_fp8r / qlinear_nvfp4 / qlinear_int4 with an
 * epilogue descriptor `epi` (NULL: the plain call); everything else about them is
 * as documented above.
 *   act       QPL_ACT_GELU_TANH: y = bf16(gelu(v)) with v the layer's fp32 result
 *             and gelu(v) = v / 2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), the tanh
 *             form used by DiT feed-forward blocks, evaluated in fp32 as
 *             v / (1 + exp(-2u)) through exp2 and a reciprocal (a few fp32 ulps)
 *   q, k, v   fused QKV projection (all three set, or all NULL): the weight is
 *             [W_q; W_k; W_v] (N = 3 heads head_dim rows) and row m of the result
 *             goes to q, k and v instead of y:
 *               part[(h tokens + token_offset + m) head_dim + e] = y[m, p d + h head_dim + e]
 *             for part p = 0, 1, 2 (q, k, v), head h, d = heads head_dim; each of
 *             q, k, v is bf16 [heads, tokens, head_dim] (the layout attention reads;
 *             token_offset places the rows, e.g. image tokens after text tokens).
 *             Requires head_dim a power of two in [8, 1024], 0 <= token_offset and
 *             token_offset + M <= tokens, 16-byte aligned q, k, v, and act NONE;
 *             y may then be NULL.  Rows of q, k, v outside the M written are left
 *             untouched.
 * Errors beyond the plain call's: QPL_ERR_ARG for an unknown act or act with QKV,
 * QPL_ERR_NULL for one or two of q, k, v, or for y NULL without them,
 * QPL_ERR_SHAPE for the QKV shape conditions above.
 */
typedef enum { QPL_ACT_NONE = 0, QPL_ACT_GELU_TANH = 1 } qpl_act;

typedef struct {
  qpl_act act;
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  int64_t heads, head_dim, tokens, token_offset;
} qpl_epilogue;

qpl_status qlinear_fp8r_ex(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                           const uint8_t* weight, const float* weight_scale, const qpl_epilogue* epi,
                           uint16_t* y, void* ws, size_t ws_bytes, void* stream);
qpl_status qlinear_nvfp4_ex(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                            const uint8_t* weight, const uint8_t* weight_scale,
                            float weight_scale_2, float input_scale, const float* smooth,
                            const uint16_t* lora_down, const uint16_t* lora_up, int64_t R,
                            const qpl_epilogue* epi, uint16_t* y, void* ws, size_t ws_bytes, void* stream);
qpl_status qlinear_int4_ex(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                           const uint8_t* weight, const float* weight_scale, const float* smooth,
                           const uint16_t* lora_down, const uint16_t* lora_up, int64_t R,
                           const qpl_epilogue* epi, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * GELU MLP of nvfp4 layers (same post and paragraph: fused GELU/MLP kernels):
 *   h = bf16(gelu(fc1(x)))      fc1 as qlinear_nvfp4 with act GELU, [M,K] -> [M,H]
 *   y = fc2(h)                  fc2 as qlinear_nvfp4, [M,H] -> [M,N]
 * GELU runs in fc1's GEMM epilogue; fc2 quantizes h with its own smoothing, input
 * scale and (fused with the quantize) low-rank down-projection, then runs its GEMM.
 * The result equals the two layers called one after the other.  Either layer may
 * carry smoothing and a low-rank branch; each layer's tensors are as in
 * qlinear_nvfp4 (weight [rows, cols/2], weight_scale [rows, cols/16], ...).
 * Workspace: qlinear_mlp_nvfp4_workspace_bytes(M, K, H, N, fc1->R, fc2->R) bytes (0
 * for invalid sizes); it starts with fc2's qlinear_nvfp4 workspace, so after the
 * call it holds fc2's quantized input as described there (codes, then slab-major
 * block scales), and the 2 M H bytes at offset qlinear_workspace_bytes(QPL_NVFP4,
 * M, H, N, fc2->R) hold h.  Errors: as qlinear_nvfp4 for either layer.
 */
typedef struct {
  const uint8_t* weight;        /* uint8 [rows, cols/2], two E2M1 codes per byte */
  const uint8_t* weight_scale;  /* E4M3 [rows, cols/16] */
  float weight_scale_2;
  float input_scale;
  const float* smooth;          /* float [cols] or NULL */
  const uint16_t* lora_down;    /* bf16 [cols, R] or NULL */
  const uint16_t* lora_up;      /* bf16 [R, rows] or NULL */
  int64_t R;
} qpl_nvfp4_layer;

size_t qlinear_mlp_nvfp4_workspace_bytes(int64_t M, int64_t K, int64_t H, int64_t N, int64_t R1, int64_t R2);
qpl_status qlinear_mlp_nvfp4(const uint16_t* x, int64_t M, int64_t K, int64_t H, int64_t N,
                             const qpl_nvfp4_layer* fc1, const qpl_nvfp4_layer* fc2,
                             uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Dequantize a weight to bf16 (guide, "Kernels" section, last paragraph: on other
 * devices the weight is dequantized to compute_dtype on every forward and the
 * layer runs as a regular linear; that linear is the caller's).
 *   QPL_FP8R:  weight uint8 E4M3 [N,K], weight_scale float [N];
 *              w[n,k] = bf16_rne(dec(w) * s[n])
 *   QPL_NVFP4: weight uint8 [N,K/2] packed E2M1, weight_scale uint8 E4M3 [N,K/16];
 *              w[n,k] = bf16_rne((e2m1(w) * dec(sf)) * weight_scale_2)
 *   weight_scale_2 is ignored for QPL_FP8R.
 *   w_bf16  bf16 [N,K]  out
 */
qpl_status dequant_weight(qpl_scheme scheme, const uint8_t* weight, const void* weight_scale,
                          float weight_scale_2, int64_t N, int64_t K,
                          uint16_t* w_bf16, void* stream);

/* Bytes of scratch that qlinear_fp8r / qlinear_nvfp4 need for these sizes
 * (0 if the sizes are invalid).  The scratch may be reused between calls that
 * are ordered on one stream. */
size_t qlinear_workspace_bytes(qpl_scheme scheme, int64_t M, int64_t K, int64_t N, int64_t R);

/*
 * Calibration helper for the nvfp4 global scales (guide, intro bullet on nvfp4:
 * `weight_scale_2` and the calibrated `input_scale`).
 *   qpl_amax_bf16: *amax (device float) = max(*amax, max_i |x[i]|) over n >= 1
 *                  bf16 values; the caller sets *amax to 0 before the first batch.
 *                  x needs 16-byte alignment; amax needs 4-byte alignment.
 *   qpl_nvfp4_global_scale: amax / (448 * 6) in fp32 (host function).
 */
qpl_status qpl_amax_bf16(const uint16_t* x, int64_t n, float* amax, void* stream);
float qpl_nvfp4_global_scale(float amax);

/*
 * Per-kernel timing (a profiling aid, off by default).  While enabled, every kernel
 * launch of the library is bracketed by two HIP events recorded on the launch's
 * stream.  qpl_timing_collect waits for all recorded events, writes per kernel
 * kind the number of launches and their summed duration in milliseconds since
 * the previous collect (arrays of QPL_KERNEL_COUNT entries, caller-owned host
 * memory), and clears the records.  Events are created by the library on first
 * use and reused.  Not thread-safe with respect to concurrent collect calls.
 */
typedef enum {
  QPL_KERNEL_QUANT_FP8_ROW = 0,     /* fp8r activation / weight quantize */
  QPL_KERNEL_QUANT_NVFP4 = 1,       /* nvfp4 quantize to packed codes */
  QPL_KERNEL_QUANT_NVFP4_LINEAR = 2, /* nvfp4 quantize inside qlinear_nvfp4 (R = 0; slab-major scales),
                                        with the weight's block scales into the GEMM's layout */
  QPL_KERNEL_GEMM_FP8R = 3,
  QPL_KERNEL_GEMM_NVFP4 = 4,
  QPL_KERNEL_GEMM_NVFP4_LOWRANK = 5, /* nvfp4 GEMM with the low-rank epilogue */
  QPL_KERNEL_LOWRANK_PREP = 6,      /* low-rank factor transposes (qlinear_int4) */
  QPL_KERNEL_DEQUANT = 7,
  QPL_KERNEL_AMAX = 8,
  QPL_KERNEL_NVFP4_PREP = 9,        /* qlinear_nvfp4's preparation when R > 0: the weight's block scales
                                       into the GEMM's layout and the low-rank factor layouts */
  QPL_KERNEL_QUANT_NVFP4_LOWRANK = 10, /* nvfp4 quantize fused with x L1 (qlinear_nvfp4, R > 0) */
  QPL_KERNEL_QUANT_W4G = 11,        /* quant_weight_awq */
  QPL_KERNEL_GEMV_W4A16 = 12,       /* qlinear_awq_w4a16 */
  QPL_KERNEL_QUANT_INT4 = 13,       /* quant_act_int4, and the INT4 quantize inside qlinear_int4 (R = 0) */
  QPL_KERNEL_INT4_EXPAND = 14,      /* INT4 weight codes -> E4M3 bytes inside qlinear_int4 */
  QPL_KERNEL_GEMM_INT4 = 15,
  QPL_KERNEL_QUANT_INT4_LOWRANK = 16, /* INT4 quantize fused with x L1 (qlinear_int4, R > 0) */
  QPL_KERNEL_GEMM_EPILOGUE = 17,    /* any GEMM with a GELU or QKV epilogue (the *_ex calls, fc1 of
                                       qlinear_mlp_nvfp4) */
  QPL_KERNEL_COUNT = 18
} qpl_kernel;

void qpl_timing_enable(int on);
/* Time only the kernel kinds whose bit (1 << kind) is set in `kinds` (0 = off);
 * an event pair costs a few microseconds of stream time per timed launch. */
void qpl_timing_select(uint32_t kinds);
qpl_status qpl_timing_collect(int64_t* launches, double* total_ms);

/* Static description of a status code. */
const char* qpl_status_str(qpl_status status);

#ifdef __cplusplus
}
#endif

#endif /* QPL_H */
