// C ABI of libqpl.so (declared in include/qpl.h): argument checks on the host,
// workspace carving and kernel launches on the caller's stream.  No entry point
// allocates memory, synchronizes, or lets a C++ exception cross the boundary.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "qpl.h"
#include "qpl_internal.h"

#define QPL_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;    // rows, columns and K each below 2^31
constexpr int64_t kMaxElems = int64_t(1) << 40;  // any operand below 2^40 elements
constexpr int64_t kMaxRank = 128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool positive_finite(float v) { return std::isfinite(v) && v > 0.0f; }

qpl_status check_dims(int64_t M, int64_t K) {
  if (M < 1 || K < 16 || K % 16 != 0 || M >= kMaxDim || K >= kMaxDim) return QPL_ERR_SHAPE;
  if (M > kMaxElems / K) return QPL_ERR_SHAPE;
  return QPL_OK;
}

qpl_status check_gemm_dims(int64_t M, int64_t K, int64_t N) {
  qpl_status s = check_dims(M, K);
  if (s != QPL_OK) return s;
  if (N < 1 || N >= kMaxDim || N > kMaxElems / K || M > kMaxElems / N) return QPL_ERR_SHAPE;
  return QPL_OK;
}

int64_t nvfp4_slabs(int64_t K) { return (K + 127) / 128; }

// The GEMMs address a 256-row tile of an operand through one buffer descriptor with
// 32-bit offsets, and an offset of 2^30 stands for "past the end": 256 rows times
// the row pitch in bytes must stay below 2^30.  fp8r and INT4 rows are K bytes,
// nvfp4 rows K/2.  The fused low-rank quantizers stage up to 128 rows of L1^T
// (2K bytes each) the same way (K <= 2^21) and store their scales through a
// descriptor below 2^31 bytes.
constexpr int64_t kMaxKBytePitch = (int64_t(1) << 30) / 256;
qpl_status check_gemm_k(qpl_scheme scheme, int64_t M, int64_t K, int64_t R) {
  const int64_t pitch = scheme == QPL_NVFP4 ? K / 2 : K;
  if (pitch >= kMaxKBytePitch) return QPL_ERR_SHAPE;
  if (R > 0) {
    if (K > (int64_t(1) << 21)) return QPL_ERR_SHAPE;
    const int64_t sc = scheme == QPL_NVFP4 ? 8 * nvfp4_slabs(K) : 4 * (K / 64);
    if (M >= (int64_t(1) << 31) / sc) return QPL_ERR_SHAPE;
  }
  return QPL_OK;
}

// The current device must be a gfx950; the answer is cached per device ordinal.
std::atomic<int> g_device_state[64];

qpl_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return QPL_ERR_DEVICE;
  }
  const int st = g_device_state[dev].load(std::memory_order_relaxed);
  if (st == 1) return QPL_OK;
  if (st == 2) return QPL_ERR_DEVICE;
  hipDeviceProp_t prop;
  bool ok = false;
  if (hipGetDeviceProperties(&prop, dev) == hipSuccess) ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  (void)hipGetLastError();
  g_device_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? QPL_OK : QPL_ERR_DEVICE;
}

qpl_status launched(hipError_t e) { return e == hipSuccess ? QPL_OK : QPL_ERR_LAUNCH; }

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

int64_t rank_pad(int64_t R) { return (R + 31) / 32 * 32; }

// Workspace layout.  fp8r: [xq: M*K bytes][xs: 4*M bytes].  nvfp4: [xq: M*K/2 packed
// E2M1 codes][xs: 8*M*S block scales slab-major [S, M, 8]], S = ceil(K/128), and, as
// part 5, [wsl: 8*N*S] the weight's block scales in the same layout.  INT4:
// [xq: M*K][w8: N*K] (code values as E4M3 bytes) and, as parts 5 and 6, the
// group-major scales [xs: 4*M*K/64][ws: 4*N*K/64].
// nvfp4 and INT4 then, when R > 0, [l1t: 2*rpad*K][t: 2*M*KL][l2t: 2*N*KL] with
// rpad = 32*ceil(R/32) and KL = 2*rpad.  Each part is rounded up to 256 bytes.
struct Layout {
  size_t off[7] = {0, 0, 0, 0, 0, 0, 0};
  size_t total = 0;
};

Layout layout(qpl_scheme scheme, int64_t M, int64_t K, int64_t N, int64_t R) {
  Layout L;
  size_t parts[7] = {0, 0, 0, 0, 0, 0, 0};
  if (scheme == QPL_FP8R) {
    parts[0] = size_t(M) * size_t(K);
    parts[1] = size_t(4) * size_t(M);
  } else {
    if (scheme == QPL_NVFP4) {
      parts[0] = size_t(M) * size_t(K / 2);
      parts[1] = size_t(8) * size_t(M) * size_t(nvfp4_slabs(K));
      parts[5] = size_t(8) * size_t(N) * size_t(nvfp4_slabs(K));
    } else {
      parts[0] = size_t(M) * size_t(K);
      parts[1] = size_t(N) * size_t(K);
      parts[5] = size_t(4) * size_t(M) * size_t(K / 64);
      parts[6] = size_t(4) * size_t(N) * size_t(K / 64);
    }
    if (R > 0) {
      const int64_t rp = rank_pad(R), kl = 2 * rp;
      parts[2] = size_t(2) * size_t(rp) * size_t(K);
      parts[3] = size_t(2) * size_t(M) * size_t(kl);
      parts[4] = size_t(2) * size_t(N) * size_t(kl);
    }
  }
  size_t o = 0;
  for (int i = 0; i < 7; ++i) {
    L.off[i] = o;
    o += round256(parts[i]);
  }
  L.total = o;
  return L;
}

// ---- per-kernel timing -------------------------------------------------------
std::atomic<uint32_t> g_timing{0u};  // bit k: time launches of kernel kind k
std::mutex g_tmu;
struct TimingRec {
  int kind;
  hipEvent_t start, stop;
};
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}

// Records an event before the launch and one after it when timing is on.
class Timed {
 public:
  Timed(qpl_kernel kind, hipStream_t s) : kind_(kind), s_(s) {
    if (!((g_timing.load(std::memory_order_relaxed) >> int(kind)) & 1u)) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    start_ = take_event();
    if (start_ && hipEventRecord(start_, s_) != hipSuccess) {
      (void)hipGetLastError();
      g_pool.push_back(start_);
      start_ = nullptr;
    }
  }
  hipError_t operator()(hipError_t launch) {
    if (!start_) return launch;
    std::lock_guard<std::mutex> lk(g_tmu);
    hipEvent_t stop = take_event();
    if (stop && hipEventRecord(stop, s_) == hipSuccess) {
      g_recs.push_back({int(kind_), start_, stop});
    } else {
      (void)hipGetLastError();
      g_pool.push_back(start_);
      if (stop) g_pool.push_back(stop);
    }
    start_ = nullptr;
    return launch;
  }

 private:
  qpl_kernel kind_;
  hipStream_t s_;
  hipEvent_t start_ = nullptr;
};

// Epilogue descriptor -> launcher form, with its checks: act known; q, k, v all
// set or all null; with them N = 3 heads head_dim, head_dim a power of two in
// [8, 1024], token_offset + M <= tokens and no activation; otherwise y set.
qpl_status epilogue_of(const qpl_epilogue* epi, int64_t M, int64_t N, const uint16_t* y, qpl::Epilogue& ep) {
  ep = qpl::Epilogue{};
  if (!epi) return y ? QPL_OK : QPL_ERR_NULL;
  if (epi->act != QPL_ACT_NONE && epi->act != QPL_ACT_GELU_TANH) return QPL_ERR_ARG;
  ep.gelu = epi->act == QPL_ACT_GELU_TANH;
  const int nset = (epi->q != nullptr) + (epi->k != nullptr) + (epi->v != nullptr);
  if (nset == 0) return y ? QPL_OK : QPL_ERR_NULL;
  if (nset != 3) return QPL_ERR_NULL;
  if (!aligned16(epi->q) || !aligned16(epi->k) || !aligned16(epi->v)) return QPL_ERR_ALIGN;
  if (ep.gelu) return QPL_ERR_ARG;
  const int64_t hd = epi->head_dim;
  if (hd < 8 || hd > 1024 || (hd & (hd - 1)) != 0) return QPL_ERR_SHAPE;
  if (epi->heads < 1 || epi->heads > kMaxDim / hd || N != 3 * epi->heads * hd) return QPL_ERR_SHAPE;
  if (epi->tokens < 1 || epi->token_offset < 0 || epi->token_offset > epi->tokens - M) return QPL_ERR_SHAPE;
  if (epi->tokens > kMaxElems / (epi->heads * hd)) return QPL_ERR_SHAPE;
  ep.qkv[0] = epi->q;
  ep.qkv[1] = epi->k;
  ep.qkv[2] = epi->v;
  ep.d = epi->heads * hd;
  ep.tokens = epi->tokens;
  ep.off = epi->token_offset;
  while ((int64_t{1} << ep.lg_hd) < hd) ++ep.lg_hd;
  return QPL_OK;
}

qpl_kernel gemm_kind(const qpl::Epilogue& ep, qpl_kernel plain) {
  return ep.gelu || ep.qkv[0] ? QPL_KERNEL_GEMM_EPILOGUE : plain;
}

// timed: record the launches for qpl_timing_collect when timing is on (the
// allocation-free variant never does: the event pool may create events).
qpl_status fp8r_linear(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                       const float* weight_scale, const qpl_epilogue* epi, uint16_t* y, void* ws, size_t ws_bytes,
                       void* stream, bool timed = true) {
  if (!x || !weight || !weight_scale || !ws) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(weight_scale) || !aligned16(y) || !aligned16(ws))
    return QPL_ERR_ALIGN;
  qpl_status s = check_gemm_dims(M, K, N);
  if (s != QPL_OK) return s;
  if ((s = check_gemm_k(QPL_FP8R, M, K, 0)) != QPL_OK) return s;
  qpl::Epilogue ep;
  if ((s = epilogue_of(epi, M, N, y, ep)) != QPL_OK) return s;
  const Layout L = layout(QPL_FP8R, M, K, N, 0);
  if (ws_bytes < L.total) return QPL_ERR_WORKSPACE;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* xq = base + L.off[0];
  float* xs = reinterpret_cast<float*>(base + L.off[1]);
  if (!timed) {
    if ((s = launched(qpl::launch_quant_fp8_row(x, M, K, xq, xs, st))) != QPL_OK) return s;
    return launched(qpl::launch_gemm_fp8r(xq, xs, weight, weight_scale, M, K, N, ep, y, st));
  }
  if ((s = launched(Timed(QPL_KERNEL_QUANT_FP8_ROW, st)(qpl::launch_quant_fp8_row(x, M, K, xq, xs, st)))) != QPL_OK)
    return s;
  return launched(Timed(gemm_kind(ep, QPL_KERNEL_GEMM_FP8R), st)(
      qpl::launch_gemm_fp8r(xq, xs, weight, weight_scale, M, K, N, ep, y, st)));
}

// ---- the allocation-free fp8r linear ----------------------------------------
// Its workspace (codes, then row scales) lives in this file-scope array: each device
// holds its own copy, at its own address, from the library's load until the process
// ends.  Host code never passes the array's name to a kernel or a copy (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kNoallocScratchBytes = size_t(QPL_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[64];

// Device address of the current device's scratch (nullptr on failure).
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

// Checks of one nvfp4 layer's tensors for a linear [N, K] (weight, scales, global
// scales, smoothing factors, low-rank factors against R).
qpl_status check_nvfp4_layer(const uint8_t* weight, const uint8_t* weight_scale, float weight_scale_2,
                             float input_scale, const float* smooth, const uint16_t* lora_down,
                             const uint16_t* lora_up, int64_t R) {
  if (!weight || !weight_scale) return QPL_ERR_NULL;
  if (!aligned16(weight) || !aligned16(weight_scale) || !aligned16(smooth)) return QPL_ERR_ALIGN;
  if (R < 0 || R > kMaxRank) return QPL_ERR_SHAPE;
  if (R > 0 && (!lora_down || !lora_up)) return QPL_ERR_NULL;
  if (R == 0 && (lora_down || lora_up)) return QPL_ERR_ARG;
  if (R > 0 && (!aligned16(lora_down) || !aligned16(lora_up))) return QPL_ERR_ALIGN;
  if (!positive_finite(weight_scale_2) || !positive_finite(input_scale) || !positive_finite(6.0f * input_scale))
    return QPL_ERR_ARG;
  // the product scales the fp32 4-bit product: finite and normal
  const float g = input_scale * weight_scale_2;
  if (!(g >= 0x1p-126f && g <= 0x1.fffffep127f)) return QPL_ERR_ARG;
  return QPL_OK;
}

// The steps of an nvfp4 linear before its GEMM, in the workspace laid out by L at
// base.  R = 0: one launch, the activation quantize into packed codes and
// slab-major block scales, whose extra workgroups relay the weight's block scales
// into the GEMM's layout.  R > 0: a preparation launch (that relay and the
// low-rank factor layouts), then the activation quantize fused with T = x L1,
// which reads L1 in the prepared layout.
qpl_status nvfp4_operands(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight_scale,
                          float input_scale, const float* smooth, const uint16_t* lora_down, const uint16_t* lora_up,
                          int64_t R, const Layout& L, uint8_t* base, hipStream_t st, qpl::LowRank& lr) {
  qpl_status s;
  uint8_t* xq = base + L.off[0];
  uint8_t* xs = base + L.off[1];
  uint8_t* wsl = base + L.off[5];
  lr = qpl::LowRank{};
  if (R > 0) {
    // SVDQuant branch: the factor layouts come with the preparation; the quantizer
    // fused with T = x L1 reads L1^T
    const int64_t kl = 2 * rank_pad(R);
    uint16_t* l1t = reinterpret_cast<uint16_t*>(base + L.off[2]);
    uint16_t* t = reinterpret_cast<uint16_t*>(base + L.off[3]);
    uint16_t* l2t = reinterpret_cast<uint16_t*>(base + L.off[4]);
    const qpl::LowRankPrep prep{lora_down, lora_up, K, N, R, kl / 2, kl, l1t, l2t};
    if ((s = launched(Timed(QPL_KERNEL_NVFP4_PREP, st)(
             qpl::launch_nvfp4_prep(weight_scale, N, K, wsl, M, xs, prep, st)))) != QPL_OK)
      return s;
    lr.t = t;
    lr.l2t = l2t;
    lr.kl = kl;
    return launched(Timed(QPL_KERNEL_QUANT_NVFP4_LOWRANK, st)(
        qpl::launch_quant_nvfp4_lowrank(x, M, K, input_scale, smooth, l1t, kl, xq, xs, t, st)));
  }
  return launched(Timed(QPL_KERNEL_QUANT_NVFP4_LINEAR, st)(
      qpl::launch_quant_nvfp4_linear(x, M, K, input_scale, smooth, xq, xs, weight_scale, N, wsl, st)));
}

qpl_status nvfp4_linear(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                        const uint8_t* weight_scale, float weight_scale_2, float input_scale, const float* smooth,
                        const uint16_t* lora_down, const uint16_t* lora_up, int64_t R, const qpl_epilogue* epi,
                        uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !ws) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return QPL_ERR_ALIGN;
  qpl_status s = check_nvfp4_layer(weight, weight_scale, weight_scale_2, input_scale, smooth, lora_down, lora_up, R);
  if (s != QPL_OK) return s;
  if ((s = check_gemm_dims(M, K, N)) != QPL_OK) return s;
  if ((s = check_gemm_k(QPL_NVFP4, M, K, R)) != QPL_OK) return s;
  qpl::Epilogue ep;
  if ((s = epilogue_of(epi, M, N, y, ep)) != QPL_OK) return s;
  const float gscale = input_scale * weight_scale_2;
  const Layout L = layout(QPL_NVFP4, M, K, N, R);
  if (ws_bytes < L.total) return QPL_ERR_WORKSPACE;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  qpl::LowRank lr;
  if ((s = nvfp4_operands(x, M, K, N, weight_scale, input_scale, smooth, lora_down, lora_up, R, L, base, st, lr)) !=
      QPL_OK)
    return s;
  return launched(Timed(gemm_kind(ep, R > 0 ? QPL_KERNEL_GEMM_NVFP4_LOWRANK : QPL_KERNEL_GEMM_NVFP4), st)(
      qpl::launch_gemm_nvfp4(base + L.off[0], base + L.off[1], weight, base + L.off[5], gscale, M, K, N, lr, ep, y,
                             st)));
}

}  // namespace

QPL_EXPORT void qpl_timing_enable(int on) { g_timing.store(on ? (1u << QPL_KERNEL_COUNT) - 1u : 0u); }

QPL_EXPORT void qpl_timing_select(uint32_t kinds) { g_timing.store(kinds & ((1u << QPL_KERNEL_COUNT) - 1u)); }

QPL_EXPORT qpl_status qpl_timing_collect(int64_t* launches, double* total_ms) {
  if (!launches || !total_ms) return QPL_ERR_NULL;
  for (int i = 0; i < QPL_KERNEL_COUNT; ++i) {
    launches[i] = 0;
    total_ms[i] = 0.0;
  }
  std::lock_guard<std::mutex> lk(g_tmu);
  qpl_status st = QPL_OK;
  for (const TimingRec& r : g_recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      (void)hipGetLastError();
      st = QPL_ERR_DEVICE;
    } else {
      launches[r.kind] += 1;
      total_ms[r.kind] += ms;
    }
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  return st;
}

QPL_EXPORT const char* qpl_status_str(qpl_status status) {
  switch (status) {
    case QPL_OK: return "ok";
    case QPL_ERR_NULL: return "a required pointer is NULL";
    case QPL_ERR_SHAPE: return "invalid shape (need M, N >= 1, K >= 16, K % 16 == 0, 0 <= R <= 128, sizes in range)";
    case QPL_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case QPL_ERR_ARG: return "invalid argument (scales must be finite and > 0; scheme; low-rank pointers vs R)";
    case QPL_ERR_WORKSPACE: return "workspace too small";
    case QPL_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case QPL_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

QPL_EXPORT float qpl_nvfp4_global_scale(float amax) { return amax / 2688.0f; }

QPL_EXPORT size_t qlinear_workspace_bytes(qpl_scheme scheme, int64_t M, int64_t K, int64_t N, int64_t R) {
  if (scheme != QPL_FP8R && scheme != QPL_NVFP4 && scheme != QPL_INT4) return 0;
  if (check_gemm_dims(M, K, N) != QPL_OK || R < 0 || R > kMaxRank) return 0;
  if (scheme == QPL_INT4 && K % 64 != 0) return 0;
  if (scheme == QPL_FP8R && R != 0) return 0;
  if (check_gemm_k(scheme, M, K, R) != QPL_OK) return 0;
  return layout(scheme, M, K, N, R).total;
}

QPL_EXPORT qpl_status quant_act_fp8_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* x_q, float* x_scale,
                                        void* stream) {
  if (!x || !x_q || !x_scale) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(x_q) || !aligned16(x_scale)) return QPL_ERR_ALIGN;
  qpl_status s = check_dims(M, K);
  if (s != QPL_OK) return s;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(Timed(QPL_KERNEL_QUANT_FP8_ROW, st)(qpl::launch_quant_fp8_row(x, M, K, x_q, x_scale, st)));
}

QPL_EXPORT qpl_status quant_act_nvfp4(const uint16_t* x, int64_t M, int64_t K, float input_scale,
                                      const float* smooth, uint8_t* x_q, uint8_t* x_block_scale, void* stream) {
  if (!x || !x_q || !x_block_scale) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(x_q) || !aligned16(x_block_scale) || !aligned16(smooth)) return QPL_ERR_ALIGN;
  qpl_status s = check_dims(M, K);
  if (s != QPL_OK) return s;
  if (!positive_finite(input_scale) || !positive_finite(6.0f * input_scale)) return QPL_ERR_ARG;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(
      Timed(QPL_KERNEL_QUANT_NVFP4, st)(qpl::launch_quant_nvfp4(x, M, K, input_scale, smooth, x_q, x_block_scale, st)));
}

QPL_EXPORT qpl_status qlinear_fp8r(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                                   const float* weight_scale, uint16_t* y, void* ws, size_t ws_bytes,
                                   void* stream) {
  return fp8r_linear(x, M, K, N, weight, weight_scale, nullptr, y, ws, ws_bytes, stream);
}

QPL_EXPORT qpl_status qlinear_fp8r_ex(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                                      const float* weight_scale, const qpl_epilogue* epi, uint16_t* y, void* ws,
                                      size_t ws_bytes, void* stream) {
  return fp8r_linear(x, M, K, N, weight, weight_scale, epi, y, ws, ws_bytes, stream);
}

QPL_EXPORT qpl_status qlinear_fp8r_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                                           const uint8_t* weight, const float* weight_scale, uint16_t* y,
                                           void* stream) {
  // the checks that need no device first, so a bad call touches no device state
  if (!x || !weight || !weight_scale || !y) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(weight_scale) || !aligned16(y)) return QPL_ERR_ALIGN;
  qpl_status s = check_gemm_dims(M, K, N);
  if (s != QPL_OK) return s;
  if ((s = check_gemm_k(QPL_FP8R, M, K, 0)) != QPL_OK) return s;
  if (layout(QPL_FP8R, M, K, N, 0).total > kNoallocScratchBytes) return QPL_ERR_WORKSPACE;
  if ((s = check_device()) != QPL_OK) return s;
  void* ws = scratch_of_current_device();
  if (!ws) return QPL_ERR_DEVICE;
  return fp8r_linear(x, M, K, N, weight, weight_scale, nullptr, y, ws, kNoallocScratchBytes, stream, false);
}

QPL_EXPORT qpl_status qlinear_nvfp4(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                                    const uint8_t* weight_scale, float weight_scale_2, float input_scale,
                                    const float* smooth, const uint16_t* lora_down, const uint16_t* lora_up,
                                    int64_t R, uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  return nvfp4_linear(x, M, K, N, weight, weight_scale, weight_scale_2, input_scale, smooth, lora_down, lora_up, R,
                      nullptr, y, ws, ws_bytes, stream);
}

QPL_EXPORT qpl_status qlinear_nvfp4_ex(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                                       const uint8_t* weight_scale, float weight_scale_2, float input_scale,
                                       const float* smooth, const uint16_t* lora_down, const uint16_t* lora_up,
                                       int64_t R, const qpl_epilogue* epi, uint16_t* y, void* ws, size_t ws_bytes,
                                       void* stream) {
  return nvfp4_linear(x, M, K, N, weight, weight_scale, weight_scale_2, input_scale, smooth, lora_down, lora_up, R,
                      epi, y, ws, ws_bytes, stream);
}

namespace {

// GELU MLP: fc1 with the GELU epilogue writes h, then fc2 runs on h (its quantize,
// fused with x L1 when it has a low-rank branch, then its GEMM).  Workspace:
// [fc2's nvfp4 layout for (M, H, N, R2), whose first parts are fc2's packed
// activation codes and slab-major block scales][h: 2 M H][fc1's nvfp4 layout for
// (M, K, H, R1)], each part rounded up to 256 bytes.
struct MlpLayout {
  size_t h = 0, fc1 = 0, total = 0;
  Layout l1, l2;
};

MlpLayout mlp_layout(int64_t M, int64_t K, int64_t H, int64_t N, int64_t R1, int64_t R2) {
  MlpLayout L;
  L.l2 = layout(QPL_NVFP4, M, H, N, R2);
  L.l1 = layout(QPL_NVFP4, M, K, H, R1);
  L.h = L.l2.total;
  L.fc1 = L.h + round256(size_t(2) * size_t(M) * size_t(H));
  L.total = L.fc1 + L.l1.total;
  return L;
}

}  // namespace

QPL_EXPORT size_t qlinear_mlp_nvfp4_workspace_bytes(int64_t M, int64_t K, int64_t H, int64_t N, int64_t R1,
                                                    int64_t R2) {
  if (check_gemm_dims(M, K, H) != QPL_OK || check_gemm_dims(M, H, N) != QPL_OK) return 0;
  if (R1 < 0 || R1 > kMaxRank || R2 < 0 || R2 > kMaxRank) return 0;
  if (check_gemm_k(QPL_NVFP4, M, K, R1) != QPL_OK || check_gemm_k(QPL_NVFP4, M, H, R2) != QPL_OK) return 0;
  return mlp_layout(M, K, H, N, R1, R2).total;
}

QPL_EXPORT qpl_status qlinear_mlp_nvfp4(const uint16_t* x, int64_t M, int64_t K, int64_t H, int64_t N,
                                        const qpl_nvfp4_layer* fc1, const qpl_nvfp4_layer* fc2, uint16_t* y,
                                        void* ws, size_t ws_bytes, void* stream) {
  if (!x || !fc1 || !fc2 || !y || !ws) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return QPL_ERR_ALIGN;
  qpl_status s = check_nvfp4_layer(fc1->weight, fc1->weight_scale, fc1->weight_scale_2, fc1->input_scale,
                                   fc1->smooth, fc1->lora_down, fc1->lora_up, fc1->R);
  if (s != QPL_OK) return s;
  if ((s = check_nvfp4_layer(fc2->weight, fc2->weight_scale, fc2->weight_scale_2, fc2->input_scale, fc2->smooth,
                             fc2->lora_down, fc2->lora_up, fc2->R)) != QPL_OK)
    return s;
  if ((s = check_gemm_dims(M, K, H)) != QPL_OK || (s = check_gemm_dims(M, H, N)) != QPL_OK) return s;
  if ((s = check_gemm_k(QPL_NVFP4, M, K, fc1->R)) != QPL_OK || (s = check_gemm_k(QPL_NVFP4, M, H, fc2->R)) != QPL_OK)
    return s;
  const MlpLayout L = mlp_layout(M, K, H, N, fc1->R, fc2->R);
  if (ws_bytes < L.total) return QPL_ERR_WORKSPACE;
  if ((s = check_device()) != QPL_OK) return s;
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + L.h);
  qpl_epilogue gelu{};
  gelu.act = QPL_ACT_GELU_TANH;
  if ((s = nvfp4_linear(x, M, K, H, fc1->weight, fc1->weight_scale, fc1->weight_scale_2, fc1->input_scale,
                        fc1->smooth, fc1->lora_down, fc1->lora_up, fc1->R, &gelu, h, base + L.fc1, L.l1.total,
                        stream)) != QPL_OK)
    return s;
  return nvfp4_linear(h, M, H, N, fc2->weight, fc2->weight_scale, fc2->weight_scale_2, fc2->input_scale,
                      fc2->smooth, fc2->lora_down, fc2->lora_up, fc2->R, nullptr, y, base, L.l2.total, stream);
}

QPL_EXPORT qpl_status quant_weight_awq(const uint16_t* w, int64_t N, int64_t K, int64_t group, uint8_t* w_q,
                                       uint16_t* w_scale, uint8_t* w_zero, void* stream) {
  if (!w || !w_q || !w_scale || !w_zero) return QPL_ERR_NULL;
  if (!aligned16(w) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(w_zero)) return QPL_ERR_ALIGN;
  if (group != 32 && group != 64 && group != 128) return QPL_ERR_ARG;
  qpl_status s = check_dims(N, K);
  if (s != QPL_OK) return s;
  if (K % group != 0) return QPL_ERR_SHAPE;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(Timed(QPL_KERNEL_QUANT_W4G, st)(qpl::launch_quant_w4g(w, N, K, (int)group, w_q, w_scale, w_zero, st)));
}

QPL_EXPORT qpl_status qlinear_awq_w4a16(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                                        const uint16_t* weight_scale, const uint8_t* weight_zero, int64_t group,
                                        uint16_t* y, void* stream) {
  if (!x || !weight || !weight_scale || !weight_zero || !y) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(weight_scale) || !aligned16(weight_zero) || !aligned16(y))
    return QPL_ERR_ALIGN;
  if (group != 32 && group != 64 && group != 128) return QPL_ERR_ARG;
  qpl_status s = check_gemm_dims(M, K, N);
  if (s != QPL_OK) return s;
  if (K % group != 0) return QPL_ERR_SHAPE;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(Timed(QPL_KERNEL_GEMV_W4A16, st)(
      qpl::launch_gemv_w4a16(x, M, K, N, weight, weight_scale, weight_zero, (int)group, y, st)));
}

QPL_EXPORT qpl_status quant_act_int4(const uint16_t* x, int64_t M, int64_t K, const float* smooth, uint8_t* x_q,
                                     float* x_scale, void* stream) {
  if (!x || !x_q || !x_scale) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(x_q) || !aligned16(x_scale) || !aligned16(smooth)) return QPL_ERR_ALIGN;
  qpl_status s = check_dims(M, K);
  if (s != QPL_OK) return s;
  if (K % 64 != 0) return QPL_ERR_SHAPE;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(Timed(QPL_KERNEL_QUANT_INT4, st)(qpl::launch_quant_int4(x, M, K, smooth, false, x_q, x_scale, st)));
}

namespace {

qpl_status int4_linear(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                              const float* weight_scale, const float* smooth, const uint16_t* lora_down,
                              const uint16_t* lora_up, int64_t R, const qpl_epilogue* epi, uint16_t* y, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!x || !weight || !weight_scale || !ws) return QPL_ERR_NULL;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(weight_scale) || !aligned16(y) || !aligned16(ws) ||
      !aligned16(smooth))
    return QPL_ERR_ALIGN;
  qpl_status s = check_gemm_dims(M, K, N);
  if (s != QPL_OK) return s;
  if (K % 64 != 0) return QPL_ERR_SHAPE;
  if (R < 0 || R > kMaxRank) return QPL_ERR_SHAPE;
  if ((s = check_gemm_k(QPL_INT4, M, K, R)) != QPL_OK) return s;
  if (R > 0 && (!lora_down || !lora_up)) return QPL_ERR_NULL;
  if (R == 0 && (lora_down || lora_up)) return QPL_ERR_ARG;
  if (R > 0 && (!aligned16(lora_down) || !aligned16(lora_up))) return QPL_ERR_ALIGN;
  qpl::Epilogue ep;
  if ((s = epilogue_of(epi, M, N, y, ep)) != QPL_OK) return s;
  const Layout L = layout(QPL_INT4, M, K, N, R);
  if (ws_bytes < L.total) return QPL_ERR_WORKSPACE;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* xq = base + L.off[0];
  uint8_t* w8 = base + L.off[1];
  float* xs = reinterpret_cast<float*>(base + L.off[5]);
  float* wst = reinterpret_cast<float*>(base + L.off[6]);
  qpl::LowRank lr;
  if (R > 0) {
    const int64_t kl = 2 * rank_pad(R);
    uint16_t* l1t = reinterpret_cast<uint16_t*>(base + L.off[2]);
    uint16_t* t = reinterpret_cast<uint16_t*>(base + L.off[3]);
    uint16_t* l2t = reinterpret_cast<uint16_t*>(base + L.off[4]);
    if ((s = launched(Timed(QPL_KERNEL_LOWRANK_PREP, st)(
             qpl::launch_lowrank_prep(lora_down, lora_up, K, N, R, kl, l1t, l2t, st)))) != QPL_OK)
      return s;
    if ((s = launched(Timed(QPL_KERNEL_QUANT_INT4_LOWRANK, st)(
             qpl::launch_quant_int4_lowrank(x, M, K, smooth, l1t, kl, xq, xs, t, st)))) != QPL_OK)
      return s;
    lr.t = t;
    lr.l2t = l2t;
    lr.kl = kl;
  } else if ((s = launched(Timed(QPL_KERNEL_QUANT_INT4, st)(
                  qpl::launch_quant_int4(x, M, K, smooth, true, xq, xs, st)))) != QPL_OK) {
    return s;
  }
  if ((s = launched(Timed(QPL_KERNEL_INT4_EXPAND, st)(
           qpl::launch_expand_int4(weight, weight_scale, N, K, w8, wst, st)))) != QPL_OK)
    return s;
  return launched(Timed(gemm_kind(ep, QPL_KERNEL_GEMM_INT4), st)(
      qpl::launch_gemm_int4(xq, xs, w8, wst, M, K, N, lr, ep, y, st)));
}

}  // namespace

QPL_EXPORT qpl_status qlinear_int4(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                                   const float* weight_scale, const float* smooth, const uint16_t* lora_down,
                                   const uint16_t* lora_up, int64_t R, uint16_t* y, void* ws, size_t ws_bytes,
                                   void* stream) {
  return int4_linear(x, M, K, N, weight, weight_scale, smooth, lora_down, lora_up, R, nullptr, y, ws, ws_bytes, stream);
}

QPL_EXPORT qpl_status qlinear_int4_ex(const uint16_t* x, int64_t M, int64_t K, int64_t N, const uint8_t* weight,
                                      const float* weight_scale, const float* smooth, const uint16_t* lora_down,
                                      const uint16_t* lora_up, int64_t R, const qpl_epilogue* epi, uint16_t* y,
                                      void* ws, size_t ws_bytes, void* stream) {
  return int4_linear(x, M, K, N, weight, weight_scale, smooth, lora_down, lora_up, R, epi, y, ws, ws_bytes, stream);
}

QPL_EXPORT qpl_status dequant_weight(qpl_scheme scheme, const uint8_t* weight, const void* weight_scale,
                                     float weight_scale_2, int64_t N, int64_t K, uint16_t* w_bf16, void* stream) {
  if (scheme != QPL_FP8R && scheme != QPL_NVFP4) return QPL_ERR_ARG;
  if (!weight || !weight_scale || !w_bf16) return QPL_ERR_NULL;
  if (!aligned16(weight) || !aligned16(weight_scale) || !aligned16(w_bf16)) return QPL_ERR_ALIGN;
  qpl_status s = check_dims(N, K);
  if (s != QPL_OK) return s;
  if (scheme == QPL_NVFP4 && !positive_finite(weight_scale_2)) return QPL_ERR_ARG;
  if ((s = check_device()) != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Timed timed(QPL_KERNEL_DEQUANT, st);
  if (scheme == QPL_FP8R)
    return launched(timed(qpl::launch_dequant_fp8r(weight, static_cast<const float*>(weight_scale), N, K, w_bf16, st)));
  return launched(timed(qpl::launch_dequant_nvfp4(weight, static_cast<const uint8_t*>(weight_scale), weight_scale_2,
                                                  N, K, w_bf16, st)));
}

QPL_EXPORT qpl_status qpl_amax_bf16(const uint16_t* x, int64_t n, float* amax, void* stream) {
  if (!x || !amax) return QPL_ERR_NULL;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(amax) & 3u) != 0) return QPL_ERR_ALIGN;
  if (n < 1 || n >= kMaxElems) return QPL_ERR_SHAPE;
  qpl_status s = check_device();
  if (s != QPL_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(Timed(QPL_KERNEL_AMAX, st)(qpl::launch_amax_bf16(x, n, amax, st)));
}
