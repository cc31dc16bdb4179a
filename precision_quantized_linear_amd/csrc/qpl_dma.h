// Global -> LDS transfers without register staging on gfx950 (buffer_load_dwordx4
// ... lds), the buffer descriptors they use and the wait-count encodings of the
// pipelines built on them.
#pragma once

#include "qpl_device.h"

namespace qpl {

// An offset past every descriptor's range: the load writes zeros, a store is dropped.
constexpr uint32_t kOutOfRange = 0x40000000u;
// gfx9 buffer descriptor word 3: raw 32-bit elements, no swizzle.
constexpr uint32_t kRawBufferWord3 = 0x00020000u;

// s_waitcnt with one counter constrained (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8).  Vector memory operations of a wavefront, loads and
// stores alike, retire from vmcnt in issue order.
#define QPL_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define QPL_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// Descriptor (scalar registers) over `bytes` bytes from `base`; bytes < 2^30.
__device__ __forceinline__ u32x4 make_desc(const void* base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  u32x4 d;
  d.x = __builtin_amdgcn_readfirstlane((uint32_t)p);
  d.y = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  d.z = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
  d.w = kRawBufferWord3;
  return d;
}

// 16 bytes per lane from global memory into LDS: lane l writes LDS bytes
// [lds_addr + 16 l, + 16); an offset past the descriptor's size writes zeros.  It
// is inline assembly so that the compiler does not wait for these loads at every
// LDS read: the pipelines count them themselves (QPL_WAIT_VMCNT).
// The LDS address and soffset are wave-uniform; readfirstlane makes them scalar
// operands even where the compiler keeps a uniform value in a vector register.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, u32x4 desc, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(desc),
                 "s"(__builtin_amdgcn_readfirstlane(soffset))
               : "memory");
}

// 4 bytes per lane from global memory into LDS: lane l writes LDS bytes
// [lds_addr + 4 l, + 4); each dword is checked against the descriptor's size on
// its own (zero past it).
__device__ __forceinline__ void dma4(uint32_t lds_addr, uint32_t voff, u32x4 desc, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(desc),
                 "s"(__builtin_amdgcn_readfirstlane(soffset))
               : "memory");
}

// LDS byte address of a __shared__ array, as a wave-uniform value.
template <class T>
__device__ __forceinline__ uint32_t lds_address(T* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)(p));
}

}  // namespace qpl
