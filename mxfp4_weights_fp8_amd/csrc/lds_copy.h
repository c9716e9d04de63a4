// Direct-to-LDS copies on gfx950 (buffer_load_dword{,x4} ... lds), shared by the
// LDS-staged GEMMs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

typedef int v4i_s __attribute__((ext_vector_type(4)));

// Buffer resource as four SGPRs (base, stride 0, size, raw access) for inline asm.
// The hardware range check compares the lane (VGPR) offset with the size, so
// callers keep every offset that can pass the end of a tensor in the lane offset;
// a size of 0 turns a copy into zeros that touch no memory.
__device__ __forceinline__ v4i_s rsrc4(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  v4i_s r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)(uint32_t)(b >> 32);
  r[2] = (int)bytes;
  r[3] = kRsrcWord3;
  return r;
}
__device__ __forceinline__ v4i_s rsrc_sized(v4i_s r, bool keep) {
  r[2] = keep ? r[2] : 0;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Lane l's data lands at M0 + l*size. Issued from inline asm so the compiler does
// not serialize later LDS reads against these writes; every use of the copied
// data is preceded by an explicit vmcnt wait and a barrier.
__device__ __forceinline__ void dma16(v4i_s r, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(v4i_s r, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "memory", "m0");
}

// s_waitcnt with only vmcnt constrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace moe
