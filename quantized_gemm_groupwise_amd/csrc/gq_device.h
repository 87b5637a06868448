// Device-side helpers shared by the HIP kernel sources (not by host-only
// translation units).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

// Raw buffer resource over [p, p + bytes): a load at an offset >= bytes
// returns 0 instead of touching memory (the hardware range check of buffer
// instructions), which replaces per-lane masks for tails and padding.
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}
// voffset (per lane) is range-checked; soffset (uniform) is added to it.
__device__ __forceinline__ uint4 ld128(Rsrc r, uint32_t off, uint32_t soff = 0) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t ld16(Rsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}
__device__ __forceinline__ uint32_t ld8(Rsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, soff, 0);
}

// (a & m) | o in one VALU op (the three operands in VGPRs; gfx9 VOP3 takes
// no literal constants).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// LDS barrier for data written to LDS only: waits for this wave's LDS
// operations, not for its outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gq
