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
// voffset (per lane) and soffset (uniform) are added; the range check is
// made on the sum, so a row cannot be reached through soffset past the
// resource's range.
__device__ __forceinline__ uint4 ld128(Rsrc r, uint32_t off, uint32_t soff = 0) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld64(Rsrc r, uint32_t off, uint32_t soff = 0) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t ld32(Rsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}
__device__ __forceinline__ uint32_t ld16(Rsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}
__device__ __forceinline__ uint32_t ld8(Rsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, soff, 0);
}
// The same loads with the nontemporal cache policy (NT): for data read
// exactly once, such as packed codes, scales and zero points streamed by a
// decode kernel, so they do not displace reused lines from the caches.
constexpr int kNT = 2;
__device__ __forceinline__ uint4 ld128_nt(Rsrc r, uint32_t off, uint32_t soff = 0) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kNT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t ld16_nt(Rsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, kNT);
}
__device__ __forceinline__ uint32_t ld8_nt(Rsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, soff, kNT);
}

// 16-bit store through a global address-space pointer.  A pointer read from
// memory (a plan's output pointer) is generic, and a generic store is a FLAT
// instruction, which counts on both the vector-memory and the LDS counters;
// while one is pending the compiler cannot wait for a given number of
// outstanding loads and falls back to waiting for all of them, which would
// stall a software pipeline at every tile.  Outputs are always in device
// memory, so the cast is exact.
typedef __attribute__((address_space(1))) uint16_t global_u16;
__device__ __forceinline__ void store_global16(uint16_t *p, int64_t i, uint16_t v) {
  ((global_u16 *)p)[i] = v;
}

// (a & m) | o in one VALU op: gfx950's three-input bitwise op with truth
// table 0xEA (bit i of the table is the result for input bits
// (a, m, o) = (i >> 2 & 1, i >> 1 & 1, i & 1)).  A builtin rather than
// inline assembly, so the compiler sees the instruction and keeps its wait
// states against in-flight matrix instructions.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  return __builtin_amdgcn_bitop3_b32(a, m, o, 0xEA);
}

// Lane exchange between two registers (gfx950 lane swaps):
//   swap32: lanes 32..63 of a  <->  lanes 0..31 of b
//   swap16: odd rows of 16 lanes of a  <->  even rows of b
__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Unpack the 8 codes of one 8-element chunk into 4 packed fp16 pairs
// (q - z) * s, pair i holding chunk elements (i, i + 4): the one fp16
// rounding per weight of the MFMA matmuls.  `t` carries the chunk's codes
// with element i at bits [B*i, B*i + B) of its low half (elements 0..3) and
// element 4 + i at the same bits of its high half; cz = -(1024 + z) and
// s2 = s, both as fp16 pairs.
template <int B>
__device__ __forceinline__ void unpack_f16_chunk(uint32_t t, half2v cz, half2v s2, half8 &out) {
  const uint32_t mask = B == 4 ? 0x000f000fu : 0x00030003u;
  const uint32_t bias = 0x64006400u;                             // 1024.0 pairs
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = and_or(t >> (B * i), mask, bias);         // 1024 + q, exact
    half2v v = __builtin_bit_cast(half2v, p);
    v = (v + cz) * s2;                                           // (q - z) exact, then * s
    out[2 * i] = v.x;
    out[2 * i + 1] = v.y;
  }
}

// LDS barrier for data written to LDS only: waits for this wave's LDS
// operations, not for its outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gq
