// Internal declarations shared by the HIP translation units of libgq.
// Nothing here is part of the public ABI (include/gq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gq.h"

namespace gq {

// Layout as the kernels see it: the bit map of GreenBitAI's Layer-mix /
// Channel-mix layouts folded into a bit mask (bit i set = block i is INT4,
// clear = INT2).  Block offsets are popcount prefixes over the mask, so no
// offset table has to live in device memory.
struct LayoutDev {
  int32_t K;
  int32_t N;
  int32_t block_n;
  int32_t nblocks;
  uint32_t int4_mask[GQ_MAX_BLOCKS / 32];
};

struct BlockInfo {
  int bits;            // 4 or 2
  uint64_t code_off;   // byte offset of the block's codes
  uint64_t grp_off;    // index of the block's first scale / zero
};

__host__ __device__ inline BlockInfo block_info(const LayoutDev &L, int blk) {
  int c4 = 0;  // INT4 blocks before blk
  const int w = blk >> 5;
  for (int i = 0; i < w; ++i) c4 += __builtin_popcount(L.int4_mask[i]);
  c4 += __builtin_popcount(L.int4_mask[w] & ((1u << (blk & 31)) - 1u));
  BlockInfo b;
  b.bits = ((L.int4_mask[w] >> (blk & 31)) & 1u) ? 4 : 2;
  const uint64_t bk = (uint64_t)L.block_n * (uint64_t)L.K;
  // INT4 rows take K/2 bytes and K/128 groups, INT2 rows K/4 bytes and K/64 groups.
  b.code_off = bk * (uint64_t)(blk + c4) / 4u;
  b.grp_off = bk * (uint64_t)(2 * blk - c4) / 128u;
  return b;
}

// Host-side helpers (layout.cpp).
gq_status make_layout(const gq_layout *in, LayoutDev *out);
gq_status check_ptr16(const void *p);
size_t linear_workspace_bytes(const LayoutDev &L, int M, gq_dtype act);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_quantize_pack(const LayoutDev &L, const float *w, uint32_t *codes,
                                uint16_t *scales, uint8_t *zeros, uint32_t *flags,
                                hipStream_t s);
hipError_t launch_fake_quant(const LayoutDev &L, const float *w, gq_dtype out, void *w_out,
                             uint32_t *flags, hipStream_t s);
hipError_t launch_dequant(const LayoutDev &L, const uint32_t *codes, const uint16_t *scales,
                          const uint8_t *zeros, gq_dtype out, void *w_out, hipStream_t s);
hipError_t launch_gemv(const LayoutDev &L, int M, gq_dtype act, const void *x,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       void *y, hipStream_t s);
hipError_t launch_gemm(const LayoutDev &L, int M, gq_dtype act, const void *x,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       void *y, void *workspace, hipStream_t s);

// Largest M served by the dot-product (GEMV) kernel; larger M goes to MFMA.
constexpr int kGemvMaxM = 4;
// Largest M served by the small-batch MFMA kernel (bf16/fp16 activations
// used as they are, no pre-pass); larger M goes to the tiled GEMM.
constexpr int kSkinnyMaxM = 32;
bool skinny_supported(const LayoutDev &L, int M);
size_t skinny_workspace_bytes(const LayoutDev &L, int M);
hipError_t launch_skinny(const LayoutDev &L, int M, gq_dtype act, const void *x,
                         const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                         void *y, void *workspace, hipStream_t s);
// Rows of x [M][K] (bf16 or fp16) as exact fp16 in natural order, [Mp][Kp]
// zero padded, with the power-of-two row exponents rexp[M] of the rescale.
hipError_t launch_prep_rows(const void *x, int M, int K, int Mp, int Kp, gq_dtype act, uint16_t *xa,
                            int *rexp, hipStream_t s);
// Sum the fp32 parts of split 256 x 256 tiles (register order of the 4-wave
// MFMA 32x32 tile: wave, 32-row block, 32-column block, element, lane) in
// part order, times 2^rexp[m], rounded; tail tile t is tile full + t of an
// m-fastest tile order.
hipError_t launch_tile_tail_reduce(const float *tail, int parts, int full, int rem, int m_tiles, int M,
                                   int N, const int *rexp, uint16_t *y, int out_fp16, hipStream_t s);
// Sum split-K fp32 partials [splits][M][N] in split order, times 2^rexp[m]
// when rexp is not null, rounded to bf16 (or fp16).
hipError_t launch_splitk_reduce(const float *part, int splits, int M, int N, const int *rexp,
                                uint16_t *y, int out_fp16, hipStream_t s);

// Data gradient dX = dY . W_hat (dx.hip).  Needs N % 8 == 0.
bool dx_supported(const LayoutDev &L, int M);
size_t dx_workspace_bytes(const LayoutDev &L, int M);
hipError_t launch_dx(const LayoutDev &L, int M, gq_dtype act, const void *dy,
                     const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros, void *dx,
                     void *workspace, hipStream_t s);

// Decode attention over a quantized KV cache (kv.hip).
gq_status kv_check(const gq_kv_cache &c);
size_t kv_workspace_bytes(const gq_kv_cache &c);
hipError_t launch_kv(const gq_kv_cache &c, const void *q, void *out, void *workspace, hipStream_t s);

// MFMA tile rows per workgroup, in 32-row blocks, for a given M.
inline int gemm_mb(int M) { return M <= 32 ? 1 : (M <= 64 ? 2 : 4); }
// Workspace of the MFMA path: fp16 activations, row exponents, split-K partials.
size_t gemm_workspace_bytes(const LayoutDev &L, int M);

// ----------------------------------------------------------- device helpers

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

}  // namespace gq
