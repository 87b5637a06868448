// Internal declarations shared by the HIP translation units of libgq.
// Nothing here is part of the public ABI (include/gq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gq.h"

namespace gq {

// Layout as the kernels see it: the bit map of GreenBitAI's Layer-mix /
// Channel-mix layouts folded into bit masks (bit i of int4_mask set: block
// i is INT4; of int8_mask: 8-bit; neither: INT2).  Block offsets are
// popcount prefixes over the masks, so no offset table has to live in
// device memory.
struct LayoutDev {
  int32_t K;
  int32_t N;
  int32_t block_n;
  int32_t nblocks;
  int32_t n8;          // 8-bit blocks in the map
  int32_t pad[3];
  uint32_t int4_mask[GQ_MAX_BLOCKS / 32];
  uint32_t int8_mask[GQ_MAX_BLOCKS / 32];
};

struct BlockInfo {
  int bits;            // 2, 4 or 8
  uint64_t code_off;   // byte offset of the block's codes
  uint64_t grp_off;    // index of the block's first scale / zero
};

// Weights per group: 64 for INT2, 128 for INT4 and 8-bit.
__host__ __device__ constexpr int group_size(int bits) { return bits == 2 ? 64 : 128; }

__host__ __device__ inline int block_bits(const LayoutDev &L, int blk) {
  const uint32_t bit = 1u << (blk & 31);
  return (L.int8_mask[blk >> 5] & bit) ? 8 : (L.int4_mask[blk >> 5] & bit) ? 4 : 2;
}

// INT4 and 8-bit blocks among blocks [a, b) of the map, added to c4 and c8.
__host__ __device__ inline void count_blocks(const LayoutDev &L, int a, int b, int &c4, int &c8) {
  for (int w = a >> 5; a < b && w <= ((b - 1) >> 5); ++w) {
    uint32_t m = ~0u;
    if (w == (a >> 5)) m &= ~0u << (a & 31);
    if (w == ((b - 1) >> 5)) m &= ~0u >> (31 - ((b - 1) & 31));
    c4 += __builtin_popcount(L.int4_mask[w] & m);
    c8 += __builtin_popcount(L.int8_mask[w] & m);
  }
}

// Block blk's width and offsets, given the INT4 (c4) and 8-bit (c8) blocks
// before it.
__host__ __device__ inline BlockInfo block_info_counted(const LayoutDev &L, int blk, int c4, int c8) {
  BlockInfo b;
  b.bits = block_bits(L, blk);
  const uint64_t bk = (uint64_t)L.block_n * (uint64_t)L.K;
  // INT2 rows take K/4 bytes and K/64 groups, INT4 rows K/2 bytes and K/128
  // groups, 8-bit rows K bytes and K/128 groups.
  b.code_off = bk * (uint64_t)(blk + c4 + 3 * c8) / 4u;
  b.grp_off = bk * (uint64_t)(2 * blk - c4 - c8) / 128u;
  return b;
}

__host__ __device__ inline BlockInfo block_info(const LayoutDev &L, int blk) {
  int c4 = 0, c8 = 0;  // INT4 and 8-bit blocks before blk
  count_blocks(L, 0, blk, c4, c8);
  return block_info_counted(L, blk, c4, c8);
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

// ------------------------------------------------------- grouped decode

// Plan of a grouped decode call (gq_group_plan / gq_linear_group).  The
// caller keeps a byte copy in device memory, which the kernels read; the
// host copy gives the launch configuration.
//
// Work is cut into row tiles of 4 * group_r(bits, M) output channels (the
// GEMV's workgroup tile).  The tiles of one bit-width and kernel configuration form
// a class, launched once.  A class is a list of segments, runs of
// consecutive tiles of one linear over which the row stride is uniform (a
// Channel-mix linear gives one segment per run of same-width blocks); each
// segment carries the device addresses of its first row's codes, scales and
// zero points, so a kernel finds any row of it with one multiply.
//
// A small class runs one workgroup per tile.  A class with many tiles runs
// as a persistent grid of G workgroups, workgroup w taking the contiguous
// range of tiles whose first packed byte (counted over the class) falls in
// [w * B / G, (w + 1) * B / G), B the class's packed bytes: equal bytes per
// workgroup however the row lengths of the class's linears differ.
constexpr uint32_t kGroupMagic = 0x50475147u;   // "GQGP"
constexpr uint32_t kGroupVersion = 3;
constexpr int kGroupMaxClasses = 27;                // 3 widths x 3 staging x 3 load-group configs
// rows per wave: 4 for INT2 rows (a row of K = 4096 is 1 KB, and four per
// wave amortize the per-tile reduction and bookkeeping; at M = 3-4 the
// wave's four rows share the matrix-core products of the decode kernel),
// else 2: INT4 and 8-bit rows carry two and four times the bytes and
// registers per row.
__host__ __device__ constexpr int group_r(int bits, int M) { return bits == 2 ? 4 : 2; }
constexpr int kGroupNL = 2;                      // 1 KB slices per load group
__host__ __device__ constexpr int group_tile(int bits, int M) { return 4 * group_r(bits, M); }   // rows per tile
constexpr int kGroupChunk = 4;                   // tiles per chunk of a persistent streamed launch
constexpr int kGroupPersistTiles = 4;            // tiles per resident workgroup to persist

struct GroupClass {
  int32_t seg0;        // first segment of the class
  int32_t nseg;        // segments
  int32_t bits;        // 4 or 2
  int32_t ss;          // x staging sub-units per thread (1, 2 or 4)
  int32_t one;         // rows of 1 or 2 slices fit one load group and staged chunk; 0: streamed
  int32_t lds;         // dynamic LDS bytes
  int32_t tiles;       // tiles in the class
  int32_t pad;
  int64_t bytes;       // packed code bytes of the class's tiles (full tiles)
};

struct GroupPlanHeader {
  uint32_t magic;
  uint32_t version;
  uint64_t bytes;      // size of the whole plan
  int32_t count;       // linears
  int32_t M;
  int32_t act;         // gq_dtype of x and y
  int32_t nclass;
  int32_t nseg;
  int32_t pad;
  uint64_t items_off;  // byte offset of GroupItemDev[count]
  uint64_t segs_off;   // byte offset of GroupSeg[nseg]
  GroupClass cls[kGroupMaxClasses];
};

struct GroupItemDev {
  LayoutDev L;
  const void *x;
  const void *codes;
  const void *scales;
  const void *zeros;
  void *y;
  int32_t uniform;     // 1: one block (no per-tile block lookup)
  int32_t pad[3];
};

struct GroupSeg {
  const uint8_t *codes;    // codes of the run's first row
  const uint16_t *scales;  // its first scale
  const uint8_t *zeros;    // its first zero point
  int64_t cbyte0;          // class code bytes of the tiles before the run
  int32_t item;
  int32_t tile0;           // first tile of the run, in the linear's tiles
  int32_t ntiles;
  int32_t ctile0;          // class tiles before the run
  int32_t rows;            // output channels in the run (its last tile may be partial)
  int32_t tile_bytes;      // code bytes of a full tile
  int32_t pad[2];
};
static_assert(sizeof(GroupSeg) == 64, "GroupSeg");

// Host: size of the plan (plan == nullptr) or the plan itself, after
// checking every item; gemv.hip.
gq_status gemv_group_plan(int count, const gq_group_item *items, int M, gq_dtype act, void *plan,
                          size_t plan_bytes, size_t *need);
// Host: sanity checks of a host plan before its launches.
gq_status gemv_group_check(const void *plan);
hipError_t launch_gemv_group(const GroupPlanHeader &H, const void *plan_dev, hipStream_t s);

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
