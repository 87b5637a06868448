// Decode GEMV (M <= 4): y = x . W_hat^T with W_hat = (q - z) * s.
//
// Weight-only quantization moves b-bit codes instead of 16-bit weights and
// dequantizes on chip ("A Survey of Low-bit Large Language Models" review,
// section 6.2: dequantization must cost less than the transfer it saves).
// This kernel is bound by HBM bandwidth: every packed byte is read once with
// a 128-bit load, unpacked in registers and never written back.
//
// Work split.  A workgroup of 4 waves owns 4R consecutive output channels,
// each wave R of them.  A packed row is cut into 1 KB slices; lane l reads
// bytes [1024 i + 16 l, +16) of slice i of each of its R rows, i.e. the
// codes of KPL = 128/b consecutive k.  Code, scale and zero loads for NL
// slices are issued as one group, so each slice waits only for its own
// bytes.  A row longer than one group is streamed group by group (keeping a
// second group in flight measured slower on the 14336-long rows: the extra
// registers cost more than the latency they hide).  Each kernel is compiled
// for one of the two cases, so the short-row kernels hold only the registers
// they use: fewer registers, more resident waves.
//
// Loads go through buffer resources, one per row for codes, scales and
// zeros, whose size is the row's own length (0 for rows past N).  A lane
// past the end of a row, or of x, gets zeros from the hardware range check
// instead of a load, and zero scales make its contribution exactly 0, so the
// kernel needs neither masks nor 64-bit address arithmetic per load.
//
// Activations.  The workgroup stages x in LDS once, already arranged as the
// code pairs come out of a packed word and laid out lane-major so reads are
// conflict-free, together with the per-lane sums sum_k x_k that the zero
// point needs.  LDS traffic has its own counter, so reading x never waits for
// outstanding code loads.
//
// Exactness.  A code q ORed into the low mantissa bits of 128.0 (bf16) or
// 1024.0 (fp16) is exactly 128+q / 1024+q; a 2-bit code two or four bits
// higher reads as 128+4q or 128+16q.  Pairs of such values feed v_dot2
// against the matching activation pairs with fp32 accumulation, one
// accumulator per position class.  Per group the zero point and scale are
// applied as s * (sum x*q - z * sum x), i.e. sum x*(q-z)*s up to fp32
// rounding.
#pragma once

#include "gq_device.h"
#include "gq_internal.h"

namespace gq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kLanes = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kLanes * kWaves;
constexpr int kStageSubMax = 4;            // x sub-units staged per thread per chunk, at most
constexpr int kLdsBytes = 65536;

template <int ACT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (ACT == 0)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
}

// Both 32-bit halves of a 64-bit value shifted right by S (one VALU op for
// two words of codes; the bits that cross into the low word are masked off
// by the caller).
template <int S>
__device__ __forceinline__ uint64_t shr64(uint64_t a) {
  uint64_t r;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "n"(S), "v"(a));
  return r;
}

// (x[i], x[i + half]) from registers holding consecutive activation pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t hi_reg, uint32_t lo_reg) {
  return __builtin_amdgcn_perm(hi_reg, lo_reg, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t hi_reg, uint32_t lo_reg) {
  return __builtin_amdgcn_perm(hi_reg, lo_reg, 0x07060302u);
}

// v read from another lane of the same row of 16 (DPP control CTRL).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Exchange halves between two registers (the lane swaps of gq_device.h on
// float bits).  Afterwards a + b holds, in lanes whose bit 5 (bit 4) is
// clear, the sum of a over the two halves, and in the others the sum of b.
__device__ __forceinline__ void swap32(float &a, float &b) {
  uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
  gq::swap32(ua, ub);
  a = __builtin_bit_cast(float, ua);
  b = __builtin_bit_cast(float, ub);
}
__device__ __forceinline__ void swap16(float &a, float &b) {
  uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
  gq::swap16(ua, ub);
  a = __builtin_bit_cast(float, ua);
  b = __builtin_bit_cast(float, ub);
}

// Sum V per-lane values over the 64 lanes of a wave.  Halving exchanges first
// (each lane keeps half of the values and adds its partner's copy of that
// half), then a butterfly on the last value.  Afterwards lane l holds the
// total of value index  sum_b bit(l, 5-b) * V/2^(b+1)  (b = 0..log2 V - 1).
// Every V adds the same lanes in the same tree -- partners at lane offsets
// 32, 16 and 8, then the mirror inside 8 lanes (l and 7 - l, which differ in
// bit 2), then offsets 2 and 1 -- so a value's total is the same bits
// whatever else is reduced with it (the decode kernels' outputs do not
// depend on rows per wave or M).
template <int V>
__device__ __forceinline__ float wave_reduce_multi(const float (&v)[V], int lane) {
  constexpr int LOGV = V == 1 ? 0 : V == 2 ? 1 : V == 4 ? 2 : V == 8 ? 3 : 4;
  static_assert((1 << LOGV) == V, "V must be a power of two <= 16");
  float cur[V];
#pragma unroll
  for (int i = 0; i < V; ++i) cur[i] = v[i];
  if constexpr (LOGV >= 1) {                   // offset 32
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      swap32(cur[i], cur[i + V / 2]);
      cur[i] += cur[i + V / 2];
    }
  }
  if constexpr (LOGV >= 2) {                   // offset 16
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      swap16(cur[i], cur[i + V / 4]);
      cur[i] += cur[i + V / 4];
    }
  }
#pragma unroll
  for (int b = 2; b < LOGV; ++b) {             // offsets 8, 4
    const int off = 32 >> b;
    const int n = V >> (b + 1);
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const float keep = upper ? cur[i + n] : cur[i];
      const float send = upper ? cur[i] : cur[i + n];
      // offset 8: row_ror:8 (lane l + 8 within a row of 16); the level of
      // bit 2: row_half_mirror (lane 7 - l within 8), the butterfly's partner
      cur[i] = keep + (off == 8 ? dpp<0x128>(send) : dpp<0x141>(send));
    }
  }
  // butterfly over the remaining G = 64/V lanes (every lane of the group
  // ends with the group total); inside a row of 16 lanes with DPP
  constexpr int G = 64 >> LOGV;
  float s = cur[0];
  if constexpr (G >= 64) {
    float t = s;
    swap32(s, t);
    s += t;
  }
  if constexpr (G >= 32) {
    float t = s;
    swap16(s, t);
    s += t;
  }
  if constexpr (G >= 16) s += dpp<0x128>(s);   // row_ror:8
  if constexpr (G >= 8) s += dpp<0x141>(s);    // row_half_mirror
  if constexpr (G >= 4) s += dpp<0x4e>(s);     // quad_perm [2,3,0,1]
  if constexpr (G >= 2) s += dpp<0xb1>(s);     // quad_perm [1,0,3,2]
  return s;
}

template <int V>
__device__ __forceinline__ int reduced_index(int lane) {
  int idx = 0, n = V;
#pragma unroll
  for (int b = 0; (1 << b) < V; ++b) {
    n >>= 1;
    if (lane & (32 >> b)) idx += n;
  }
  return idx;
}

// Slot of lane l's x pairs in the 64 slots (1 KB) of a staged row-slice
// ms = m * nslice + slice: l XOR 4 * (ms mod 4).  A permutation, so the
// dot-product path's reads (each lane its own slot) stay conflict-free; for
// the matrix-core path, whose lanes 4b + j read row j of one slot in 16
// lanes at a time, rows that differ in ms mod 4 land on different LDS banks
// (without it the rows, 8 KB apart, hit the same banks).
__device__ __forceinline__ int pair_slot(int l, int ms) { return l ^ ((ms & 3) << 2); }

// Geometry of one bit-width.
template <int BITS>
struct Geo {
  static constexpr int G = group_size(BITS);            // group size
  static constexpr int KPL = 128 / BITS;                // k per lane per slice
  static constexpr int SK = KPL * kLanes;               // k per slice
  static constexpr int PW = KPL / 2;                    // activation pair words per lane-slice
  static constexpr int NSUM = BITS == 2 ? 2 : 1;        // floats per lane-slice in the sum table
  static constexpr int SPU = KPL / 16;                  // staging sub-units per lane-slice
};

// Stage x[:, k0 : k0 + nslice*SK] into LDS:
//   pairs: uint4 [m][slice][quad q][lane]  words 4q..4q+3 of the lane's pair list
//   sums:  float [m][slice][s][lane]       INT4: sum x; INT2: sum x and B*(X1+X4/4+X16/16)
// Units are (m, slice, lane) triples of KPL activations, each cut into SPU
// sub-units of 16 activations (one INT2 code word, two INT4 code words).
// Thread t stages sub-units t, t + 256, ...; the SPU sub-units of a unit sit
// in consecutive lanes, which combine their partial sums with DPP.  The
// loads of all SS sub-units are issued unconditionally (sub-units past the
// end read out of range and get zeros), so the wait before the stores counts
// exactly; stage_x_store skips the arithmetic of sub-units no thread of the
// workgroup owns.  SS is chosen at launch as the fewest sub-units (1, 2 or
// 4) that stage a whole row: every register held for staging is one less
// wave per SIMD.
template <int SS>
struct StageRegs {
  uint32_t raw[SS][8];
};

template <int BITS, int M, int SS>
__device__ __forceinline__ void stage_x_load(StageRegs<SS> &st, Rsrc xr, uint32_t xbytes, int K,
                                             int k0, int nslice) {
  using Gm = Geo<BITS>;
  const int subs = M * nslice * kLanes * Gm::SPU;
#pragma unroll
  for (int j = 0; j < SS; ++j) {
    const int su = (int)threadIdx.x + j * kThreads;
    const int unit = su / Gm::SPU, part = su % Gm::SPU;
    const int lane = unit & (kLanes - 1);
    const int ms = unit >> 6;                   // m * nslice + slice
    const int m = ms / nslice, sl = ms - m * nslice;
    const int kk = k0 + sl * Gm::SK + lane * Gm::KPL + part * 16;
    const bool ok = su < subs && kk < K;        // K is a multiple of 64
    const uint32_t off = ok ? ((uint32_t)m * (uint32_t)K + (uint32_t)kk) * 2u : xbytes;
    const uint4 a = ld128(xr, off), b = ld128(xr, off + 16u);
    st.raw[j][0] = a.x; st.raw[j][1] = a.y; st.raw[j][2] = a.z; st.raw[j][3] = a.w;
    st.raw[j][4] = b.x; st.raw[j][5] = b.y; st.raw[j][6] = b.z; st.raw[j][7] = b.w;
  }
}

template <int BITS, int ACT, int M, int SS>
__device__ __forceinline__ void stage_x_store(const StageRegs<SS> &st, int nslice, uint4 *pairs,
                                              float *sums) {
  using Gm = Geo<BITS>;
  constexpr uint32_t ONES = ACT == 0 ? 0x3f803f80u : 0x3c003c00u;
  constexpr float BIASF = ACT == 0 ? 128.f : 1024.f;
  const int subs = M * nslice * kLanes * Gm::SPU;
#pragma unroll
  for (int j = 0; j < SS; ++j) {
    if (j * kThreads >= subs) break;            // uniform: nothing left to stage
    const int su = (int)threadIdx.x + j * kThreads;
    const int unit = su / Gm::SPU, part = su % Gm::SPU;
    const int lane = unit & (kLanes - 1);
    const int ms = unit >> 6;
    const uint32_t *q = st.raw[j];
    uint32_t p[8];
    float s0, s1;
    if constexpr (BITS == 4) {
      // code word w covers k 8w..8w+7: pairs (k_t, k_{t+4}), t = 0..3
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        p[4 * w + 0] = pair_lo(q[4 * w + 2], q[4 * w + 0]);
        p[4 * w + 1] = pair_hi(q[4 * w + 2], q[4 * w + 0]);
        p[4 * w + 2] = pair_lo(q[4 * w + 3], q[4 * w + 1]);
        p[4 * w + 3] = pair_hi(q[4 * w + 3], q[4 * w + 1]);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) s = dot2<ACT>(p[t], ONES, s);
      s += dpp<0xb1>(s);                        // the other sub-unit of the unit
      s0 = s;
      s1 = 0.f;
    } else if constexpr (BITS == 8) {
      // code word w covers k 4w..4w+3: pairs (k_4w, k_4w+2), (k_4w+1, k_4w+3)
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        p[2 * w] = pair_lo(q[2 * w + 1], q[2 * w]);
        p[2 * w + 1] = pair_hi(q[2 * w + 1], q[2 * w]);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) s = dot2<ACT>(p[t], ONES, s);
      s0 = s;                                   // one sub-unit per unit: nothing to combine
      s1 = 0.f;
    } else {
      // the code word covers k 0..15: pairs (k_i, k_{i+8}); classes by
      // position in the word: i = 0,3,6 -> 1x, 1,4,7 -> 4x, 2,5 -> 16x
      float c1 = 0.f, c4 = 0.f, c16 = 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        p[2 * a] = pair_lo(q[a + 4], q[a]);         // (x_{2a}, x_{2a+8})
        p[2 * a + 1] = pair_hi(q[a + 4], q[a]);     // (x_{2a+1}, x_{2a+9})
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i % 3 == 0) c1 = dot2<ACT>(p[i], ONES, c1);
        else if (i % 3 == 1) c4 = dot2<ACT>(p[i], ONES, c4);
        else c16 = dot2<ACT>(p[i], ONES, c16);
      }
      // the four sub-units of the unit
      c1 += dpp<0xb1>(c1); c4 += dpp<0xb1>(c4); c16 += dpp<0xb1>(c16);
      c1 += dpp<0x4e>(c1); c4 += dpp<0x4e>(c4); c16 += dpp<0x4e>(c16);
      s0 = c1 + c4 + c16;
      s1 = BIASF * fmaf(c16, 0.0625f, fmaf(c4, 0.25f, c1));
    }
    if (su < subs) {                            // LDS slot exists
      uint4 *dst = pairs + (ms * (Gm::PW / 4) + 2 * part) * kLanes + pair_slot(lane, ms);
      dst[0] = make_uint4(p[0], p[1], p[2], p[3]);
      dst[kLanes] = make_uint4(p[4], p[5], p[6], p[7]);
      if (part == 0) {
        float *sdst = sums + (ms * Gm::NSUM) * kLanes + lane;
        sdst[0] = s0;
        if constexpr (BITS == 2) sdst[kLanes] = s1;
      }
    }
  }
}

template <int BITS, int R, int NL>
struct LoadGroup {
  uint4 cw[NL][R];
  uint32_t sb[NL][R];
  uint32_t zb[NL][R];
};

// Row resources of one wave: codes, scales and zeros of each of its R rows.
template <int R>
struct RowRsrc {
  Rsrc c[R], s[R], z[R];
  uint32_t rb, gpr;           // row bytes and groups per row (matrix-core path)
};

// INT2 rows at M = 3-4 with four rows per wave run on the matrix cores (the
// 16-block 4x4x4 MFMA); every other case on v_dot2.  The dot-product path
// issues 8 v_dot2 per 16 codes and activation row, the matrix-core path a
// fixed 4 instructions per 16 codes for all rows together plus the group's
// scale arithmetic per row.  Measured on MI355X (Llama-3-8B up/gate, one
// launch; the 224-linear Layer-mix pass, grouped; dot-product against
// matrix core): M = 2 7.8 against 8.2 us and 0.545 against 0.523 ms,
// M = 3 10.2 against 9.0 us and 0.73 against 0.58 ms, M = 4 12.0 against
// 9.8 us and 0.92 against 0.62 ms.
__host__ __device__ constexpr bool mfma_decode(int bits, int M, int R) {
  return bits == 2 && M >= 3 && R == 4;
}

// Resources of a wave's R consecutive rows (row r at codes + r * RB, ...;
// `live` of them exist, the rest load zeros).  The dot-product path keeps
// one resource per row.  The matrix-core path reads any of its four rows
// from any lane, so c[0], s[0], z[0] span the live rows together (rows are
// contiguous in a block) and the lanes add the row offset themselves.
template <int BITS, int M, int R>
__device__ __forceinline__ void make_row_rsrc(RowRsrc<R> &rr, const uint8_t *codes,
                                              const uint16_t *scales, const uint8_t *zeros,
                                              uint32_t RB, uint32_t GPR, int live) {
  if constexpr (mfma_decode(BITS, M, R)) {
    // a clamp compiles to a vector min/max; the row count is uniform, and a
    // resource whose size sits in a vector register makes every load a
    // loop over its distinct values, so it is taken back to a scalar
    const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane(live < 0 ? 0 : live > R ? R : live);
    rr.rb = RB;
    rr.gpr = GPR;
    rr.c[0] = make_rsrc(codes, n * RB);
    rr.s[0] = make_rsrc(scales, n * 2u * GPR);
    rr.z[0] = make_rsrc(zeros, n * GPR);
#pragma unroll
    for (int r = 1; r < R; ++r) rr.c[r] = rr.s[r] = rr.z[r] = rr.c[0];
  } else {
    rr.rb = RB;
    rr.gpr = GPR;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool ok = r < live;
      rr.c[r] = make_rsrc(codes + (uint64_t)r * RB, ok ? RB : 0u);
      rr.s[r] = make_rsrc(scales + (uint64_t)r * GPR, ok ? 2u * GPR : 0u);
      rr.z[r] = make_rsrc(zeros + (uint64_t)r * GPR, ok ? GPR : 0u);
    }
  }
}

// Slices >= lim (LIM) are not loaded: they belong to the next staged chunk.
constexpr uint32_t kOutOfRange = 0x80000000u;   // beyond any row resource

template <int BITS, int R, int NL, bool LIM, bool MF = false>
__device__ __forceinline__ void issue_group(LoadGroup<BITS, R, NL> &g, int slice0, int lim,
                                            int lane, const RowRsrc<R> &rr) {
  using Gm = Geo<BITS>;
  if constexpr (MF) {
    // INT2 on the matrix cores: lane 4b + j loads row j's 16-byte chunks
    // b, b + 16, b + 32, b + 48 of each slice (one quantization group of
    // 64 codes each), with that group's scale and zero point.  A chunk
    // past its row's end gets an out-of-range offset (the shared resource
    // would otherwise reach into the next row).
    const uint32_t j = (uint32_t)(lane & 3), b = (uint32_t)(lane >> 2);
    const uint32_t RB = rr.rb, GPR = rr.gpr;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int sl = slice0 + i;
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const uint32_t c = b + 16u * (uint32_t)u;
        const uint32_t in_row = (uint32_t)sl * 1024u + 16u * c;
        const uint32_t gi = (uint32_t)sl * 64u + c;
        const bool ok = in_row < RB && (!LIM || sl < lim);
        const uint32_t off = ok ? j * RB + in_row : kOutOfRange;
        const uint32_t goff = ok ? j * GPR + gi : kOutOfRange;
        g.cw[i][u] = ld128_nt(rr.c[0], off);
        g.sb[i][u] = ld16_nt(rr.s[0], ok ? 2u * goff : kOutOfRange);
        g.zb[i][u] = ld8_nt(rr.z[0], goff);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int sl = slice0 + i;
    // a lane past the row end reads nothing: its offsets are out of range
    // of the row's resources, so codes, scale and zero come back as 0
    uint32_t off = (uint32_t)(sl * 1024 + lane * 16);
    uint32_t gi = (uint32_t)(sl * Gm::SK + lane * Gm::KPL) / Gm::G;
    if (LIM && sl >= lim) off = gi = kOutOfRange;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      g.cw[i][r] = ld128_nt(rr.c[r], off);
      g.sb[i][r] = ld16_nt(rr.s[r], gi == kOutOfRange ? gi : 2u * gi);
      g.zb[i][r] = ld8_nt(rr.z[r], gi);
    }
  }
}

typedef short mf_s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 mf_h16x4 __attribute__((ext_vector_type(4)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));

// 16 independent 4x4x4 products: lanes 4b..4b+3 form block b; lane 4b + i
// supplies row i of A and column i of B (4 k each, as two registers of
// pairs), and after the instruction lane 4b + j holds D[0..3][j] of its
// block.
template <int ACT>
__device__ __forceinline__ mf_f32x4 mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                          mf_f32x4 c) {
  const uint2 a = make_uint2(a0, a1), b = make_uint2(b0, b1);
  if constexpr (ACT == 0)
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(mf_s16x4, a),
                                                  __builtin_bit_cast(mf_s16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(mf_h16x4, a),
                                              __builtin_bit_cast(mf_h16x4, b), c, 0, 0, 0);
}

// INT2 at M = 3-4 on the matrix cores.  A wave's four rows share k: lane
// 4b + j holds, for each of its four 16-byte chunks (one group of 64 codes
// of row j), the codes as exact bias values in the B operand, and the same
// lane supplies activation row j at the same k in the A operand (lanes
// past M read row 0: rows m >= M of D are never used), read from the x
// pairs the staging wrote for that chunk.  The 16 blocks are 16 groups.  Codes unpack as on the dot-product path --
// pairs (q_i, q_i+8) at weights 1, 4 and 16 -- and each weight class
// accumulates in its own D, so after the group's 16 instructions lane
// 4b + j holds, for activation rows m = 0..3,
//   D1 + D4/4 + D16/16 = sum x*q + B * (X1 + X4/4 + X16/16)
// of row j and the group, exactly the dot-product path's p1 + p4/4 + p16/16,
// and applies the group's scale and zero point (its own loads) the same
// way.  acc[m] is then row j's partial sum over this lane's chunks.
template <int ACT, int M, int NL>
__device__ __forceinline__ void compute_group_mfma(const LoadGroup<2, 4, NL> &g, int slice0,
                                                   int nslice_row, int chunk_slice0, int lane,
                                                   const uint4 *pairs, const float *sums,
                                                   int chunk_nslice, float (&acc)[M]) {
  using Gm = Geo<2>;
  constexpr uint32_t bias = ACT == 0 ? 0x43004300u : 0x64006400u;
  const uint32_t m1 = 0x00030003u, m4 = 0x000c000cu, m16 = 0x00300030u;
  const int j = lane & 3, b = lane >> 2;
  const bool xrow = j < M;                       // this lane's activation row exists
  const mf_f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int sl = slice0 + i;
    if (sl < nslice_row) {
      const int lsl = sl - chunk_slice0;
      const int msx = (xrow ? j : 0) * chunk_nslice + lsl;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = b + 16 * u;                // chunk (group) within the slice
        const uint4 *xsrc = pairs + (msx * (Gm::PW / 4)) * kLanes + pair_slot(c, msx);
        mf_f32x4 d1 = zero4, d4 = zero4, d16 = zero4;
        uint32_t pq6 = 0, pq7 = 0, px6 = 0, px7 = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t wv = w == 0 ? g.cw[i][u].x : w == 1 ? g.cw[i][u].y : w == 2 ? g.cw[i][u].z : g.cw[i][u].w;
          const uint32_t w0 = wv, w6 = wv >> 6, w12 = wv >> 12;
          const uint32_t q0 = and_or(w0, m1, bias), q1 = and_or(w0, m4, bias);
          const uint32_t q2 = and_or(w0, m16, bias), q3 = and_or(w6, m1, bias);
          const uint32_t q4 = and_or(w6, m4, bias), q5 = and_or(w6, m16, bias);
          const uint32_t q6 = and_or(w12, m1, bias), q7 = and_or(w12, m4, bias);
          // lanes past M read activation row 0 (the same words as lane
          // 4b, so no extra LDS banks): they feed rows m >= M of D, which
          // are never used
          const uint4 xa = xsrc[(2 * w) * kLanes], xb4 = xsrc[(2 * w + 1) * kLanes];
          // pair t of the word: xa.x..w = pairs 0..3, xb4.x..w = pairs 4..7
          d1 = mfma4<ACT>(xa.x, xa.w, q0, q3, d1);
          d4 = mfma4<ACT>(xa.y, xb4.x, q1, q4, d4);
          d16 = mfma4<ACT>(xa.z, xb4.y, q2, q5, d16);
          if (w % 2 == 0) {
            pq6 = q6; pq7 = q7; px6 = xb4.z; px7 = xb4.w;
          } else {
            d1 = mfma4<ACT>(px6, xb4.z, pq6, q6, d1);
            d4 = mfma4<ACT>(px7, xb4.w, pq7, q7, d4);
          }
        }
        const float S = f16_bits_to_f32((uint16_t)g.sb[i][u]);
        const float zz = (float)g.zb[i][u];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const int ms = m * chunk_nslice + lsl;
          const float *sp = sums + (ms * Gm::NSUM) * kLanes + c;
          const float xs = sp[0], xbs = sp[kLanes];
          const float xq = fmaf(d16[m], 0.0625f, fmaf(d4[m], 0.25f, d1[m])) - xbs;
          acc[m] = fmaf(S, fmaf(-zz, xs, xq), acc[m]);
        }
      }
    }
  }
}

// Matrix-core path: after compute_group_mfma, lane 4b + j holds row j's
// partial sums over its chunks; the 16 lanes of a row are summed (offsets
// 4 and 8 inside each row of 16 lanes, then across rows of 16 and halves),
// in the same tree for every row and M, and lane 4m + j stores y[m][n0 + j].
template <int ACT, int M>
__device__ __forceinline__ void mfma_reduce_store(const float (&acc)[M], int lane, int n0,
                                                  int nlim, int N, uint16_t *y) {
  float tot[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = acc[m];
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
    float t = v;
    swap16(v, t);
    v += t;
    t = v;
    swap32(v, t);
    v += t;
    tot[m] = v;
  }
  const int j = lane & 3, m = lane >> 2;
  if (m < M && n0 + j < nlim) {
    float v = tot[0];
#pragma unroll
    for (int k = 1; k < M; ++k)
      if (m == k) v = tot[k];
    store_global16(y, (int64_t)m * N + n0 + j, ACT == 0 ? f32_to_bf16_rne(v) : f32_to_f16_bits(v));
  }
}

// The x pairs of one slice are read from LDS a chunk at a time (the pairs
// one code word, or one pair of INT4 words, multiplies), and every row of the
// wave consumes a chunk before the next is read: only one chunk of x per M
// row is held in registers.  Each row's accumulation order does not depend
// on this interleaving.
template <int BITS, int ACT, int M, int R, int NL>
__device__ __forceinline__ void compute_group(const LoadGroup<BITS, R, NL> &g, int slice0,
                                              int nslice_row, int chunk_slice0, int lane,
                                              const uint4 *pairs, const float *sums,
                                              int chunk_nslice, float (&acc)[R][M]) {
  using Gm = Geo<BITS>;
  constexpr uint32_t BIAS = ACT == 0 ? 0x43004300u : 0x64006400u;   // 128.0 / 1024.0 pairs
  constexpr float BIASF = ACT == 0 ? 128.f : 1024.f;
  const uint32_t bias = BIAS;
  if constexpr (mfma_decode(BITS, M, R)) {
    compute_group_mfma<ACT, M, NL>(g, slice0, nslice_row, chunk_slice0, lane, pairs, sums,
                                   chunk_nslice, acc[0]);
    return;
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int sl = slice0 + i;
    if (sl < nslice_row) {
    const int lsl = sl - chunk_slice0;          // slice within the staged chunk
    float xs[M], xb[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int ms = m * chunk_nslice + lsl;
      const float *s = sums + (ms * Gm::NSUM) * kLanes + lane;
      xs[m] = s[0];
      if constexpr (BITS == 2) xb[m] = s[kLanes];
    }
    // x pair words [8c, 8c + 8) of row m of this slice
    auto read_chunk = [&](int c, uint32_t (&xc)[M][8]) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int ms = m * chunk_nslice + lsl;
        const uint4 *src = pairs + (ms * (Gm::PW / 4)) * kLanes + pair_slot(lane, ms);
        const uint4 a = src[(2 * c) * kLanes], b = src[(2 * c + 1) * kLanes];
        xc[m][0] = a.x; xc[m][1] = a.y; xc[m][2] = a.z; xc[m][3] = a.w;
        xc[m][4] = b.x; xc[m][5] = b.y; xc[m][6] = b.z; xc[m][7] = b.w;
      }
    };
    if constexpr (BITS == 4) {
      // nibble t of each 16-bit half of word w gives the pair for
      // activation pair 4w + t; words (0,1) and (2,3) are shifted as one
      // 64-bit value, the bits that cross into the low word are masked off
      const uint32_t mask = 0x000f000fu;
      float pa[R][M], pb[R][M];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) pa[r][m] = pb[r][m] = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t xc[M][8];
        read_chunk(h, xc);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t lo = h ? g.cw[i][r].z : g.cw[i][r].x, hi = h ? g.cw[i][r].w : g.cw[i][r].y;
          const uint64_t w64 = ((uint64_t)hi << 32) | lo;
          uint64_t sh[4];
          sh[0] = w64;
          sh[1] = shr64<4>(w64);
          sh[2] = shr64<8>(w64);
          sh[3] = shr64<12>(w64);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t q0 = and_or((uint32_t)sh[t], mask, bias);
            const uint32_t q1 = and_or((uint32_t)(sh[t] >> 32), mask, bias);
#pragma unroll
            for (int m = 0; m < M; ++m) {
              pa[r][m] = dot2<ACT>(q0, xc[m][t], pa[r][m]);
              pb[r][m] = dot2<ACT>(q1, xc[m][4 + t], pb[r][m]);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float S = f16_bits_to_f32((uint16_t)g.sb[i][r]);
        const float zz = (float)g.zb[i][r];
#pragma unroll
        for (int m = 0; m < M; ++m)
          acc[r][m] = fmaf(S, fmaf(-(BIASF + zz), xs[m], pa[r][m] + pb[r][m]), acc[r][m]);
      }
    } else if constexpr (BITS == 8) {
      // byte b of code word w is the code of k = 4w + b.  Its low nibble l
      // and high nibble h go through the 4-bit bias trick separately: pl and
      // ph accumulate (B + l) x and (B + h) x, and with X = sum x,
      // sum q x = 16 (ph - B X) + (pl - B X)
      const uint32_t mask = 0x000f000fu;
      float pl[R][M], ph[R][M];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) pl[r][m] = ph[r][m] = 0.f;
      uint32_t xc[M][8];
      read_chunk(0, xc);
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t wv = w == 0 ? g.cw[i][r].x : w == 1 ? g.cw[i][r].y : w == 2 ? g.cw[i][r].z : g.cw[i][r].w;
          const uint32_t l02 = and_or(wv, mask, bias), h02 = and_or(wv >> 4, mask, bias);
          const uint32_t l13 = and_or(wv >> 8, mask, bias), h13 = and_or(wv >> 12, mask, bias);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            pl[r][m] = dot2<ACT>(l02, xc[m][2 * w], pl[r][m]);
            ph[r][m] = dot2<ACT>(h02, xc[m][2 * w], ph[r][m]);
            pl[r][m] = dot2<ACT>(l13, xc[m][2 * w + 1], pl[r][m]);
            ph[r][m] = dot2<ACT>(h13, xc[m][2 * w + 1], ph[r][m]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float S = f16_bits_to_f32((uint16_t)g.sb[i][r]);
        const float zz = (float)g.zb[i][r];
#pragma unroll
        for (int m = 0; m < M; ++m)
          acc[r][m] = fmaf(S, fmaf(-(17.f * BIASF + zz), xs[m], fmaf(16.f, ph[r][m], pl[r][m])), acc[r][m]);
      }
    } else {
      const uint32_t m1 = 0x00030003u, m4 = 0x000c000cu, m16 = 0x00300030u;
      float p1[R][M], p4[R][M], p16[R][M];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) p1[r][m] = p4[r][m] = p16[r][m] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t xq[M][8];
        read_chunk(w, xq);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t wv = w == 0 ? g.cw[i][r].x : w == 1 ? g.cw[i][r].y : w == 2 ? g.cw[i][r].z : g.cw[i][r].w;
          const uint32_t w0 = wv, w6 = wv >> 6, w12 = wv >> 12;
          const uint32_t q0 = and_or(w0, m1, bias), q1 = and_or(w0, m4, bias);
          const uint32_t q2 = and_or(w0, m16, bias), q3 = and_or(w6, m1, bias);
          const uint32_t q4 = and_or(w6, m4, bias), q5 = and_or(w6, m16, bias);
          const uint32_t q6 = and_or(w12, m1, bias), q7 = and_or(w12, m4, bias);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            p1[r][m] = dot2<ACT>(q0, xq[m][0], p1[r][m]);
            p4[r][m] = dot2<ACT>(q1, xq[m][1], p4[r][m]);
            p16[r][m] = dot2<ACT>(q2, xq[m][2], p16[r][m]);
            p1[r][m] = dot2<ACT>(q3, xq[m][3], p1[r][m]);
            p4[r][m] = dot2<ACT>(q4, xq[m][4], p4[r][m]);
            p16[r][m] = dot2<ACT>(q5, xq[m][5], p16[r][m]);
            p1[r][m] = dot2<ACT>(q6, xq[m][6], p1[r][m]);
            p4[r][m] = dot2<ACT>(q7, xq[m][7], p4[r][m]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float S = f16_bits_to_f32((uint16_t)g.sb[i][r]);
        const float zz = (float)g.zb[i][r];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          // sum x*q = p1 + p4/4 + p16/16 - B*(X1 + X4/4 + X16/16)
          const float xq = fmaf(p16[r][m], 0.0625f, fmaf(p4[r][m], 0.25f, p1[r][m])) - xb[m];
          acc[r][m] = fmaf(S, fmaf(-zz, xs[m], xq), acc[r][m]);
        }
      }
    }
    }
  }
}

// Slices per staged chunk for a bit-width and M: each thread stages at most
// ss sub-units and the chunk fits kLdsBytes.
__host__ __device__ constexpr int chunk_slices(int bits, int M, int ss) {
  const int pw = 64 / bits, nsum = bits == 2 ? 2 : 1;
  const int by_units = ss * kThreads / (M * kLanes * (8 / bits));
  const int by_lds = kLdsBytes / (M * kLanes * 4 * (pw + nsum));
  return by_units < by_lds ? by_units : by_lds;
}

__host__ __device__ constexpr int stage_bytes(int bits, int M, int nslice_row, int ss) {
  const int pw = 64 / bits, nsum = bits == 2 ? 2 : 1;
  const int ch = chunk_slices(bits, M, ss);
  const int c = nslice_row < ch ? nslice_row : ch;
  return M * c * kLanes * 4 * (pw + nsum);
}

// One workgroup: stage x chunk by chunk, stream the wave's R rows.
// ONE: every row of the layout fits one load group and one staged chunk
// (chosen at launch, so each kernel holds the registers of one path only).
// stage == false: x of this linear is already in LDS from the workgroup's
// previous row tile (only when a row fits one staged chunk; the caller keeps
// the workgroup's waves in step).
template <int BITS, int ACT, int M, int R, int NL, int SS, bool ONE>
__device__ __forceinline__ void gemv_block(const LayoutDev &L, const BlockInfo &bi, int blk,
                                           int n0, bool active, const uint16_t *__restrict__ x,
                                           const uint8_t *__restrict__ codes,
                                           const uint16_t *__restrict__ scales,
                                           const uint8_t *__restrict__ zeros,
                                           uint16_t *__restrict__ y, uint32_t *lds,
                                           bool stage = true) {
  using Gm = Geo<BITS>;
  const int lane = threadIdx.x & (kLanes - 1);
  const int K = L.K;
  const int RB = K * BITS / 8;               // bytes per packed row
  const int GPR = K / Gm::G;                 // groups per row
  const int nslice_row = (RB + 1023) >> 10;
  // slices per staged chunk: every thread stages at most SS sub-units and
  // the chunk fits the LDS budget
  constexpr int CHUNK = chunk_slices(BITS, M, SS);
  static_assert(CHUNK >= 1, "chunk");
  static_assert(CHUNK * M * kLanes * 4 * (Gm::PW + Gm::NSUM) <= kLdsBytes, "lds");
  const int r0 = n0 - blk * L.block_n;
  RowRsrc<R> rr;
  {
    // rows past N (ragged tail, or a wave past the end) get empty resources:
    // they load zeros and never store
    const int live = L.N - n0;
    const uint64_t row = live > 0 ? (uint64_t)r0 : 0u;
    make_row_rsrc<BITS, M, R>(rr, codes + bi.code_off + row * (uint64_t)RB,
                              scales + bi.grp_off + row * (uint64_t)GPR,
                              zeros + bi.grp_off + row * (uint64_t)GPR, (uint32_t)RB, (uint32_t)GPR, live);
  }
  const uint32_t xbytes = (uint32_t)(M * K) * 2u;
  const Rsrc xr = make_rsrc(x, xbytes);
  // the LDS arena holds min(CHUNK, nslice_row) slices: pairs, then sums
  const int cslices = nslice_row < CHUNK ? nslice_row : CHUNK;
  uint4 *pairs = reinterpret_cast<uint4 *>(lds);
  float *sums = reinterpret_cast<float *>(lds + M * cslices * Gm::PW * kLanes);
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  if constexpr (ONE) {
    // whole row in one load group and one staged chunk: straight-line code,
    // so slice i waits only for the loads issued before it
    LoadGroup<BITS, R, NL> g;
    StageRegs<SS> st;
    if (stage) stage_x_load<BITS, M, SS>(st, xr, xbytes, K, 0, nslice_row);
    __builtin_amdgcn_sched_barrier(0);
    issue_group<BITS, R, NL, false, mfma_decode(BITS, M, R)>(g, 0, nslice_row, lane, rr);
    __builtin_amdgcn_sched_barrier(0);
    if (stage) {
      stage_x_store<BITS, ACT, M, SS>(st, nslice_row, pairs, sums);
      lds_barrier();
    }
    compute_group<BITS, ACT, M, R, NL>(g, 0, nslice_row, 0, lane, pairs, sums, nslice_row, acc);
  } else {
    // a row that fits one chunk keeps x staged when stage is false
    const bool restage = stage || nslice_row > CHUNK;
    for (int c0 = 0; c0 < nslice_row; c0 += CHUNK) {
      const int cn = nslice_row - c0 < CHUNK ? nslice_row - c0 : CHUNK;
      const int cend = c0 + cn;
      if (c0 > 0) lds_barrier();               // previous chunk fully read
      LoadGroup<BITS, R, NL> g;
      StageRegs<SS> st;
      if (restage) stage_x_load<BITS, M, SS>(st, xr, xbytes, K, c0 * Gm::SK, cn);
      __builtin_amdgcn_sched_barrier(0);
      issue_group<BITS, R, NL, true, mfma_decode(BITS, M, R)>(g, c0, cend, lane, rr);
      __builtin_amdgcn_sched_barrier(0);
      if (restage) {
        stage_x_store<BITS, ACT, M, SS>(st, cn, pairs, sums);
        lds_barrier();
      }
      for (int s = c0;;) {
        compute_group<BITS, ACT, M, R, NL>(g, s, cend, c0, lane, pairs, sums, cn, acc);
        s += NL;
        if (s >= cend) break;
        issue_group<BITS, R, NL, true, mfma_decode(BITS, M, R)>(g, s, cend, lane, rr);
      }
    }
  }
  if (!active) return;
  if constexpr (mfma_decode(BITS, M, R)) {
    mfma_reduce_store<ACT, M>(acc[0], lane, n0, L.N, L.N, y);
    return;
  } else {
  // wave reduction of the R*M partial sums, then one lane per value stores
  constexpr int V0 = R * M;
  constexpr int V = V0 <= 1 ? 1 : V0 <= 2 ? 2 : V0 <= 4 ? 4 : V0 <= 8 ? 8 : 16;
  float vals[V];
#pragma unroll
  for (int v = 0; v < V; ++v) vals[v] = v < V0 ? acc[v / M][v % M] : 0.f;
  const float tot = wave_reduce_multi<V>(vals, lane);
  const int idx = reduced_index<V>(lane);
  if ((lane & ((64 / V) - 1)) == 0 && idx < V0) {
    const int r = idx / M, m = idx % M;
    if (n0 + r < L.N)
      store_global16(y, (int64_t)m * L.N + n0 + r, ACT == 0 ? f32_to_bf16_rne(tot) : f32_to_f16_bits(tot));
  }
  }
}

}  // namespace
}  // namespace gq
