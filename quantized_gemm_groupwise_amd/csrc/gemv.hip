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
#include <string.h>

#include <mutex>

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
      cur[i] = keep + (off == 8 ? dpp<0x128>(send) : __shfl_xor(send, off));
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
      uint4 *dst = pairs + (ms * (Gm::PW / 4) + 2 * part) * kLanes + lane;
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
};

// Slices >= lim (LIM) are not loaded: they belong to the next staged chunk.
constexpr uint32_t kOutOfRange = 0x80000000u;   // beyond any row resource

template <int BITS, int R, int NL, bool LIM>
__device__ __forceinline__ void issue_group(LoadGroup<BITS, R, NL> &g, int slice0, int lim,
                                            int lane, const RowRsrc<R> &rr) {
  using Gm = Geo<BITS>;
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
        const uint4 *src = pairs + (ms * (Gm::PW / 4)) * kLanes + lane;
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
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // rows past N (ragged tail, or a wave past the end) get empty resources:
    // they load zeros and never store
    const bool live = n0 + r < L.N;
    const uint64_t row = live ? (uint64_t)(r0 + r) : 0u;
    rr.c[r] = make_rsrc(codes + bi.code_off + row * (uint64_t)RB, live ? (uint32_t)RB : 0u);
    rr.s[r] = make_rsrc(scales + bi.grp_off + row * (uint64_t)GPR, live ? 2u * GPR : 0u);
    rr.z[r] = make_rsrc(zeros + bi.grp_off + row * (uint64_t)GPR, live ? (uint32_t)GPR : 0u);
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
    issue_group<BITS, R, NL, false>(g, 0, nslice_row, lane, rr);
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
      issue_group<BITS, R, NL, true>(g, c0, cend, lane, rr);
      __builtin_amdgcn_sched_barrier(0);
      if (restage) {
        stage_x_store<BITS, ACT, M, SS>(st, cn, pairs, sums);
        lds_barrier();
      }
      for (int s = c0;;) {
        compute_group<BITS, ACT, M, R, NL>(g, s, cend, c0, lane, pairs, sums, cn, acc);
        s += NL;
        if (s >= cend) break;
        issue_group<BITS, R, NL, true>(g, s, cend, lane, rr);
      }
    }
  }
  if (!active) return;
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

// BITSEL: 4, 2 or 8 for a uniform (Layer-mix) linear; 0 for a Channel-mix
// layout of INT4 and INT2 blocks and 1 for one that also has 8-bit blocks,
// where the workgroup reads its block's width from the bit masks (the 4R
// rows of a workgroup never straddle two blocks).
template <int ACT, int M, int R, int NL, int BITSEL, int SS, bool ONE>
__global__ __launch_bounds__(kThreads) void gemv_kernel(LayoutDev L, const uint16_t *__restrict__ x,
                                                        const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        const uint8_t *__restrict__ zeros,
                                                        uint16_t *__restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int nb = (int)blockIdx.x * kWaves * R;
  const int n0 = nb + wave * R;
  const bool active = n0 < L.N;                // inactive waves still stage x
  // the launch picks SS so that a chunk holds at least one slice of every
  // bit-width in the layout; other combinations are never launched
  constexpr bool ok4 = chunk_slices(4, M, SS) >= 1, ok2 = chunk_slices(2, M, SS) >= 1;
  constexpr bool ok8 = chunk_slices(8, M, SS) >= 1;
  if constexpr (BITSEL == 4) {
    BlockInfo bi = {4, 0, 0};
    if constexpr (ok4)
      gemv_block<4, ACT, M, R, NL, SS, ONE>(L, bi, 0, n0, active, x, codes, scales, zeros, y, lds);
  } else if constexpr (BITSEL == 2) {
    BlockInfo bi = {2, 0, 0};
    if constexpr (ok2)
      gemv_block<2, ACT, M, R, NL, SS, ONE>(L, bi, 0, n0, active, x, codes, scales, zeros, y, lds);
  } else if constexpr (BITSEL == 8) {
    BlockInfo bi = {8, 0, 0};
    if constexpr (ok8)
      gemv_block<8, ACT, M, R, NL, SS, ONE>(L, bi, 0, n0, active, x, codes, scales, zeros, y, lds);
  } else if constexpr (ok4 && ok2 && (BITSEL == 0 || ok8)) {
    const int blk = nb / L.block_n;
    const BlockInfo bi = block_info(L, blk);
    const int bits = __builtin_amdgcn_readfirstlane(bi.bits);
    if (bits == 4)
      gemv_block<4, ACT, M, R, NL, SS, ONE>(L, bi, blk, n0, active, x, codes, scales, zeros, y, lds);
    else if (BITSEL == 1 && bits == 8)
      gemv_block<8, ACT, M, R, NL, SS, ONE>(L, bi, blk, n0, active, x, codes, scales, zeros, y, lds);
    else
      gemv_block<2, ACT, M, R, NL, SS, ONE>(L, bi, blk, n0, active, x, codes, scales, zeros, y, lds);
  }
}

// ------------------------------------------------------- grouped decode

// Buffer resources of a wave's R rows starting at output channel n0 (rows
// past N get empty resources: they load zeros and are never stored).
template <int BITS, int R>
__device__ __forceinline__ void tile_rows(const LayoutDev &L, const BlockInfo &bi, int blk, int n0,
                                          const uint8_t *codes, const uint16_t *scales,
                                          const uint8_t *zeros, RowRsrc<R> &rr) {
  using Gm = Geo<BITS>;
  const int RB = L.K * BITS / 8, GPR = L.K / Gm::G;
  const int r0 = n0 - blk * L.block_n;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = n0 + r < L.N;
    const uint64_t row = live ? (uint64_t)(r0 + r) : 0u;
    rr.c[r] = make_rsrc(codes + bi.code_off + row * (uint64_t)RB, live ? (uint32_t)RB : 0u);
    rr.s[r] = make_rsrc(scales + bi.grp_off + row * (uint64_t)GPR, live ? 2u * GPR : 0u);
    rr.z[r] = make_rsrc(zeros + bi.grp_off + row * (uint64_t)GPR, live ? (uint32_t)GPR : 0u);
  }
}

// The wave's R * M sums reduced across lanes; one lane per output stores
// y[m][n0 + r] (row stride N) for n0 + r < nlim.
template <int ACT, int M, int R>
__device__ __forceinline__ void reduce_store(const float (&acc)[R][M], int lane, int n0, int nlim,
                                             int N, uint16_t *y) {
  constexpr int V0 = R * M;
  constexpr int V = V0 <= 1 ? 1 : V0 <= 2 ? 2 : V0 <= 4 ? 4 : V0 <= 8 ? 8 : 16;
  float vals[V];
#pragma unroll
  for (int v = 0; v < V; ++v) vals[v] = v < V0 ? acc[v / M][v % M] : 0.f;
  const float tot = wave_reduce_multi<V>(vals, lane);
  const int idx = reduced_index<V>(lane);
  if ((lane & ((64 / V) - 1)) == 0 && idx < V0) {
    const int r = idx / M, m = idx % M;
    if (n0 + r < nlim)
      store_global16(y, (int64_t)m * N + n0 + r, ACT == 0 ? f32_to_bf16_rne(tot) : f32_to_f16_bits(tot));
  }
}

// Position in a class's tile list: segment si, tile t of that segment; T is
// the class tile index, [T0, T1) the workgroup's current chunk.
struct TilePos {
  int si, t, T, T0, T1;
};

// Row resources of a wave's R rows at run-relative row rw of segment S:
// rows past the run's end get empty resources (they load zeros and are
// never stored).
template <int BITS, int R>
__device__ __forceinline__ void seg_rows(const GroupSeg &S, int rw, int K, RowRsrc<R> &rr) {
  using Gm = Geo<BITS>;
  const uint32_t RB = (uint32_t)(K * BITS / 8), GPR = (uint32_t)(K / Gm::G);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = rw + r < S.rows;
    const uint64_t row = live ? (uint64_t)(rw + r) : 0u;
    rr.c[r] = make_rsrc(S.codes + row * RB, live ? RB : 0u);
    rr.s[r] = make_rsrc(S.scales + row * GPR, live ? 2u * GPR : 0u);
    rr.z[r] = make_rsrc(S.zeros + row * GPR, live ? GPR : 0u);
  }
}

// Grouped decode, one class of a plan.  Every tile runs the single-linear
// kernel's arithmetic and order, so the outputs are the same bits as one
// gq_linear call per linear.  x of a linear is staged once per workgroup
// while consecutive tiles stay in that linear.  Every branch below depends
// only on the workgroup and the plan, so the waves of a workgroup meet the
// same barriers.
//
// PIPE (persistent launch; every row fits one load group and one staged
// chunk): workgroup w of G takes the contiguous tile range of its share of
// the class's bytes and walks it segment by segment, software pipelined --
// each wave issues the loads of its next tile before it works on the
// current one, so two tiles of codes are in flight per wave.  Segment data
// is read once per segment and a tile's row resources are a multiply-add
// from the segment's base addresses.  The pipeline restarts where the
// linear changes (x must be restaged first).
//
// Otherwise workgroup w takes the class's chunks of `chunk` tiles
// w, w + G, ... (a grid of one workgroup per tile when chunk is 1 and G the
// tile count) and runs each tile with the single-linear kernel's workgroup
// body (rows in one load group when ONE, else streamed group by group).
template <int ACT, int M, int BITS, int SS, int NL, bool ONE, bool PIPE>
__global__ __launch_bounds__(kThreads) void gemv_group_kernel(const uint8_t *__restrict__ plan,
                                                              int cls, int chunk) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  constexpr int R = group_r(BITS);
  constexpr int kTile = group_tile(BITS);
  using Gm = Geo<BITS>;
  if constexpr (chunk_slices(BITS, M, SS) < 1) {
    return;                                 // never launched: SS too small for M
  } else {
  const GroupPlanHeader &H = *reinterpret_cast<const GroupPlanHeader *>(plan);
  const GroupClass &C = H.cls[cls];
  const GroupSeg *segs = reinterpret_cast<const GroupSeg *>(plan + H.segs_off) + C.seg0;
  const GroupItemDev *items = reinterpret_cast<const GroupItemDev *>(plan + H.items_off);
  const int nseg = C.nseg;
  const int G = gridDim.x, w = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int lane = threadIdx.x & (kLanes - 1);

  if constexpr (ONE && PIPE) {
    // byte range [lo, hi) of the class; the tiles whose first byte is in it
    const int64_t lo = C.bytes * w / G, hi = C.bytes * (w + 1) / G;
    int ls = 0;
    {
      int a = 0, b = nseg - 1;              // last segment starting at or before lo
      while (a < b) {
        const int mid = (a + b + 1) >> 1;
        if (segs[mid].cbyte0 <= lo) a = mid;
        else b = mid - 1;
      }
      ls = a;
    }
    int lt = (int)((lo - segs[ls].cbyte0 + segs[ls].tile_bytes - 1) / segs[ls].tile_bytes);
    if (lt >= segs[ls].ntiles) {
      if (++ls >= nseg) return;
      lt = 0;
    }
    // Load cursor: the tile whose loads are issued next.  Its segment's
    // fields are read from the plan once per segment and kept in scalar
    // registers (stores through y could alias the plan, so fields read
    // again after a store would be loaded again); within a segment the
    // cursor steps by one tile with a few adds.
    int64_t lcb;                            // class byte of the cursor's tile
    int64_t ltb;                            // bytes per tile of its segment
    int lend;                               // tiles of the segment
    int litem;                              // its linear
    const uint8_t *pc;                      // codes of the wave's first row in the tile
    const uint16_t *ps;                     // its scales
    const uint8_t *pz;                      // its zero points
    int lrows;                              // rows of the run from that row on
    int ln0, lnlim;                         // that row in the linear; end of the run
    int K = 0;                              // K of the linear being worked on
    uint32_t RB = 0, GPR = 0;               // row bytes and groups per row
    auto open_seg = [&](int sg, int tt) {
      const GroupSeg &S = segs[sg];
      const int rw = tt * kTile + wave * R;
      lcb = S.cbyte0 + (int64_t)tt * S.tile_bytes;
      ltb = S.tile_bytes;
      lend = S.ntiles;
      litem = S.item;
      const int Ks = items[litem].L.K;
      const uint32_t rb = (uint32_t)(Ks * BITS / 8), gpr = (uint32_t)(Ks / Gm::G);
      pc = S.codes + (uint64_t)rw * rb;
      ps = S.scales + (uint64_t)rw * gpr;
      pz = S.zeros + (uint64_t)rw * gpr;
      lrows = S.rows - rw;
      ln0 = S.tile0 * kTile + rw;
      lnlim = S.tile0 * kTile + S.rows;
    };
    // step the cursor to the next tile of the range; false past its end
    auto advance = [&]() -> bool {
      if (++lt < lend) {
        lcb += ltb;
        pc += kTile * RB;
        ps += kTile * GPR;
        pz += kTile * GPR;
        lrows -= kTile;
        ln0 += kTile;
      } else {
        if (ls + 1 >= nseg) return false;
        ++ls;
        lt = 0;
        open_seg(ls, 0);
      }
      return lcb < hi;
    };
    // issue the loads of the cursor's tile into gl (or, when `none`, the
    // same number of loads of empty resources); rows past the run's end get
    // empty resources
    auto issue_cursor = [&](LoadGroup<BITS, R, NL> &gl, bool none) {
      RowRsrc<R> rr;
      if (!none) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool live = lrows > r;
          rr.c[r] = make_rsrc(pc + r * RB, live ? RB : 0u);
          rr.s[r] = make_rsrc(ps + r * GPR, live ? 2u * GPR : 0u);
          rr.z[r] = make_rsrc(pz + r * GPR, live ? GPR : 0u);
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) rr.c[r] = rr.s[r] = rr.z[r] = make_rsrc(plan, 0u);
      }
      issue_group<BITS, R, NL, false>(gl, 0, NL, lane, rr);
    };
    open_seg(ls, lt);
    if (lcb >= hi) return;

    uint4 *pairs = reinterpret_cast<uint4 *>(lds);
    int item = litem;
    const uint16_t *yp = nullptr;
    int yN = 0;
    auto stage = [&](int it) {
      const GroupItemDev &I = items[it];
      K = I.L.K;
      RB = (uint32_t)(K * BITS / 8);
      GPR = (uint32_t)(K / Gm::G);
      yp = reinterpret_cast<const uint16_t *>(I.y);
      yN = I.L.N;
      const int ns = (K * BITS / 8 + 1023) >> 10;
      const uint32_t xbytes = (uint32_t)(M * K) * 2u;
      StageRegs<SS> st;
      stage_x_load<BITS, M, SS>(st, make_rsrc(I.x, xbytes), xbytes, K, 0, ns);
      stage_x_store<BITS, ACT, M, SS>(st, ns, pairs,
                                      reinterpret_cast<float *>(lds + M * ns * Gm::PW * kLanes));
      lds_barrier();
    };
    // Work on the tile whose codes are in g (outputs from row n0, run end
    // nlim), after issuing the loads of the next tile of the same linear
    // into gn; returns false when the range is done.  The loads into gn are
    // issued on every path (with empty resources when there is no next tile
    // in this linear, so they return zeros without touching memory): the
    // wait before the work on g then counts only g's loads.
    int sn0 = 0, snlim = 0;                 // rows of the tile being worked on
    auto step = [&](LoadGroup<BITS, R, NL> &g, LoadGroup<BITS, R, NL> &gn) -> bool {
      const bool more = advance();
      const bool same = more && litem == item;
      issue_cursor(gn, !same);
      const int ns = (K * BITS / 8 + 1023) >> 10;
      const float *sm = reinterpret_cast<const float *>(lds + M * ns * Gm::PW * kLanes);
      float acc[R][M];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
      compute_group<BITS, ACT, M, R, NL>(g, 0, ns, 0, lane, pairs, sm, ns, acc);
      // rows past the run (a partial last tile) are past N: not stored
      reduce_store<ACT, M, R>(acc, lane, sn0, snlim, yN, const_cast<uint16_t *>(yp));
      if (!more) return false;
      if (!same) {
        // the next tile is in another linear: restage x, then its loads
        item = litem;
        lds_barrier();
        stage(item);
        issue_cursor(gn, false);
      }
      sn0 = ln0;
      snlim = lnlim;
      return true;
    };
    stage(item);
    LoadGroup<BITS, R, NL> ga, gb;
    issue_cursor(ga, false);
    sn0 = ln0;
    snlim = lnlim;
    while (true) {
      if (!step(ga, gb)) break;
      if (!step(gb, ga)) break;
    }
  } else {
  const int tiles = C.tiles;
  // the segment holding class tile T
  auto seg_of_tile = [&](int T) -> int {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (segs[mid].ctile0 <= T) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  // chunks w, w + G, ... of `chunk` tiles
  if ((int64_t)w * chunk >= tiles) return;
  TilePos pos;
  pos.T0 = pos.T = w * chunk;
  pos.T1 = pos.T + chunk < tiles ? pos.T + chunk : tiles;
  pos.si = seg_of_tile(pos.T);
  pos.t = pos.T - segs[pos.si].ctile0;
  // normalize p (after p.t and p.T advanced by one) to a real tile, and say
  // whether the workgroup has one
  auto settle = [&](TilePos &p) -> bool {
    if (p.T >= p.T1) {                      // next chunk of this workgroup
      if ((int64_t)p.T0 + (int64_t)G * chunk >= tiles) return false;
      p.T0 = p.T = p.T0 + G * chunk;
      p.T1 = p.T + chunk < tiles ? p.T + chunk : tiles;
      p.si = seg_of_tile(p.T);
      p.t = p.T - segs[p.si].ctile0;
      return true;
    }
    while (p.t >= segs[p.si].ntiles) {
      ++p.si;
      p.t = 0;
    }
    return true;
  };
  int prev_item = -1;
  do {
    const int item = segs[pos.si].item;
    const GroupItemDev &I = items[item];
    const LayoutDev &L = I.L;
    const int nb = (segs[pos.si].tile0 + pos.t) * kTile;
    const int n0 = nb + wave * R;
    const int ns = (L.K * BITS / 8 + 1023) >> 10;
    // restage when the linear changes, or every tile when a row does not
    // fit one staged chunk; the barrier lets every wave finish reading
    // the previous x first
    const bool stage = item != prev_item || ns > chunk_slices(BITS, M, SS);
    if (stage && prev_item >= 0) lds_barrier();
    BlockInfo bi = {BITS, 0, 0};
    int blk = 0;
    if (!I.uniform) {
      blk = nb / L.block_n;
      bi = block_info(L, blk);
    }
    gemv_block<BITS, ACT, M, R, NL, SS, ONE>(
        L, bi, blk, n0, n0 < L.N, reinterpret_cast<const uint16_t *>(I.x),
        reinterpret_cast<const uint8_t *>(I.codes), reinterpret_cast<const uint16_t *>(I.scales),
        reinterpret_cast<const uint8_t *>(I.zeros), reinterpret_cast<uint16_t *>(I.y), lds, stage);
    prev_item = item;
    ++pos.t;
    ++pos.T;
  } while (settle(pos));
  }
  }
}

template <int ACT, int M, int R, int NL, int SS>
hipError_t launch_rows(const LayoutDev &L, int bitsel, const void *x, const uint32_t *codes,
                       const uint16_t *scales, const uint8_t *zeros, void *y, hipStream_t s) {
  const int blocks = (L.N + kWaves * R - 1) / (kWaves * R);
  const uint16_t *xp = reinterpret_cast<const uint16_t *>(x);
  const uint8_t *cp = reinterpret_cast<const uint8_t *>(codes);
  uint16_t *yp = reinterpret_cast<uint16_t *>(y);
  const dim3 g(blocks), b(kThreads);
  const int ns4 = (L.K * 4 / 8 + 1023) / 1024, ns2 = (L.K * 2 / 8 + 1023) / 1024;
  const int ns8 = (L.K + 1023) / 1024;
  const int s4 = stage_bytes(4, M, ns4, SS), s2 = stage_bytes(2, M, ns2, SS);
  const int s8 = stage_bytes(8, M, ns8, SS);
  const bool one4 = ns4 <= NL && ns4 <= chunk_slices(4, M, SS);
  const bool one2 = ns2 <= NL && ns2 <= chunk_slices(2, M, SS);
  const bool one8 = ns8 <= NL && ns8 <= chunk_slices(8, M, SS);
  if (bitsel == 4) {
    if (one4)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 4, SS, true>), g, b, s4, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 4, SS, false>), g, b, s4, s, L, xp, cp, scales, zeros, yp);
  } else if (bitsel == 2) {
    if (one2)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 2, SS, true>), g, b, s2, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 2, SS, false>), g, b, s2, s, L, xp, cp, scales, zeros, yp);
  } else if (bitsel == 8) {
    if (one8)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 8, SS, true>), g, b, s8, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 8, SS, false>), g, b, s8, s, L, xp, cp, scales, zeros, yp);
  } else if (bitsel == 0) {
    const int sm = s4 > s2 ? s4 : s2;
    if (one4 && one2)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 0, SS, true>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 0, SS, false>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
  } else {
    // a map with 8-bit blocks: rows stream unless every width fits one group
    const int sm = s4 > s2 ? (s4 > s8 ? s4 : s8) : (s2 > s8 ? s2 : s8);
    if (one4 && one2 && one8)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 1, SS, true>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 1, SS, false>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
  }
  return hipGetLastError();
}

template <int ACT, int M, int SS>
hipError_t launch_r(const LayoutDev &L, int bitsel, bool two, int ns, const void *x,
                    const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros, void *y,
                    hipStream_t s) {
  if (ns <= 1)
    return two ? launch_rows<ACT, M, 2, 1, SS>(L, bitsel, x, codes, scales, zeros, y, s)
               : launch_rows<ACT, M, 1, 1, SS>(L, bitsel, x, codes, scales, zeros, y, s);
  return two ? launch_rows<ACT, M, 2, 2, SS>(L, bitsel, x, codes, scales, zeros, y, s)
             : launch_rows<ACT, M, 1, 2, SS>(L, bitsel, x, codes, scales, zeros, y, s);
}

template <int ACT, int M>
hipError_t launch_m(const LayoutDev &L, const void *x, const uint32_t *codes,
                    const uint16_t *scales, const uint8_t *zeros, void *y, hipStream_t s) {
  int n4 = 0, n8 = 0;
  for (int i = 0; i < L.nblocks; ++i) {
    const int b = block_bits(L, i);
    n4 += b == 4;
    n8 += b == 8;
  }
  const int n2 = L.nblocks - n4 - n8;
  const int bitsel = n4 == L.nblocks ? 4 : n2 == L.nblocks ? 2 : n8 == L.nblocks ? 8 : (n8 ? 1 : 0);
  // Load groups of two 1 KB slices (one for rows of a single slice), issued
  // one group ahead; two rows per wave once N gives >= 2048 waves.  Measured
  // on MI355X over the Llama-3-8B decode shapes: issuing a whole long row at
  // once, or more rows per wave, leaves fewer waves to cover HBM latency.
  const int widest = n8 ? 8 : (n4 ? 4 : 2);
  const int ns = (L.K * widest / 8 + 1023) / 1024;
  const bool two = L.N >= 4096;
  // staging sub-units per thread that hold a whole row of x (an INT2 slice
  // carries twice the activations of an INT4 one, an 8-bit slice half)
  const int ns4 = (L.K * 4 / 8 + 1023) / 1024, ns2 = (L.K * 2 / 8 + 1023) / 1024;
  const int ns8 = (L.K + 1023) / 1024;
  const int u4 = n4 ? M * kLanes * 2 * ns4 : 0, u2 = n2 ? M * kLanes * 4 * ns2 : 0;
  const int u8 = n8 ? M * kLanes * ns8 : 0;
  const int um = u4 > u2 ? (u4 > u8 ? u4 : u8) : (u2 > u8 ? u2 : u8);
  const int need = (um + kThreads - 1) / kThreads;
  if (need <= 1) return launch_r<ACT, M, 1>(L, bitsel, two, ns, x, codes, scales, zeros, y, s);
  if (need <= 2) return launch_r<ACT, M, 2>(L, bitsel, two, ns, x, codes, scales, zeros, y, s);
  return launch_r<ACT, M, kStageSubMax>(L, bitsel, two, ns, x, codes, scales, zeros, y, s);
}

template <int ACT>
hipError_t launch_act(const LayoutDev &L, int M, const void *x, const uint32_t *codes,
                      const uint16_t *scales, const uint8_t *zeros, void *y, hipStream_t s) {
  switch (M) {
    case 1: return launch_m<ACT, 1>(L, x, codes, scales, zeros, y, s);
    case 2: return launch_m<ACT, 2>(L, x, codes, scales, zeros, y, s);
    case 3: return launch_m<ACT, 3>(L, x, codes, scales, zeros, y, s);
    default: return launch_m<ACT, 4>(L, x, codes, scales, zeros, y, s);
  }
}

typedef void (*GroupKernel)(const uint8_t *, int, int);

// one: 0 streamed rows, 1 rows of one slice (one-slice load groups), 2 rows
// of two slices; pipe: the software-pipelined persistent body
template <int ACT, int M, int BITS, int SS>
GroupKernel group_kernel_ss(int one, bool pipe) {
  if (one == 1)
    return pipe ? gemv_group_kernel<ACT, M, BITS, SS, 1, true, true> : gemv_group_kernel<ACT, M, BITS, SS, 1, true, false>;
  if (one == 2)
    return pipe ? gemv_group_kernel<ACT, M, BITS, SS, 2, true, true> : gemv_group_kernel<ACT, M, BITS, SS, 2, true, false>;
  return gemv_group_kernel<ACT, M, BITS, SS, kGroupNL, false, false>;
}

template <int ACT, int M, int BITS>
GroupKernel group_kernel_bits(int ss, int one, bool pipe) {
  if (chunk_slices(BITS, M, ss) < 1) return nullptr;   // not a configuration the plan picks
  if (ss == 1) return group_kernel_ss<ACT, M, BITS, 1>(one, pipe);
  if (ss == 2) return group_kernel_ss<ACT, M, BITS, 2>(one, pipe);
  return group_kernel_ss<ACT, M, BITS, 4>(one, pipe);
}

template <int ACT, int M>
GroupKernel group_kernel_m(int bits, int ss, int one, bool pipe) {
  if (bits == 8) return group_kernel_bits<ACT, M, 8>(ss, one, pipe);
  return bits == 4 ? group_kernel_bits<ACT, M, 4>(ss, one, pipe) : group_kernel_bits<ACT, M, 2>(ss, one, pipe);
}

GroupKernel group_kernel(int act, int M, int bits, int ss, int one, bool pipe) {
  const bool bf = act == GQ_BF16;
  switch (M) {
    case 1: return bf ? group_kernel_m<0, 1>(bits, ss, one, pipe) : group_kernel_m<1, 1>(bits, ss, one, pipe);
    case 2: return bf ? group_kernel_m<0, 2>(bits, ss, one, pipe) : group_kernel_m<1, 2>(bits, ss, one, pipe);
    case 3: return bf ? group_kernel_m<0, 3>(bits, ss, one, pipe) : group_kernel_m<1, 3>(bits, ss, one, pipe);
    default: return bf ? group_kernel_m<0, 4>(bits, ss, one, pipe) : group_kernel_m<1, 4>(bits, ss, one, pipe);
  }
}

// Resident workgroups per CU of a kernel at an LDS size, and CUs of the
// current device; each queried once and kept.
int resident_grid(GroupKernel k, int lds) {
  struct Entry { GroupKernel k; int lds; int dev; int grid; };
  static std::mutex mu;
  static Entry cache[256];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].k == k && cache[i].lds == lds && cache[i].dev == dev) return cache[i].grid;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(k), kThreads,
                                                   lds) != hipSuccess)
    return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int grid = per_cu * cus;
  if (used < 256) cache[used++] = {k, lds, dev, grid};
  return grid;
}

// Kernel configuration of one bit-width of a linear: the single-linear
// launch's choices (staging sub-units, one load group per row or streamed
// rows), with R and NL fixed for the group.
struct WidthCfg {
  int ss, one, lds;
};

WidthCfg width_cfg(int bits, int K, int M) {
  const int ns = (K * bits / 8 + 1023) / 1024;
  const int units = M * kLanes * (8 / bits) * ns;
  const int need = (units + kThreads - 1) / kThreads;
  WidthCfg c;
  c.ss = need <= 1 ? 1 : (need <= 2 ? 2 : kStageSubMax);
  // one-load-group rows: 1 or 2 slices (the load group's size), else 0
  c.one = (ns <= kGroupNL && ns <= chunk_slices(bits, M, c.ss)) ? ns : 0;
  c.lds = stage_bytes(bits, M, ns, c.ss);
  return c;
}

// key of a kernel class: width (4, 2, 8 -> 0, 16, 32), then staging and
// load-group configuration
inline int class_key(int bits, const WidthCfg &c) { return (bits == 4 ? 0 : bits == 2 ? 16 : 32) + c.ss * 3 + c.one; }
inline int key_bits(int key) { return key < 16 ? 4 : key < 32 ? 2 : 8; }

}  // namespace

gq_status gemv_group_plan(int count, const gq_group_item *items, int M, gq_dtype act, void *plan,
                          size_t plan_bytes, size_t *need) {
  if (!items) return GQ_ERR_NULL_ARG;
  if (count < 1 || count > 65535 || M < 1 || M > kGemvMaxM) return GQ_ERR_SHAPE;
  if (act != GQ_BF16 && act != GQ_FP16) return GQ_ERR_DTYPE;
  // pass 1: check every item, count segments and classes
  int nkeys = 0, keys[kGroupMaxClasses];
  int64_t nseg = 0;
  for (int i = 0; i < count; ++i) {
    const gq_group_item &it = items[i];
    LayoutDev L;
    gq_status st = make_layout(&it.layout, &L);
    if (st != GQ_OK) return st;
    if (L.N == 0) continue;
    if ((st = check_ptr16(it.x)) != GQ_OK) return st;
    if ((st = check_ptr16(it.codes)) != GQ_OK) return st;
    if (!it.scales || !it.zeros || !it.y) return GQ_ERR_NULL_ARG;
    if (((uintptr_t)it.scales & 1u) || ((uintptr_t)it.y & 1u)) return GQ_ERR_ALIGNMENT;
    int prev = -1;
    for (int b = 0; b < L.nblocks; ++b) {
      const int bits = block_info(L, b).bits;
      if (bits != prev) ++nseg;
      prev = bits;
      const int key = class_key(bits, width_cfg(bits, L.K, M));
      bool seen = false;
      for (int k = 0; k < nkeys; ++k) seen |= keys[k] == key;
      if (!seen) keys[nkeys++] = key;   // at most 3 widths x 3 x 3 = 27 keys
    }
  }
  if (nseg > INT32_MAX / 2) return GQ_ERR_SHAPE;
  const size_t items_off = (sizeof(GroupPlanHeader) + 15) & ~(size_t)15;
  const size_t segs_off = items_off + (size_t)count * sizeof(GroupItemDev);
  const size_t bytes = segs_off + (size_t)nseg * sizeof(GroupSeg);
  if (need) *need = bytes;
  if (!plan) return GQ_OK;
  if (plan_bytes < bytes) return GQ_ERR_WORKSPACE;
  uint8_t *P = static_cast<uint8_t *>(plan);
  memset(P, 0, bytes);
  GroupPlanHeader &H = *reinterpret_cast<GroupPlanHeader *>(P);
  H.magic = kGroupMagic;
  H.version = kGroupVersion;
  H.bytes = bytes;
  H.count = count;
  H.M = M;
  H.act = act;
  H.items_off = items_off;
  H.segs_off = segs_off;
  GroupItemDev *dst = reinterpret_cast<GroupItemDev *>(P + items_off);
  for (int i = 0; i < count; ++i) {
    GroupItemDev &D = dst[i];
    make_layout(&items[i].layout, &D.L);
    D.x = items[i].x;
    D.codes = items[i].codes;
    D.scales = items[i].scales;
    D.zeros = items[i].zeros;
    D.y = items[i].y;
    D.uniform = D.L.nblocks == 1;
  }
  // classes in key order; inside a class, linears in call order and their
  // runs of same-width blocks in block order
  for (int a = 1; a < nkeys; ++a)
    for (int b = a; b > 0 && keys[b - 1] > keys[b]; --b) {
      const int tk = keys[b]; keys[b] = keys[b - 1]; keys[b - 1] = tk;
    }
  GroupSeg *segs = reinterpret_cast<GroupSeg *>(P + segs_off);
  int si = 0;
  for (int k = 0; k < nkeys; ++k) {
    GroupClass &C = H.cls[k];
    C.seg0 = si;
    C.bits = key_bits(keys[k]);
    C.ss = (keys[k] & 15) / 3;
    C.one = (keys[k] & 15) % 3;
    int tiles = 0;
    int64_t cbytes = 0;
    for (int i = 0; i < count; ++i) {
      const LayoutDev &L = dst[i].L;
      if (L.N == 0) continue;
      const WidthCfg c = width_cfg(C.bits, L.K, M);
      if (class_key(C.bits, c) != keys[k]) continue;
      for (int b = 0; b < L.nblocks;) {
        if (block_info(L, b).bits != C.bits) { ++b; continue; }
        int e = b;
        while (e < L.nblocks && block_info(L, e).bits == C.bits) ++e;
        const int tile = group_tile(C.bits);
        const int t0 = b * L.block_n / tile;
        const int t1 = e == L.nblocks ? (L.N + tile - 1) / tile : e * L.block_n / tile;
        const BlockInfo bi = block_info(L, b);
        const int64_t rb = (int64_t)L.K * C.bits / 8;
        GroupSeg &S = segs[si++];
        S.codes = reinterpret_cast<const uint8_t *>(items[i].codes) + bi.code_off;
        S.scales = static_cast<const uint16_t *>(items[i].scales) + bi.grp_off;
        S.zeros = static_cast<const uint8_t *>(items[i].zeros) + bi.grp_off;
        S.item = i;
        S.tile0 = t0;
        S.ntiles = t1 - t0;
        S.ctile0 = tiles;
        S.rows = (e == L.nblocks ? L.N : e * L.block_n) - b * L.block_n;
        S.tile_bytes = (int32_t)(rb * tile);
        S.cbyte0 = cbytes;
        tiles += S.ntiles;
        cbytes += (int64_t)S.ntiles * S.tile_bytes;
        b = e;
      }
      if (c.lds > C.lds) C.lds = c.lds;
    }
    C.nseg = si - C.seg0;
    C.tiles = tiles;
    C.bytes = cbytes;
  }
  H.nclass = nkeys;
  H.nseg = si;
  return GQ_OK;
}

gq_status gemv_group_check(const void *plan) {
  if (!plan) return GQ_ERR_NULL_ARG;
  const GroupPlanHeader &H = *static_cast<const GroupPlanHeader *>(plan);
  if (H.magic != kGroupMagic || H.version != kGroupVersion) return GQ_ERR_SHAPE;
  if (H.count < 1 || H.M < 1 || H.M > kGemvMaxM || (H.act != GQ_BF16 && H.act != GQ_FP16))
    return GQ_ERR_SHAPE;
  if (H.nclass < 0 || H.nclass > kGroupMaxClasses || H.nseg < 0) return GQ_ERR_SHAPE;
  if (H.items_off + (uint64_t)H.count * sizeof(GroupItemDev) > H.segs_off ||
      H.segs_off + (uint64_t)H.nseg * sizeof(GroupSeg) != H.bytes)
    return GQ_ERR_SHAPE;
  int seg = 0;
  for (int c = 0; c < H.nclass; ++c) {
    const GroupClass &C = H.cls[c];
    if (C.seg0 != seg || C.nseg < 1 || (C.bits != 4 && C.bits != 2 && C.bits != 8) ||
        (C.ss != 1 && C.ss != 2 && C.ss != 4) || C.one < 0 || C.one > kGroupNL || C.lds < 0 ||
        C.lds > kLdsBytes || C.tiles < 1 || C.bytes < C.tiles)
      return GQ_ERR_SHAPE;
    seg += C.nseg;
  }
  return seg == H.nseg ? GQ_OK : GQ_ERR_SHAPE;
}

hipError_t launch_gemv_group(const GroupPlanHeader &H, const void *plan_dev, hipStream_t s) {
  const uint8_t *p = static_cast<const uint8_t *>(plan_dev);
  for (int c = 0; c < H.nclass; ++c) {
    const GroupClass &C = H.cls[c];
    // a class with many tiles per resident workgroup runs as a persistent
    // grid (software pipelined over a byte-balanced contiguous tile range
    // when its rows fit one load group, else taking chunks of kGroupChunk
    // tiles in turn); a small one as one workgroup per tile (the hardware
    // dispatcher then overlaps the workgroups' start and end, and no
    // workgroup pays the pipeline's extra registers for a single tile)
    const GroupKernel kp = group_kernel(H.act, H.M, C.bits, C.ss, C.one, true);
    if (!kp) return hipErrorInvalidConfiguration;
    const int resident = resident_grid(kp, C.lds);
    if (resident <= 0) return hipErrorInvalidConfiguration;
    const bool persist = (int64_t)C.tiles >= (int64_t)kGroupPersistTiles * resident;
    const GroupKernel k = persist ? kp : group_kernel(H.act, H.M, C.bits, C.ss, C.one, false);
    const int chunk = persist ? kGroupChunk : 1;
    const int grid = persist ? (resident < C.tiles ? resident : C.tiles) : C.tiles;
    hipLaunchKernelGGL(k, dim3(grid), dim3(kThreads), C.lds, s, p, c, chunk);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemv(const LayoutDev &L, int M, gq_dtype act, const void *x,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       void *y, hipStream_t s) {
  if (act == GQ_BF16) return launch_act<0>(L, M, x, codes, scales, zeros, y, s);
  return launch_act<1>(L, M, x, codes, scales, zeros, y, s);
}

}  // namespace gq
