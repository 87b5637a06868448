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
  static constexpr int G = BITS == 4 ? 128 : 64;       // group size
  static constexpr int KPL = 128 / BITS;                // k per lane per slice
  static constexpr int SK = KPL * kLanes;               // k per slice
  static constexpr int PW = KPL / 2;                    // activation pair words per lane-slice
  static constexpr int NSUM = BITS == 4 ? 1 : 2;        // floats per lane-slice in the sum table
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
      g.cw[i][r] = ld128(rr.c[r], off);
      g.sb[i][r] = ld16(rr.s[r], gi == kOutOfRange ? gi : 2u * gi);
      g.zb[i][r] = ld8(rr.z[r], gi);
    }
  }
}

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
    uint32_t xp[M][Gm::PW];
    float xs[M], xb[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int ms = m * chunk_nslice + lsl;
      const uint4 *src = pairs + (ms * (Gm::PW / 4)) * kLanes + lane;
#pragma unroll
      for (int q = 0; q < Gm::PW / 4; ++q) {
        const uint4 t = src[q * kLanes];
        xp[m][4 * q + 0] = t.x; xp[m][4 * q + 1] = t.y;
        xp[m][4 * q + 2] = t.z; xp[m][4 * q + 3] = t.w;
      }
      const float *s = sums + (ms * Gm::NSUM) * kLanes + lane;
      xs[m] = s[0];
      if constexpr (BITS == 2) xb[m] = s[kLanes];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t wv[4] = {g.cw[i][r].x, g.cw[i][r].y, g.cw[i][r].z, g.cw[i][r].w};
      const float S = f16_bits_to_f32((uint16_t)g.sb[i][r]);
      const float zz = (float)g.zb[i][r];
      if constexpr (BITS == 4) {
        // nibble t of each 16-bit half of word w gives the pair for
        // activation pair 4w + t; words (0,1) and (2,3) are shifted as one
        // 64-bit value, the bits that cross into the low word are masked off
        const uint32_t mask = 0x000f000fu;
        float pa[M], pb[M];
#pragma unroll
        for (int m = 0; m < M; ++m) pa[m] = pb[m] = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint64_t w64 = ((uint64_t)wv[2 * h + 1] << 32) | wv[2 * h];
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
              pa[m] = dot2<ACT>(q0, xp[m][4 * (2 * h) + t], pa[m]);
              pb[m] = dot2<ACT>(q1, xp[m][4 * (2 * h + 1) + t], pb[m]);
            }
          }
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
          acc[r][m] = fmaf(S, fmaf(-(BIASF + zz), xs[m], pa[m] + pb[m]), acc[r][m]);
      } else {
        const uint32_t m1 = 0x00030003u, m4 = 0x000c000cu, m16 = 0x00300030u;
        float p1[M], p4[M], p16[M];
#pragma unroll
        for (int m = 0; m < M; ++m) p1[m] = p4[m] = p16[m] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t w0 = wv[w], w6 = wv[w] >> 6, w12 = wv[w] >> 12;
          const uint32_t q0 = and_or(w0, m1, bias), q1 = and_or(w0, m4, bias);
          const uint32_t q2 = and_or(w0, m16, bias), q3 = and_or(w6, m1, bias);
          const uint32_t q4 = and_or(w6, m4, bias), q5 = and_or(w6, m16, bias);
          const uint32_t q6 = and_or(w12, m1, bias), q7 = and_or(w12, m4, bias);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const uint32_t *xq = &xp[m][8 * w];
            p1[m] = dot2<ACT>(q0, xq[0], p1[m]);
            p4[m] = dot2<ACT>(q1, xq[1], p4[m]);
            p16[m] = dot2<ACT>(q2, xq[2], p16[m]);
            p1[m] = dot2<ACT>(q3, xq[3], p1[m]);
            p4[m] = dot2<ACT>(q4, xq[4], p4[m]);
            p16[m] = dot2<ACT>(q5, xq[5], p16[m]);
            p1[m] = dot2<ACT>(q6, xq[6], p1[m]);
            p4[m] = dot2<ACT>(q7, xq[7], p4[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          // sum x*q = p1 + p4/4 + p16/16 - B*(X1 + X4/4 + X16/16)
          const float xq = fmaf(p16[m], 0.0625f, fmaf(p4[m], 0.25f, p1[m])) - xb[m];
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
  const int pw = bits == 4 ? 16 : 32, nsum = bits == 4 ? 1 : 2;
  const int by_units = ss * kThreads / (M * kLanes * (bits == 4 ? 2 : 4));
  const int by_lds = kLdsBytes / (M * kLanes * 4 * (pw + nsum));
  return by_units < by_lds ? by_units : by_lds;
}

__host__ __device__ constexpr int stage_bytes(int bits, int M, int nslice_row, int ss) {
  const int pw = bits == 4 ? 16 : 32, nsum = bits == 4 ? 1 : 2;
  const int ch = chunk_slices(bits, M, ss);
  const int c = nslice_row < ch ? nslice_row : ch;
  return M * c * kLanes * 4 * (pw + nsum);
}

// One workgroup: stage x chunk by chunk, stream the wave's R rows.
// ONE: every row of the layout fits one load group and one staged chunk
// (chosen at launch, so each kernel holds the registers of one path only).
template <int BITS, int ACT, int M, int R, int NL, int SS, bool ONE>
__device__ __forceinline__ void gemv_block(const LayoutDev &L, const BlockInfo &bi, int blk,
                                           int n0, bool active, const uint16_t *__restrict__ x,
                                           const uint8_t *__restrict__ codes,
                                           const uint16_t *__restrict__ scales,
                                           const uint8_t *__restrict__ zeros,
                                           uint16_t *__restrict__ y, uint32_t *lds) {
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
    stage_x_load<BITS, M, SS>(st, xr, xbytes, K, 0, nslice_row);
    __builtin_amdgcn_sched_barrier(0);
    issue_group<BITS, R, NL, false>(g, 0, nslice_row, lane, rr);
    __builtin_amdgcn_sched_barrier(0);
    stage_x_store<BITS, ACT, M, SS>(st, nslice_row, pairs, sums);
    lds_barrier();
    compute_group<BITS, ACT, M, R, NL>(g, 0, nslice_row, 0, lane, pairs, sums, nslice_row, acc);
  } else {
    for (int c0 = 0; c0 < nslice_row; c0 += CHUNK) {
      const int cn = nslice_row - c0 < CHUNK ? nslice_row - c0 : CHUNK;
      const int cend = c0 + cn;
      if (c0 > 0) lds_barrier();               // previous chunk fully read
      LoadGroup<BITS, R, NL> g;
      StageRegs<SS> st;
      stage_x_load<BITS, M, SS>(st, xr, xbytes, K, c0 * Gm::SK, cn);
      __builtin_amdgcn_sched_barrier(0);
      issue_group<BITS, R, NL, true>(g, c0, cend, lane, rr);
      __builtin_amdgcn_sched_barrier(0);
      stage_x_store<BITS, ACT, M, SS>(st, cn, pairs, sums);
      lds_barrier();
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
      y[(int64_t)m * L.N + n0 + r] = ACT == 0 ? f32_to_bf16_rne(tot) : f32_to_f16_bits(tot);
  }
}

// BITSEL: 4 or 2 for a uniform (Layer-mix) linear, 0 for a Channel-mix
// layout where the workgroup reads its block's width from the bit mask (the
// 4R rows of a workgroup never straddle two blocks).
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
  if constexpr (BITSEL == 4) {
    BlockInfo bi = {4, 0, 0};
    if constexpr (ok4)
      gemv_block<4, ACT, M, R, NL, SS, ONE>(L, bi, 0, n0, active, x, codes, scales, zeros, y, lds);
  } else if constexpr (BITSEL == 2) {
    BlockInfo bi = {2, 0, 0};
    if constexpr (ok2)
      gemv_block<2, ACT, M, R, NL, SS, ONE>(L, bi, 0, n0, active, x, codes, scales, zeros, y, lds);
  } else if constexpr (ok4 && ok2) {
    const int blk = nb / L.block_n;
    const BlockInfo bi = block_info(L, blk);
    if (__builtin_amdgcn_readfirstlane(bi.bits) == 4)
      gemv_block<4, ACT, M, R, NL, SS, ONE>(L, bi, blk, n0, active, x, codes, scales, zeros, y, lds);
    else
      gemv_block<2, ACT, M, R, NL, SS, ONE>(L, bi, blk, n0, active, x, codes, scales, zeros, y, lds);
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
  const int s4 = stage_bytes(4, M, ns4, SS), s2 = stage_bytes(2, M, ns2, SS);
  const bool one4 = ns4 <= NL && ns4 <= chunk_slices(4, M, SS);
  const bool one2 = ns2 <= NL && ns2 <= chunk_slices(2, M, SS);
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
  } else {
    const int sm = s4 > s2 ? s4 : s2;
    if (one4 && one2)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 0, SS, true>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 0, SS, false>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
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
  uint32_t any4 = 0, all4 = ~0u;
  for (int i = 0; i < L.nblocks; ++i) {
    const uint32_t b = (L.int4_mask[i >> 5] >> (i & 31)) & 1u;
    any4 |= b;
    all4 &= b;
  }
  const int bitsel = all4 ? 4 : (any4 ? 0 : 2);
  // Load groups of two 1 KB slices (one for rows of a single slice), issued
  // one group ahead; two rows per wave once N gives >= 2048 waves.  Measured
  // on MI355X over the Llama-3-8B decode shapes: issuing a whole long row at
  // once, or more rows per wave, leaves fewer waves to cover HBM latency.
  const int ns = (L.K * (any4 ? 4 : 2) / 8 + 1023) / 1024;
  const bool two = L.N >= 4096;
  // staging sub-units per thread that hold a whole row of x (INT2 slices
  // carry twice the activations of INT4 ones)
  const int ns4 = (L.K * 4 / 8 + 1023) / 1024, ns2 = (L.K * 2 / 8 + 1023) / 1024;
  const int u4 = any4 ? M * kLanes * 2 * ns4 : 0, u2 = all4 ? 0 : M * kLanes * 4 * ns2;
  const int need = ((u4 > u2 ? u4 : u2) + kThreads - 1) / kThreads;
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

}  // namespace

hipError_t launch_gemv(const LayoutDev &L, int M, gq_dtype act, const void *x,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       void *y, hipStream_t s) {
  if (act == GQ_BF16) return launch_act<0>(L, M, x, codes, scales, zeros, y, s);
  return launch_act<1>(L, M, x, codes, scales, zeros, y, s);
}

}  // namespace gq
