// Small-batch matmul (4 < M <= 32): y = x . W_hat^T on the MFMA units, for
// the decode and short-prefill batches between the dot-product kernel
// (M <= 4) and the tiled prefill GEMM.
//
// "A Survey of Low-bit Large Language Models" review, sections 5.2 and 6.2:
// weight-only quantization dequantizes the weights and multiplies them with
// floating-point activations.  Here nothing is rounded on the way: a code q
// ORed into the mantissa of 128.0 (bf16) or 1024.0 (fp16) is exactly B + q,
// the MFMA forms sum_k x_k (B + q_k) for one quantization group with exact
// products and fp32 accumulation, and the group's scale and zero point are
// applied afterwards in fp32:
//     y += s * (sum_k x_k (B + q_k) - (B + z) * sum_k x_k).
// The group sums of x come from a second MFMA with an all-ones operand.
// bf16 activations are used as they are (no conversion pass).
//
// MFMA v_mfma_f32_16x16x32: A = x (16 rows of M per block), B = codes of 16
// output channels.  Lane l holds channel / row l % 16 and a chunk of 8
// consecutive k for lane group g = l / 16.  Every MFMA stays inside one
// quantization group:
//   INT4 (one group per 128-k step): MFMA i takes chunk 4g + i, so a lane's
//        16 code bytes of the step are one contiguous load;
//   INT2 (two groups per step): MFMAs 0, 1 take chunks 2g + i of the first
//        group and MFMAs 2, 3 chunks 8 + 2g + (i - 2) of the second.  A lane
//        loads 16 bytes covering two steps and a 4 x 4 exchange between the
//        lane groups (gfx950 lane swaps) hands every lane its chunks.
// B fragments hold code pairs in k order, so x is used exactly as stored.
//
// Work split.  A workgroup of 4 waves is CW channel groups (16 channels each,
// one wave) times KW k-ways (CW * KW = 4).  Wide layers use KW = 1 (64
// channels share every staged x tile); narrow ones use KW = 2 or 4, the
// k-ways' partial sums meeting in LDS at the end, so enough workgroups exist
// without a second pass over the output.  Only a linear too narrow for that
// splits K across workgroups, whose fp32 partials the split-K reduction sums
// in split order.  Each wave's k range is walked in phases of PH steps with
// everything double-buffered: while phase p is computed, phase p + 1's x
// tiles land in LDS (buffer loads that write LDS directly, row-major with an
// XOR swizzle so the MFMA operand reads are conflict-free), its codes land in
// registers and its scales and zero points are fetched.  One barrier per
// phase.  Every result is summed in a fixed order: the kernel is
// deterministic.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int SK_WAVES = 4;
constexpr int SK_STEP = 128;                    // k per step
constexpr int SK_SLOTS = 8;                     // steps x k-ways x 16-row blocks per phase
constexpr int SK_XBLK = 256;                    // 16-byte LDS slots per 16-row x block of a step
constexpr uint32_t SK_OOB = 0x80000000u;        // beyond every buffer resource

template <int ACT>
__device__ __forceinline__ floatx4 mfma16(uint4 a, uint4 b, floatx4 c) {
  if constexpr (ACT == 0)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// k chunk (of the 16 in a step) that lane group g feeds to MFMA i
template <int BITS>
__device__ __forceinline__ int sk_chunk(int g, int i) {
  if constexpr (BITS == 4) return 4 * g + i;
  else return i < 2 ? 2 * g + i : 8 + 2 * g + (i - 2);
}

// B fragment from the 8 codes of a chunk, as pairs (B + q_2t, B + q_2t+1).
//   INT4: w holds q_0..q_7 in nibbles 0..7; byte t of w and of w >> 4 carry
//         q_2t and q_2t+1 in their low nibbles.
//   INT2: v (16 bits, zero-extended) holds q_0..q_7 in bit pairs 0..7;
//         u = v | v << 14 carries q_2t at bit 4t and q_2t+1 at bit 16 + 4t.
template <int BITS>
__device__ __forceinline__ uint4 unpack_chunk(uint32_t w, uint32_t bias) {
  uint4 b;
  if constexpr (BITS == 4) {
    const uint32_t hi = w >> 4, m = 0x000f000fu;
    b.x = and_or(__builtin_amdgcn_perm(hi, w, 0x0c040c00u), m, bias);
    b.y = and_or(__builtin_amdgcn_perm(hi, w, 0x0c050c01u), m, bias);
    b.z = and_or(__builtin_amdgcn_perm(hi, w, 0x0c060c02u), m, bias);
    b.w = and_or(__builtin_amdgcn_perm(hi, w, 0x0c070c03u), m, bias);
  } else {
    const uint32_t u = w | (w << 14), m = 0x00030003u;
    b.x = and_or(u, m, bias);
    b.y = and_or(u >> 4, m, bias);
    b.z = and_or(u >> 8, m, bias);
    b.w = and_or(u >> 12, m, bias);
  }
  return b;
}

// Lane-group exchange on gfx950 (the leading s_nop covers the wait states
// the swaps need after a VALU write of their operands):
//   swap32: lanes 32..63 of a  <->  lanes 0..31 of b
//   swap16: odd rows of 16 lanes of a  <->  even rows of b
__device__ __forceinline__ void swap32u(uint32_t &a, uint32_t &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap16u(uint32_t &a, uint32_t &b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// Lane group g holds words 4g .. 4g + 3 of a 16-word block in (v[0..3]);
// afterwards it holds words g, 4 + g, 8 + g, 12 + g.
__device__ __forceinline__ void transpose4(uint32_t (&v)[4]) {
  swap32u(v[0], v[2]);
  swap32u(v[1], v[3]);
  swap16u(v[0], v[1]);
  swap16u(v[2], v[3]);
}

template <int MB, int KW, int BITS>
struct SkGeo {
  static constexpr int CW = SK_WAVES / KW;            // channel groups
  static constexpr int NC = 16 * CW;                  // channels per workgroup
  static constexpr int PH = SK_SLOTS / (KW * MB);     // steps per k-way per phase
  static constexpr int GPS = BITS == 4 ? 1 : 2;       // groups per step
  static constexpr int G = PH * GPS;                  // groups per channel and k-way per phase
  static constexpr int NCL = BITS == 4 ? PH : PH / 2; // 16-byte code loads per lane per phase
  static constexpr int SPT = (64 * G + 255) / 256;    // scale entries per thread per phase
  static_assert(PH >= 2 && NC * KW == 64, "geometry");
};

struct SkArgs {
  int M, K, N;
  int s0, s1;              // the workgroup's steps (its split of K)
  int sw;                  // steps per k-way
  int np;                  // phases (even)
  int n0;                  // first output channel of the workgroup
  int rw0;                 // row of n0 inside its block
  int nvalid;              // channels of the workgroup below N
  int nsplit;
  uint16_t *y;
  float *part;             // [nsplit][M][N] fp32
};

template <int ACT, int MB, int KW, int BITS>
__device__ __forceinline__ void skinny_tile(const SkArgs &a, Rsrc xr, Rsrc cr, Rsrc sr, Rsrc zr,
                                            uint32_t RB, uint32_t GPR, uint4 *xb0, uint4 *xb1,
                                            float2 *sb0, float2 *sb1, float *red) {
  using Gm = SkGeo<MB, KW, BITS>;
  constexpr int CW = Gm::CW, PH = Gm::PH, GPS = Gm::GPS, G = Gm::G, NCL = Gm::NCL;
  constexpr int SPT = Gm::SPT;
  constexpr uint32_t BIAS = ACT == 0 ? 0x43004300u : 0x64006400u;   // 128.0 / 1024.0 pairs
  constexpr uint32_t ONES = ACT == 0 ? 0x3f803f80u : 0x3c003c00u;
  constexpr float BIASF = ACT == 0 ? 128.f : 1024.f;
  constexpr uint32_t STEPB = SK_STEP * BITS / 8;     // code bytes per channel per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave / CW, cg = wave % CW;
  const int g = lane >> 4, r = lane & 15;
  const int cl = 16 * cg + r;                        // the lane's channel in the tile
  const bool ch_ok = cl < a.nvalid;
  auto kbeg = [&](int k) { return a.s0 + k * a.sw; };
  auto kend = [&](int k) { return min(a.s0 + (k + 1) * a.sw, a.s1); };
  const int kb = kbeg(kw), ke = kend(kw);

  // ---- x DMA: per phase 4 * SK_SLOTS loads of 1 KB (4 rows x 128 k);
  // wave w issues loads 8w .. 8w + 7.  Load j fills rows 4(j&3) .. +3 of
  // block b = j/4 = (k-way * PH + step) * MB + mb; lane l takes row
  // rr = 4(j&3) + l/16 of the block and writes slot 16 rr + l%16, which holds
  // chunk (l%16) ^ rr of that row.
  constexpr int XL = 4 * SK_SLOTS / SK_WAVES;        // DMA loads per wave per phase
  uint32_t xrow[XL];                                 // byte offset of the lane's row and chunk
  int xkc[XL];                                       // k of the lane's chunk within a step
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int j = XL * wave + q;
    const int b = j >> 2, mb = b % MB;
    const int rr = 4 * (j & 3) + (lane >> 4);
    const int row = 16 * mb + rr;
    const int c = (lane & 15) ^ rr;
    xkc[q] = 8 * c;
    xrow[q] = row < a.M ? ((uint32_t)row * (uint32_t)a.K + (uint32_t)(8 * c)) * 2u : SK_OOB;
  }
  auto issue_x = [&](int p, uint4 *dst) {
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      const int j = XL * wave + q;
      const int b = j >> 2;
      const int kwb = b / (PH * MB), st = (b / MB) % PH;
      const int gs = kbeg(kwb) + p * PH + st;
      const bool ok = xrow[q] != SK_OOB && gs < kend(kwb) && gs * SK_STEP + xkc[q] < a.K;
      const uint32_t off = ok ? xrow[q] + (uint32_t)gs * (SK_STEP * 2) : SK_OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(dst + b * SK_XBLK + 64 * (j & 3)), 16,
                                               off, 0, 0, 0);
    }
  };

  // ---- codes of the lane's channel and k-way, straight to registers.
  // INT4: one 16-byte load per step (chunks 4g .. 4g + 3); INT2: one per
  // two steps (lane group g gets bytes 16g .. 16g + 15 of the pair's 64).
  const uint32_t crow = ch_ok ? (uint32_t)(a.rw0 + cl) * RB : SK_OOB;
  auto issue_codes = [&](int p, uint32_t (*dst)[4]) {
#pragma unroll
    for (int s = 0; s < NCL; ++s) {
      int gs, lstep;
      if constexpr (BITS == 4) {
        gs = kb + p * PH + s;
        lstep = gs;
      } else {
        gs = kb + p * PH + 2 * s;
        lstep = gs + (g >> 1);
      }
      const uint32_t off = (crow != SK_OOB && lstep < ke) ? crow + (uint32_t)gs * STEPB + 16u * g
                                                          : SK_OOB;
      const uint4 v = ld128(cr, off);
      dst[s][0] = v.x; dst[s][1] = v.y; dst[s][2] = v.z; dst[s][3] = v.w;
    }
  };

  // ---- scales and zero points: entry u = (channel, k-way) pair u / G, group
  // u % G of the phase; staged in LDS as (S, -(B + z)) at [group][pair].
  // Groups past the k-way's range or past K get S = 0.
  uint32_t sv[SPT], zv[SPT];
  bool sok[SPT];
  auto issue_scales = [&](int p) {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int u = tid + 256 * j;
      const int pi = u / G, gi = u % G;
      const int c = pi / KW, k = pi % KW;
      const int gs = kbeg(k) + p * PH + gi / GPS, h = gi % GPS;
      const bool ok = u < 64 * G && c < a.nvalid && gs < kend(k) && gs * SK_STEP + h * 64 < a.K;
      const uint32_t gidx = ok ? (uint32_t)(a.rw0 + c) * GPR + (uint32_t)(gs * GPS + h) : SK_OOB / 4u;
      sok[j] = ok;
      sv[j] = ld16(sr, 2u * gidx);
      zv[j] = ld8(zr, gidx);
    }
  };
  auto store_scales = [&](float2 *dst) {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int u = tid + 256 * j;
      if (u < 64 * G) {
        const int pi = u / G, gi = u % G;
        dst[gi * 64 + pi] = make_float2(sok[j] ? f16_bits_to_f32((uint16_t)sv[j]) : 0.f,
                                        -(BIASF + (float)zv[j]));
      }
    }
  };

  floatx4 yacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) yacc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint4 ones = make_uint4(ONES, ONES, ONES, ONES);
  const int pidx = cl * KW + kw;                     // the lane's (channel, k-way) pair

  auto compute = [&](const uint4 *xb, const float2 *sb, uint32_t (*cw)[4]) {
    if constexpr (BITS == 2) {
#pragma unroll
      for (int s = 0; s < NCL; ++s) transpose4(cw[s]);
    }
#pragma unroll
    for (int st = 0; st < PH; ++st) {
      floatx4 gacc[MB], gsum[MB];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w;
        if constexpr (BITS == 4) {
          w = cw[st][i];
        } else {
          const uint32_t t = cw[st >> 1][2 * (st & 1) + (i >> 1)];
          w = (i & 1) ? (t >> 16) : (t & 0xffffu);
        }
        const uint4 b = unpack_chunk<BITS>(w, BIAS);
        const bool first = BITS == 4 ? i == 0 : (i & 1) == 0;   // first MFMA of a group
        const int slot = 16 * r + (sk_chunk<BITS>(g, i) ^ r);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint4 av = xb[((kw * PH + st) * MB + mb) * SK_XBLK + slot];
          gacc[mb] = mfma16<ACT>(av, b, first ? zero4 : gacc[mb]);
          gsum[mb] = mfma16<ACT>(av, ones, first ? zero4 : gsum[mb]);
        }
        const bool last = BITS == 4 ? i == 3 : (i & 1) == 1;
        if (last) {
          const int h = BITS == 4 ? 0 : (i >> 1);
          const float2 sc = sb[(st * GPS + h) * 64 + pidx];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              yacc[mb][e] = fmaf(sc.x, fmaf(sc.y, gsum[mb][e], gacc[mb][e]), yacc[mb][e]);
          // apply the group here: deferring the corrections would keep every
          // group's MFMA results of the phase live
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(yacc[mb]));
        }
      }
    }
  };

  // ---- phases: compute p while p + 1 is in flight (loads of phases past
  // the k-way's range are out of range: no traffic, zeros)
  uint32_t c0[NCL][4], c1[NCL][4];
  issue_scales(0);
  issue_x(0, xb0);
  issue_codes(0, c0);
  store_scales(sb0);
  lds_barrier();
  for (int p = 0; p < a.np; p += 2) {
    issue_scales(p + 1);
    issue_x(p + 1, xb1);
    issue_codes(p + 1, c1);
    compute(xb0, sb0, c0);
    store_scales(sb1);
    lds_barrier();
    issue_scales(p + 2);
    issue_x(p + 2, xb0);
    issue_codes(p + 2, c0);
    compute(xb1, sb1, c1);
    store_scales(sb0);
    lds_barrier();
  }

  // ---- k-ways meet in LDS, summed in k-way order
  if constexpr (KW > 1) {
    if (kw > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[(((kw - 1) * CW + cg) * MB * 4 + mb * 4 + e) * 64 + lane] = yacc[mb][e];
    }
    lds_barrier();
    if (kw > 0) return;
#pragma unroll
    for (int k = 1; k < KW; ++k)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          yacc[mb][e] += red[(((k - 1) * CW + cg) * MB * 4 + mb * 4 + e) * 64 + lane];
  }

  // ---- results: lane l holds channel cl, rows 16 mb + 4 g + e
  if (!ch_ok) return;
  const int ncol = a.n0 + cl;
  if (a.nsplit == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mb + 4 * g + e;
        if (m < a.M)
          a.y[(int64_t)m * a.N + ncol] = ACT == 0 ? f32_to_bf16_rne(yacc[mb][e])
                                                  : f32_to_f16_bits(yacc[mb][e]);
      }
    return;
  }
  // split K: this split's fp32 partial tile, summed by the split-K reduction
  const int split = (int)blockIdx.y;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * mb + 4 * g + e;
      if (m < a.M) a.part[((int64_t)split * a.M + m) * a.N + ncol] = yacc[mb][e];
    }
}

// BITSEL: 4 or 2 for a uniform (Layer-mix) linear, 0 for Channel-mix blocks
// of either width (the channels of a workgroup lie in one block).
template <int ACT, int MB, int KW, int BITSEL>
__global__ __launch_bounds__(64 * SK_WAVES) void skinny_kernel(
    LayoutDev L, int M, const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ y, float *__restrict__ part, int sps, int sw, int np) {
  // double-buffered x tiles and (scale, zero) tables; separate arrays so the
  // wait before reading one buffer does not cover the loads into the other
  constexpr int GMAX = SK_SLOTS / (KW * MB) * (BITSEL == 4 ? 1 : 2);
  __shared__ __attribute__((aligned(16))) uint4 xb0[SK_SLOTS * SK_XBLK];
  __shared__ __attribute__((aligned(16))) uint4 xb1[SK_SLOTS * SK_XBLK];
  __shared__ __attribute__((aligned(16))) float2 sb0[64 * GMAX];
  __shared__ __attribute__((aligned(16))) float2 sb1[64 * GMAX];
  __shared__ __attribute__((aligned(16))) float red[KW > 1 ? 3 * 64 * 4 * MB : 1];
  // the x tiles start zeroed: every slot a load does not fill stays finite
  for (int i = (int)threadIdx.x; i < SK_SLOTS * SK_XBLK; i += 64 * SK_WAVES) {
    xb0[i] = make_uint4(0u, 0u, 0u, 0u);
    xb1[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  lds_barrier();
  constexpr int NC = 16 * (SK_WAVES / KW);
  const int nsteps = (L.K + SK_STEP - 1) / SK_STEP;
  SkArgs a;
  a.M = M; a.K = L.K; a.N = L.N;
  a.s0 = (int)blockIdx.y * sps;
  a.s1 = min(a.s0 + sps, nsteps);
  a.sw = sw; a.np = np;
  a.nsplit = (int)gridDim.y;
  const int n0 = (int)blockIdx.x * NC;
  a.n0 = n0;
  a.nvalid = L.N - n0 < NC ? L.N - n0 : NC;
  a.y = y; a.part = part;
  const int blk = n0 / L.block_n;
  a.rw0 = n0 - blk * L.block_n;
  BlockInfo bi;
  if constexpr (BITSEL == 0) {
    bi = block_info(L, blk);
  } else {
    bi.bits = BITSEL; bi.code_off = 0; bi.grp_off = 0;
  }
  const int bits = BITSEL ? BITSEL : __builtin_amdgcn_readfirstlane(bi.bits);
  const uint32_t RB = (uint32_t)(L.K * bits / 8);
  const uint32_t GPR = (uint32_t)(bits == 4 ? L.K / 128 : L.K / 64);
  const Rsrc xr = make_rsrc(x, (uint32_t)M * (uint32_t)L.K * 2u);
  const Rsrc cr = make_rsrc(codes + bi.code_off, (uint32_t)L.block_n * RB);
  const Rsrc sr = make_rsrc(scales + bi.grp_off, (uint32_t)L.block_n * GPR * 2u);
  const Rsrc zr = make_rsrc(zeros + bi.grp_off, (uint32_t)L.block_n * GPR);
  if (BITSEL != 2 && bits == 4)
    skinny_tile<ACT, MB, KW, 4>(a, xr, cr, sr, zr, RB, GPR, xb0, xb1, sb0, sb1, red);
  else if constexpr (BITSEL != 4)
    skinny_tile<ACT, MB, KW, 2>(a, xr, cr, sr, zr, RB, GPR, xb0, xb1, sb0, sb1, red);
}

struct SkPlan {
  int mb, kw, tiles, nsplit, sps, sw, np;
  size_t part_bytes;
};

// Launch shape.  16-row blocks: 1 for M <= 16, else 2.  k-ways: the fewest
// that give at least kSkFill workgroups (more k-ways stage more x per code
// byte), at most 4 / blocks (a phase holds at least two steps).  K is split
// across workgroups only while fewer than kSkMinTiles would exist.  Workspace:
// fp32 partials [nsplit][M][N] when K is split.
constexpr int kSkFill = 224;
constexpr int kSkMinTiles = 48;

inline SkPlan skinny_plan(const LayoutDev &L, int M) {
  SkPlan p;
  p.mb = M <= 16 ? 1 : 2;
  const int kwmax = 4 / p.mb;
  p.kw = kwmax;
  for (int kw = 1; kw <= kwmax; kw *= 2) {
    if ((L.N + 64 / kw - 1) / (64 / kw) >= kSkFill) {
      p.kw = kw;
      break;
    }
  }
  p.tiles = (L.N + 64 / p.kw - 1) / (64 / p.kw);
  const int ph = SK_SLOTS / (p.kw * p.mb);
  const int nsteps = (L.K + SK_STEP - 1) / SK_STEP;
  p.nsplit = 1;
  while (p.tiles * p.nsplit < kSkMinTiles && nsteps >= 2 * p.nsplit * p.kw * ph) p.nsplit *= 2;
  p.sps = (nsteps + p.nsplit - 1) / p.nsplit;
  p.nsplit = (nsteps + p.sps - 1) / p.sps;
  p.sw = (p.sps + p.kw - 1) / p.kw;
  p.np = (p.sw + ph - 1) / ph;
  p.np += p.np & 1;
  p.part_bytes = p.nsplit > 1 ? ((size_t)p.nsplit * (size_t)M * (size_t)L.N * 4u + 255u) & ~(size_t)255u
                              : 0u;
  return p;
}

template <int ACT, int MB, int KW>
hipError_t launch_kw(const LayoutDev &L, int M, const SkPlan &p, const void *x,
                     const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros, void *y,
                     void *workspace, hipStream_t s) {
  float *part = reinterpret_cast<float *>(workspace);
  uint16_t *yp = reinterpret_cast<uint16_t *>(y);
  uint32_t any4 = 0, all4 = ~0u;
  for (int i = 0; i < L.nblocks; ++i) {
    const uint32_t b = (L.int4_mask[i >> 5] >> (i & 31)) & 1u;
    any4 |= b;
    all4 &= b;
  }
  const dim3 grid(p.tiles, p.nsplit), block(64 * SK_WAVES);
  const uint16_t *xp = reinterpret_cast<const uint16_t *>(x);
  const uint8_t *cp = reinterpret_cast<const uint8_t *>(codes);
  if (all4)
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, KW, 4>), grid, block, 0, s, L, M, xp, cp, scales, zeros,
                       yp, part, p.sps, p.sw, p.np);
  else if (!any4)
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, KW, 2>), grid, block, 0, s, L, M, xp, cp, scales, zeros,
                       yp, part, p.sps, p.sw, p.np);
  else
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, KW, 0>), grid, block, 0, s, L, M, xp, cp, scales, zeros,
                       yp, part, p.sps, p.sw, p.np);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  return launch_splitk_reduce(part, p.nsplit, M, L.N, nullptr, yp, ACT, s);
}

template <int ACT>
hipError_t launch_act(const LayoutDev &L, int M, const void *x, const uint32_t *codes,
                      const uint16_t *scales, const uint8_t *zeros, void *y, void *workspace,
                      hipStream_t s) {
  const SkPlan p = skinny_plan(L, M);
  if (p.mb == 1) {
    if (p.kw == 1) return launch_kw<ACT, 1, 1>(L, M, p, x, codes, scales, zeros, y, workspace, s);
    if (p.kw == 2) return launch_kw<ACT, 1, 2>(L, M, p, x, codes, scales, zeros, y, workspace, s);
    return launch_kw<ACT, 1, 4>(L, M, p, x, codes, scales, zeros, y, workspace, s);
  }
  if (p.kw == 1) return launch_kw<ACT, 2, 1>(L, M, p, x, codes, scales, zeros, y, workspace, s);
  return launch_kw<ACT, 2, 2>(L, M, p, x, codes, scales, zeros, y, workspace, s);
}

}  // namespace

bool skinny_supported(const LayoutDev &L, int M) {
  return M > kGemvMaxM && M <= kSkinnyMaxM && (uint64_t)M * (uint64_t)L.K * 2u < (1ull << 31) &&
         (uint64_t)L.block_n * (uint64_t)L.K / 2u < (1ull << 31);
}

size_t skinny_workspace_bytes(const LayoutDev &L, int M) { return skinny_plan(L, M).part_bytes; }

hipError_t launch_skinny(const LayoutDev &L, int M, gq_dtype act, const void *x,
                         const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                         void *y, void *workspace, hipStream_t s) {
  if (act == GQ_BF16) return launch_act<0>(L, M, x, codes, scales, zeros, y, workspace, s);
  return launch_act<1>(L, M, x, codes, scales, zeros, y, workspace, s);
}

}  // namespace gq
