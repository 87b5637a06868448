// Small-batch matmul (4 < M <= 32): y = x . W_hat^T on the MFMA units, for
// the decode and short-prefill batches between the dot-product kernel
// (M <= 4) and the tiled prefill GEMM.
//
// "A Survey of Low-bit Large Language Models" review, sections 5.2 and 6.2:
// weight-only quantization dequantizes the weights and multiplies them with
// floating-point activations.  Here nothing is rounded on the way: a code q
// ORed into the mantissa of 128.0 (bf16) or 1024.0 (fp16) is exactly B + q,
// and -(B + z) is exact too, so for one quantization group the MFMAs form
//     sum_k x_k (B + q_k) + sum_k x_k * -(B + z) = sum_k x_k (q_k - z)
// with exact products and fp32 accumulation; the group's scale is applied
// afterwards in fp32.  bf16 activations are used as they are.
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
// Work split.  A workgroup of 8 waves (two per SIMD) is CW channel groups
// (16 channels each, one wave) times KW k-ways (CW * KW = 8); the k-ways'
// partial sums meet in LDS at the end.  The launch shape (k-ways, steps per
// k-way, K splits) comes from a time model of the layer.  x reaches LDS by
// buffer loads that write LDS directly (row-major, XOR-swizzled so the MFMA
// operand reads are conflict-free; lanes past M, K or the range read zeros),
// in chunks of 4 steps held in a ring of two buffers, one barrier per chunk:
// the first steps compute while later chunks are still on their way.  The
// scales and zero points come as 16-byte runs into LDS before the first
// barrier.  Each wave streams its codes straight to registers in step order,
// starting with a short window (a long burst from every wave of the chip
// queues the x and scale loads the first barrier waits for behind it) that
// grows by two loads a step, so codes return in step order and the
// multiplications overlap the transfer.  A layer whose k range does not fit
// one workgroup splits K across workgroups; their fp32 partials are summed
// in split order by the split-K reduction.  Every result is summed in a
// fixed order: the kernel is deterministic.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int SK_WAVES = 8;                     // two per SIMD
constexpr int SK_THREADS = 64 * SK_WAVES;
constexpr int SK_PAIRS = 16 * SK_WAVES;         // (channel, k-way) pairs per workgroup
constexpr int SK_STEP = 128;                    // k per step
constexpr int SK_XCAP = 32;                     // x blocks (step x k-way x 16 rows) in LDS
constexpr int SK_SWMAX = 16;                    // steps per wave (code registers)
constexpr int SK_XSC = 4;                       // steps per x chunk
constexpr int SK_CWIN = 12;                     // code loads in flight per lane
constexpr int SK_CW0 = 2;                       // code loads issued before the first barrier
constexpr int SK_CW1 = 4;                       // ... and right after it
constexpr int SK_CRAMP = 2;                     // code loads per step until the window is full
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

// Lane group g holds words 4g .. 4g + 3 of a 16-word block in (v[0..3]);
// afterwards it holds words g, 4 + g, 8 + g, 12 + g.
// (gfx950 lane swaps: swap32 exchanges lane groups 0, 1 of one register
// with 2, 3 of the other, swap16 groups 1, 3 with 0, 2.)
__device__ __forceinline__ void transpose4(uint32_t (&v)[4]) {
  swap32(v[0], v[2]);
  swap32(v[1], v[3]);
  swap16(v[0], v[1]);
  swap16(v[2], v[3]);
}

template <int MB, int KW, int SWC, int BITS>
struct SkGeo {
  static constexpr int CW = SK_WAVES / KW;            // channel groups
  static constexpr int NC = 16 * CW;                  // channels per workgroup
  static constexpr int SC = SWC < SK_XSC ? SWC : SK_XSC;   // steps per x chunk
  static constexpr int XCH = SWC / SC;                // x chunks
  static constexpr int NXB = XCH > 1 ? 2 : 1;         // chunk buffers in LDS (a ring)
  static constexpr int XS = KW * SC * MB * SK_XBLK;   // 16-byte slots per chunk buffer
  static constexpr int GPS = BITS == 4 ? 1 : 2;       // groups per step
  static constexpr int R = SWC * GPS;                 // groups per (channel, k-way)
  static constexpr int PS = (2 * R + 14 + 15) / 16;   // 16-byte scale pieces per (channel, k-way)
  static constexpr int PZ = (R + 15 + 15) / 16;       // 16-byte zero pieces
  static constexpr int NCL = BITS == 4 ? SWC : SWC / 2;   // 16-byte code loads per lane
  static_assert(NC * KW == SK_PAIRS && NXB * KW * SC * MB <= SK_XCAP && SWC <= SK_SWMAX &&
                    SWC % 4 == 0 && SWC % SC == 0 && (KW * SC) % 2 == 0,
                "geometry");
};

struct SkArgs {
  int M, K, N;
  int s0, s1;              // the workgroup's steps (its split of K)
  int sw;                  // steps per k-way
  int n0;                  // first output channel of the workgroup
  int rw0;                 // row of n0 inside its block
  int nvalid;              // channels of the workgroup below N
  int nsplit;
  uint32_t g_blk;          // index of the block's first scale / zero
  uint16_t *y;
  float *part;             // [nsplit][M][N] fp32
};

template <int ACT, int MB, int KW, int SWC, int BITS>
__device__ __forceinline__ void skinny_tile(const SkArgs &a, Rsrc xr, Rsrc cr, Rsrc sr, Rsrc zr,
                                            uint32_t RB, uint32_t GPR, uint4 *xb0, uint4 *xb1, uint4 *ss,
                                            uint4 *zz) {
  using Gm = SkGeo<MB, KW, SWC, BITS>;
  constexpr int CW = Gm::CW, GPS = Gm::GPS, NCL = Gm::NCL, PS = Gm::PS, PZ = Gm::PZ;
  constexpr int SC = Gm::SC, XCH = Gm::XCH;
  constexpr uint32_t BIAS = ACT == 0 ? 0x43004300u : 0x64006400u;   // 128.0 / 1024.0 pairs
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

  // ---- x, in chunks of SC steps held in a ring of two LDS buffers: chunk c
  // sits in buffer c % 2, its block (k-way * SC + sl) * MB + mb holding 16
  // rows x 128 k of step c * SC + sl.  Wave w loads rows 4q .. 4q + 3
  // (q = w % 4) of every other block (1 KB per load); lane l takes row
  // rr = 4q + l/16 and fills slot 16 rr + l%16 with chunk (l%16) ^ rr of that
  // row.  Rows past M are not loaded (their MFMA output rows are discarded).
  // Chunk c + 1 is requested once every wave has passed the barrier that
  // ends chunk c - 1, the last reader of its buffer.
  auto xbuf = [&](int c) { return (c & 1) ? xb1 : xb0; };
  auto x_dma = [&](int c) {
    constexpr int BS = SK_WAVES / 4;                  // waves per row quarter
    const int qq = wave & 3, bset = wave >> 2;
    const int rr = 4 * qq + (lane >> 4);
    const int cc = (lane & 15) ^ rr;
    uint4 *dst = xbuf(c);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = 16 * mb + rr;
      if (16 * mb + 4 * qq < a.M) {                   // uniform
        const uint32_t rowoff = row < a.M ? ((uint32_t)row * (uint32_t)a.K + (uint32_t)(8 * cc)) * 2u
                                          : SK_OOB;
#pragma unroll
        for (int tt = 0; tt < KW * SC / BS; ++tt) {
          const int t = tt * BS + bset;
          const int kwb = t / SC, sl = t % SC;
          const int gs = kbeg(kwb) + c * SC + sl;
          const bool ok = rowoff != SK_OOB && gs < kend(kwb) && gs * SK_STEP + 8 * cc < a.K;
          const uint32_t off = ok ? rowoff + (uint32_t)gs * (SK_STEP * 2) : SK_OOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xr, (lds_void *)(dst + (t * MB + mb) * SK_XBLK + 64 * qq), 16, off, 0, 0, 0);
        }
      }
    }
  };
  x_dma(0);

  // ---- scales and zero points: for each (channel, k-way) pair the runs of
  // its groups, read as 16-byte pieces from the 16-byte boundary at or below
  // the run's start (the arrays start 16-byte aligned)
  constexpr int SPS = (SK_PAIRS * PS + SK_THREADS - 1) / SK_THREADS;
  constexpr int SPZ = (SK_PAIRS * PZ + SK_THREADS - 1) / SK_THREADS;
  uint4 spv[SPS], zpv[SPZ];
  auto run_start = [&](int pair) {
    return a.g_blk + (uint32_t)(a.rw0 + pair / KW) * GPR + (uint32_t)(kbeg(pair % KW) * GPS);
  };
#pragma unroll
  for (int j = 0; j < SPS; ++j) {
    const int u = tid + SK_THREADS * j, pair = u / PS, piece = u % PS;
    const bool ok = u < SK_PAIRS * PS && pair / KW < a.nvalid;
    spv[j] = ld128_nt(sr, ok ? ((2u * run_start(pair)) & ~15u) + 16u * piece : SK_OOB);
  }
#pragma unroll
  for (int j = 0; j < SPZ; ++j) {
    const int u = tid + SK_THREADS * j, pair = u / PZ, piece = u % PZ;
    const bool ok = u < SK_PAIRS * PZ && pair / KW < a.nvalid;
    zpv[j] = ld128_nt(zr, ok ? (run_start(pair) & ~15u) + 16u * piece : SK_OOB);
  }

  // ---- codes of the lane's channel and k-way, straight to registers.
  // INT4: one 16-byte load per step (chunks 4g .. 4g + 3); INT2: one per
  // two steps (lane group g gets bytes 16g .. 16g + 15 of the pair's 64).
  // Code loads are issued in step order, so they return in step order and
  // each step computes as soon as its codes are in.  Only CW0 are requested
  // before the first barrier: a larger burst from every wave of the chip
  // would queue the x and scale loads the barrier waits for behind it.
  // From there the window grows by CRAMP loads per step up to CWIN.
  constexpr int CWIN = NCL < SK_CWIN ? NCL : SK_CWIN;
  constexpr int CW0 = NCL < SK_CW0 ? NCL : SK_CW0;
  constexpr int CW1 = NCL < SK_CW1 ? NCL : SK_CW1;
  // code loads issued before step st computes
  auto ctarget = [&](int st) {
    int t = CW1 + SK_CRAMP * st;
    const int u = (BITS == 4 ? st : st / 2) + CWIN;
    t = t < u ? t : u;
    return t < NCL ? t : NCL;
  };
  uint32_t cw[NCL][4];
  const uint32_t crow = ch_ok ? (uint32_t)(a.rw0 + cl) * RB : SK_OOB;
  auto load_codes = [&](int s) {
    const int gs = BITS == 4 ? kb + s : kb + 2 * s;
    const int lstep = BITS == 4 ? gs : gs + (g >> 1);
    const uint32_t off = (crow != SK_OOB && lstep < ke) ? crow + (uint32_t)gs * STEPB + 16u * g
                                                        : SK_OOB;
    const uint4 v = ld128_nt(cr, off);
    cw[s][0] = v.x; cw[s][1] = v.y; cw[s][2] = v.z; cw[s][3] = v.w;
  };
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < CW0; ++s) load_codes(s);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int j = 0; j < SPS; ++j)
    if (tid + SK_THREADS * j < SK_PAIRS * PS) ss[tid + SK_THREADS * j] = spv[j];
#pragma unroll
  for (int j = 0; j < SPZ; ++j)
    if (tid + SK_THREADS * j < SK_PAIRS * PZ) zz[tid + SK_THREADS * j] = zpv[j];
  lds_barrier();
  if constexpr (XCH > 1) x_dma(1);
#pragma unroll
  for (int s = CW0; s < CW1; ++s) load_codes(s);

  floatx4 yacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) yacc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // the lane's scale and zero runs in LDS
  const int pidx = cl * KW + kw;
  const uint32_t g0 = a.g_blk + (uint32_t)(a.rw0 + cl) * GPR + (uint32_t)(kb * GPS);
  const uint16_t *srun = reinterpret_cast<const uint16_t *>(
      reinterpret_cast<const uint8_t *>(ss + pidx * PS) + ((2u * g0) & 15u));
  const uint8_t *zrun = reinterpret_cast<const uint8_t *>(zz + pidx * PZ) + (g0 & 15u);

  // Per group the MFMAs accumulate sum x (B + q) and, against a constant
  // operand -(B + z) (exact in bf16 / fp16 for z <= 15), sum x * -(B + z)
  // into the same registers: the result is sum x (q - z), scaled by s in
  // fp32 afterwards.  Software-pipelined over steps: while step st is
  // multiplied, the A fragments, scales and zero points of step st + 1 are
  // read from LDS, the codes of a later step are requested, and the scaling
  // of step st - 1 is applied (its MFMA results are complete by then).
  // Steps past the k-way's range add zeros.
  constexpr uint32_t NEGB = ACT == 0 ? 0xc300c300u : 0xe400e400u;   // -(B + 0) pairs
  uint4 av[2][4][MB];
  float sc[3][GPS];
  uint32_t zp[2][GPS];
  // partial accumulators per (group, row block): with one row block the
  // chunks alternate between two, so no MFMA waits for the one just issued
  constexpr int NP = MB == 1 ? 2 : 1;
  floatx4 gacc[2][GPS][MB][NP];
  auto read_step = [&](int st, uint4 (&A)[4][MB], float (&S)[GPS], uint32_t (&Z)[GPS]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 16 * r + (sk_chunk<BITS>(g, i) ^ r);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        A[i][mb] = xbuf(st / SC)[((kw * SC + st % SC) * MB + mb) * SK_XBLK + slot];
    }
#pragma unroll
    for (int h = 0; h < GPS; ++h) {
      const int gs = kb + st;
      // groups past the k-way's range or past K, and channels past N, get
      // scale 0 (their x or codes read as zeros)
      const bool ok = ch_ok && gs < ke && gs * SK_STEP + h * 64 < a.K;
      const float sraw = f16_bits_to_f32(srun[st * GPS + h]);
      S[h] = ok ? sraw : 0.f;
      const uint32_t z = zrun[st * GPS + h];
      Z[h] = NEGB | z | (z << 16);
    }
  };
  auto scale_step = [&](const floatx4 (&ga)[GPS][MB][NP], const float (&S)[GPS]) {
#pragma unroll
    for (int h = 0; h < GPS; ++h)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) yacc[mb][e] = fmaf(S[h], ga[h][mb][p][e], yacc[mb][e]);
    // keep the scaling here: otherwise it is all moved after the last step
    // and every step's MFMA results stay live
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(yacc[mb]));
  };
  read_step(0, av[0], sc[0], zp[0]);
#pragma unroll
  for (int st = 0; st < SWC; ++st) {
    const int cur = st & 1;
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < SWC && (st + 1) % SC == 0) {
      // the next x chunk is in (every wave's DMA of it is complete), and the
      // buffer of the one just finished is free for the chunk after
      lds_barrier();
      if ((st + 1) / SC + 1 < XCH) x_dma((st + 1) / SC + 1);
    }
    if (st + 1 < SWC) read_step(st + 1, av[cur ^ 1], sc[(st + 1) % 3], zp[cur ^ 1]);
#pragma unroll
    for (int s = ctarget(st); s < ctarget(st + 1); ++s) load_codes(s);
    if constexpr (BITS == 2) {
      if ((st & 1) == 0) transpose4(cw[st >> 1]);
    }
    uint4 bq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w;
      if constexpr (BITS == 4) {
        w = cw[st][i];
      } else {
        const uint32_t t = cw[st >> 1][2 * (st & 1) + (i >> 1)];
        w = (i & 1) ? (t >> 16) : (t & 0xffffu);
      }
      bq[i] = unpack_chunk<BITS>(w, BIAS);
    }
    // chunks in pairs: the data MFMAs of both, then their zero-point MFMAs,
    // so every MFMA's accumulator was last written two MFMAs earlier
#pragma unroll
    for (int ip = 0; ip < 4; ip += 2) {
#pragma unroll
      for (int i = ip; i < ip + 2; ++i) {
        const int h = BITS == 4 ? 0 : (i >> 1);
        const int p = NP == 2 ? (i & 1) : 0;
        const bool first = (BITS == 4 ? i : (i & 1)) < NP;   // first MFMA of its accumulator
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          gacc[cur][h][mb][p] = mfma16<ACT>(av[cur][i][mb], bq[i], first ? zero4 : gacc[cur][h][mb][p]);
      }
#pragma unroll
      for (int i = ip; i < ip + 2; ++i) {
        const int h = BITS == 4 ? 0 : (i >> 1);
        const int p = NP == 2 ? (i & 1) : 0;
        const uint4 zb = make_uint4(zp[cur][h], zp[cur][h], zp[cur][h], zp[cur][h]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          gacc[cur][h][mb][p] = mfma16<ACT>(av[cur][i][mb], zb, gacc[cur][h][mb][p]);
      }
    }
    if (st > 0) scale_step(gacc[cur ^ 1], sc[(st - 1) % 3]);
  }
  __builtin_amdgcn_sched_barrier(0);
  scale_step(gacc[(SWC - 1) & 1], sc[(SWC - 1) % 3]);

  // ---- k-ways meet in LDS (the x tiles' space, free once every wave is
  // done with it), summed in k-way order
  if constexpr (KW > 1) {
    float *red = reinterpret_cast<float *>(xb0);
    lds_barrier();
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
template <int ACT, int MB, int KW, int SWC, int BITSEL>
__global__ __launch_bounds__(SK_THREADS) void skinny_kernel(
    LayoutDev L, int M, const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ y, float *__restrict__ part, int sps, int sw) {
  using G2 = SkGeo<MB, KW, SWC, BITSEL == 4 ? 4 : 2>;   // the larger scale runs
  __shared__ __attribute__((aligned(16))) uint4 xb0[G2::XS];
  __shared__ __attribute__((aligned(16))) uint4 xb1[G2::NXB > 1 ? G2::XS : 1];
  __shared__ __attribute__((aligned(16))) uint4 ss[SK_PAIRS * G2::PS];
  __shared__ __attribute__((aligned(16))) uint4 zz[SK_PAIRS * G2::PZ];
  static_assert((KW - 1) * (SK_WAVES / KW) * MB * 4 * 64 <= G2::XS * 4, "reduction space");
  constexpr int NC = 16 * (SK_WAVES / KW);
  const int nsteps = (L.K + SK_STEP - 1) / SK_STEP;
  SkArgs a;
  a.M = M; a.K = L.K; a.N = L.N;
  a.s0 = (int)blockIdx.y * sps;
  a.s1 = min(a.s0 + sps, nsteps);
  a.sw = sw;
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
  a.g_blk = (uint32_t)bi.grp_off;
  const uint32_t gend = a.g_blk + (uint32_t)L.block_n * GPR;   // past the block's groups
  const Rsrc xr = make_rsrc(x, (uint32_t)M * (uint32_t)L.K * 2u);
  const Rsrc cr = make_rsrc(codes + bi.code_off, (uint32_t)L.block_n * RB);
  const Rsrc sr = make_rsrc(scales, 2u * gend);
  const Rsrc zr = make_rsrc(zeros, gend);
  if (BITSEL != 2 && bits == 4)
    skinny_tile<ACT, MB, KW, SWC, 4>(a, xr, cr, sr, zr, RB, GPR, xb0, xb1, ss, zz);
  else if constexpr (BITSEL != 4)
    skinny_tile<ACT, MB, KW, SWC, 2>(a, xr, cr, sr, zr, RB, GPR, xb0, xb1, ss, zz);
}

struct SkPlan {
  int mb, kw, swc, tiles, nsplit, sps, sw;
  size_t part_bytes;
};

// Launch shape, from a rough time model in units of one step of one wave:
// the busiest CU works through ceil(workgroups / CUs) k ranges of sw steps,
// each round of resident workgroups adds a latency of about 8, and
// splitting K adds about 16 for the second pass.  16-row blocks: 1 for
// M <= 16, else 2.  Capacity: x for KW * steps * blocks <= 32 block-steps
// in LDS, at most 32 steps per wave.  Workspace: fp32 partials
// [nsplit][M][N] when K is split.
constexpr int kCUs = 256;

// x blocks resident in LDS: one chunk buffer, or a ring of two
__host__ __device__ constexpr int skinny_x_blocks(int mb, int kw, int swc) {
  return (swc > SK_XSC ? 2 : 1) * kw * (swc < SK_XSC ? swc : SK_XSC) * mb;
}

inline size_t skinny_lds_bytes(int mb, int kw, int swc) {
  const int r = swc * 2;                              // sized for INT2 runs
  return (size_t)skinny_x_blocks(mb, kw, swc) * SK_XBLK * 16 +
         (size_t)SK_PAIRS * 16 * ((2 * r + 29) / 16 + (r + 30) / 16);
}

// Launch shape from a time model (us), fitted on MI355X to per-wave
// timestamps of this kernel and to forced launch shapes on the Llama-3-8B
// layers: a workgroup step takes ~0.27 us with one 16-row block and ~0.65 us
// with two; the weights, and at half weight the x tiles every workgroup
// reads from L2 (M x its K range), stream at ~5 TB/s over the CUs that have
// work; a round of workgroups past the first costs ~3 us, a K split the
// reduction launch (~2 us) and ~0.5 us per split.
inline SkPlan skinny_plan(const LayoutDev &L, int M) {
  SkPlan best{};
  double best_cost = 1e30;
  const int mb = M <= 16 ? 1 : 2;
  const int nsteps = (L.K + SK_STEP - 1) / SK_STEP;
  double wbytes = 0.0;                                // packed codes, scales and zeros
  for (int i = 0; i < L.nblocks; ++i) {
    const bool b4 = (L.int4_mask[i >> 5] >> (i & 31)) & 1u;
    wbytes += (double)L.block_n * L.K * (b4 ? 0.5 + 3.0 / 128 : 0.25 + 3.0 / 64);
  }
  for (int kw = 2; kw <= 8 / mb; kw *= 2) {
    const int nc = 16 * (SK_WAVES / kw);
    const int tiles = (L.N + nc - 1) / nc;
    int cap = 0;                                       // most steps per k-way
    for (int c = 4; c <= SK_SWMAX; c *= 2)
      if (skinny_x_blocks(mb, kw, c) <= SK_XCAP) cap = c;
    if (cap < 4) continue;
    for (int ns = 1; ns <= nsteps; ++ns) {
      const int sps = (nsteps + ns - 1) / ns;
      const int nsplit = (nsteps + sps - 1) / sps;
      if (nsplit != ns) continue;
      const int sw = (sps + kw - 1) / kw;
      if (sw > cap) continue;
      const int swc = sw <= 4 ? 4 : sw <= 8 ? 8 : 16;
      const int per_cu = max(1, min(2, (int)((160u * 1024u) / skinny_lds_bytes(mb, kw, swc))));
      const int wgs = tiles * nsplit;
      const int rounds = (wgs + kCUs * per_cu - 1) / (kCUs * per_cu);
      const double xbytes = (double)tiles * M * L.K * 2.0;
      const double t_bw = (wbytes + 0.5 * xbytes) / (5.0e6 * (wgs < kCUs ? wgs : kCUs) / kCUs);
      const double t_comp = (double)((wgs + kCUs - 1) / kCUs) * sw * (mb == 1 ? 0.27 : 0.65);
      const double t_split = nsplit > 1 ? 2.0 + 0.5 * nsplit : 0.0;
      const double cost = (t_bw > t_comp ? t_bw : t_comp) + 3.0 * (rounds - 1) + t_split;
      if (cost < best_cost) {
        best_cost = cost;
        best.mb = mb; best.kw = kw; best.swc = swc; best.tiles = tiles;
        best.nsplit = nsplit; best.sps = sps; best.sw = sw;
      }
      if (wgs >= kCUs) break;                         // more splits only add cost
    }
  }
  best.part_bytes = best.nsplit > 1
                        ? ((size_t)best.nsplit * (size_t)M * (size_t)L.N * 4u + 255u) & ~(size_t)255u
                        : 0u;
  return best;
}

template <int ACT, int MB, int KW, int SWC>
hipError_t launch_cfg(const LayoutDev &L, int M, const SkPlan &p, const void *x,
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
  const dim3 grid(p.tiles, p.nsplit), block(SK_THREADS);
  const uint16_t *xp = reinterpret_cast<const uint16_t *>(x);
  const uint8_t *cp = reinterpret_cast<const uint8_t *>(codes);
  if (all4)
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, KW, SWC, 4>), grid, block, 0, s, L, M, xp, cp, scales,
                       zeros, yp, part, p.sps, p.sw);
  else if (!any4)
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, KW, SWC, 2>), grid, block, 0, s, L, M, xp, cp, scales,
                       zeros, yp, part, p.sps, p.sw);
  else
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, KW, SWC, 0>), grid, block, 0, s, L, M, xp, cp, scales,
                       zeros, yp, part, p.sps, p.sw);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  return launch_splitk_reduce(part, p.nsplit, M, L.N, nullptr, yp, ACT, s);
}

template <int ACT, int MB, int KW>
hipError_t launch_kw(const LayoutDev &L, int M, const SkPlan &p, const void *x,
                     const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros, void *y,
                     void *workspace, hipStream_t s) {
  constexpr bool ok8 = skinny_x_blocks(MB, KW, 8) <= SK_XCAP;
  constexpr bool ok16 = skinny_x_blocks(MB, KW, 16) <= SK_XCAP;
  if (p.swc == 4)
    return launch_cfg<ACT, MB, KW, 4>(L, M, p, x, codes, scales, zeros, y, workspace, s);
  if constexpr (ok8) {
    if (p.swc == 8)
      return launch_cfg<ACT, MB, KW, 8>(L, M, p, x, codes, scales, zeros, y, workspace, s);
  }
  if constexpr (ok16) {
    if (p.swc == 16)
      return launch_cfg<ACT, MB, KW, 16>(L, M, p, x, codes, scales, zeros, y, workspace, s);
  }
  return hipErrorInvalidValue;
}

template <int ACT>
hipError_t launch_act(const LayoutDev &L, int M, const void *x, const uint32_t *codes,
                      const uint16_t *scales, const uint8_t *zeros, void *y, void *workspace,
                      hipStream_t s) {
  const SkPlan p = skinny_plan(L, M);
  if (p.mb == 1) {
    if (p.kw == 2) return launch_kw<ACT, 1, 2>(L, M, p, x, codes, scales, zeros, y, workspace, s);
    if (p.kw == 4) return launch_kw<ACT, 1, 4>(L, M, p, x, codes, scales, zeros, y, workspace, s);
    return launch_kw<ACT, 1, 8>(L, M, p, x, codes, scales, zeros, y, workspace, s);
  }
  if (p.kw == 2) return launch_kw<ACT, 2, 2>(L, M, p, x, codes, scales, zeros, y, workspace, s);
  return launch_kw<ACT, 2, 4>(L, M, p, x, codes, scales, zeros, y, workspace, s);
}

}  // namespace

bool skinny_supported(const LayoutDev &L, int M) {
  if (M <= kGemvMaxM || M > kSkinnyMaxM) return false;
  if ((uint64_t)M * (uint64_t)L.K * 2u >= (1ull << 31)) return false;
  if ((uint64_t)L.block_n * (uint64_t)L.K / 2u >= (1ull << 31)) return false;
  // scale byte offsets of the whole layer stay below 2^31
  uint64_t groups = 0;
  for (int i = 0; i < L.nblocks; ++i)
    groups += (uint64_t)L.block_n * (uint64_t)(((L.int4_mask[i >> 5] >> (i & 31)) & 1u) ? L.K / 128 : L.K / 64);
  return 2u * groups < (1ull << 31);
}

size_t skinny_workspace_bytes(const LayoutDev &L, int M) { return skinny_plan(L, M).part_bytes; }

hipError_t launch_skinny(const LayoutDev &L, int M, gq_dtype act, const void *x,
                         const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                         void *y, void *workspace, hipStream_t s) {
  if (act == GQ_BF16) return launch_act<0>(L, M, x, codes, scales, zeros, y, workspace, s);
  return launch_act<1>(L, M, x, codes, scales, zeros, y, workspace, s);
}

}  // namespace gq
