// Data gradient through the packed weights: dX = dY . W_hat, the product the
// backward pass needs for y = x . W_hat^T, i.e.
//     dX[m][k] = sum_n dY[m][n] * W_hat[n][k],   W_hat = (q - z) * s.
// GreenBitAI's full-parameter fine-tuning of the low-bit model and Bitorch
// Engine's quantization-aware training run this product in their backward
// pass ("只需单卡 RTX 3090 低比特量化训练就能实现 LLaMA-3 8B 全参微调", Q-SFT
// and Bitorch Engine paragraphs).  The arithmetic is the forward matmul's:
// each weight is rounded once to fp16 ("A Survey of Low-bit Large Language
// Models", sections 5.2 and 6.2: dequantize, then an FP16 matmul), dY is
// rescaled per row by a power of two so that its fp16 form is exact, the
// MFMAs accumulate in fp32, and x 2^e and round-to-nearest-even end it.
//
// Work split.  A workgroup of 4 waves computes a 256 (m) x 256 (k) tile of
// dX, each wave 64 columns and all 256 rows (eight 32-row blocks times two
// 32-column blocks of MFMA 32x32x16).  The reduction runs over n in steps of
// 128; dY's 256 x 128 slice of a step reaches LDS by buffer loads that write
// LDS directly, one step ahead, into the other of two buffers, in the layout
// the forward matmul uses for x (sub-step t reduces over n-chunks t and
// 8 + t of the step).
//
// The weight operand.  A packed word holds consecutive k of one row n, but a
// lane of the MFMA weight operand needs 8 consecutive n of one k.  So each
// wave unpacks the 16 x 64 weight block of a sub-step itself -- a lane takes
// one row and 16 consecutive k, with that row's scale and zero point -- and
// writes it transposed into a private LDS block ([k][n] fp16), from which it
// reads its operand fragments back.  LDS operations of one wave complete in
// issue order, so the exchange needs no barrier.  A 128-row step lies inside
// one Channel-mix block (blocks are multiples of 128 rows), so the bit width
// is uniform per step.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int DX_NT = 128;                              // n per step
constexpr int DX_MB = 8;                                // 32-row blocks per wave
constexpr int DX_NW = 4;                                // waves, 64 columns each
constexpr int DX_TM = 32 * DX_MB;                       // 256 rows of dX
constexpr int DX_TK = 64 * DX_NW;                       // 256 columns of dX
constexpr int DX_TILE_BYTES = DX_TM * DX_NT * 2;        // 64 KB of dY per step
constexpr int DX_DMA = DX_TILE_BYTES / (1024 * DX_NW);  // 1 KB LDS loads per wave per step
constexpr int DX_WBLK = 148 * 4;                        // dwords of a wave's weight block
constexpr uint32_t kOobDx = 0x80000000u;                // beyond every resource

// The INT4 mask of the layout in the lanes of two registers: lane l holds
// word l and the number of INT4 blocks before it.  A step's block is then
// found with two lane reads instead of a walk over the mask in the kernel
// arguments (a chain of dependent scalar loads, ~1.5 us per step when it
// ran twice per step on a 224-block layout).
struct MaskLanes {
  uint32_t word, pre;
};

__device__ __forceinline__ MaskLanes mask_lanes(const LayoutDev &L, int lane) {
  MaskLanes ml{0u, 0u};
#pragma unroll
  for (int i = 0; i < GQ_MAX_BLOCKS / 32; ++i) {
    const uint32_t m = L.int4_mask[i];
    ml.word = lane == i ? m : ml.word;
    ml.pre += i < lane ? (uint32_t)__builtin_popcount(m) : 0u;
  }
  return ml;
}

__device__ __forceinline__ BlockInfo block_of(const LayoutDev &L, const MaskLanes &ml, int blk) {
  const int wi = blk >> 5;
  const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)ml.word, wi);
  const uint32_t c4 = (uint32_t)__builtin_amdgcn_readlane((int)ml.pre, wi) +
                      (uint32_t)__builtin_popcount(word & ((1u << (blk & 31)) - 1u));
  BlockInfo b;
  b.bits = ((word >> (blk & 31)) & 1u) ? 4 : 2;
  const uint64_t bk = (uint64_t)L.block_n * (uint64_t)L.K;
  b.code_off = bk * (uint64_t)(blk + c4) / 4u;
  b.grp_off = bk * (uint64_t)(2 * blk - (int)c4) / 128u;
  return b;
}

struct DxArgs {
  int M, N, K, Np;
  int m0, k0w;             // tile row origin; the wave's first column
  int st0, st1;            // n steps [st0, st1) of this workgroup (even count)
  bool kact;               // the wave's columns lie below K
  const int *rexp;
  uint16_t *dx;            // bf16/fp16 output, or
  float *part;             // the fp32 partial [M][K] of this split, or
  float *tail;             // the fp32 part of a split tail tile (register order)
  int out_fp16;
};

__device__ __forceinline__ void dx_wave(const LayoutDev &L, const DxArgs &g, uint4 *As0, uint4 *As1,
                                        uint32_t *Wb, Rsrc xr, Rsrc cr, Rsrc sr, Rsrc zr, int wave) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 31;
  const int h = lane >> 5;
  // weight block lane roles: lane (ri, cj) loads row ri of the sub-step,
  // columns 16 cj .. 16 cj + 15.  Lanes ri and ri ^ 1 then swap halves, so
  // that the even lane holds rows (ri, ri + 1) x columns 16 cj .. + 7 and the
  // odd one rows (ri - 1, ri) x columns 16 cj + 8 .. + 15: column group
  // g = 2 cj + odd of 8 columns, one dword (two rows) per column.
  const int ri = lane & 15, cj = lane >> 4;
  const MaskLanes ml = mask_lanes(L, lane);
  const bool odd = ri & 1;
  // Wb holds column 8g + c, rows 8hh .. 8hh + 7 (hh = half of the 16
  // rows) in 16-byte chunk 9 (8 hh + g) + 4 hh + c.  LDS has 32 banks and
  // serves a dword write half a wave per cycle: the 32 lanes of a half
  // (4 groups g, both hh, 4 row pairs) then hit 32 different banks, since
  // 9 (8 hh + g) + 4 hh = g + 4 hh (mod 8).  An operand read (8 lanes, one
  // group, 8 columns) covers 8 consecutive chunks.
  const uint32_t wbase = (uint32_t)(4 * (9 * (8 * (ri >> 3) + 2 * cj + (odd ? 1 : 0)) + 4 * (ri >> 3)) +
                                    ((ri >> 1) & 3));
  const uint32_t rbase = (uint32_t)(4 * (9 * (8 * h + (j >> 3)) + 4 * h + (j & 7)));
  // partner's scale and zero join the lane's own as (row a, row b) halves
  const uint32_t ssel = odd ? 0x01000504u : 0x05040100u;
  const uint32_t zsel = odd ? 0x0c020c06u : 0x0c060c02u;

  // dY tile DMA (the forward matmul's x tile): load i (= DX_DMA * wave + p)
  // writes slots 64 i .. 64 i + 63, rows 4i .. 4i + 3; lane l -> row
  // 4i + l/16, chunk (l%16) ^ (row & 15), row & 15 = 4 (i & 3) + l/16
  uint32_t dv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    dv[q] = (uint32_t)(((lane >> 4) * g.Np + (((lane & 15) ^ (4 * q + (lane >> 4))) * 8)) * 2);
  auto dma_a = [&](int st, uint4 *dst, int p0, int np) {
#pragma unroll
    for (int p = p0; p < p0 + np; ++p) {
      const int i = DX_DMA * wave + p;
      const uint32_t soff = (uint32_t)(((g.m0 + 4 * i) * g.Np + st * DX_NT) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(dst + 64 * i), 16, dv[p & 3], soff,
                                               0, 0);
    }
  };
  // operand reads: lane (j, h) of block mb, sub-step t reads row 32 mb + j,
  // chunk 8h + t, i.e. slot chunk ((8h) ^ (j & 8)) | (t ^ (j & 7))
  const uint32_t rb = (uint32_t)(j * 16 + ((8 * h) ^ (j & 8)));

  // block of a step (clamped: padding steps past N load nothing anyway)
  auto step_block = [&](int st) {
    int blk = st * DX_NT / L.block_n;
    return blk < L.nblocks ? blk : L.nblocks - 1;
  };

  // Weights of a step: lane (ri, cj) loads, for each sub-step t, the codes
  // of row n0 + 8t + (ri & 7) + 64 (ri >> 3) for columns k0w + 16 cj .. + 15,
  // and the scale and zero point of that row for t = cj and t = cj + 4
  // (spread to the other lanes later).  One 64-bit code load per row for
  // both widths: INT4 takes its 16 columns (8 bytes); INT2 takes the
  // 8-byte-aligned window holding its 4 bytes (a row is a multiple of 16
  // bytes, so the window stays in the row), whose high dword is the one
  // lanes with odd cj need.  (A load that differs by width would be a
  // branch, and merging its two sides made the compiler wait for the
  // loads.)  Offsets are computed at the top of a step; the loads issue
  // over its first sub-steps, between the dY tile loads.
  struct WAddr {
    uint32_t co[8], so[2], zo[2];
  };
  auto waddr = [&](int st, WAddr &A) {
    const int blk = step_block(st);
    const BlockInfo bi = block_of(L, ml, blk);
    const int bits = bi.bits;
    const uint32_t RB = (uint32_t)(L.K * bits / 8);
    const uint32_t GPR = (uint32_t)(bits == 4 ? L.K / 128 : L.K / 64);
    const uint32_t gcol = (uint32_t)(g.k0w / (bits == 4 ? 128 : 64));
    const uint32_t ccol = (uint32_t)((g.k0w + 16 * cj) * bits / 8);
    const uint32_t ccw = bits == 4 ? ccol : (ccol & ~7u);
    auto row_ok = [&](int t, uint32_t &r) {
      const int n = st * DX_NT + 8 * t + (ri & 7) + 64 * (ri >> 3);
      r = (uint32_t)(n - blk * L.block_n);
      return g.kact && n < g.N;
    };
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t r;
      A.co[t] = row_ok(t, r) ? (uint32_t)bi.code_off + r * RB + ccw : kOobDx;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t r;
      const bool ok = row_ok(cj + 4 * u, r);
      const uint32_t gi = (uint32_t)bi.grp_off + r * GPR + gcol;
      A.so[u] = ok ? 2u * gi : kOobDx;
      A.zo[u] = ok ? gi : kOobDx;
    }
  };

  // Per-step constants of the unpacking.  The bit width enters as shift,
  // mask and byte selectors rather than a branch: two copies of the MFMA
  // loop under a branch make the register allocator spill the
  // accumulators.  sel0 / sel1 put columns 0..3 / 4..7 of the lane's group
  // for row a in the low half and for row b in the high half (INT4: bytes
  // 0-1 / 2-3 of the group's word; INT2: byte 0 / 1 of the even lane's,
  // 2 / 3 of the odd lane's 16-code word).
  struct Sel {
    bool b4;
    uint32_t xmask, sh, mask, sel0, sel1;
  };
  auto sel_of = [&](int st) {
    Sel S;
    S.b4 = block_of(L, ml, step_block(st)).bits == 4;
    S.xmask = (S.b4 || !(cj & 1)) ? ~0u : 0u;   // word x holds the lane's columns 0..7
    S.sh = S.b4 ? 4u : 2u;
    S.mask = S.b4 ? 0x000f000fu : 0x00030003u;
    S.sel0 = S.b4 ? 0x05040100u : (odd ? 0x0c060c02u : 0x0c040c00u);
    S.sel1 = S.b4 ? 0x07060302u : (odd ? 0x0c070c03u : 0x0c050c01u);
    return S;
  };
  // scale | zero << 16 of row ri for every sub-step: lane (ri, cj) holds
  // sub-steps cj and cj + 4; two lane swaps copy the row of lanes c to all
  // four
  auto spread_sz = [&](const uint32_t *sv, const uint32_t *zv, uint32_t *szb) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t a = sv[u] | (zv[u] << 16), b = a;
      swap16(a, b);                    // a: rows (0, 0, 2, 2), b: rows (1, 1, 3, 3)
      uint32_t a2 = a, b2 = b;
      swap32(a, a2);                   // a: row 0 everywhere, a2: row 2
      swap32(b, b2);                   // b: row 1, b2: row 3
      szb[4 * u + 0] = a;
      szb[4 * u + 1] = b;
      szb[4 * u + 2] = a2;
      szb[4 * u + 3] = b2;
    }
  };
  // unpack the lane's 2 rows x 8 columns of one sub-step and write them to
  // weight block wb, one dword (rows a, b) per column
  auto make_b = [&](uint32_t *wb, const uint2 code, uint32_t sz, const Sel &S) {
    // a select between the two loaded words written as a bit blend: as a
    // select the compiler turns it into an indexed access and moves the
    // code registers to scratch
    const uint32_t ox = (code.x & S.xmask) | (code.y & ~S.xmask);
    const uint32_t oy = S.b4 ? code.y : ox;   // INT2: all 16 columns in one word
    // even lanes keep columns 0..7 and send 8..15, odd lanes the reverse
    const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(
        0, (int)(odd ? ox : oy), 0xB1, 0xF, 0xF, false);   // lanes l <-> l ^ 1
    const uint32_t wa = odd ? recv : ox;
    const uint32_t wbw = odd ? oy : recv;
    const uint32_t szp = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sz, 0xB1, 0xF, 0xF, false);
    // -(1024 + z) for rows a and b: the zero bytes under an fp16 -1024
    const half2v cz = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(szp, sz, zsel) | 0xE400E400u);
    const half2v s2 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(szp, sz, ssel));
    const uint32_t tw[2] = {__builtin_amdgcn_perm(wbw, wa, S.sel0), __builtin_amdgcn_perm(wbw, wa, S.sel1)};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // 1024 + q of column 4c + e for rows a and b, then (q - z) s
        const uint32_t p = and_or(tw[c] >> (S.sh * e), S.mask, 0x64006400u);
        const half2v v = (__builtin_bit_cast(half2v, p) + cz) * s2;
        wb[wbase + 4 * (4 * c + e)] = __builtin_bit_cast(uint32_t, v);
      }
  };
  // B operand of lane (j, h): rows 8h .. 8h + 7 of column 32 nb + j
  auto read_b = [&](const uint32_t *wb, half8 *bf) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bf[nb] = *reinterpret_cast<const half8 *>(&wb[rbase + 144 * nb]);
  };
  auto read_a = [&](const uint4 *tile, int t, half8 *af) {
    const uint32_t slot = rb + (uint32_t)(t ^ (j & 7));
#pragma unroll
    for (int mb = 0; mb < DX_MB; ++mb) af[mb] = __builtin_bit_cast(half8, tile[mb * 512 + slot]);
  };
  uint32_t *const Wb0 = Wb, *const Wb1 = Wb + DX_WBLK;

  floatx16 acc[DX_MB][2];
#pragma unroll
  for (int mb = 0; mb < DX_MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;
  half8 af[2][DX_MB], bf[2][2];

  // One n step from dY tile `cur`, with the step's codes bc and spread
  // scales szc.  Sub-step t multiplies operands read during sub-step t - 1,
  // reads those of t + 1 and unpacks the weights of t + 2 into the block
  // that sub-step t emptied (two blocks, alternating).  The step also
  // loads the next step's dY tile into `nxt` and its weights into (bn, sn,
  // zn); sub-steps 6 and 7 unpack the next step's first two sub-steps, and
  // the barrier that makes `nxt` visible sits before sub-step 7, which reads
  // the next step's first dY operands.  On the last step the "next" step is
  // the same step again, so every load stays unconditional.
  auto step = [&](int st, const uint4 *cur, uint4 *nxt, const uint2 *bc, const uint32_t *szc,
                  uint2 *bn, uint32_t *sn, uint32_t *zn, uint32_t *szn) {
    const int sn_ = st + 1 < g.st1 ? st + 1 : st;
    WAddr A;
    waddr(sn_, A);
    const Sel Sc = sel_of(st), Sn = sel_of(sn_);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int c = t & 1, n = c ^ 1;
      // one scheduling region per sub-step: without it the scheduler sinks
      // the operand reads of sub-step t + 1 to just before their MFMAs,
      // behind this sub-step's weight writes, and waits for them there
      __builtin_amdgcn_sched_barrier(0);
      if (t == 7) {
        __builtin_amdgcn_sched_barrier(0);
        // every wave's part of the next dY tile has landed, and no wave
        // reads `cur` any more
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      // loads: the next dY tile over sub-steps 0..3, the next weights'
      // scales and zero points with sub-step 0 and codes with 1 and 2
      if (t < 4) dma_a(sn_, nxt, (DX_DMA / 4) * t, DX_DMA / 4);
      if (t == 0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          sn[u] = ld16(sr, A.so[u]);
          zn[u] = ld8(zr, A.zo[u]);
        }
      }
      if (t == 1 || t == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) bn[4 * (t - 1) + q] = ld64(cr, A.co[4 * (t - 1) + q]);
      }
      if (t == 5) spread_sz(sn, zn, szn);
      // operands of sub-step t + 1 (of the next step's sub-step 0 at t = 7)
      read_b(n ? Wb1 : Wb0, bf[n]);
      read_a(t < 7 ? cur : nxt, (t + 1) & 7, af[n]);
      // weights of sub-step t + 2 into the block sub-step t used
      if (t < 6)
        make_b(c ? Wb1 : Wb0, bc[t + 2], szc[t + 2], Sc);
      else
        make_b(c ? Wb1 : Wb0, bn[t - 6], szn[t - 6], Sn);
#pragma unroll
      for (int mb = 0; mb < DX_MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][mb], bf[c][nb], acc[mb][nb], 0, 0, 0);
      // one wave per SIMD: the loads, operand reads, unpacking and weight
      // writes of this sub-step issue between its MFMAs
      const int nvm = t == 0 ? DX_DMA / 4 + 4 : (t < 3 ? DX_DMA / 4 + 4 : (t == 3 ? DX_DMA / 4 : 0));
#pragma unroll
      for (int i = 0; i < 2 * DX_MB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
        if (i < nvm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);          // global load
        if (i < DX_MB + 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // operand read
        if (i < 12) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);           // VALU
        if (i >= 2 && i < 10) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); // weight write
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  uint2 b0[8], b1[8];
  uint32_t s0[2], s1[2], z0[2], z1[2], szA[8], szB[8];
  {
    // first step: its dY tile, weights and the first two weight blocks
    WAddr A;
    waddr(g.st0, A);
    dma_a(g.st0, As0, 0, DX_DMA);
#pragma unroll
    for (int t = 0; t < 8; ++t) b0[t] = ld64(cr, A.co[t]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s0[u] = ld16(sr, A.so[u]);
      z0[u] = ld8(zr, A.zo[u]);
    }
    lds_barrier();
    const Sel S0 = sel_of(g.st0);
    spread_sz(s0, z0, szA);
    make_b(Wb0, b0[0], szA[0], S0);
    make_b(Wb1, b0[1], szA[1], S0);
    read_b(Wb0, bf[0]);
    read_a(As0, 0, af[0]);
  }
  for (int st = g.st0; st < g.st1; st += 2) {
    step(st, As0, As1, b0, szA, b1, s1, z1, szB);
    step(st + 1, As1, As0, b1, szB, b0, s0, z0, szA);
  }

  if (g.tail) {
    // part of a split tail tile: the accumulators in register order
    // (wave, mb, nb, e, lane), 256 contiguous bytes per store
#pragma unroll
    for (int mb = 0; mb < DX_MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          g.tail[(((wave * DX_MB + mb) * 2 + nb) * 16 + e) * 64 + lane] = acc[mb][nb][e];
    return;
  }
  if (!g.kact) return;
  // lane (j, h) holds column k0w + 32 nb + j and rows 8(e/4) + 4h + e%4 of
  // each 32-row block
  if (g.part) {
#pragma unroll
    for (int mb = 0; mb < DX_MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = g.m0 + mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int k = g.k0w + 32 * nb + j;
          if (m < g.M && k < g.K) g.part[(int64_t)m * g.K + k] = acc[mb][nb][e];
        }
      }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < DX_MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = g.m0 + mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      const int ex = m < g.M ? g.rexp[m] : 0;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int k = g.k0w + 32 * nb + j;
        const float v = ldexpf(acc[mb][nb][e], ex);
        if (m < g.M && k < g.K)
          g.dx[(int64_t)m * g.K + k] = g.out_fp16 ? f32_to_f16_bits(v) : f32_to_bf16_rne(v);
      }
    }
}

__global__ __launch_bounds__(64 * DX_NW, 1) void dx_kernel(
    LayoutDev L, int M, int Np, uint32_t ya_bytes, int m_tiles, const uint16_t *__restrict__ ya,
    const int *__restrict__ rexp, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, uint32_t code_bytes,
    uint32_t groups, uint16_t *__restrict__ dx, int out_fp16, int steps_per_split,
    float *__restrict__ part, int tail_full, int tail_parts, int tail_per) {
  __shared__ __attribute__((aligned(16))) uint4 As0[DX_TILE_BYTES / 16];
  __shared__ __attribute__((aligned(16))) uint4 As1[DX_TILE_BYTES / 16];
  __shared__ __attribute__((aligned(16))) uint32_t Wb[DX_NW * 2 * DX_WBLK];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // tile order: m fastest, so the workgroups on one XCD (every 8th id)
  // share one m tile of dY in that XCD's L2; ids past tail_full are the
  // parts of the split tail tiles
  const int id = (int)blockIdx.x;
  const bool tpart = id >= tail_full;
  const int tile = tpart ? tail_full + (id - tail_full) / tail_parts : id;
  const int pidx = tpart ? (id - tail_full) % tail_parts : 0;
  const int m_tile = tile % m_tiles, k_tile = tile / m_tiles;
  const int nsteps = Np / DX_NT;
  DxArgs g;
  g.M = M; g.N = L.N; g.K = L.K; g.Np = Np;
  g.m0 = m_tile * DX_TM;
  g.k0w = k_tile * DX_TK + wave * 64;
  g.kact = g.k0w < L.K;
  if (tpart) {
    g.st0 = pidx * tail_per;
    g.st1 = min(g.st0 + tail_per, nsteps);
  } else {
    g.st0 = (int)blockIdx.y * steps_per_split;
    g.st1 = min(g.st0 + steps_per_split, nsteps);
  }
  g.rexp = rexp;
  g.dx = dx;
  g.part = gridDim.y > 1 ? part + (size_t)blockIdx.y * (size_t)M * (size_t)L.K : nullptr;
  g.tail = tpart ? part + (size_t)(id - tail_full) * (DX_TM * DX_TK) : nullptr;
  g.out_fp16 = out_fp16;
  const Rsrc xr = make_rsrc(ya, ya_bytes);
  const Rsrc cr = make_rsrc(codes, code_bytes);
  const Rsrc sr = make_rsrc(scales, 2u * groups);
  const Rsrc zr = make_rsrc(zeros, groups);
  dx_wave(L, g, As0, As1, Wb + wave * 2 * DX_WBLK, xr, cr, sr, zr, wave);
}

// dX = 0 for an empty reduction (N == 0): a fill kernel rather than a
// memset, so that the call can be captured in a graph.
__global__ __launch_bounds__(256) void dx_zero_kernel(uint16_t *__restrict__ dx, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dx[i] = 0;
}

// dY rows padded to whole 256-row tiles, n to whole pairs of 128 steps.
// Fewer tiles than CUs: the n range of every tile is split (fp32 partials
// [splits][M][K]).  More: the tiles of an incomplete last round are cut
// along n into `parts` pieces that run side by side (fp32 parts of those
// tiles), one tile per CU at a time either way.
constexpr int kDxCUs = 256;

struct DxWs {
  int Mp, Np, tiles, splits, per;
  int full, rem, parts, tper;     // tail split
  size_t a_bytes, e_bytes, p_bytes;
};

inline size_t round256(size_t v) { return (v + 255u) & ~(size_t)255u; }

inline DxWs dx_workspace_of(const LayoutDev &L, int M) {
  DxWs w;
  w.Np = (L.N + 2 * DX_NT - 1) / (2 * DX_NT) * (2 * DX_NT);
  w.Mp = (M + DX_TM - 1) / DX_TM * DX_TM;
  w.a_bytes = round256((size_t)w.Mp * (size_t)w.Np * 2u);
  w.e_bytes = round256((size_t)(M > 0 ? M : 1) * 4u);
  w.tiles = (w.Mp / DX_TM) * ((L.K + DX_TK - 1) / DX_TK);
  const int nsteps = w.Np / DX_NT;
  // split n until the tiles fill the CUs, keeping >= 8 steps per split
  int sp = 1;
  while (w.tiles * sp < kDxCUs && nsteps / (2 * sp) >= 8 && sp < 16) sp *= 2;
  w.per = ((nsteps + sp - 1) / sp + 1) & ~1;             // even
  w.splits = (nsteps + w.per - 1) / w.per;
  w.p_bytes = w.splits > 1 ? (size_t)w.splits * (size_t)M * (size_t)L.K * 4u : 0u;
  // tail split of the last round, parts of >= 16 steps
  w.full = w.tiles;
  w.rem = 0;
  w.parts = 1;
  w.tper = nsteps;
  if (w.splits == 1 && w.tiles > kDxCUs && w.tiles % kDxCUs) {
    const int rem = w.tiles % kDxCUs;
    int parts = kDxCUs / rem < 4 ? kDxCUs / rem : 4;
    while (parts > 1 && nsteps / parts < 16) --parts;
    if (parts > 1) {
      w.rem = rem;
      w.parts = parts;
      w.full = w.tiles - rem;
      w.tper = ((nsteps + parts - 1) / parts + 1) & ~1;
      w.p_bytes = (size_t)rem * parts * DX_TM * DX_TK * 4u;
    }
  }
  return w;
}

}  // namespace

bool dx_supported(const LayoutDev &L, int M) {
  if (L.N % 8 != 0) return false;                        // dY rows in 16-byte pieces
  const DxWs w = dx_workspace_of(L, M);
  if (w.a_bytes >= ((size_t)1 << 31)) return false;
  uint64_t code_bytes = 0, groups = 0;
  for (int i = 0; i < L.nblocks; ++i) {
    const bool b4 = (L.int4_mask[i >> 5] >> (i & 31)) & 1u;
    code_bytes += (uint64_t)L.block_n * L.K / (b4 ? 2 : 4);
    groups += (uint64_t)L.block_n * L.K / (b4 ? 128 : 64);
  }
  return code_bytes < ((uint64_t)1 << 31) && 2u * groups < ((uint64_t)1 << 31);
}

size_t dx_workspace_bytes(const LayoutDev &L, int M) {
  if (M <= 0 || L.N == 0 || L.K == 0) return 0;
  const DxWs w = dx_workspace_of(L, M);
  return w.a_bytes + w.e_bytes + w.p_bytes;
}

hipError_t launch_dx(const LayoutDev &L, int M, gq_dtype act, const void *dy,
                     const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros, void *dx,
                     void *workspace, hipStream_t s) {
  if (L.N == 0) {
    const size_t n = (size_t)M * (size_t)L.K;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(dx_zero_kernel, dim3(blocks < 4096 ? (unsigned)blocks : 4096u), dim3(256), 0, s,
                       reinterpret_cast<uint16_t *>(dx), n);
    return hipGetLastError();
  }
  const DxWs w = dx_workspace_of(L, M);
  uint16_t *ya = reinterpret_cast<uint16_t *>(workspace);
  int *rexp = reinterpret_cast<int *>(reinterpret_cast<char *>(workspace) + w.a_bytes);
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + w.a_bytes + w.e_bytes);
  hipError_t err = launch_prep_rows(dy, M, L.N, w.Mp, w.Np, act, ya, rexp, s);
  if (err != hipSuccess) return err;
  uint64_t code_bytes = 0, groups = 0;
  for (int i = 0; i < L.nblocks; ++i) {
    const bool b4 = (L.int4_mask[i >> 5] >> (i & 31)) & 1u;
    code_bytes += (uint64_t)L.block_n * L.K / (b4 ? 2 : 4);
    groups += (uint64_t)L.block_n * L.K / (b4 ? 128 : 64);
  }
  const int m_tiles = w.Mp / DX_TM;
  const int out_fp16 = act == GQ_FP16 ? 1 : 0;
  uint16_t *dxp = reinterpret_cast<uint16_t *>(dx);
  hipLaunchKernelGGL(dx_kernel, dim3(w.full + w.rem * w.parts, w.splits), dim3(64 * DX_NW), 0, s, L, M,
                     w.Np, (uint32_t)w.a_bytes, m_tiles, ya, rexp,
                     reinterpret_cast<const uint8_t *>(codes), scales, zeros, (uint32_t)code_bytes,
                     (uint32_t)groups, dxp, out_fp16, w.per, part, w.full, w.parts, w.tper);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (w.splits > 1) return launch_splitk_reduce(part, w.splits, M, L.K, rexp, dxp, out_fp16, s);
  if (w.rem > 0)
    return launch_tile_tail_reduce(part, w.parts, w.full, w.rem, m_tiles, M, L.K, rexp, dxp, out_fp16, s);
  return hipSuccess;
}

}  // namespace gq
