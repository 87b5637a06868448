// Prefill GEMM (M > 4): y = x . W_hat^T on the MFMA matrix cores.
//
// "A Survey of Low-bit Large Language Models" review, sections 5.2 and 6.2:
// weight-only quantization dequantizes the weights and runs an FP16 matmul.
// Here each weight is dequantized in registers to fp16 as
// fp16((q - z) * s) -- (q - z) is formed exactly, the product is rounded once
// -- and fed to v_mfma_f32_32x32x16_f16 with fp32 accumulation.  The
// dequantized matrix never touches memory.
//
// Activations arrive as bf16.  A pre-pass rescales each row of x by a power
// of two 2^-e (e chosen from the row's largest magnitude) so every bf16
// value lands exactly in fp16, and the epilogue multiplies by 2^e.  The
// pre-pass also permutes each 8-element chunk of k to the order
// (0,4,1,5,2,6,3,7): that is the order in which the packed-word unpacking
// below produces code pairs, so A and B agree on k inside each MFMA.
//
// Tiles: a workgroup of 4 waves computes a (32*MB) x 256 tile of y.  Wave w
// owns output columns [64w, 64w+64) as two 32-column MFMA blocks and all
// 32*MB rows.  The x tile goes through LDS (double buffered, one barrier per
// 64-deep k step); the packed codes of the wave's own columns go straight
// from HBM to registers, so every code is unpacked exactly once per tile.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));


// ---------------------------------------------------------------- pre-pass

// One workgroup per row of the padded activation matrix xa [Mp][Kp]: largest
// magnitude, exponent, rescale, convert, permute (PERM).  Rows m >= M and
// columns k >= K are written as zeros, so the GEMM reads whole tiles without
// masks.  act 0: bf16 input (rescaled), act 1: fp16 input (copied).
template <int ACT, bool PERM>
__global__ __launch_bounds__(256) void prep_x_kernel(const uint16_t *__restrict__ x, int M, int K,
                                                     int Kp, uint16_t *__restrict__ xa,
                                                     int *__restrict__ rexp) {
  const int m = blockIdx.x;
  uint16_t *out = xa + (int64_t)m * Kp;
  if (m >= M) {
    for (int c = threadIdx.x * 8; c < Kp; c += 256 * 8)
      *reinterpret_cast<uint4 *>(out + c) = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const uint16_t *row = x + (int64_t)m * K;
  __shared__ float red[4];
  int e = 0;
  // each thread keeps kPrepLoads 16-byte loads in flight: one at a time
  // left the pass waiting on memory latency (a 57 KB row is 14 loads per
  // thread)
  constexpr int kPrepLoads = 4;
  if (ACT == 0) {
    float amax = 0.f;
    for (int c0 = threadIdx.x * 8; c0 < K; c0 += kPrepLoads * 256 * 8) {
      uint4 v[kPrepLoads];
#pragma unroll
      for (int u = 0; u < kPrepLoads; ++u) {
        const int c = c0 + u * 256 * 8;
        v[u] = c < K ? *reinterpret_cast<const uint4 *>(row + c) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kPrepLoads; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (amax > 0.f && __builtin_isfinite(amax)) {
      int ex;
      frexpf(amax, &ex);        // amax = f * 2^ex, f in [0.5, 1)
      e = ex - 16;              // amax * 2^-e in [2^15, 2^16)
    }
  }
  if (threadIdx.x == 0) rexp[m] = e;
  for (int c0 = threadIdx.x * 8; c0 < Kp; c0 += kPrepLoads * 256 * 8) {
    uint4 vin[kPrepLoads];
#pragma unroll
    for (int u = 0; u < kPrepLoads; ++u) {
      const int c = c0 + u * 256 * 8;
      vin[u] = c < K ? *reinterpret_cast<const uint4 *>(row + c) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kPrepLoads; ++u) {
    const int c = c0 + u * 256 * 8;
    if (c >= Kp) break;
    if (c >= K) {
      *reinterpret_cast<uint4 *>(out + c) = make_uint4(0u, 0u, 0u, 0u);
      continue;
    }
    const uint4 v = vin[u];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint16_t h[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ACT == 0) {
        h[2 * i] = f32_to_f16_bits(ldexpf(__uint_as_float(w[i] << 16), -e));
        h[2 * i + 1] = f32_to_f16_bits(ldexpf(__uint_as_float(w[i] & 0xffff0000u), -e));
      } else {
        h[2 * i] = (uint16_t)(w[i] & 0xffffu);
        h[2 * i + 1] = (uint16_t)(w[i] >> 16);
      }
    }
    uint4 o;
    if (PERM) {
      // chunk order (0,4,1,5,2,6,3,7)
      o.x = (uint32_t)h[0] | ((uint32_t)h[4] << 16);
      o.y = (uint32_t)h[1] | ((uint32_t)h[5] << 16);
      o.z = (uint32_t)h[2] | ((uint32_t)h[6] << 16);
      o.w = (uint32_t)h[3] | ((uint32_t)h[7] << 16);
    } else {
      o.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
      o.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
      o.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
      o.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
    }
    *reinterpret_cast<uint4 *>(out + c) = o;
    }
  }
}

// ------------------------------------------------------------------- GEMM

constexpr int KT = 128;                   // k per main-loop step
constexpr int LDA = KT + 8;               // halfs per LDS row (conflict-free b128 reads)

struct GemmArgs {
  int K, Kp, N, M, m0, nw;
  int kt0, nkt;                           // first k step and number of k steps
  const uint16_t *xa;
  const int *rexp;
  uint16_t *y;                            // bf16/fp16 output (split == 0)
  float *part;                            // fp32 partial [M][N] of this split (split != 0)
  int out_fp16;
};

// Main loop and epilogue of one wave; BITS is the bit-width of the wave's
// 64 columns (one Channel-mix block never splits a wave).  Every wave of the
// workgroup runs the same number of steps and barriers, including waves
// whose columns lie beyond N (they only help load the x tile).
template <int BITS, int MB, int NW, bool SPLIT>
__device__ __forceinline__ void gemm_wave(const GemmArgs &g, uint16_t (*As)[32 * MB * LDA],
                                          bool wave_active, const uint8_t *const *crow,
                                          const uint16_t *const *srow, const uint8_t *const *zrow,
                                          const bool *cvalid) {
  constexpr int RPP = 64 * NW / 16;       // A rows per load pass (16 threads per 256-byte row)
  constexpr int PASSES = 32 * MB / RPP;
  static_assert(PASSES * RPP == 32 * MB, "A tile rows");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h = lane >> 5;
  const int K = g.K;

  // A tile loads: thread -> (row = p*16 + tid/16, 16-byte chunk tid%16)
  const int arow = tid >> 4;
  const int achunk = tid & 15;
  uint4 areg[PASSES];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int m = g.m0 + p * RPP + arow;
      const int kk = kt * KT + achunk * 8;
      const bool ok = m < g.M && kk < K;              // rows past M, k past K (INT2 tail) read 0
      const int mc = m < g.M ? m : g.M - 1;           // clamped: always a valid address
      const uint4 v = *reinterpret_cast<const uint4 *>(g.xa + (int64_t)mc * g.Kp + (kk < K ? kk : 0));
      const uint32_t keep = ok ? 0xffffffffu : 0u;
      areg[p] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
      *reinterpret_cast<uint4 *>(&As[buf][(p * RPP + arow) * LDA + achunk * 8]) = areg[p];
  };
  // B codes: lane half h takes chunks 8h..8h+7 of the step (INT4: 8 words,
  // INT2: 4 words); both halves of an INT4 step share one group, each INT2
  // half lies in its own group.
  constexpr int BW = BITS == 4 ? 8 : 4;   // code words per lane per step
  uint32_t bcur[2][BW], bnext[2][BW];
  uint32_t scur[2], snext[2], zcur[2], znext[2];
  auto load_b = [&](int kt, uint32_t (*dst)[BW], uint32_t *sd, uint32_t *zd) {
    // the half step past K (INT2 layers with K % 128 == 64) reads row start
    // and gets scale 0, so it adds exactly 0
    const bool kok = kt * KT + h * (KT / 2) < K;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint8_t *src = crow[nb] + (kok ? (size_t)kt * (KT * BITS / 8) + h * (BW * 4) : 0);
#pragma unroll
      for (int q = 0; q < BW / 4; ++q) {
        const uint4 v = *reinterpret_cast<const uint4 *>(src + 16 * q);
        dst[nb][4 * q + 0] = v.x; dst[nb][4 * q + 1] = v.y;
        dst[nb][4 * q + 2] = v.z; dst[nb][4 * q + 3] = v.w;
      }
      const int gi = kok ? (BITS == 4 ? kt : 2 * kt + h) : 0;
      const uint32_t keep = (cvalid[nb] && kok) ? 0xffffffffu : 0u;   // invalid: scale 0
      sd[nb] = (uint32_t)srow[nb][gi] & keep;
      zd[nb] = (uint32_t)zrow[nb][gi];
    }
  };

  floatx16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;

  const int kend = g.kt0 + g.nkt;
  load_a(g.kt0);
  load_b(g.kt0, bcur, scur, zcur);
  store_a(0);
  lds_barrier();
  int cur = 0;
  for (int kt = g.kt0; kt < kend; ++kt) {
    // prefetch the next step; on the last step reload the same step (the
    // loads stay unconditional so the wait counts are exact)
    const int kn = kt + 1 < kend ? kt + 1 : kt;
    __builtin_amdgcn_sched_barrier(0);
    load_a(kn);
    load_b(kn, bnext, snext, znext);
    __builtin_amdgcn_sched_barrier(0);
    half2v cz[2], s2[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint16_t zb = f32_to_f16_bits(-(1024.f + (float)zcur[nb]));
      s2[nb] = __builtin_bit_cast(half2v, scur[nb] | (scur[nb] << 16));
      cz[nb] = __builtin_bit_cast(half2v, (uint32_t)zb | ((uint32_t)zb << 16));
    }
    // software pipeline over the 8 sub-steps of 16 k: the A fragments and
    // the unpacked B fragments of sub-step t+1 are produced while the MFMAs
    // of sub-step t run
    auto read_a = [&](int t, half8 *af) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *reinterpret_cast<const half8 *>(&As[cur][(mb * 32 + j) * LDA + (8 * h + t) * 8]);
    };
    auto make_b = [&](int t, half8 *bf) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if constexpr (BITS == 4) {
          unpack_f16_chunk<4>(bcur[nb][t], cz[nb], s2[nb], bf[nb]);
        } else {
          const uint32_t wv = bcur[nb][t >> 1];
          // bytes (b0, b0, b1, b1) for the low chunk, (b2, b2, b3, b3) for the high one
          const uint32_t tc = __builtin_amdgcn_perm(wv, wv, (t & 1) ? 0x03030202u : 0x01010000u);
          unpack_f16_chunk<2>(tc, cz[nb], s2[nb], bf[nb]);
        }
      }
    };
    half8 af[MB], bf[2][2];
    make_b(0, bf[0]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int c = t & 1, n = c ^ 1;
      read_a(t, af);
      if (t + 1 < 8) make_b(t + 1, bf[n]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mb], bf[c][nb], acc[mb][nb], 0, 0, 0);
      // the next step's x tile goes to the other LDS buffer half-way through
      // this step (that buffer was released by the previous barrier), so the
      // LDS writes overlap the remaining MFMAs
      if (t == 3) store_a(cur ^ 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    cur ^= 1;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int w = 0; w < BW; ++w) bcur[nb][w] = bnext[nb][w];
      scur[nb] = snext[nb];
      zcur[nb] = znext[nb];
    }
  }
  (void)wave_active;

  if (!wave_active) return;
  // epilogue: lane (j, h) holds column nw + 32nb + j and rows 8(e/4) + 4h + e%4
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = g.m0 + mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (m >= g.M) continue;
      const int ex = SPLIT ? 0 : g.rexp[m];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int n = g.nw + 32 * nb + j;
        if (n >= g.N) continue;
        if constexpr (SPLIT) {
          g.part[(int64_t)m * g.N + n] = acc[mb][nb][e];
        } else {
          const float v = ldexpf(acc[mb][nb][e], ex);
          g.y[(int64_t)m * g.N + n] = g.out_fp16 ? f32_to_f16_bits(v) : f32_to_bf16_rne(v);
        }
      }
    }
  }
}

template <int MB, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW, 1) void gemm_kernel(LayoutDev L, int M, int Kp, int m_tiles, int n_tiles,
                                                   int ksteps_per_split,
                                                   const uint16_t *__restrict__ xa,
                                                   const int *__restrict__ rexp,
                                                   const uint8_t *__restrict__ codes,
                                                   const uint16_t *__restrict__ scales,
                                                   const uint8_t *__restrict__ zeros,
                                                   uint16_t *__restrict__ y, float *__restrict__ part,
                                                   int out_fp16) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][32 * MB * LDA];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = threadIdx.x & 31;
  // tile order: m fastest, so the workgroups resident at one time share the
  // same packed-weight columns
  const int tile = (int)blockIdx.x;
  const int m_tile = tile % m_tiles;
  const int n_tile = tile / m_tiles;
  const int split = (int)blockIdx.y;
  GemmArgs g;
  g.K = L.K; g.Kp = Kp; g.N = L.N; g.M = M;
  g.m0 = m_tile * 32 * MB;
  g.nw = n_tile * (64 * NW) + wave * 64;
  const int ksteps = (L.K + KT - 1) / KT;
  g.kt0 = split * ksteps_per_split;
  g.nkt = ksteps - g.kt0 < ksteps_per_split ? ksteps - g.kt0 : ksteps_per_split;
  g.xa = xa; g.rexp = rexp; g.y = y; g.out_fp16 = out_fp16;
  g.part = part + (int64_t)split * M * L.N;
  const bool wave_active = g.nw < L.N;

  int bits = 4;
  const uint8_t *crow[2];
  const uint16_t *srow[2];
  const uint8_t *zrow[2];
  bool cvalid[2];
  // waves past N read column 0's block (valid memory) and never store
  const int nref = wave_active ? g.nw : 0;
  const int blk = nref / L.block_n;
  const BlockInfo bi = block_info(L, blk);
  bits = __builtin_amdgcn_readfirstlane(bi.bits);
  const int RB = L.K * bits / 8;
  const int GPR = bits == 4 ? L.K / 128 : L.K / 64;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = nref + 32 * nb + j;
    cvalid[nb] = wave_active && n < L.N;
    const int r = (cvalid[nb] ? n : nref) - blk * L.block_n;
    crow[nb] = codes + bi.code_off + (uint64_t)r * (uint64_t)RB;
    srow[nb] = scales + bi.grp_off + (uint64_t)r * (uint64_t)GPR;
    zrow[nb] = zeros + bi.grp_off + (uint64_t)r * (uint64_t)GPR;
  }
  (void)n_tiles;
  if (bits == 4)
    gemm_wave<4, MB, NW, SPLIT>(g, As, wave_active, crow, srow, zrow, cvalid);
  else
    gemm_wave<2, MB, NW, SPLIT>(g, As, wave_active, crow, srow, zrow, cvalid);
}

// ------------------------------------------------------- large-M GEMM
//
// M >= 256: a workgroup of 4 waves (one per SIMD) computes a 256 x 256 tile.
// Wave w owns columns [64w, 64w + 64) as two 32-column MFMA blocks and all
// 256 rows as eight 32-row blocks, so each unpacked code pair feeds eight
// MFMAs (half the dequantization work per MFMA of the 128-row tile).  The
// 8 x 2 accumulator blocks (256 fp32 per lane) live in the AGPRs.
//
// The x tile of the next k step travels HBM/L2 -> LDS by buffer loads that
// write LDS directly (no registers, no LDS store instructions), issued at
// the start of the current step into the other of two LDS buffers; the
// barrier at the end of the step is the only wait for it.  In LDS a tile is
// 256 rows x 16 chunks of 16 bytes, chunk c of row r in slot
// 16 r + (c ^ (r & 15)): the XOR spreads the MFMA operand reads (32
// consecutive rows, one chunk) over all banks.  Codes, scales and zeros go
// to registers through resources over the wave's Channel-mix block (columns
// past N read out of range and get zeros), also one step ahead.
constexpr int BIG_MB = 8;
constexpr int BIG_NW = 4;
constexpr int BIG_TM = 32 * BIG_MB;              // 256 rows
constexpr int BIG_TN = 64 * BIG_NW;              // 256 columns
constexpr int BIG_TILE_BYTES = BIG_TM * KT * 2;  // 64 KB
constexpr int BIG_DMA = BIG_TILE_BYTES / (1024 * BIG_NW);   // 1 KB LDS loads per wave per tile
constexpr uint32_t kOob = 0x80000000u;           // beyond every resource

typedef __attribute__((address_space(3))) void lds_void;

struct BigArgs {
  int K, Kp, N, M, m0;
  int kt0, kt1;                                  // k steps [kt0, kt1) of this workgroup (even count)
  float *tail;                                   // fp32 partial tile of a split tail tile, or null
  const int *rexp;
  uint16_t *y;
  int out_fp16;
};

template <int BITS>
__device__ __forceinline__ void big_wave(const BigArgs &g, uint4 *As0, uint4 *As1, Rsrc xr,
                                         Rsrc cr, Rsrc sr, Rsrc zr, const uint32_t (&cbase)[2],
                                         const uint32_t (&sbase)[2], const uint32_t (&zbase)[2],
                                         bool wave_active, int wave, int ncol0) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 31;
  const int h = lane >> 5;

  // x tile DMA: load i (= BIG_DMA * wave + p) writes slots 64 i .. 64 i + 63,
  // i.e. rows 4i .. 4i + 3; lane l -> row 4i + l/16, chunk (l%16) ^ (row & 15)
  // with row & 15 = 4 (i & 3) + l/16
  uint32_t dv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    dv[q] = (uint32_t)(((lane >> 4) * g.Kp + (((lane & 15) ^ (4 * q + (lane >> 4))) * 8)) * 2);
  // loads p0 .. p0 + np - 1 of the wave's BIG_DMA
  auto dma_a = [&](int kt, uint4 *dst, int p0, int np) {
#pragma unroll
    for (int p = p0; p < p0 + np; ++p) {
      const int i = BIG_DMA * wave + p;
      const uint32_t soff = (uint32_t)(((g.m0 + 4 * i) * g.Kp + kt * KT) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(dst + 64 * i), 16, dv[p & 3], soff,
                                               0, 0);
    }
  };
  // x loads per sub-step, over the first four: the last ones then have
  // half a step to land before the barrier that waits for them
  constexpr int DMA_PER_SUB = BIG_DMA / 4;
  // MFMA operand reads: lane (j, h) of 32-row block mb, sub-step t reads row
  // 32 mb + j, chunk 8h + t, i.e. slot chunk ((8h) ^ (j & 8)) | (t ^ (j & 7))
  const uint32_t rb = (uint32_t)(j * 16 + ((8 * h) ^ (j & 8)));   // in 16-byte slots

  // codes: lane half h takes chunks 8h..8h+7 of the step (INT4: 8 words,
  // INT2: 4 words); INT4 steps are one group, INT2 halves one group each
  constexpr int BW = BITS == 4 ? 8 : 4;
  constexpr uint32_t STEPB = KT * BITS / 8;       // code bytes per column per step
  constexpr uint32_t STEPG = BITS == 4 ? 1 : 2;   // groups per step
  auto load_b = [&](int kt, uint32_t (*dst)[BW], uint32_t *sd, uint32_t *zd) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t co = cbase[nb] + (uint32_t)kt * STEPB;
#pragma unroll
      for (int q = 0; q < BW / 4; ++q) {
        const uint4 v = ld128(cr, co + 16u * q);
        dst[nb][4 * q + 0] = v.x; dst[nb][4 * q + 1] = v.y;
        dst[nb][4 * q + 2] = v.z; dst[nb][4 * q + 3] = v.w;
      }
      sd[nb] = ld16(sr, sbase[nb] + (uint32_t)kt * (2 * STEPG));
      zd[nb] = ld8(zr, zbase[nb] + (uint32_t)kt * STEPG);
    }
  };

  floatx16 acc[BIG_MB][2];
#pragma unroll
  for (int mb = 0; mb < BIG_MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;

  // one k step from LDS tile `cur` with codes (bc, sc, zc); starts the
  // next step's x DMA into `nxt` and its codes into (bn, sn, zn).  On the
  // last step both reload the same step, so every load stays unconditional.
  auto step = [&](int kt, const uint4 *cur, uint4 *nxt, const uint32_t (*bc)[BW],
                  const uint32_t *sc, const uint32_t *zc, uint32_t (*bn)[BW], uint32_t *sn,
                  uint32_t *zn) {
    const int kn = kt + 1 < g.kt1 ? kt + 1 : kt;
    __builtin_amdgcn_sched_barrier(0);
    load_b(kn, bn, sn, zn);
    __builtin_amdgcn_sched_barrier(0);
    // the half step past K (INT2 rows with K % 128 == 64) gets scale 0;
    // its x columns are zero padding
    const bool kok = kt * KT + h * (KT / 2) < g.K;
    half2v cz[2], s2[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t sv = kok ? sc[nb] : 0u;
      const uint16_t zb = f32_to_f16_bits(-(1024.f + (float)zc[nb]));
      s2[nb] = __builtin_bit_cast(half2v, sv | (sv << 16));
      cz[nb] = __builtin_bit_cast(half2v, (uint32_t)zb | ((uint32_t)zb << 16));
    }
    auto read_a = [&](int t, half8 *af) {
      const uint32_t slot = rb + (uint32_t)(t ^ (j & 7));
#pragma unroll
      for (int mb = 0; mb < BIG_MB; ++mb)
        af[mb] = __builtin_bit_cast(half8, cur[mb * 512 + slot]);
    };
    auto make_b = [&](int t, half8 *bf) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if constexpr (BITS == 4) {
          unpack_f16_chunk<4>(bc[nb][t], cz[nb], s2[nb], bf[nb]);
        } else {
          const uint32_t wv = bc[nb][t >> 1];
          const uint32_t tc = __builtin_amdgcn_perm(wv, wv, (t & 1) ? 0x03030202u : 0x01010000u);
          unpack_f16_chunk<2>(tc, cz[nb], s2[nb], bf[nb]);
        }
      }
    };
    half8 af[2][BIG_MB], bf[2][2];
    read_a(0, af[0]);
    make_b(0, bf[0]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int c = t & 1, n = c ^ 1;
      // the next tile's x arrives a few loads per sub-step: issued in one
      // burst after the barrier, the four waves' loads queued in the
      // address unit for ~1 us while no MFMA ran
      if (t < 4) dma_a(kn, nxt, DMA_PER_SUB * t, DMA_PER_SUB);
      if (t + 1 < 8) {
        read_a(t + 1, af[n]);
        make_b(t + 1, bf[n]);
      }
#pragma unroll
      for (int mb = 0; mb < BIG_MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][mb], bf[c][nb], acc[mb][nb], 0, 0, 0);
      // one wave per SIMD: the next sub-step's operand reads and unpacking
      // must issue while this sub-step's MFMAs execute, so interleave them
      // (MFMA, 2 VALU, 1 LDS read, MFMA, ...)
#pragma unroll
      for (int i = 0; i < 2 * BIG_MB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
        if (t < 4 && i < DMA_PER_SUB) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // x load
        if (t + 1 < 8) {
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);          // VALU
          if (i < BIG_MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next tile's DMA has landed in every wave's part once all waves
    // pass this barrier
    lds_barrier();
  };

  uint32_t b0[2][BW], b1[2][BW], s0[2], s1[2], z0[2], z1[2];
  dma_a(g.kt0, As0, 0, BIG_DMA);
  load_b(g.kt0, b0, s0, z0);
  lds_barrier();
  // kt1 - kt0 is even: x is zero-padded to a multiple of 256 in k, and steps
  // past K get scale 0
  for (int kt = g.kt0; kt < g.kt1; kt += 2) {
    step(kt, As0, As1, b0, s0, z0, b1, s1, z1);
    step(kt + 1, As1, As0, b1, s1, z1, b0, s0, z0);
  }

  if (g.tail) {
    // part of a split tail tile: the fp32 accumulators in register order
    // (wave, mb, nb, e, lane), 256 contiguous bytes per store; the tail
    // reduction sums the parts and writes y
#pragma unroll
    for (int mb = 0; mb < BIG_MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          g.tail[(((wave * BIG_MB + mb) * 2 + nb) * 16 + e) * 64 + (threadIdx.x & 63)] = acc[mb][nb][e];
    return;
  }
  if (!wave_active) return;
  // epilogue: lane (j, h) holds column ncol0 + 32nb + j and rows
  // 8(e/4) + 4h + e%4 of each 32-row block
#pragma unroll
  for (int mb = 0; mb < BIG_MB; ++mb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = g.m0 + mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (m >= g.M) continue;
      const int ex = g.rexp[m];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int n = ncol0 + 32 * nb + j;
        if (n >= g.N) continue;
        const float v = ldexpf(acc[mb][nb][e], ex);
        g.y[(int64_t)m * g.N + n] = g.out_fp16 ? f32_to_f16_bits(v) : f32_to_bf16_rne(v);
      }
    }
  }
}

// Tail split.  With one 256 x 256 tile per CU at a time, a tile count that
// is not a multiple of the CU count leaves the last round partly idle.  The
// last `rem` tiles (rem = tiles mod CUs) are therefore cut along K into
// `parts` pieces of whole step pairs, run as rem * parts workgroups of the
// last round, and summed in part order by gemm_tail_reduce_kernel.
constexpr int kBigCUs = 256;
constexpr int BIG_TILE_ELEMS = BIG_TM * BIG_TN;

struct TailPlan {
  int tiles, full, rem, parts, per;   // per: k steps per part (even)
  size_t bytes;                       // fp32 partial tiles
};

inline TailPlan tail_plan(int tiles, int nkt) {
  TailPlan t;
  t.tiles = tiles;
  t.rem = tiles % kBigCUs;
  t.parts = t.rem ? kBigCUs / t.rem : 1;
  if (t.parts > 4) t.parts = 4;
  // a part keeps at least 8 step pairs; a tail that fills most of a round
  // is left whole
  while (t.parts > 1 && nkt / t.parts < 16) --t.parts;
  if (t.rem == 0 || t.parts < 2) {
    t.rem = 0;
    t.parts = 1;
  }
  t.full = tiles - t.rem;
  t.per = ((nkt + t.parts - 1) / t.parts + 1) & ~1;
  t.bytes = (size_t)t.rem * t.parts * BIG_TILE_ELEMS * 4u;
  return t;
}

// One thread per 4 consecutive lanes of a register-order row: 16-byte
// loads of each part, 4 consecutive output columns of one output row.
__global__ __launch_bounds__(256) void gemm_tail_reduce_kernel(const float *__restrict__ tail, int parts,
                                                               int full, int m_tiles, int M, int N,
                                                               const int *__restrict__ rexp,
                                                               uint16_t *__restrict__ y, int out_fp16) {
  const int t = (int)blockIdx.y;                                // tail tile index
  const int q = 4 * ((int)blockIdx.x * 256 + (int)threadIdx.x);  // first element, register order
  if (q >= BIG_TILE_ELEMS) return;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = 0; p < parts; ++p) {
    const float4 u = *reinterpret_cast<const float4 *>(tail + ((size_t)t * parts + p) * BIG_TILE_ELEMS + q);
    v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
  }
  const int lane = q & 63, e = (q >> 6) & 15, nb = (q >> 10) & 1, mb = (q >> 11) & (BIG_MB - 1);
  const int wave = q >> 14;
  const int tile = full + t;
  const int m = (tile % m_tiles) * BIG_TM + mb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
  const int n = (tile / m_tiles) * BIG_TN + wave * 64 + 32 * nb + (lane & 31);
  if (m >= M) return;
  const int ex = rexp[m];
  const float r[4] = {v.x, v.y, v.z, v.w};
  uint16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float w = ldexpf(r[i], ex);
    o[i] = out_fp16 ? f32_to_f16_bits(w) : f32_to_bf16_rne(w);
  }
  uint16_t *dst = y + (int64_t)m * N + n;
  if (n + 3 < N && ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0)) {
    *reinterpret_cast<uint2 *>(dst) = make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                  (uint32_t)o[2] | ((uint32_t)o[3] << 16));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n + i < N) dst[i] = o[i];
  }
}

__global__ __launch_bounds__(64 * BIG_NW, 1) void gemm_big_kernel(
    LayoutDev L, int M, int Kp, uint32_t xa_bytes, int m_tiles, const uint16_t *__restrict__ xa,
    const int *__restrict__ rexp, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros,
    uint16_t *__restrict__ y, int out_fp16, int tail_full, int tail_parts, int tail_per,
    float *__restrict__ tail) {
  __shared__ __attribute__((aligned(16))) uint4 As0[BIG_TILE_BYTES / 16];
  __shared__ __attribute__((aligned(16))) uint4 As1[BIG_TILE_BYTES / 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane & 31;
  const int h = lane >> 5;
  // tile order: m fastest, so the workgroups on one XCD (every 8th id)
  // share one m tile of x in that XCD's L2
  // workgroups past tail_full are parts of the split tail tiles
  const int id = (int)blockIdx.x;
  const int nkt = Kp / KT;
  const bool part = id >= tail_full;
  const int tile = part ? tail_full + (id - tail_full) / tail_parts : id;
  const int pidx = part ? (id - tail_full) % tail_parts : 0;
  const int m_tile = tile % m_tiles;
  const int n_tile = tile / m_tiles;
  BigArgs g;
  g.K = L.K; g.Kp = Kp; g.N = L.N; g.M = M;
  g.m0 = m_tile * BIG_TM;
  g.kt0 = part ? pidx * tail_per : 0;
  g.kt1 = part ? min(g.kt0 + tail_per, nkt) : nkt;
  g.tail = part ? tail + (size_t)(id - tail_full) * BIG_TILE_ELEMS : nullptr;
  g.rexp = rexp; g.y = y; g.out_fp16 = out_fp16;
  const int ncol0 = n_tile * BIG_TN + wave * 64;
  const bool wave_active = ncol0 < L.N;
  // waves past N read column 0's block through empty offsets and never store
  const int nref = wave_active ? ncol0 : 0;
  const int blk = nref / L.block_n;
  const BlockInfo bi = block_info(L, blk);
  const int bits = __builtin_amdgcn_readfirstlane(bi.bits);
  const uint32_t RB = (uint32_t)(L.K * bits / 8);
  const uint32_t GPR = (uint32_t)(bits == 4 ? L.K / 128 : L.K / 64);
  const Rsrc xr = make_rsrc(xa, xa_bytes);
  const Rsrc cr = make_rsrc(codes + bi.code_off, (uint32_t)L.block_n * RB);
  const Rsrc sr = make_rsrc(scales + bi.grp_off, (uint32_t)L.block_n * GPR * 2u);
  const Rsrc zr = make_rsrc(zeros + bi.grp_off, (uint32_t)L.block_n * GPR);
  uint32_t cbase[2], sbase[2], zbase[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = nref + 32 * nb + j;
    const bool valid = wave_active && n < L.N;
    const uint32_t r = (uint32_t)(n - blk * L.block_n);
    if (bits == 4) {
      cbase[nb] = valid ? r * RB + 32u * h : kOob;
      sbase[nb] = valid ? r * GPR * 2u : kOob;
      zbase[nb] = valid ? r * GPR : kOob;
    } else {
      cbase[nb] = valid ? r * RB + 16u * h : kOob;
      sbase[nb] = valid ? (r * GPR + h) * 2u : kOob;
      zbase[nb] = valid ? r * GPR + h : kOob;
    }
  }
  if (bits == 4)
    big_wave<4>(g, As0, As1, xr, cr, sr, zr, cbase, sbase, zbase, wave_active, wave, ncol0);
  else
    big_wave<2>(g, As0, As1, xr, cr, sr, zr, cbase, sbase, zbase, wave_active, wave, ncol0);
}

// Sum the split-K partials in split order, rescale by 2^e (rexp may be
// null: no rescale), round.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int splits,
                                                            int M, int N, const int *__restrict__ rexp,
                                                            uint16_t *__restrict__ y, int out_fp16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += part[(int64_t)k * total + i];
  const int m = (int)(i / N);
  const float v = rexp ? ldexpf(s, rexp[m]) : s;
  y[i] = out_fp16 ? f32_to_f16_bits(v) : f32_to_bf16_rne(v);
}

template <int MB, int NW>
hipError_t launch_tiles(const LayoutDev &L, int M, int Kp, int splits, const uint16_t *xa, const int *rexp,
                        const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                        void *y, float *part, int out_fp16, hipStream_t s) {
  const int m_tiles = (M + 32 * MB - 1) / (32 * MB);
  const int n_tiles = (L.N + 64 * NW - 1) / (64 * NW);
  const int ksteps = (L.K + KT - 1) / KT;
  const int per = (ksteps + splits - 1) / splits;
  const int nsplit = (ksteps + per - 1) / per;
  const uint8_t *c = reinterpret_cast<const uint8_t *>(codes);
  uint16_t *yp = reinterpret_cast<uint16_t *>(y);
  if (nsplit == 1) {
    hipLaunchKernelGGL((gemm_kernel<MB, NW, false>), dim3(m_tiles * n_tiles, 1), dim3(64 * NW), 0, s, L,
                       M, Kp, m_tiles, n_tiles, per, xa, rexp, c, scales, zeros, yp, part, out_fp16);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_kernel<MB, NW, true>), dim3(m_tiles * n_tiles, nsplit), dim3(64 * NW), 0, s,
                     L, M, Kp, m_tiles, n_tiles, per, xa, rexp, c, scales, zeros, yp, part, out_fp16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)M * L.N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     part, nsplit, M, L.N, rexp, yp, out_fp16);
  return hipGetLastError();
}

// Split-K factor: enough workgroups to cover the CUs twice when the tile
// grid alone is small; the K range of a split stays >= 4 steps.
inline int choose_splits(const LayoutDev &L, int M, int mb) {
  const int m_tiles = (M + 32 * mb - 1) / (32 * mb);
  const int nt = mb == 4 ? 512 : 256;
  const int n_tiles = (L.N + nt - 1) / nt;
  const int tiles = m_tiles * n_tiles;
  const int ksteps = (L.K + KT - 1) / KT;
  int sp = 1;
  while (tiles * sp < 512 && ksteps / (sp * 2) >= 4 && sp < 16) sp *= 2;
  return sp;
}

}  // namespace

namespace {

// Workspace layout: fp16 activations [Mp][Kp] (zero padded to whole
// 256-row tiles and pairs of 128-k steps), row exponents [M], split-K
// partials [S][M][N] (tiled kernel) or the fp32 parts of the split tail
// tiles (256 x 256 kernel).
struct Workspace {
  int Mp, Kp;
  size_t a_bytes, e_bytes, p_bytes;
};

inline size_t round256(size_t v) { return (v + 255u) & ~(size_t)255u; }

// The 256 x 256 kernel needs M >= 256, enough tiles to fill the chip and
// 32-bit buffer offsets (x and each Channel-mix block below 2 GiB).
inline bool use_big(const LayoutDev &L, int M, const Workspace &w) {
  if (M < BIG_TM) return false;
  const int64_t tiles = (int64_t)((M + BIG_TM - 1) / BIG_TM) * ((L.N + BIG_TN - 1) / BIG_TN);
  if (tiles < 128) return false;
  if (w.a_bytes >= ((size_t)1 << 31)) return false;
  if ((uint64_t)L.block_n * (uint64_t)L.K / 2u >= ((uint64_t)1 << 31)) return false;
  return true;
}

inline Workspace workspace_of(const LayoutDev &L, int M) {
  Workspace w;
  w.Kp = (L.K + 2 * KT - 1) / (2 * KT) * (2 * KT);   // whole pairs of k steps
  w.Mp = (M + BIG_TM - 1) / BIG_TM * BIG_TM;
  w.a_bytes = round256((size_t)w.Mp * (size_t)w.Kp * 2u);
  w.e_bytes = round256((size_t)M * 4u);
  w.p_bytes = 0;
  if (!use_big(L, M, w)) {
    const int sp = choose_splits(L, M, gemm_mb(M));
    if (sp > 1) w.p_bytes = (size_t)sp * (size_t)M * (size_t)L.N * 4u;
  } else {
    const int tiles = (w.Mp / BIG_TM) * ((L.N + BIG_TN - 1) / BIG_TN);
    w.p_bytes = tail_plan(tiles, w.Kp / KT).bytes;
  }
  return w;
}

}  // namespace

hipError_t launch_tile_tail_reduce(const float *tail, int parts, int full, int rem, int m_tiles, int M,
                                   int N, const int *rexp, uint16_t *y, int out_fp16, hipStream_t s) {
  hipLaunchKernelGGL(gemm_tail_reduce_kernel, dim3(BIG_TILE_ELEMS / 1024, rem), dim3(256), 0, s, tail, parts,
                     full, m_tiles, M, N, rexp, y, out_fp16);
  return hipGetLastError();
}

hipError_t launch_prep_rows(const void *x, int M, int K, int Mp, int Kp, gq_dtype act, uint16_t *xa,
                            int *rexp, hipStream_t s) {
  const uint16_t *xin = reinterpret_cast<const uint16_t *>(x);
  if (act == GQ_BF16)
    hipLaunchKernelGGL((prep_x_kernel<0, false>), dim3(Mp), dim3(256), 0, s, xin, M, K, Kp, xa, rexp);
  else
    hipLaunchKernelGGL((prep_x_kernel<1, false>), dim3(Mp), dim3(256), 0, s, xin, M, K, Kp, xa, rexp);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *part, int splits, int M, int N, const int *rexp,
                                uint16_t *y, int out_fp16, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     part, splits, M, N, rexp, y, out_fp16);
  return hipGetLastError();
}

hipError_t launch_gemm(const LayoutDev &L, int M, gq_dtype act, const void *x,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       void *y, void *workspace, hipStream_t s) {
  const Workspace w = workspace_of(L, M);
  uint16_t *xa = reinterpret_cast<uint16_t *>(workspace);
  int *rexp = reinterpret_cast<int *>(reinterpret_cast<char *>(workspace) + w.a_bytes);
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + w.a_bytes + w.e_bytes);
  const uint16_t *xin = reinterpret_cast<const uint16_t *>(x);
  if (act == GQ_BF16)
    hipLaunchKernelGGL((prep_x_kernel<0, true>), dim3(w.Mp), dim3(256), 0, s, xin, M, L.K, w.Kp, xa, rexp);
  else
    hipLaunchKernelGGL((prep_x_kernel<1, true>), dim3(w.Mp), dim3(256), 0, s, xin, M, L.K, w.Kp, xa, rexp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int out_fp16 = act == GQ_FP16 ? 1 : 0;
  if (use_big(L, M, w)) {
    const int m_tiles = w.Mp / BIG_TM;
    const int n_tiles = (L.N + BIG_TN - 1) / BIG_TN;
    const TailPlan t = tail_plan(m_tiles * n_tiles, w.Kp / KT);
    uint16_t *yp = reinterpret_cast<uint16_t *>(y);
    hipLaunchKernelGGL(gemm_big_kernel, dim3(t.full + t.rem * t.parts), dim3(64 * BIG_NW), 0, s, L, M,
                       w.Kp, (uint32_t)w.a_bytes, m_tiles, xa, rexp,
                       reinterpret_cast<const uint8_t *>(codes), scales, zeros, yp, out_fp16, t.full,
                       t.parts, t.per, part);
    err = hipGetLastError();
    if (err != hipSuccess || t.rem == 0) return err;
    hipLaunchKernelGGL(gemm_tail_reduce_kernel, dim3(BIG_TILE_ELEMS / 1024, t.rem), dim3(256), 0, s, part,
                       t.parts, t.full, m_tiles, M, L.N, rexp, yp, out_fp16);
    return hipGetLastError();
  }
  const int mb = gemm_mb(M);
  const int sp = choose_splits(L, M, mb);
  if (mb == 1) return launch_tiles<1, 4>(L, M, w.Kp, sp, xa, rexp, codes, scales, zeros, y, part, out_fp16, s);
  if (mb == 2) return launch_tiles<2, 4>(L, M, w.Kp, sp, xa, rexp, codes, scales, zeros, y, part, out_fp16, s);
  return launch_tiles<4, 8>(L, M, w.Kp, sp, xa, rexp, codes, scales, zeros, y, part, out_fp16, s);
}

size_t gemm_workspace_bytes(const LayoutDev &L, int M) {
  const Workspace w = workspace_of(L, M);
  return w.a_bytes + w.e_bytes + w.p_bytes;
}

}  // namespace gq
