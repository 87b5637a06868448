// Small-batch matmul (4 < M <= 32): y = x . W_hat^T on the MFMA units,
// for the decode and short-prefill batches between the dot-product kernel
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
// output channels.  Lane l holds channel l % 16 and the k chunk (8 k) of lane
// group g = l / 16.  Every MFMA stays inside one quantization group:
//   INT4 (one group per 128-k step): MFMA i takes chunk 4g + i, so a lane's
//        16 code bytes of the step are contiguous;
//   INT2 (two groups per step): MFMAs 0, 1 take chunks 2g + i of the first
//        group and MFMAs 2, 3 chunks 8 + 2g + (i - 2) of the second; a lane
//        reads two 4-byte pieces.
// Code pairs come out of a word as elements (t, t + 4) of a chunk, so the x
// fragments are staged in LDS in the chunk order (0,4,1,5,2,6,3,7).
//
// Work split: a workgroup of 4 waves owns 64 output channels (16 per wave)
// and SK_S consecutive k steps.  It issues every load of its work at once --
// x for all its steps (staged through LDS in the order above) and its codes,
// scales and zeros straight into registers -- so a workgroup pays one memory
// round trip, and the many workgroups of the grid keep HBM busy.  When K has
// more than SK_S steps, each workgroup writes an fp32 partial tile to the
// workspace and the split-K reduction sums them in split order.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int SK_WAVES = 4;
constexpr int SK_COLS = 16 * SK_WAVES;         // output channels per workgroup
constexpr int SK_STEP = 128;                    // k per step
constexpr int SK_S = 8;                         // k steps per workgroup
constexpr uint32_t SK_OOB = 0x80000000u;

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

// (x[a], x[a + 4]) pairs of an 8-element chunk held as 4 words of pairs
__device__ __forceinline__ uint4 chunk_order(uint4 v) {
  uint4 o;
  o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return o;
}

// (g, i) of the lane group and MFMA that take k chunk c of a step
template <int BITS>
__device__ __forceinline__ void sk_chunk_owner(int c, int &g, int &i) {
  if constexpr (BITS == 4) {
    g = c >> 2;
    i = c & 3;
  } else {
    g = (c & 7) >> 1;
    i = (c >> 3) * 2 + (c & 1);
  }
}

struct SkArgs {
  int M, K, N, nsteps, st0;
  int n0;                  // first output channel of the workgroup
  int rw0;                 // block row of the workgroup's first channel
  int nvalid;              // channels of the workgroup below N
  int nsplit;
  uint16_t *y;
  float *part;             // [nsplit][M][N] fp32
};

constexpr int SK_CSTRIDE = SK_S * 8 + 4;   // INT2 code words per staged channel (padded)

template <int ACT, int MB, int BITS>
__device__ __forceinline__ void skinny_tile(const SkArgs &a, Rsrc xr, uint32_t xbytes, Rsrc cr,
                                            Rsrc sr, Rsrc zr, uint32_t RB, uint32_t GPR,
                                            uint4 *xbuf, uint16_t *sbuf, uint8_t *zbuf,
                                            uint32_t *cbuf) {
  constexpr int XS = SK_S / MB;                                  // steps per x phase
  constexpr int XPT = 16 * MB * XS * 16 / (64 * SK_WAVES);       // 16-byte x units per thread
  constexpr int GPS = BITS == 4 ? 1 : 2;                         // groups per step
  constexpr int NG = SK_S * GPS;                                 // groups per channel
  constexpr int GPT = 64 * NG / (64 * SK_WAVES);                 // scales per thread
  constexpr uint32_t BIAS = ACT == 0 ? 0x43004300u : 0x64006400u;   // 128.0 / 1024.0 pairs
  constexpr uint32_t ONES = ACT == 0 ? 0x3f803f80u : 0x3c003c00u;
  constexpr float BIASF = ACT == 0 ? 128.f : 1024.f;
  constexpr uint32_t STEPB = SK_STEP * BITS / 8;    // code bytes per channel per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int ch = 16 * wave + (lane & 15);            // the lane's channel in the tile
  const bool ch_ok = ch < a.nvalid;

  // ---- x, read along k (1 KB per wave load), XS steps per phase: unit u ->
  // row u / (16 XS), chunk c of step st; staged at slot
  // ((st * 4 + i) * MB + mb) * 64 + l of the MFMA operand that uses it, in
  // pair order
  uint4 xs[XPT];
  auto load_x = [&](int ph) {
#pragma unroll
    for (int p = 0; p < XPT; ++p) {
      const int u = tid + p * 64 * SK_WAVES;
      const int row = u / (16 * XS);
      const int cc = u % (16 * XS);
      const int k = (a.st0 + ph * XS + (cc >> 4)) * SK_STEP + 8 * (cc & 15);
      // rows past M and k past K read out of range: zeros
      const uint32_t off = (row < a.M && k < a.K)
                               ? ((uint32_t)row * (uint32_t)a.K + (uint32_t)k) * 2u : xbytes;
      xs[p] = ld128(xr, off);
    }
  };
  auto store_x = [&]() {
#pragma unroll
    for (int p = 0; p < XPT; ++p) {
      const int u = tid + p * 64 * SK_WAVES;
      const int row = u / (16 * XS);
      const int cc = u % (16 * XS);
      int gg, ii;
      sk_chunk_owner<BITS>(cc & 15, gg, ii);
      const int slot = (((cc >> 4) * 4 + ii) * MB + (row >> 4)) * 64 + 16 * gg + (row & 15);
      xbuf[slot] = chunk_order(xs[p]);
    }
  };
  load_x(0);
  // ---- scales and zeros of the tile's channels, read along each channel
  uint32_t sv[GPT], zv[GPT];
#pragma unroll
  for (int p = 0; p < GPT; ++p) {
    const int u = tid + p * 64 * SK_WAVES;
    const int c = u / NG, j = u % NG;
    const uint32_t gi = c < a.nvalid ? (uint32_t)(a.rw0 + c) * GPR + (uint32_t)(a.st0 * GPS + j)
                                     : SK_OOB / 4u;
    sv[p] = ld16(sr, 2u * gi);
    zv[p] = ld8(zr, gi);
  }
  // ---- codes: INT2 staged through LDS (each channel's 256 bytes read
  // contiguously); INT4 straight to registers (64 bytes per channel and step)
  uint32_t c4[BITS == 4 ? SK_S * 4 : 1];
  uint4 c2[BITS == 2 ? 4 : 1];
  if constexpr (BITS == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int u = tid + p * 64 * SK_WAVES;
      const int c = u >> 4, q = u & 15;
      const uint32_t off = c < a.nvalid ? (uint32_t)(a.rw0 + c) * RB + (uint32_t)a.st0 * STEPB + 16u * q
                                        : SK_OOB;
      c2[p] = ld128(cr, off);
    }
  } else {
    const uint32_t cb = ch_ok ? (uint32_t)(a.rw0 + ch) * RB + 16u * g : SK_OOB;
#pragma unroll
    for (int st = 0; st < SK_S; ++st) {
      const bool live = a.st0 + st < a.nsteps;
      const uint4 v = ld128(cr, live ? cb + (uint32_t)(a.st0 + st) * STEPB : SK_OOB);
      c4[4 * st + 0] = v.x; c4[4 * st + 1] = v.y; c4[4 * st + 2] = v.z; c4[4 * st + 3] = v.w;
    }
  }
  // ---- to LDS (each wait covers only loads issued before the data it needs)
  store_x();
#pragma unroll
  for (int p = 0; p < GPT; ++p) {
    const int u = tid + p * 64 * SK_WAVES;
    sbuf[u] = (uint16_t)sv[p];
    zbuf[u] = (uint8_t)zv[p];
  }
  if constexpr (BITS == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int u = tid + p * 64 * SK_WAVES;
      const int c = u >> 4, q = u & 15;
      uint32_t *d = cbuf + c * SK_CSTRIDE + 4 * q;
      d[0] = c2[p].x; d[1] = c2[p].y; d[2] = c2[p].z; d[3] = c2[p].w;
    }
  }
  lds_barrier();
  if constexpr (XS < SK_S) load_x(1);     // second x phase, into the free registers

  floatx4 yacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) yacc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint4 ones = make_uint4(ONES, ONES, ONES, ONES);

#pragma unroll
  for (int st = 0; st < SK_S; ++st) {
    if constexpr (XS < SK_S) {
      static_assert(SK_S == 2 * XS, "two x phases");
      if (st == XS) {
        // second x phase: its loads were issued before the first computed
        lds_barrier();
        store_x();
        lds_barrier();
      }
    }
    const int step = a.st0 + st;
    if (step >= a.nsteps) break;                     // uniform
    uint32_t w2[2];
    if constexpr (BITS == 2) {
      w2[0] = cbuf[ch * SK_CSTRIDE + st * 8 + g];
      w2[1] = cbuf[ch * SK_CSTRIDE + st * 8 + 4 + g];
    }
    floatx4 gacc[MB], gsum[MB];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // B fragment of MFMA i: four pairs (B + q_t, B + q_{t+4})
      uint32_t wv;
      if constexpr (BITS == 4) {
        wv = c4[4 * st + i];
      } else {
        const uint32_t w = w2[i >> 1];
        wv = __builtin_amdgcn_perm(w, w, (i & 1) ? 0x03030202u : 0x01010000u);
      }
      constexpr uint32_t MASK = BITS == 4 ? 0x000f000fu : 0x00030003u;
      uint4 b;
      b.x = and_or(wv, MASK, BIAS);
      b.y = and_or(wv >> BITS, MASK, BIAS);
      b.z = and_or(wv >> (2 * BITS), MASK, BIAS);
      b.w = and_or(wv >> (3 * BITS), MASK, BIAS);
      const bool first = BITS == 4 ? i == 0 : (i & 1) == 0;   // first MFMA of a group
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4 av = xbuf[(((st % XS) * 4 + i) * MB + mb) * 64 + lane];
        gacc[mb] = mfma16<ACT>(av, b, first ? zero4 : gacc[mb]);
        gsum[mb] = mfma16<ACT>(av, ones, first ? zero4 : gsum[mb]);
      }
      const bool last = BITS == 4 ? i == 3 : (i & 1) == 1;
      if (last) {
        const int gi = BITS == 4 ? 0 : (i >> 1);
        // a group past K (the half step of INT2 rows with K % 128 == 64)
        // gets scale 0; its x columns are zero
        const bool kok = step * SK_STEP + gi * 64 < a.K;
        const int j = ch * NG + st * GPS + gi;
        const float S = kok ? f16_bits_to_f32(sbuf[j]) : 0.f;
        const float c = -(BIASF + (float)zbuf[j]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            yacc[mb][e] = fmaf(S, fmaf(c, gsum[mb][e], gacc[mb][e]), yacc[mb][e]);
      }
    }
  }

  // ---- results: lane l holds channel ch, rows 16 mb + 4 g + e
  if (!ch_ok) return;
  const int ncol = a.n0 + ch;
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
// of either width (the 64 channels of a workgroup lie in one block).
template <int ACT, int MB, int BITSEL>
__global__ __launch_bounds__(64 * SK_WAVES) void skinny_kernel(LayoutDev L, int M,
                                                              const uint16_t *__restrict__ x,
                                                              const uint8_t *__restrict__ codes,
                                                              const uint16_t *__restrict__ scales,
                                                              const uint8_t *__restrict__ zeros,
                                                              uint16_t *__restrict__ y,
                                                              float *__restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint4 xbuf[SK_S * 4 * 64];   // one x phase
  __shared__ __attribute__((aligned(16))) uint16_t sbuf[64 * SK_S * 2];
  __shared__ __attribute__((aligned(16))) uint8_t zbuf[64 * SK_S * 2];
  __shared__ __attribute__((aligned(16))) uint32_t cbuf[BITSEL == 4 ? 4 : 64 * SK_CSTRIDE];
  SkArgs a;
  a.M = M; a.K = L.K; a.N = L.N;
  a.nsteps = (L.K + SK_STEP - 1) / SK_STEP;
  a.nsplit = (int)gridDim.y;
  a.st0 = (int)blockIdx.y * SK_S;
  const int n0 = (int)blockIdx.x * SK_COLS;       // one Channel-mix block per workgroup
  a.nvalid = L.N - n0 < SK_COLS ? L.N - n0 : SK_COLS;
  a.n0 = n0;
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
  const uint32_t xbytes = (uint32_t)M * (uint32_t)L.K * 2u;
  const Rsrc xr = make_rsrc(x, xbytes);
  const Rsrc cr = make_rsrc(codes + bi.code_off, (uint32_t)L.block_n * RB);
  const Rsrc sr = make_rsrc(scales + bi.grp_off, (uint32_t)L.block_n * GPR * 2u);
  const Rsrc zr = make_rsrc(zeros + bi.grp_off, (uint32_t)L.block_n * GPR);
  if (BITSEL != 2 && bits == 4)
    skinny_tile<ACT, MB, 4>(a, xr, xbytes, cr, sr, zr, RB, GPR, xbuf, sbuf, zbuf, cbuf);
  else if constexpr (BITSEL != 4)
    skinny_tile<ACT, MB, 2>(a, xr, xbytes, cr, sr, zr, RB, GPR, xbuf, sbuf, zbuf, cbuf);
}

struct SkPlan {
  int tiles, nsplit;
  size_t part_bytes;
};

// Workspace: fp32 partials [nsplit][M][N] when K has more than SK_S steps.
inline SkPlan skinny_plan(const LayoutDev &L, int M) {
  SkPlan p;
  p.tiles = (L.N + SK_COLS - 1) / SK_COLS;
  const int nsteps = (L.K + SK_STEP - 1) / SK_STEP;
  p.nsplit = (nsteps + SK_S - 1) / SK_S;
  p.part_bytes = p.nsplit > 1 ? ((size_t)p.nsplit * (size_t)M * (size_t)L.N * 4u + 255u) & ~(size_t)255u
                              : 0u;
  return p;
}

template <int ACT, int MB>
hipError_t launch_mb(const LayoutDev &L, int M, const void *x, const uint32_t *codes,
                     const uint16_t *scales, const uint8_t *zeros, void *y, void *workspace,
                     hipStream_t s) {
  const SkPlan p = skinny_plan(L, M);
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
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, 4>), grid, block, 0, s, L, M, xp, cp, scales, zeros, yp, part);
  else if (!any4)
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, 2>), grid, block, 0, s, L, M, xp, cp, scales, zeros, yp, part);
  else
    hipLaunchKernelGGL((skinny_kernel<ACT, MB, 0>), grid, block, 0, s, L, M, xp, cp, scales, zeros, yp, part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  return launch_splitk_reduce(part, p.nsplit, M, L.N, nullptr, yp, ACT, s);
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
  if (act == GQ_BF16)
    return M <= 16 ? launch_mb<0, 1>(L, M, x, codes, scales, zeros, y, workspace, s)
                   : launch_mb<0, 2>(L, M, x, codes, scales, zeros, y, workspace, s);
  return M <= 16 ? launch_mb<1, 1>(L, M, x, codes, scales, zeros, y, workspace, s)
                 : launch_mb<1, 2>(L, M, x, codes, scales, zeros, y, workspace, s);
}

}  // namespace gq
