// Decode GEMV (M <= 4): y = x . W_hat^T with W_hat = (q - z) * s.
//
// Weight-only quantization moves b-bit codes instead of 16-bit weights and
// dequantizes on chip ("A Survey of Low-bit Large Language Models" review,
// section 6.2: dequantization cost must stay below the transfer time it
// saves).  This kernel is bound by HBM bandwidth: every packed byte is read
// once with a 128-bit load, unpacked in registers and never written back.
//
// Exactness: a code q (4 or 2 bits) ORed into the low mantissa bits of the
// constant 128.0 (bf16) or 1024.0 (fp16) is the exact value 128+q / 1024+q.
// A packed pair of such values feeds v_dot2 against the matching pair of
// activations, so the inner loop computes P = sum x*(B+q) in fp32.  Per group
// the zero point and scale are applied as s * (P - (B+z) * sum x), which is
// sum x*(q-z)*s with fp32 rounding only.
#include "gq_internal.h"

namespace gq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kLanes = 64;
constexpr int kWaves = 4;

template <int ACT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (ACT == 0)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
}

// Pair of activations (x[i], x[i + half]) for code pair i of a word, from
// registers holding consecutive activation pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t hi_reg, uint32_t lo_reg) {
  return __builtin_amdgcn_perm(hi_reg, lo_reg, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t hi_reg, uint32_t lo_reg) {
  return __builtin_amdgcn_perm(hi_reg, lo_reg, 0x07060302u);
}

template <int BITS, int ACT, int M, int R>
__device__ __forceinline__ void gemv_rows(const LayoutDev &L, const BlockInfo &bi, int blk, int n0,
                                          const uint16_t *__restrict__ x,
                                          const uint8_t *__restrict__ codes,
                                          const uint16_t *__restrict__ scales,
                                          const uint8_t *__restrict__ zeros,
                                          uint16_t *__restrict__ y) {
  constexpr int G = BITS == 4 ? 128 : 64;
  constexpr int KPL = 128 / BITS;            // weights per lane per 16-byte load
  constexpr int XR = KPL / 2;                // activation registers (pairs) per row of x
  constexpr uint32_t BIAS = ACT == 0 ? 0x43004300u : 0x64006400u;   // 128.0 / 1024.0
  constexpr uint32_t ONES = ACT == 0 ? 0x3f803f80u : 0x3c003c00u;   // 1.0, 1.0
  constexpr float BIASF = ACT == 0 ? 128.f : 1024.f;
  constexpr uint32_t MASK = BITS == 4 ? 0x000f000fu : 0x00030003u;
  const int lane = threadIdx.x & (kLanes - 1);
  const int K = L.K;
  const int RB = K * BITS / 8;               // bytes per packed row
  const int GPR = K / G;                     // groups per row
  const int r0 = n0 - blk * L.block_n;
  const uint8_t *crow[R];
  const uint16_t *srow[R];
  const uint8_t *zrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = (n0 + r < L.N) ? r0 + r : r0;     // ragged tail: recompute row 0
    crow[r] = codes + bi.code_off + (uint64_t)rr * (uint64_t)RB;
    srow[r] = scales + bi.grp_off + (uint64_t)rr * (uint64_t)GPR;
    zrow[r] = zeros + bi.grp_off + (uint64_t)rr * (uint64_t)GPR;
  }
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  for (int off = lane * 16; off < RB; off += kLanes * 16) {
    const int k0 = off * (8 / BITS);
    const int gi = k0 / G;
    uint4 cw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) cw[r] = *reinterpret_cast<const uint4 *>(crow[r] + off);
    uint32_t xr[M][XR];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4 *xp = reinterpret_cast<const uint4 *>(x + (int64_t)m * K + k0);
#pragma unroll
      for (int v = 0; v < XR / 4; ++v) {
        const uint4 t = xp[v];
        xr[m][4 * v + 0] = t.x; xr[m][4 * v + 1] = t.y;
        xr[m][4 * v + 2] = t.z; xr[m][4 * v + 3] = t.w;
      }
    }
    float sc[R], zb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sc[r] = f16_bits_to_f32(srow[r][gi]);
      zb[r] = BIASF + (float)zrow[r][gi];
    }
    // activation pairs in the order the code pairs come out of a word, and
    // the sum of the lane's activations per row of x.
    uint32_t xp[M][XR];
    float xs[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t *q = &xr[m][w * (XR / 4)];
        if constexpr (BITS == 4) {
          xp[m][4 * w + 0] = pair_lo(q[2], q[0]);
          xp[m][4 * w + 1] = pair_hi(q[2], q[0]);
          xp[m][4 * w + 2] = pair_lo(q[3], q[1]);
          xp[m][4 * w + 3] = pair_hi(q[3], q[1]);
        } else {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            xp[m][8 * w + 2 * a + 0] = pair_lo(q[a + 4], q[a]);
            xp[m][8 * w + 2 * a + 1] = pair_hi(q[a + 4], q[a]);
          }
        }
#pragma unroll
        for (int i = 0; i < XR / 4; ++i) s = dot2<ACT>(q[i], ONES, s);
      }
      xs[m] = s;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t wv[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
      float p[M];
#pragma unroll
      for (int m = 0; m < M; ++m) p[m] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int i = 0; i < 32 / BITS / 2; ++i) {
          const uint32_t qp = ((wv[w] >> (BITS * i)) & MASK) | BIAS;
#pragma unroll
          for (int m = 0; m < M; ++m) p[m] = dot2<ACT>(qp, xp[m][(32 / BITS / 2) * w + i], p[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = fmaf(sc[r], fmaf(-zb[r], xs[m], p[m]), acc[r][m]);
    }
  }
  // wave reduction, then lane 0 stores
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      acc[r][m] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (n0 + r >= L.N) break;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = acc[r][m];
        y[(int64_t)m * L.N + n0 + r] = ACT == 0 ? f32_to_bf16_rne(v) : f32_to_f16_bits(v);
      }
    }
  }
}

// BITSEL: 4 or 2 for a uniform (Layer-mix) linear, 0 for a Channel-mix
// layout where each wave reads its block's width from the bit mask.
template <int ACT, int M, int R, int BITSEL>
__global__ __launch_bounds__(kWaves * kLanes) void gemv_kernel(LayoutDev L,
                                                               const uint16_t *__restrict__ x,
                                                               const uint8_t *__restrict__ codes,
                                                               const uint16_t *__restrict__ scales,
                                                               const uint8_t *__restrict__ zeros,
                                                               uint16_t *__restrict__ y) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int n0 = ((int)blockIdx.x * kWaves + wave) * R;
  if (n0 >= L.N) return;
  if constexpr (BITSEL == 4) {
    BlockInfo bi = {4, 0, 0};
    gemv_rows<4, ACT, M, R>(L, bi, 0, n0, x, codes, scales, zeros, y);
  } else if constexpr (BITSEL == 2) {
    BlockInfo bi = {2, 0, 0};
    gemv_rows<2, ACT, M, R>(L, bi, 0, n0, x, codes, scales, zeros, y);
  } else {
    const int blk = n0 / L.block_n;
    const BlockInfo bi = block_info(L, blk);
    if (__builtin_amdgcn_readfirstlane(bi.bits) == 4)
      gemv_rows<4, ACT, M, R>(L, bi, blk, n0, x, codes, scales, zeros, y);
    else
      gemv_rows<2, ACT, M, R>(L, bi, blk, n0, x, codes, scales, zeros, y);
  }
}

template <int ACT, int M, int R>
hipError_t launch_rows(const LayoutDev &L, const void *x, const uint32_t *codes,
                       const uint16_t *scales, const uint8_t *zeros, void *y, hipStream_t s) {
  const int waves = (L.N + R - 1) / R;
  const int blocks = (waves + kWaves - 1) / kWaves;
  const uint16_t *xp = reinterpret_cast<const uint16_t *>(x);
  const uint8_t *cp = reinterpret_cast<const uint8_t *>(codes);
  uint16_t *yp = reinterpret_cast<uint16_t *>(y);
  // uniform layouts get a kernel specialised on the bit-width
  uint32_t any4 = 0, all4 = ~0u;
  for (int i = 0; i < L.nblocks; ++i) {
    const uint32_t b = (L.int4_mask[i >> 5] >> (i & 31)) & 1u;
    any4 |= b;
    all4 &= b;
  }
  if (all4)
    hipLaunchKernelGGL((gemv_kernel<ACT, M, R, 4>), dim3(blocks), dim3(kWaves * kLanes), 0, s, L, xp,
                       cp, scales, zeros, yp);
  else if (!any4)
    hipLaunchKernelGGL((gemv_kernel<ACT, M, R, 2>), dim3(blocks), dim3(kWaves * kLanes), 0, s, L, xp,
                       cp, scales, zeros, yp);
  else
    hipLaunchKernelGGL((gemv_kernel<ACT, M, R, 0>), dim3(blocks), dim3(kWaves * kLanes), 0, s, L, xp,
                       cp, scales, zeros, yp);
  return hipGetLastError();
}

template <int ACT, int M>
hipError_t launch_m(const LayoutDev &L, const void *x, const uint32_t *codes,
                    const uint16_t *scales, const uint8_t *zeros, void *y, hipStream_t s) {
  // Rows per wave: as many as keep >= 1024 waves in flight (4 per CU), so
  // each activation load is shared by several packed rows; fewer rows for
  // larger M to bound the accumulator registers.
  constexpr int RMAX = M <= 2 ? 8 : 4;
  if (RMAX >= 8 && (L.N + 7) / 8 >= 1024) return launch_rows<ACT, M, 8>(L, x, codes, scales, zeros, y, s);
  if ((L.N + 3) / 4 >= 1024) return launch_rows<ACT, M, 4>(L, x, codes, scales, zeros, y, s);
  if ((L.N + 1) / 2 >= 1024) return launch_rows<ACT, M, 2>(L, x, codes, scales, zeros, y, s);
  return launch_rows<ACT, M, 1>(L, x, codes, scales, zeros, y, s);
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
