// Quantize + pack and dequantize kernels for gfx950.
//
// Quantizer: GreenBitAI's group-wise MinMax quantizer (two-stage
// quantization paragraph: round-to-nearest, INT4 with groups of 128, INT2
// with groups of 64) with the affine map of section 2.2 of
// "大模型量化实战：从原理到4-bit部署的完整指南": s = (x_max - x_min)/(2^b - 1),
// z = round(-x_min/s), Q(x) = round(x/s) + z.  The scale is stored as fp16
// (nearest even) and the zero point and codes are computed from the stored
// scale; z and the codes are clamped to [0, 2^b - 1].  A group whose zero
// point had to be clamped (all its values of one sign, away from 0) sets
// GQ_FLAG_ZERO_CLAMPED: its codes saturate at the clamp.
//
// Dequantizer: (q - z) * s, the "Zero Point" formula of "Low-bit
// Quantization: Slimming Large Models to the Extreme".
//
// Fake quantization (quantize, then dequantize, in one pass): the forward of
// quantization-aware training with FakeQuantize modules ("大模型量化实战",
// section 5.2: the forward quantizes and dequantizes, the gradient flows
// through in FP32).  Same groups, scale, zero point and codes as the packing
// quantizer; the output is (c - z) * s, exact in fp32, rounded to nearest
// even for bf16 / fp16.
#include "gq_internal.h"

namespace gq {
namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kSeg = 512;          // weights per wave-segment: 64 lanes x 8
constexpr int kLanes = 64;

// One wave quantizes the 512-weight segment [k0, k0 + 512) of row n.  Lane l
// holds weights k0 + 8l .. k0 + 8l + 7; a group of g weights spans g/8
// consecutive lanes, so the min/max reduction is a butterfly over g/8 lanes.
// MODE kPack writes codes, scale and zero point; the other modes write the
// fake-quantized weights of the lane to orow (0 bf16, 1 fp16, 2 fp32).
constexpr int kPack = -1;
template <int BITS, int MODE>
__device__ __forceinline__ void quant_segment(const float *__restrict__ wrow, int K, int kl,
                                              uint8_t *__restrict__ crow,
                                              uint16_t *__restrict__ srow,
                                              uint8_t *__restrict__ zrow, void *__restrict__ orow,
                                              uint32_t *flags) {
  constexpr int G = BITS == 4 ? 128 : 64;
  constexpr int LPG = G / 8;  // lanes per group
  const bool active = kl < K;
  float v[8];
  if (active) {
    const float4 a = *reinterpret_cast<const float4 *>(wrow + kl);
    const float4 b = *reinterpret_cast<const float4 *>(wrow + kl + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  float lo = v[0], hi = v[0];
  bool finite = __builtin_isfinite(v[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    lo = fminf(lo, v[i]);
    hi = fmaxf(hi, v[i]);
    finite = finite && __builtin_isfinite(v[i]);
  }
  int nonfinite = finite ? 0 : 1;
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
    nonfinite |= __shfl_xor(nonfinite, off);
  }
  finite = nonfinite == 0;   // whole group
  const float qm = (float)((1 << BITS) - 1);
  const float s32 = (hi - lo) / qm;          // correctly rounded fp32 divide
  _Float16 s16 = (_Float16)s32;              // nearest even
  if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
  const float S = (float)s16;
  const float zr = rintf(-lo / S);
  const float z = fminf(fmaxf(zr, 0.f), qm);
  const bool zclamp = zr < 0.f || zr > qm;   // a group of one sign, away from 0
  uint32_t packed = 0;
  float fq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = fminf(fmaxf(rintf(v[i] / S) + z, 0.f), qm);
    packed |= ((uint32_t)c) << (BITS * i);
    fq[i] = (c - z) * S;                     // exact: |c - z| <= 15, S has 11 bits
  }
  if (MODE != kPack) {
    if (active) {
      if (MODE == 2) {
        float *o = reinterpret_cast<float *>(orow) + kl;
        *reinterpret_cast<float4 *>(o) = make_float4(fq[0], fq[1], fq[2], fq[3]);
        *reinterpret_cast<float4 *>(o + 4) = make_float4(fq[4], fq[5], fq[6], fq[7]);
      } else {
        uint32_t h[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint16_t a = MODE == 0 ? f32_to_bf16_rne(fq[2 * p]) : f32_to_f16_bits(fq[2 * p]);
          const uint16_t b = MODE == 0 ? f32_to_bf16_rne(fq[2 * p + 1]) : f32_to_f16_bits(fq[2 * p + 1]);
          h[p] = (uint32_t)a | ((uint32_t)b << 16);
        }
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(orow) + kl) = make_uint4(h[0], h[1], h[2], h[3]);
      }
    }
    if (flags) {
      uint32_t f = finite ? 0u : GQ_FLAG_NONFINITE;
      if (finite && __builtin_isinf(S)) f |= GQ_FLAG_SCALE_OVERFLOW;
      else if (finite && zclamp) f |= GQ_FLAG_ZERO_CLAMPED;
      if (f && active) atomicOr(flags, f);
    }
    return;
  }
  if (!active) return;
  if (BITS == 4) {
    *reinterpret_cast<uint32_t *>(crow + (kl >> 1)) = packed;
  } else {
    *reinterpret_cast<uint16_t *>(crow + (kl >> 2)) = (uint16_t)packed;
  }
  const int lane = threadIdx.x & (kLanes - 1);
  if ((lane & (LPG - 1)) == 0) {
    const int gi = kl / G;
    srow[gi] = __builtin_bit_cast(uint16_t, s16);
    zrow[gi] = (uint8_t)z;
  }
  if (flags) {
    uint32_t f = finite ? 0u : GQ_FLAG_NONFINITE;
    if (finite && __builtin_isinf(S)) f |= GQ_FLAG_SCALE_OVERFLOW;
    else if (finite && zclamp) f |= GQ_FLAG_ZERO_CLAMPED;
    if (f) atomicOr(flags, f);
  }
}

template <int MODE>
__global__ __launch_bounds__(kWaves * kLanes) void quantize_pack_kernel(
    LayoutDev L, const float *__restrict__ w, uint8_t *__restrict__ codes,
    uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros, void *__restrict__ wout,
    uint32_t *flags, int segs_per_row) {
  const int wave = threadIdx.x / kLanes;
  const int lane = threadIdx.x & (kLanes - 1);
  const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t total = (int64_t)L.N * segs_per_row;
  if (gw >= total) return;
  const int n = (int)(gw / segs_per_row);
  const int seg = (int)(gw - (int64_t)n * segs_per_row);
  const int blk = n / L.block_n;
  const int r = n - blk * L.block_n;
  const BlockInfo bi = block_info(L, blk);
  const float *wrow = w + (int64_t)n * L.K;
  const int kl = seg * kSeg + lane * 8;
  void *orow = nullptr;
  if (MODE != kPack)
    orow = reinterpret_cast<uint8_t *>(wout) + (int64_t)n * L.K * (MODE == 2 ? 4 : 2);
  if (bi.bits == 4) {
    uint8_t *crow = MODE == kPack ? codes + bi.code_off + (uint64_t)r * (uint64_t)(L.K / 2) : nullptr;
    const uint64_t g0 = bi.grp_off + (uint64_t)r * (uint64_t)(L.K / 128);
    quant_segment<4, MODE>(wrow, L.K, kl, crow, MODE == kPack ? scales + g0 : nullptr,
                           MODE == kPack ? zeros + g0 : nullptr, orow, flags);
  } else {
    uint8_t *crow = MODE == kPack ? codes + bi.code_off + (uint64_t)r * (uint64_t)(L.K / 4) : nullptr;
    const uint64_t g0 = bi.grp_off + (uint64_t)r * (uint64_t)(L.K / 64);
    quant_segment<2, MODE>(wrow, L.K, kl, crow, MODE == kPack ? scales + g0 : nullptr,
                           MODE == kPack ? zeros + g0 : nullptr, orow, flags);
  }
}

// ------------------------------------------------------------ dequant

// One thread expands one packed uint32 word: 8 INT4 or 16 INT2 weights.
template <int OUT>  // 0 bf16, 1 fp16, 2 fp32
__global__ __launch_bounds__(256) void dequant_kernel(LayoutDev L, const uint8_t *__restrict__ codes,
                                                      const uint16_t *__restrict__ scales,
                                                      const uint8_t *__restrict__ zeros,
                                                      void *__restrict__ out, int chunks_per_row) {
  const int64_t row_chunk = blockIdx.x;
  const int n = (int)(row_chunk / chunks_per_row);
  const int chunk = (int)(row_chunk - (int64_t)n * chunks_per_row);
  if (n >= L.N) return;
  const int blk = n / L.block_n;
  const int r = n - blk * L.block_n;
  const BlockInfo bi = block_info(L, blk);
  const int bits = bi.bits;
  const int per = 32 / bits;                 // codes per word
  const int words = L.K / per;               // words per row
  const int j = chunk * 256 + (int)threadIdx.x;
  if (j >= words) return;
  const int g = bits == 4 ? 128 : 64;
  const uint32_t *crow =
      reinterpret_cast<const uint32_t *>(codes + bi.code_off + (uint64_t)r * (uint64_t)(L.K * bits / 8));
  const uint64_t g0 = bi.grp_off + (uint64_t)r * (uint64_t)(L.K / g);
  const uint32_t wd = crow[j];
  const int k0 = j * per;
  const int gi = k0 / g;                     // a word never straddles a group
  const float S = f16_bits_to_f32(scales[g0 + gi]);
  const float z = (float)zeros[g0 + gi];
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t obase = (int64_t)n * L.K + k0;
  if (OUT == 2) {
    float *o = reinterpret_cast<float *>(out) + obase;
    for (int i = 0; i < per; i += 4) {
      float4 q;
      q.x = ((float)((wd >> (bits * (i + 0))) & mask) - z) * S;
      q.y = ((float)((wd >> (bits * (i + 1))) & mask) - z) * S;
      q.z = ((float)((wd >> (bits * (i + 2))) & mask) - z) * S;
      q.w = ((float)((wd >> (bits * (i + 3))) & mask) - z) * S;
      *reinterpret_cast<float4 *>(o + i) = q;
    }
  } else {
    uint16_t *o = reinterpret_cast<uint16_t *>(out) + obase;
    for (int i = 0; i < per; i += 8) {
      uint32_t h[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = ((float)((wd >> (bits * (i + 2 * p))) & mask) - z) * S;
        const float b = ((float)((wd >> (bits * (i + 2 * p + 1))) & mask) - z) * S;
        const uint16_t ha = OUT == 0 ? f32_to_bf16_rne(a) : f32_to_f16_bits(a);
        const uint16_t hb = OUT == 0 ? f32_to_bf16_rne(b) : f32_to_f16_bits(b);
        h[p] = (uint32_t)ha | ((uint32_t)hb << 16);
      }
      *reinterpret_cast<uint4 *>(o + i) = make_uint4(h[0], h[1], h[2], h[3]);
    }
  }
}

}  // namespace

hipError_t launch_quantize_pack(const LayoutDev &L, const float *w, uint32_t *codes,
                                uint16_t *scales, uint8_t *zeros, uint32_t *flags,
                                hipStream_t s) {
  if (L.N == 0) return hipSuccess;
  const int segs = (L.K + kSeg - 1) / kSeg;
  const int64_t waves = (int64_t)L.N * segs;
  const int64_t blocks = (waves + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(quantize_pack_kernel<kPack>, dim3((unsigned)blocks), dim3(kWaves * kLanes), 0, s,
                     L, w, reinterpret_cast<uint8_t *>(codes), scales, zeros, nullptr, flags, segs);
  return hipGetLastError();
}

hipError_t launch_fake_quant(const LayoutDev &L, const float *w, gq_dtype out, void *w_out,
                             uint32_t *flags, hipStream_t s) {
  if (L.N == 0) return hipSuccess;
  const int segs = (L.K + kSeg - 1) / kSeg;
  const int64_t waves = (int64_t)L.N * segs;
  const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves)), block(kWaves * kLanes);
  switch (out) {
    case GQ_BF16:
      hipLaunchKernelGGL(quantize_pack_kernel<0>, grid, block, 0, s, L, w, nullptr, nullptr, nullptr, w_out, flags, segs);
      break;
    case GQ_FP16:
      hipLaunchKernelGGL(quantize_pack_kernel<1>, grid, block, 0, s, L, w, nullptr, nullptr, nullptr, w_out, flags, segs);
      break;
    default:
      hipLaunchKernelGGL(quantize_pack_kernel<2>, grid, block, 0, s, L, w, nullptr, nullptr, nullptr, w_out, flags, segs);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const LayoutDev &L, const uint32_t *codes, const uint16_t *scales,
                          const uint8_t *zeros, gq_dtype out, void *w_out, hipStream_t s) {
  if (L.N == 0) return hipSuccess;
  const int max_words = L.K / 8;  // INT4 rows have the most words
  const int chunks = (max_words + 255) / 256;
  const dim3 grid((unsigned)((int64_t)L.N * chunks));
  const uint8_t *c = reinterpret_cast<const uint8_t *>(codes);
  switch (out) {
    case GQ_BF16: hipLaunchKernelGGL(dequant_kernel<0>, grid, dim3(256), 0, s, L, c, scales, zeros, w_out, chunks); break;
    case GQ_FP16: hipLaunchKernelGGL(dequant_kernel<1>, grid, dim3(256), 0, s, L, c, scales, zeros, w_out, chunks); break;
    default: hipLaunchKernelGGL(dequant_kernel<2>, grid, dim3(256), 0, s, L, c, scales, zeros, w_out, chunks); break;
  }
  return hipGetLastError();
}

}  // namespace gq
