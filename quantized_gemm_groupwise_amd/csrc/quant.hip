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
#include <mutex>

#include "gq_internal.h"

namespace gq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kSeg = 512;          // weights per wave-segment: 64 lanes x 8
constexpr int kLanes = 64;

// One wave quantizes the 512-weight segment [k0, k0 + 512) of row n.  Lane l
// holds weights k0 + 8l .. k0 + 8l + 7; a group of g weights spans g/8
// consecutive lanes, so the min/max reduction is a butterfly over g/8 lanes.
// MODE kPack writes codes, scale and zero point; the other modes write the
// fake-quantized weights of the lane to orow (0 bf16, 1 fp16, 2 fp32).
constexpr int kPack = -1;
// v: the lane's 8 weights (zeros for lanes past the row end, active false).
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

template <int BITS, int MODE>
__device__ __forceinline__ void quant_segment(const float (&v)[8], bool active, int kl,
                                              uint8_t *__restrict__ crow,
                                              uint16_t *__restrict__ srow,
                                              uint8_t *__restrict__ zrow, void *__restrict__ orow,
                                              uint32_t *flags) {
  constexpr int G = group_size(BITS);
  constexpr int LPG = G / 8;  // lanes per group: 16 (one DPP row) or 8 (half a row)
  const int lane = threadIdx.x & (kLanes - 1);
  // IEEE 754-2019 minimum / maximum (NaN-propagating, v_minimum3 /
  // v_maximum3): they need no operand canonicalization, and a group holding
  // NaN gets unspecified codes anyway (it is flagged below)
  auto mn = [](float a, float b) { return __builtin_elementwise_minimum(a, b); };
  auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  float lo = mn(mn(mn(v[0], v[1]), mn(v[2], v[3])), mn(mn(v[4], v[5]), mn(v[6], v[7])));
  float hi = mx(mx(mx(v[0], v[1]), mx(v[2], v[3])), mx(mx(v[4], v[5]), mx(v[6], v[7])));
  // butterfly inside the group's lanes: xor 1, xor 2 (quads), then the
  // mirrors that pair the quads of a half row and the halves of a row
  lo = mn(lo, dppf<0xb1>(lo));
  hi = mx(hi, dppf<0xb1>(hi));
  lo = mn(lo, dppf<0x4e>(lo));
  hi = mx(hi, dppf<0x4e>(hi));
  lo = mn(lo, dppf<0x141>(lo));             // row_half_mirror
  hi = mx(hi, dppf<0x141>(hi));
  if constexpr (LPG == 16) {
    lo = mn(lo, dppf<0x140>(lo));           // row_mirror
    hi = mx(hi, dppf<0x140>(hi));
  }
  // NaN or Inf anywhere in the group: minimum / maximum propagate NaN, and
  // an infinity is an extreme, so the group is finite exactly when its
  // reduced lo and hi are
  const bool finite = __builtin_isfinite(lo) && __builtin_isfinite(hi);
  const float qm = (float)((1 << BITS) - 1);
  const float s32 = (hi - lo) / qm;          // correctly rounded fp32 divide
  _Float16 s16 = (_Float16)s32;              // nearest even
  if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
  const float S = (float)s16;
  // round(x / S) with x / S the correctly rounded fp32 quotient, for -lo
  // (the zero point) and the 8 weights.  Only the integer a quotient rounds
  // to matters, so it is taken from x * (1/S) (relative error below 2^-22
  // against x / S) wherever that lies clear of the midpoints n + 1/2; a lane
  // with a quotient within the margin of a midpoint (ties among them)
  // divides exactly instead.
  const float rS = __builtin_amdgcn_rcpf(S);
  auto near_mid = [](float q, float n) {
    return fabsf(q - n) >= fmaf(-fabsf(q), 0x1p-20f, 0.5f - 0x1p-30f);
  };
  const float zq = -lo * rS;
  float zr = rintf(zq);
  bool exact = near_mid(zq, zr);
  float qn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = v[i] * rS;
    qn[i] = rintf(q);
    exact |= near_mid(q, qn[i]);
  }
  if (exact) {
    zr = rintf(-lo / S);
#pragma unroll
    for (int i = 0; i < 8; ++i) qn[i] = rintf(v[i] / S);
  }
  const float z = __builtin_amdgcn_fmed3f(zr, 0.f, qm);
  const bool zclamp = zr < 0.f || zr > qm;   // a group of one sign, away from 0
  // the lane's 8 codes, packed: 32 bits (INT4), 16 (INT2) or 64 (8-bit,
  // one byte per code: lo holds codes 0..3, hi codes 4..7)
  uint32_t packed = 0, packed_hi = 0;
  float fq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = __builtin_amdgcn_fmed3f(qn[i] + z, 0.f, qm);
    if (BITS == 8 && i >= 4) packed_hi |= ((uint32_t)c) << (8 * (i - 4));
    else packed |= ((uint32_t)c) << (BITS * i);
    fq[i] = (c - z) * S;                     // exact: |c - z| <= 255, S has 11 bits
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
  if (BITS == 8) {
    *reinterpret_cast<uint2 *>(crow + kl) = make_uint2(packed, packed_hi);
  } else if (BITS == 4) {
    *reinterpret_cast<uint32_t *>(crow + (kl >> 1)) = packed;
  } else {
    *reinterpret_cast<uint16_t *>(crow + (kl >> 2)) = (uint16_t)packed;
  }
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

// The layout's 512-weight segments, numbered row by row, are dealt to the
// grid's waves in turn: wave g takes segments g, g + W, g + 2W, ... (W the
// waves of the grid), so at any moment the waves read neighbouring segments
// of the matrix.  A wave loads the next two of its segments before it works
// on the current one, so it keeps three segments' reads in flight.  The
// grid holds as many waves as the chip keeps resident.  Positions advance by
// W segments with adds only (row, segment of the row, block, row in the
// block), no division per segment.
template <int MODE>
__global__ __launch_bounds__(kWaves * kLanes) void quantize_pack_kernel(
    LayoutDev L, const float *__restrict__ w, uint8_t *__restrict__ codes,
    uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros, void *__restrict__ wout,
    uint32_t *flags, int segs_per_row) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int lane = threadIdx.x & (kLanes - 1);
  const int nw = (int)gridDim.x * kWaves;
  const int gw = (int)blockIdx.x * kWaves + wave;
  const int spr = segs_per_row;
  if ((int64_t)gw >= (int64_t)L.N * spr) return;
  const int K = L.K;
  const int dq = nw / spr, dr = nw - dq * spr;   // a step of nw segments: dq rows and dr segments
  auto advance = [&](int &n, int &sg) {
    n += dq;
    sg += dr;
    if (sg >= spr) {
      sg -= spr;
      ++n;
    }
  };
  // loads of segment (n, sg); past the last row or the row end: nothing
  auto load = [&](int n, int sg, float (&v)[8]) {
    const int kl = sg * kSeg + lane * 8;
    if (n < L.N && kl < K) {
      const float *src = w + (int64_t)n * K + kl;
      const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src));
      const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + 4));
      v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
      v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
  };
  int n = gw / spr, seg = gw - (gw / spr) * spr;  // current segment
  int ln = n, ls = seg;                           // the segment loaded next
  float cur[8], nx1[8];
  load(ln, ls, cur);
  advance(ln, ls);
  load(ln, ls, nx1);
  advance(ln, ls);
  // the current row's block, and the row within it
  int blk = n / L.block_n;
  int r = n - blk * L.block_n;
  int c4 = 0, c8 = 0;                              // INT4 and 8-bit blocks before blk
  count_blocks(L, 0, blk, c4, c8);
  BlockInfo bi = block_info_counted(L, blk, c4, c8);
  while (n < L.N) {
    float nx2[8];
    load(ln, ls, nx2);
    advance(ln, ls);
    const int kl = seg * kSeg + lane * 8;
    const bool active = kl < K;
    void *orow = nullptr;
    if (MODE != kPack) orow = reinterpret_cast<uint8_t *>(wout) + (int64_t)n * K * (MODE == 2 ? 4 : 2);
    if (bi.bits == 4) {
      uint8_t *crow = MODE == kPack ? codes + bi.code_off + (uint64_t)r * (uint64_t)(K / 2) : nullptr;
      const uint64_t g0 = bi.grp_off + (uint64_t)r * (uint64_t)(K / 128);
      quant_segment<4, MODE>(cur, active, kl, crow, MODE == kPack ? scales + g0 : nullptr,
                             MODE == kPack ? zeros + g0 : nullptr, orow, flags);
    } else if (bi.bits == 8) {
      uint8_t *crow = MODE == kPack ? codes + bi.code_off + (uint64_t)r * (uint64_t)K : nullptr;
      const uint64_t g0 = bi.grp_off + (uint64_t)r * (uint64_t)(K / 128);
      quant_segment<8, MODE>(cur, active, kl, crow, MODE == kPack ? scales + g0 : nullptr,
                             MODE == kPack ? zeros + g0 : nullptr, orow, flags);
    } else {
      uint8_t *crow = MODE == kPack ? codes + bi.code_off + (uint64_t)r * (uint64_t)(K / 4) : nullptr;
      const uint64_t g0 = bi.grp_off + (uint64_t)r * (uint64_t)(K / 64);
      quant_segment<2, MODE>(cur, active, kl, crow, MODE == kPack ? scales + g0 : nullptr,
                             MODE == kPack ? zeros + g0 : nullptr, orow, flags);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      cur[i] = nx1[i];
      nx1[i] = nx2[i];
    }
    const int n0 = n;
    advance(n, seg);
    r += n - n0;
    if (r >= L.block_n && n < L.N) {
      // blocks passed, counted without a division; the running counts of
      // INT4 and 8-bit blocks take the passed blocks' bits of the map
      const int blk0 = blk;
      do {
        r -= L.block_n;
        ++blk;
      } while (r >= L.block_n);
      count_blocks(L, blk0, blk, c4, c8);
      bi = block_info_counted(L, blk, c4, c8);
    }
  }
}

// Workgroups of quantize_pack_kernel<MODE> the current device keeps
// resident (queried once per kernel and device), capped by the work.
template <int MODE>
int quant_grid(int64_t waves) {
  static std::mutex mu;
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int per = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    per = cached[dev];
    if (!per) {
      int per_cu = 0, cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &per_cu, reinterpret_cast<const void *>(quantize_pack_kernel<MODE>), kWaves * kLanes, 0) !=
              hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        per_cu = cus = 0;
      per = per_cu * cus;
      if (per > 0) cached[dev] = per;
    }
  }
  if (per <= 0) per = 2048;
  const int64_t need = (waves + kWaves - 1) / kWaves;
  return (int)(need < per ? need : per);
}

// ------------------------------------------------------------ dequant

// One thread expands one packed uint32 word: 8 INT4, 16 INT2 or 4 8-bit
// weights.
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
  const int g = group_size(bits);
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
  if (bits == 8) {
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = ((float)((wd >> (8 * i)) & 255u) - z) * S;
    if (OUT == 2) {
      *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + obase) = make_float4(q[0], q[1], q[2], q[3]);
    } else {
      uint32_t h[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint16_t ha = OUT == 0 ? f32_to_bf16_rne(q[2 * p]) : f32_to_f16_bits(q[2 * p]);
        const uint16_t hb = OUT == 0 ? f32_to_bf16_rne(q[2 * p + 1]) : f32_to_f16_bits(q[2 * p + 1]);
        h[p] = (uint32_t)ha | ((uint32_t)hb << 16);
      }
      *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + obase) = make_uint2(h[0], h[1]);
    }
  } else if (OUT == 2) {
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
  const int blocks = quant_grid<kPack>(waves);
  hipLaunchKernelGGL(quantize_pack_kernel<kPack>, dim3((unsigned)blocks), dim3(kWaves * kLanes), 0, s,
                     L, w, reinterpret_cast<uint8_t *>(codes), scales, zeros, nullptr, flags, segs);
  return hipGetLastError();
}

hipError_t launch_fake_quant(const LayoutDev &L, const float *w, gq_dtype out, void *w_out,
                             uint32_t *flags, hipStream_t s) {
  if (L.N == 0) return hipSuccess;
  const int segs = (L.K + kSeg - 1) / kSeg;
  const int64_t waves = (int64_t)L.N * segs;
  const dim3 block(kWaves * kLanes);
  switch (out) {
    case GQ_BF16:
      hipLaunchKernelGGL(quantize_pack_kernel<0>, dim3(quant_grid<0>(waves)), block, 0, s, L, w, nullptr, nullptr, nullptr, w_out, flags, segs);
      break;
    case GQ_FP16:
      hipLaunchKernelGGL(quantize_pack_kernel<1>, dim3(quant_grid<1>(waves)), block, 0, s, L, w, nullptr, nullptr, nullptr, w_out, flags, segs);
      break;
    default:
      hipLaunchKernelGGL(quantize_pack_kernel<2>, dim3(quant_grid<2>(waves)), block, 0, s, L, w, nullptr, nullptr, nullptr, w_out, flags, segs);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const LayoutDev &L, const uint32_t *codes, const uint16_t *scales,
                          const uint8_t *zeros, gq_dtype out, void *w_out, hipStream_t s) {
  if (L.N == 0) return hipSuccess;
  const int max_words = L.n8 > 0 ? L.K / 4 : L.K / 8;  // words of the widest row
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
