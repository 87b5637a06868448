// Decode attention over a group-wise quantized KV cache.  The review of "A
// Survey of Low-bit Large Language Models" lists KV-cache compression among
// the uses of low-bit formats (FP16 down to INT4 / INT2) and three of its
// techniques: a quantization window (only tokens beyond the window are
// quantized), keeping the newest keys unquantized, and outlier handling.
// Here the cache of a sequence is the packed format of gq_quantize_pack with
// one row per token (groups of 128 / 64 features along each row), the newest
// tokens sit in a dense bf16 window, and one decode step computes, per query
// head h with key/value head h / G (G = query heads per key/value head),
//     out = softmax(q . K^T / sqrt(D)) . V     over packed tokens + window.
// Outlier handling is not implemented.
//
// Work split (flash-decoding).  kv_packed_kernel: a workgroup of 4 waves
// takes 4 key/value heads of one sequence (one per wave) over a range of at
// most 64 packed tokens (2 tiles of 32).  It issues every load of the range
// at once: K tiles by buffer loads that write LDS directly, V tiles into
// registers; pass 1 starts once the K half has landed, and the V tiles are
// written to LDS after it:
//   pass 1, q . K^T on MFMA 16x16x32 f16: A = q of the G query heads
//     (rescaled per head by a power of two so that its fp16 form is exact),
//     B = the codes as exact 1024 + c, and a second MFMA per 32 features with
//     B = the exact constant -(1024 + z), so the accumulator holds
//     sum q (c - z) with no rounding before accumulation; the token's scale
//     is applied in fp32 and the scores are kept in LDS;
//   one max per head over the range; p = exp(s - max) once per token and
//     head, in place of the score;
//   pass 2, P . V on fp32 VALU: lane (features 8f .. 8f + 7, tokens = lane
//     group mod 4) accumulates p S c per feature and p S z per head, so the
//     zero point costs one FMA per token and head.
// (An online softmax over each 32-token tile spent most of its time in the
// per-tile cross-lane reductions.)  Each workgroup writes its (max, sum,
// unnormalised output) per head; workgroup s then does the same for the
// s-th 32 tokens of the window (one wave per head); kv_combine_kernel
// merges the parts with the log-sum-exp rule.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int KV_D = 128;                         // head dimension
constexpr int KV_TT = 32;                         // tokens per tile
constexpr int KV_HG = 4;                          // key/value heads per workgroup (one per wave)
constexpr int KV_SEG = KV_HG * KV_D / 2;          // code bytes per token of 4 INT4 heads
constexpr int KV_TILE = KV_TT * KV_SEG;           // 8 KB
constexpr int KV_TPS = 64;                        // packed tokens per workgroup (2 tiles)
constexpr int KV_NT = KV_TPS / KV_TT;             // tiles per workgroup
constexpr int KV_NS_MAX = 2048;                   // parts per (sequence, head)
constexpr uint32_t kOobKv = 0x80000000u;

struct KvArgs {
  int B, Hq, Hkv, bits, tp, tw;
  int tps;               // packed tokens per split (a multiple of KV_TT)
  int nsp;               // packed splits per sequence
  int nwp;               // 32-token window parts per sequence
  int ns;                // parts per (sequence, head): packed splits, then 32-token window parts
  uint32_t row_bytes;    // code bytes of one token row (all heads)
  uint32_t row_groups;   // groups of one token row
  float scale;           // 1 / sqrt(D)
};

// A part: m (running max), l (sum of exp(s - m)) and o (sum of exp(s - m) v)
// of one (sequence, part, query head); m = -inf and l = 0 for a part that saw
// no token.
__device__ __forceinline__ size_t part_index(const KvArgs &a, int b, int s, int h) {
  return ((size_t)b * a.ns + s) * a.Hq + h;
}

// Cross-lane sums and maxima in registers: DPP moves within rows of 16
// lanes (quad swaps, then the half-row and row mirrors), lane swaps across
// rows; every lane receives the result.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dppf<0xB1>(v);          // lane ^ 1
  v += dppf<0x4E>(v);          // lane ^ 2
  v += dppf<0x141>(v);         // mirror within 8
  return v + dppf<0x140>(v);   // mirror within 16
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  return fmaxf(v, dppf<0x140>(v));
}
// v + v of lane ^ 16, v + v of lane ^ 32 (and the maxima)
__device__ __forceinline__ float add_x16(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  swap16(x, y);
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float add_x32(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  swap32(x, y);
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float max_x16(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  swap16(x, y);
  return fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}
__device__ __forceinline__ float max_x32(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  swap32(x, y);
  return fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}

// Ordering of LDS values that one lane of a wave stores and others load.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One 32-token part of the dense bf16 window ([B][tw][Hkv][D]) for key/value
// head kh, by one wave: its (max, sum, unnormalised output) for the G query
// heads.  qs: this wave's LDS scratch, G * (D + 32) floats.
template <int G>
__device__ __forceinline__ void window_part(const KvArgs &a, int wp, int b, int kh, int lane,
                                            const uint16_t *__restrict__ q, const uint16_t *__restrict__ kw,
                                            const uint16_t *__restrict__ vw, float *qs,
                                            float *__restrict__ part_o, float *__restrict__ part_ml) {
  float *pl = qs + G * KV_D;                       // weights [G][32]
  const int t0 = wp * KV_TT;
  const int nt = a.tw - t0 < KV_TT ? a.tw - t0 : KV_TT;
  const size_t tstride = (size_t)a.Hkv * KV_D;
  // q of the G query heads, fp32
  const uint16_t *qh = q + ((size_t)b * a.Hq + (size_t)kh * G) * KV_D;
  for (int c = lane; c < G * KV_D / 8; c += 64) {
    const uint4 v = *reinterpret_cast<const uint4 *>(qh + 8 * c);
    const uint32_t uu[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qs[8 * c + 2 * i] = bf16_bits_to_f32((uint16_t)(uu[i] & 0xffffu));
      qs[8 * c + 2 * i + 1] = bf16_bits_to_f32((uint16_t)(uu[i] >> 16));
    }
  }
  wave_lds_sync();
  // scores: lane -> token lane / 2, features 64 (lane & 1) .. + 63
  const int t = lane >> 1, hf = lane & 1;
  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.f;
  if (t < nt) {
    const uint16_t *krow = kw + ((size_t)b * a.tw + t0 + t) * tstride + (size_t)kh * KV_D + 64 * hf;
#pragma unroll 2
    for (int c = 0; c < 8; ++c) {
      const uint4 v = *reinterpret_cast<const uint4 *>(krow + 8 * c);
      const uint32_t uu[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float k0 = bf16_bits_to_f32((uint16_t)(uu[i] & 0xffffu));
        const float k1 = bf16_bits_to_f32((uint16_t)(uu[i] >> 16));
        const int d = 64 * hf + 8 * c + 2 * i;
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = fmaf(qs[g * KV_D + d + 1], k1, fmaf(qs[g * KV_D + d], k0, acc[g]));
      }
    }
  }
  float mx[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float v = acc[g] + dppf<0xB1>(acc[g]);          // the two halves of the token
    const float sc = t < nt ? v * a.scale : -__builtin_inff();
    const float m = max_x32(max_x16(max16(sc)));
    const float p = t < nt ? __expf(sc - m) : 0.f;
    const float l = add_x32(add_x16(sum16(hf == 0 ? p : 0.f)));
    mx[g] = m;
    sm[g] = l;
    if (hf == 0) pl[g * KV_TT + t] = p;
  }
  wave_lds_sync();
  // P . V: lane -> features 2 lane, 2 lane + 1
  float o[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) o[g][0] = o[g][1] = 0.f;
  const uint16_t *vrow = vw + ((size_t)b * a.tw + t0) * tstride + (size_t)kh * KV_D + 2 * lane;
#pragma unroll 4
  for (int tt = 0; tt < nt; ++tt) {
    const uint32_t v2 = *reinterpret_cast<const uint32_t *>(vrow + tt * tstride);
    const float v0 = bf16_bits_to_f32((uint16_t)(v2 & 0xffffu)), v1 = bf16_bits_to_f32((uint16_t)(v2 >> 16));
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pg = pl[g * KV_TT + tt];
      o[g][0] = fmaf(pg, v0, o[g][0]);
      o[g][1] = fmaf(pg, v1, o[g][1]);
    }
  }
  const int part = a.nsp + wp;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const size_t pi = part_index(a, b, part, kh * G + g);
    *reinterpret_cast<float2 *>(part_o + pi * KV_D + 2 * lane) = make_float2(o[g][0], o[g][1]);
    if (lane == 0) {
      part_ml[2 * pi] = mx[g];
      part_ml[2 * pi + 1] = sm[g];
    }
  }
}

// (8 query heads per key/value head: 3 waves per SIMD asked for, 2 by default)
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G == 8 ? 3 : 1))) void kv_packed_kernel(KvArgs a, const uint16_t *__restrict__ q,
                                                        const uint8_t *__restrict__ kc,
                                                        const uint16_t *__restrict__ ks,
                                                        const uint8_t *__restrict__ kz,
                                                        const uint8_t *__restrict__ vc,
                                                        const uint16_t *__restrict__ vs,
                                                        const uint8_t *__restrict__ vz,
                                                        uint32_t code_bytes, uint32_t groups,
                                                        const uint16_t *__restrict__ kw,
                                                        const uint16_t *__restrict__ vw,
                                                        float *__restrict__ part_o,
                                                        float *__restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) uint4 TK[KV_NT][KV_TILE / 16];     // K tiles
  __shared__ __attribute__((aligned(16))) uint4 TV[KV_NT][KV_TILE / 16];     // V tiles
  __shared__ uint32_t SZ[KV_HG][2 * KV_NT][KV_TT][2];   // scale | zero << 16 per tile, token, group
  constexpr int SCW = G <= 4 ? 4 : 8;
  __shared__ __attribute__((aligned(16))) float SC[KV_HG][KV_TPS][SCW];     // scores, then weights

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int kh0 = blockIdx.z * KV_HG;
  const int kh = kh0 + w;
  const bool active = kh < a.Hkv;
  const int split = blockIdx.x;
  // workgroup `split` takes packed split `split` (if any), then window part
  // `split` (if any), so the window adds no workgroups while nsp >= nwp
  if (split < a.nsp) [&]() {
  const uint32_t hbytes = (uint32_t)(KV_D * a.bits / 8);          // code bytes per token and head
  // code bytes per token of the group's 4 heads (past the last head the
  // bytes of the next token row are loaded and not used)
  const uint32_t seg = (uint32_t)KV_HG * hbytes;
  const uint32_t seg_off = (uint32_t)kh0 * hbytes;
  const int gph = a.bits == 4 ? 1 : 2;                            // groups per head
  const int t_begin = split * a.tps;
  const int t_end = t_begin + a.tps < a.tp ? t_begin + a.tps : a.tp;
  const int ntiles = (t_end - t_begin + KV_TT - 1) / KV_TT;
  const Rsrc kcr = make_rsrc(kc, code_bytes), vcr = make_rsrc(vc, code_bytes);
  const Rsrc ksr = make_rsrc(ks, 2u * groups), kzr = make_rsrc(kz, groups);
  const Rsrc vsr = make_rsrc(vs, 2u * groups), vzr = make_rsrc(vz, groups);
  const size_t row0 = (size_t)b * a.tp;                           // first token row of the sequence

  // tile tau of K or V: instruction i < ninst carries 1 KB = 1024 / seg
  // tokens, lane l -> token i * (1024 / seg) + l / (seg / 16), 16-byte piece
  // l % (seg / 16); each wave issues instructions w and w + 4 (past ninst or
  // past the range the offset is out of range: the load writes zeros to LDS
  // inside the tile), so every wave issues the same number of loads
  const int lpt = (int)(seg / 16);                                // lanes per token
  const int ninst = (int)(KV_TT * seg / 1024);                    // 8 (INT4) or 4 (INT2)
  auto tile_off = [&](int tau, int i) -> uint32_t {
    const int tok = i * (64 / lpt) + lane / lpt;
    const int t = t_begin + tau * KV_TT + tok;
    return (i < ninst && t < t_end) ? (uint32_t)((row0 + t) * a.row_bytes) + seg_off + 16u * (lane % lpt)
                                    : kOobKv;
  };
  // scales and zero points of the wave's head for tile tau: lane -> token
  // lane % 32, group lane / 32 (INT4 has one group per head)
  auto load_sz = [&](int tau, bool isv, uint32_t &sv, uint32_t &zv) {
    const int tok = lane & 31, grp = (lane >> 5) & (gph - 1);
    const int t = t_begin + tau * KV_TT + tok;
    const bool ok = active && t < t_end;
    const uint32_t gi = ok ? (uint32_t)((row0 + t) * a.row_groups) + (uint32_t)(kh * gph + grp) : kOobKv;
    sv = ld16(isv ? vsr : ksr, ok ? 2u * gi : kOobKv);
    zv = ld8(isv ? vzr : kzr, gi);
  };

  // q of the G query heads of this wave's head: A operand of 16x16x32,
  // lane l -> head l % 16 (zero past G), features 32 kb + 8 (l / 16) + i in
  // the order (0,4,1,5,2,6,3,7) the codes unpack in; each head rescaled by
  // 2^-e so that its largest magnitude lies in [2^15, 2^16) (exact in fp16)
  const int r = lane & 15, kq = lane >> 4;
  half8 qa[4];
  float fr[4];          // per accumulator row 4 kq + i: 2^e / sqrt(D)
  {
    float qv[4][8];
    float amax = 0.f;
    const bool qok = active && r < G;
    const uint16_t *qrow = q + ((size_t)b * a.Hq + (size_t)(qok ? kh * G + r : 0)) * KV_D;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint4 v = *reinterpret_cast<const uint4 *>(qrow + 32 * kb + 8 * kq);
      const uint32_t uu[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[kb][2 * i] = qok ? bf16_bits_to_f32((uint16_t)(uu[i] & 0xffffu)) : 0.f;
        qv[kb][2 * i + 1] = qok ? bf16_bits_to_f32((uint16_t)(uu[i] >> 16)) : 0.f;
        amax = fmaxf(amax, fmaxf(fabsf(qv[kb][2 * i]), fabsf(qv[kb][2 * i + 1])));
      }
    }
    amax = max_x32(max_x16(amax));
    int e = 0;
    if (amax > 0.f && __builtin_isfinite(amax)) {
      int ex;
      frexpf(amax, &ex);
      e = ex - 16;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qa[kb][2 * i] = (_Float16)ldexpf(qv[kb][i], -e);
        qa[kb][2 * i + 1] = (_Float16)ldexpf(qv[kb][i + 4], -e);
      }
    const float f = ldexpf(a.scale, e);
#pragma unroll
    for (int i = 0; i < 4; ++i) fr[i] = __shfl(f, 4 * kq + i);
  }

  float mrow[4];        // running max of accumulator rows 4 kq + i over this lane's tokens
#pragma unroll
  for (int i = 0; i < 4; ++i) mrow[i] = -__builtin_inff();

  // every load of the range at once: K scales and zero points, K tiles
  // (loads that write LDS directly), V scales and zero points, V tiles into
  // registers (written to LDS after pass 1: the compiler cannot tell loads
  // that write LDS apart, and would make the first LDS read of pass 1 wait
  // for all of them)
  uint32_t szs[2 * KV_NT], szz[2 * KV_NT];
  uint4 vt[KV_NT][2];
#pragma unroll
  for (int tau = 0; tau < KV_NT; ++tau) load_sz(tau, false, szs[tau], szz[tau]);
  // (with a lambda call among the builtin's arguments the host pass of the
  // compiler drops the kernel's launch stub: the offset goes first into a
  // variable)
  auto dma_k = [&](uint4 *dst, int tau, int i) {
    const uint32_t off = tile_off(tau, i);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kcr, (lds_void *)(dst + 64 * i), 16, off, 0, 0, 0);
  };
#pragma unroll
  for (int tau = 0; tau < KV_NT; ++tau)
#pragma unroll
    for (int j = 0; j < 2; ++j) dma_k(TK[tau], tau, w + 4 * j);
#pragma unroll
  for (int tau = 0; tau < KV_NT; ++tau) load_sz(tau, true, szs[KV_NT + tau], szz[KV_NT + tau]);
#pragma unroll
  for (int tau = 0; tau < KV_NT; ++tau)
#pragma unroll
    for (int j = 0; j < 2; ++j) vt[tau][j] = ld128(vcr, tile_off(tau, w + 4 * j));
#pragma unroll
  for (int u = 0; u < KV_NT; ++u) SZ[w][u][lane & 31][lane >> 5] = szs[u] | (szz[u] << 16);
  lds_barrier();

  // ---- pass 1: scores of each tile's two 16-token blocks
  for (int u = 0; u < (active ? ntiles : 0); ++u) {
    const uint8_t *tb8 = reinterpret_cast<const uint8_t *>(TK[u]);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int n = 16 * blk + r;                 // token of this lane's B column
      const uint32_t sz0 = SZ[w][u][n][0], sz1 = SZ[w][u][n][gph - 1];
      floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        half8 bv;
        const uint32_t base = (uint32_t)n * seg + (uint32_t)w * hbytes;
        uint32_t t4, mask, shift;
        if (a.bits == 4) {
          t4 = *reinterpret_cast<const uint32_t *>(tb8 + base + (uint32_t)(16 * kb + 4 * kq));
          mask = 0x000f000fu;
          shift = 4;
        } else {
          const uint32_t uu = *reinterpret_cast<const uint16_t *>(tb8 + base + (uint32_t)(8 * kb + 2 * kq));
          t4 = __builtin_amdgcn_perm(uu, uu, 0x0c010c00u);
          mask = 0x00030003u;
          shift = 2;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2v pp = __builtin_bit_cast(half2v, and_or(t4 >> (shift * i), mask, 0x64006400u));
          bv[2 * i] = pp.x;
          bv[2 * i + 1] = pp.y;
        }
        const uint32_t zz = (a.bits == 4 || kb < 2) ? sz0 : sz1;
        const _Float16 zb = (_Float16)(-(1024.f + (float)(zz >> 16)));
        half8 zv;
#pragma unroll
        for (int i = 0; i < 8; ++i) zv[i] = zb;
        if (a.bits == 4 || kb < 2) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], bv, acc0, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], zv, acc0, 0, 0, 0);
        } else {
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], bv, acc1, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], zv, acc1, 0, 0, 0);
        }
      }
      const float s0 = f16_bits_to_f32((uint16_t)(sz0 & 0xffffu));
      const float s1 = f16_bits_to_f32((uint16_t)(sz1 & 0xffffu));
      const int trel = u * KV_TT + n;             // token within the range
      const bool valid = t_begin + trel < t_end;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float raw = a.bits == 4 ? s0 * acc0[i] : s0 * acc0[i] + s1 * acc1[i];
        const float sc = valid ? raw * fr[i] : -__builtin_inff();
        mrow[i] = fmaxf(mrow[i], sc);
        if (4 * kq + i < G) SC[w][trel][4 * kq + i] = sc;
      }
    }
  }

  // the V half to LDS: scales and zero points, tiles
#pragma unroll
  for (int u = KV_NT; u < 2 * KV_NT; ++u) SZ[w][u][lane & 31][lane >> 5] = szs[u] | (szz[u] << 16);
#pragma unroll
  for (int tau = 0; tau < KV_NT; ++tau)
#pragma unroll
    for (int j = 0; j < 2; ++j) TV[tau][64 * (w + 4 * j) + lane] = vt[tau][j];
  lds_barrier();
  if (!active) return;

  // the range's max per head, from the lanes' running maxima of their rows;
  // head g is row g % 4 of lane group g / 4, read from its first lane (a
  // conditional LDS store read back by the other lanes is not ordered for
  // the compiler: it served the storing lane its own value and loaded the
  // others before the store)
  float mh[G];
  {
    float mxr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mxr[i] = max16(mrow[i]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
      mh[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mxr[g & 3]), 16 * (g >> 2)));
  }
  // the scores other lanes stored are read below: order them for the wave
  wave_lds_sync();

  // ---- weights p = exp(s - max), once per (token, head): lane -> token
  // `lane` of the range (invalid tokens hold -inf, so p = 0); their sums
  float lsum[G];
  {
    const bool have = lane < KV_TT * ntiles;
    float pv[SCW];
#pragma unroll
    for (int g = 0; g < SCW; g += 4) {
      const float4 v4 = have ? *reinterpret_cast<const float4 *>(&SC[w][lane][g]) : make_float4(0.f, 0.f, 0.f, 0.f);
      pv[g] = v4.x; pv[g + 1] = v4.y; pv[g + 2] = v4.z; pv[g + 3] = v4.w;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = have ? __expf(pv[g] - mh[g]) : 0.f;
      pv[g] = p;
      lsum[g] = add_x32(add_x16(sum16(p)));
    }
#pragma unroll
    for (int g = 0; g < SCW; g += 4)
      if (have) *reinterpret_cast<float4 *>(&SC[w][lane][g]) = make_float4(pv[g], pv[g + 1], pv[g + 2], pv[g + 3]);
  }
  wave_lds_sync();

  // ---- pass 2: P . V, lane -> features 8 fs .. 8 fs + 7, tokens 4 j + kq
  float o[G][8], Z[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Z[g] = 0.f;
#pragma unroll
    for (int f = 0; f < 8; ++f) o[g][f] = 0.f;
  }
  const int fs = r;
  const int vg = a.bits == 4 ? 0 : (fs >> 3);        // group of these features
  for (int tau = 0; tau < ntiles; ++tau) {
    const uint8_t *tb8 = reinterpret_cast<const uint8_t *>(TV[tau]);
    const int u = KV_NT + tau;
    constexpr int UNR = G <= 4 ? 2 : 1;         // registers: 8 heads leave no room for two tokens
#pragma unroll UNR
    for (int jj = 0; jj < KV_TT / 4; ++jj) {
      const int t = 4 * jj + kq;
      const int trel = tau * KV_TT + t;
      const uint32_t base = (uint32_t)t * seg + (uint32_t)w * hbytes;
      float c[8];
      if (a.bits == 4) {
        // even and odd nibbles to bytes, bytes to float
        const uint32_t cw = *reinterpret_cast<const uint32_t *>(tb8 + base + 4u * fs);
        const uint32_t lo = cw & 0x0f0f0f0fu, hi = (cw >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          c[2 * k] = (float)((lo >> (8 * k)) & 0xffu);
          c[2 * k + 1] = (float)((hi >> (8 * k)) & 0xffu);
        }
      } else {
        const uint32_t cw = *reinterpret_cast<const uint16_t *>(tb8 + base + 2u * fs);
#pragma unroll
        for (int f = 0; f < 8; ++f) c[f] = (float)((cw >> (2 * f)) & 3u);
      }
      const uint32_t sz = SZ[w][u][t][vg];
      const float S = f16_bits_to_f32((uint16_t)(sz & 0xffffu));
      const float zf = (float)(sz >> 16);
      float pv[SCW];
#pragma unroll
      for (int g = 0; g < SCW; g += 4) {
        const float4 v4 = *reinterpret_cast<const float4 *>(&SC[w][trel][g]);
        pv[g] = v4.x; pv[g + 1] = v4.y; pv[g + 2] = v4.z; pv[g + 3] = v4.w;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pw = pv[g] * S;
        Z[g] = fmaf(pw, zf, Z[g]);
#pragma unroll
        for (int f = 0; f < 8; ++f) o[g][f] = fmaf(pw, c[f], o[g][f]);
      }
    }
  }

  // sum the four token lane groups, subtract the zero-point term
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Z[g] = add_x32(add_x16(Z[g]));
#pragma unroll
    for (int f = 0; f < 8; ++f) o[g][f] = add_x32(add_x16(o[g][f]));
  }
  if (kq == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const size_t pi = part_index(a, b, split, kh * G + g);
      float *dst = part_o + pi * KV_D + 8 * r;
      *reinterpret_cast<float4 *>(dst) = make_float4(o[g][0] - Z[g], o[g][1] - Z[g], o[g][2] - Z[g], o[g][3] - Z[g]);
      *reinterpret_cast<float4 *>(dst + 4) = make_float4(o[g][4] - Z[g], o[g][5] - Z[g], o[g][6] - Z[g], o[g][7] - Z[g]);
      if (r == 0) {
        part_ml[2 * pi] = mh[g];
        part_ml[2 * pi + 1] = lsum[g];
      }
    }
  }
  }();
  if (split < a.nwp) {
    // the window part's scratch is the tile memory (two waves in each of
    // TK, TV: 2 G (D + 32) floats <= 16 KB): wait for every wave
    if (split < a.nsp) __syncthreads();
    if (active)
      window_part<G>(a, split, b, kh, lane, q, kw, vw, reinterpret_cast<float *>(w < 2 ? &TK[0][0] : &TV[0][0]) + (w & 1) * (G * KV_D + G * KV_TT),
                     part_o, part_ml);
  }
}

constexpr int KV_TW_MAX = 1024;

// out[b][h] = sum_s o_s e^(m_s - M) / sum_s l_s e^(m_s - M), M = max_s m_s,
// over the parts that saw tokens; bf16, round to nearest even.  One
// workgroup per (sequence, head, 4 Q features): thread (part slice ps of
// SL, features 4 dq .. 4 dq + 3) loads KC parts of its slice at once (every
// SL-th part; 12 x 32 covers a 32K-token context in one round trip), the
// wave takes their max, and the thread adds them with
// weights e^(m_s - max) into a running (max, sum, output) that is rescaled
// when a later chunk raises the max; the SL slices are merged the same way
// at the end.  SL = 32 (a quarter of the features per workgroup) when there
// are few (sequence, head) pairs, SL = 8 (all features) otherwise.
template <int SL>
__global__ __launch_bounds__(256) void kv_combine_kernel(KvArgs a, const float *__restrict__ part_o,
                                                         const float *__restrict__ part_ml,
                                                         uint16_t *__restrict__ out) {
  constexpr int Q = 256 / SL;                      // feature quads per workgroup
  constexpr int KC = SL == 32 ? 12 : 8;            // parts per slice loaded at once
  __shared__ float4 acc_s[SL][Q];
  __shared__ float2 ml_s[SL];
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int tid = threadIdx.x;
  const int ps = tid / Q, dq = tid % Q;
  const int f0 = 4 * Q * blockIdx.y;
  float M = -__builtin_inff(), L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < a.ns; s0 += KC * SL) {
    float2 ml[KC];
    float4 v[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      // unconditional loads (a part past the end reads the last part and is
      // given a zero sum below): a load under a branch was waited for inside
      // its branch, one round trip per part
      const int sp = s0 + ps + SL * k;
      const size_t pi = part_index(a, b, sp < a.ns ? sp : a.ns - 1, h);
      ml[k] = *reinterpret_cast<const float2 *>(part_ml + 2 * pi);
      v[k] = *reinterpret_cast<const float4 *>(part_o + pi * KV_D + f0 + 4 * dq);
    }
    __builtin_amdgcn_sched_barrier(0);             // every load issued before the first use
#pragma unroll
    for (int k = 0; k < KC; ++k)
      if (s0 + ps + SL * k >= a.ns) ml[k].y = 0.f;
    float cm = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < KC; ++k)
      if (ml[k].y > 0.f) cm = fmaxf(cm, ml[k].x);
#pragma unroll
    for (int d = Q; d < 64; d <<= 1) cm = fmaxf(cm, __shfl_xor(cm, d));
    // no branch here: the loads above would be moved into it
    const float Mn = fmaxf(M, cm);
    const float Ms = Mn > -__builtin_inff() ? Mn : 0.f;
    const float ca = __expf(M - Ms);               // 0 while M = -inf
    L *= ca;
    acc.x *= ca;
    acc.y *= ca;
    acc.z *= ca;
    acc.w *= ca;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const float e = ml[k].y > 0.f ? __expf(ml[k].x - Ms) : 0.f;
      L = fmaf(e, ml[k].y, L);
      acc.x = fmaf(e, v[k].x, acc.x);
      acc.y = fmaf(e, v[k].y, acc.y);
      acc.z = fmaf(e, v[k].z, acc.z);
      acc.w = fmaf(e, v[k].w, acc.w);
    }
    M = Mn;
  }
  acc_s[ps][dq] = acc;
  if (dq == 0) ml_s[ps] = make_float2(M, L);
  __syncthreads();
  if (tid < 4 * Q) {
    float Mx = -__builtin_inff();
#pragma unroll 8
    for (int k = 0; k < SL; ++k)
      if (ml_s[k].y > 0.f) Mx = fmaxf(Mx, ml_s[k].x);
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int k = 0; k < SL; ++k) {
      const float2 ml = ml_s[k];
      if (ml.y > 0.f) {
        const float e = __expf(ml.x - Mx);
        num = fmaf(reinterpret_cast<const float *>(&acc_s[k][0])[tid], e, num);
        den = fmaf(ml.y, e, den);
      }
    }
    out[((size_t)b * a.Hq + h) * KV_D + f0 + tid] = f32_to_bf16_rne(num / den);
  }
}

struct KvPlan {
  KvArgs a;
  int ngroups;
  size_t o_bytes, ml_bytes;
};

inline size_t round256(size_t v) { return (v + 255u) & ~(size_t)255u; }

inline KvPlan kv_plan(const gq_kv_cache &c) {
  KvPlan p;
  KvArgs &a = p.a;
  a.B = c.batch;
  a.Hq = c.q_heads;
  a.Hkv = c.kv_heads;
  a.bits = c.bits;
  a.tp = c.t_packed;
  a.tw = c.t_window;
  a.row_bytes = (uint32_t)(c.kv_heads * KV_D * c.bits / 8);
  a.row_groups = (uint32_t)(c.kv_heads * KV_D / (c.bits == 4 ? 128 : 64));
  a.scale = 1.0f / sqrtf((float)KV_D);
  p.ngroups = (c.kv_heads + KV_HG - 1) / KV_HG;
  // a fixed 64 tokens per workgroup: all of its tiles are loaded at once
  const int tps = KV_TPS;
  a.tps = tps;
  const int nsplit = a.tp > 0 ? (a.tp + tps - 1) / tps : 0;
  a.nsp = nsplit;
  a.nwp = (a.tw + KV_TT - 1) / KV_TT;
  a.ns = nsplit + a.nwp;
  p.o_bytes = round256((size_t)a.B * a.ns * a.Hq * KV_D * 4u);
  p.ml_bytes = round256((size_t)a.B * a.ns * a.Hq * 2 * 4u);
  return p;
}

template <int G>
hipError_t launch_kv_g(const KvPlan &p, const gq_kv_cache &c, const void *q, void *out, float *po,
                       float *pml, hipStream_t s) {
  const KvArgs &a = p.a;
  const uint16_t *qq = reinterpret_cast<const uint16_t *>(q);
  const uint64_t code_bytes = (uint64_t)a.B * a.tp * a.row_bytes;
  const uint64_t groups = (uint64_t)a.B * a.tp * a.row_groups;
  hipLaunchKernelGGL((kv_packed_kernel<G>), dim3(a.nsp > a.nwp ? a.nsp : a.nwp, a.B, p.ngroups), dim3(256), 0, s, a, qq,
                     reinterpret_cast<const uint8_t *>(c.k_codes), c.k_scales, c.k_zeros,
                     reinterpret_cast<const uint8_t *>(c.v_codes), c.v_scales, c.v_zeros,
                     (uint32_t)code_bytes, (uint32_t)groups, reinterpret_cast<const uint16_t *>(c.k_window),
                     reinterpret_cast<const uint16_t *>(c.v_window), po, pml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.B * a.Hq >= 512)
    hipLaunchKernelGGL(kv_combine_kernel<8>, dim3(a.B * a.Hq, 1), dim3(256), 0, s, a, po, pml,
                       reinterpret_cast<uint16_t *>(out));
  else
    hipLaunchKernelGGL(kv_combine_kernel<32>, dim3(a.B * a.Hq, KV_D / 32), dim3(256), 0, s, a, po, pml,
                       reinterpret_cast<uint16_t *>(out));
  return hipGetLastError();
}

}  // namespace

gq_status kv_check(const gq_kv_cache &c) {
  if (c.batch < 1 || c.kv_heads < 1 || c.q_heads < 1 || c.q_heads % c.kv_heads) return GQ_ERR_SHAPE;
  const int G = c.q_heads / c.kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return GQ_ERR_SHAPE;
  if (c.head_dim != KV_D) return GQ_ERR_SHAPE;
  if (c.bits != 4 && c.bits != 2) return GQ_ERR_BITS;
  if (c.t_packed < 0 || c.t_window < 0 || c.t_window > KV_TW_MAX) return GQ_ERR_SHAPE;
  if ((int64_t)c.t_packed + c.t_window < 1) return GQ_ERR_SHAPE;
  // parts per (sequence, head): packed splits of at most 64 tokens plus
  // window parts of 32
  if ((int64_t)(c.t_packed + KV_TPS - 1) / KV_TPS + (c.t_window + KV_TT - 1) / KV_TT > KV_NS_MAX)
    return GQ_ERR_SHAPE;
  const uint64_t code_bytes = (uint64_t)c.batch * c.t_packed * c.kv_heads * KV_D * c.bits / 8;
  if (code_bytes >= ((uint64_t)1 << 31)) return GQ_ERR_SHAPE;
  return GQ_OK;
}

size_t kv_workspace_bytes(const gq_kv_cache &c) {
  const KvPlan p = kv_plan(c);
  return p.o_bytes + p.ml_bytes;
}

hipError_t launch_kv(const gq_kv_cache &c, const void *q, void *out, void *workspace, hipStream_t s) {
  const KvPlan p = kv_plan(c);
  float *po = reinterpret_cast<float *>(workspace);
  float *pml = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + p.o_bytes);
  switch (c.q_heads / c.kv_heads) {
    case 1: return launch_kv_g<1>(p, c, q, out, po, pml, s);
    case 2: return launch_kv_g<2>(p, c, q, out, po, pml, s);
    case 4: return launch_kv_g<4>(p, c, q, out, po, pml, s);
    default: return launch_kv_g<8>(p, c, q, out, po, pml, s);
  }
}

}  // namespace gq
