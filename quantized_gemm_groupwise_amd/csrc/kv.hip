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
// most 256 packed tokens, in two passes over tiles of 32 tokens whose codes
// reach LDS by buffer loads that write LDS directly, one tile ahead (the K
// tiles, then the V tiles, as one stream):
//   pass 1, q . K^T on MFMA 16x16x32 f16: A = q of the G query heads
//     (rescaled per head by a power of two so that its fp16 form is exact),
//     B = the codes as exact 1024 + c, and a second MFMA per 32 features with
//     B = the exact constant -(1024 + z), so the accumulator holds
//     sum q (c - z) with no rounding before accumulation; the token's scale
//     is applied in fp32 and the scores are kept in LDS;
//   one max per head over the range;
//   pass 2, P . V on fp32 VALU: lane (features 8f .. 8f + 7, tokens = lane
//     group mod 4) takes p = exp(s - max) and accumulates p S c per feature
//     and p S z per head, so the zero point costs one FMA per token and head.
// (An online softmax over each 32-token tile spent most of its time in the
// per-tile cross-lane reductions.)  Each workgroup writes its (max, sum,
// unnormalised output) per head; the first workgroups do the same for each 32
// tokens of the window; kv_combine_kernel merges the parts with the
// log-sum-exp rule.
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
    const float v = acc[g] + __shfl_xor(acc[g], 1);
    const float sc = t < nt ? v * a.scale : -__builtin_inff();
    float m = sc;
#pragma unroll
    for (int d = 2; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
    const float p = t < nt ? __expf(sc - m) : 0.f;
    float l = p;
#pragma unroll
    for (int d = 2; d < 64; d <<= 1) l += __shfl_xor(l, d);
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

template <int G>
__global__ __launch_bounds__(256) void kv_packed_kernel(KvArgs a, const uint16_t *__restrict__ q,
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
  __shared__ __attribute__((aligned(16))) uint4 T[2 * KV_NT][KV_TILE / 16];   // K tiles, then V tiles
  __shared__ uint32_t SZ[KV_HG][2 * KV_NT][KV_TT][2];   // scale | zero << 16 per tile, token, group
  constexpr int SCW = G <= 4 ? 4 : 8;
  __shared__ __attribute__((aligned(16))) float SC[KV_HG][KV_TPS][SCW];     // scores, then weights

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int kh0 = blockIdx.z * KV_HG;
  const int kh = kh0 + w;
  const bool active = kh < a.Hkv;
  if ((int)blockIdx.x < a.nwp) {
    // the first workgroups take the window's 32-token parts (they start
    // with the first round of workgroups), in the tile memory
    if (active)
      window_part<G>(a, blockIdx.x, b, kh, lane, q, kw, vw, reinterpret_cast<float *>(&T[0][0]) + w * (G * KV_D + G * KV_TT),
                     part_o, part_ml);
    return;
  }
  const int split = blockIdx.x - a.nwp;
  const int nh = a.Hkv - kh0 < KV_HG ? a.Hkv - kh0 : KV_HG;      // heads of this group
  const uint32_t hbytes = (uint32_t)(KV_D * a.bits / 8);          // code bytes per token and head
  const uint32_t seg = (uint32_t)nh * hbytes;                     // code bytes per token, this group
  const uint32_t seg_off = (uint32_t)kh0 * hbytes;
  const int gph = a.bits == 4 ? 1 : 2;                            // groups per head
  const int t_begin = split * a.tps;
  const int t_end = t_begin + a.tps < a.tp ? t_begin + a.tps : a.tp;
  const int ntiles = (t_end - t_begin + KV_TT - 1) / KV_TT;
  const Rsrc kcr = make_rsrc(kc, code_bytes), vcr = make_rsrc(vc, code_bytes);
  const Rsrc ksr = make_rsrc(ks, 2u * groups), kzr = make_rsrc(kz, groups);
  const Rsrc vsr = make_rsrc(vs, 2u * groups), vzr = make_rsrc(vz, groups);
  const size_t row0 = (size_t)b * a.tp;                           // first token row of the sequence

  // tile u of the stream: K tile u for u < ntiles, V tile u - ntiles after.
  // Instruction i of a tile carries 1 KB = 1024 / seg tokens, lane l ->
  // token i * (1024 / seg) + l / (seg / 16), 16-byte piece l % (seg / 16);
  // every offset goes in the per-lane (range-checked) offset
  const int lpt = (int)(seg / 16);                                // lanes per token
  const int ninst = (int)(KV_TT * seg / 1024);                    // >= 1
  auto dma_tile = [&](int u, uint4 *dst) {
    const bool isv = u >= ntiles;
    const int tau = isv ? u - ntiles : u;
    for (int i = w; i < ninst; i += 4) {
      const int tok = i * (64 / lpt) + lane / lpt;
      const int t = t_begin + tau * KV_TT + tok;
      const uint32_t off = t < a.tp ? (uint32_t)((row0 + t) * a.row_bytes) + seg_off + 16u * (lane % lpt)
                                    : kOobKv;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? vcr : kcr, (lds_void *)(dst + 64 * i), 16, off, 0, 0, 0);
    }
  };
  // scales and zero points of the wave's head for tile u: lane -> token
  // lane % 32, group lane / 32 (INT4 has one group per head)
  auto load_sz = [&](int u, uint32_t &sv, uint32_t &zv) {
    const bool isv = u >= ntiles;
    const int tau = isv ? u - ntiles : u;
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
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
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

  // every tile of the range at once (K tiles, then V tiles), one barrier
  const int nu = 2 * ntiles;
  for (int u = 0; u < nu; ++u) dma_tile(u, T[u]);
  {
    uint32_t szs[2 * KV_NT], szz[2 * KV_NT];
#pragma unroll
    for (int u = 0; u < 2 * KV_NT; ++u)
      if (u < nu) load_sz(u, szs[u], szz[u]);
#pragma unroll
    for (int u = 0; u < 2 * KV_NT; ++u)
      if (u < nu) SZ[w][u][lane & 31][lane >> 5] = szs[u] | (szz[u] << 16);
  }
  lds_barrier();
  if (!active || ntiles == 0) return;

  // ---- pass 1: scores of each tile's two 16-token blocks
  for (int u = 0; u < ntiles; ++u) {
    const uint8_t *tb8 = reinterpret_cast<const uint8_t *>(T[u]);
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
      float mx = mrow[i];
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
      mxr[i] = mx;
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
      float sm = p;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) sm += __shfl_xor(sm, d);
      lsum[g] = sm;
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
  for (int u = ntiles; u < nu; ++u) {
    const uint8_t *tb8 = reinterpret_cast<const uint8_t *>(T[u]);
    const int tau = u - ntiles;
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
    Z[g] += __shfl_xor(Z[g], 16);
    Z[g] += __shfl_xor(Z[g], 32);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      o[g][f] += __shfl_xor(o[g][f], 16);
      o[g][f] += __shfl_xor(o[g][f], 32);
    }
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
}

constexpr int KV_TW_MAX = 1024;

// out[b][h] = sum_s o_s e^(m_s - M) / sum_s l_s e^(m_s - M), M = max_s m_s,
// over the parts that saw tokens; bf16, round to nearest even.  One
// workgroup per (sequence, head, quarter of the features): thread (part
// slice ps of 32, features 4 dq .. 4 dq + 3 of the quarter) merges every
// 32nd part into a running (max, sum, output) in one pass over the parts,
// then the 32 slices are merged the same way.
__global__ __launch_bounds__(256) void kv_combine_kernel(KvArgs a, const float *__restrict__ part_o,
                                                         const float *__restrict__ part_ml,
                                                         uint16_t *__restrict__ out) {
  __shared__ float4 acc_s[32][8];
  __shared__ float2 ml_s[32];
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int tid = threadIdx.x;
  const int ps = tid >> 3, dq = tid & 7;
  const int f0 = 32 * blockIdx.y;
  float M = -__builtin_inff(), L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = ps; s < a.ns; s += 32) {
    const size_t pi = part_index(a, b, s, h);
    const float2 ml = *reinterpret_cast<const float2 *>(part_ml + 2 * pi);
    const float4 v = *reinterpret_cast<const float4 *>(part_o + pi * KV_D + f0 + 4 * dq);
    if (ml.y > 0.f) {
      const float Mn = fmaxf(M, ml.x);
      const float ca = __expf(M - Mn), cb = __expf(ml.x - Mn);     // ca = 0 while M = -inf
      L = fmaf(L, ca, ml.y * cb);
      acc.x = fmaf(acc.x, ca, v.x * cb);
      acc.y = fmaf(acc.y, ca, v.y * cb);
      acc.z = fmaf(acc.z, ca, v.z * cb);
      acc.w = fmaf(acc.w, ca, v.w * cb);
      M = Mn;
    }
  }
  acc_s[ps][dq] = acc;
  if (dq == 0) ml_s[ps] = make_float2(M, L);
  __syncthreads();
  if (tid < 32) {
    float Mx = -__builtin_inff();
#pragma unroll 8
    for (int k = 0; k < 32; ++k)
      if (ml_s[k].y > 0.f) Mx = fmaxf(Mx, ml_s[k].x);
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
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
  hipLaunchKernelGGL((kv_packed_kernel<G>), dim3(a.nwp + a.nsp, a.B, p.ngroups), dim3(256), 0, s, a, qq,
                     reinterpret_cast<const uint8_t *>(c.k_codes), c.k_scales, c.k_zeros,
                     reinterpret_cast<const uint8_t *>(c.v_codes), c.v_scales, c.v_zeros,
                     (uint32_t)code_bytes, (uint32_t)groups, reinterpret_cast<const uint16_t *>(c.k_window),
                     reinterpret_cast<const uint16_t *>(c.v_window), po, pml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_combine_kernel, dim3(a.B * a.Hq, KV_D / 32), dim3(256), 0, s, a, po, pml,
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
