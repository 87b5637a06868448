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
// takes 4 key/value heads of one sequence (one per wave) over a range of
// packed tokens, in tiles of 32 tokens whose codes reach LDS by buffer loads
// that write LDS directly, one tile ahead.  Per tile and wave:
//   q . K^T on MFMA 16x16x32 f16: A = q of the G query heads (rescaled per
//     head by a power of two so that its fp16 form is exact), B = the codes
//     as exact 1024 + c, and a second MFMA per 32 features with B = the exact
//     constant -(1024 + z), so the accumulator holds sum q (c - z) with no
//     rounding before accumulation; the token's scale is applied in fp32.
//   online softmax per head (running max, sum);
//   P . V on fp32 VALU: lane (features 8f .. 8f + 7, tokens = lane group
//     mod 4) accumulates p S c per feature and p S z per head, so the zero
//     point costs one FMA per token and head.
// Each workgroup writes its (max, sum, unnormalised output) per head;
// kv_window_kernel does the same for the window tokens; kv_combine_kernel
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
constexpr uint32_t kOobKv = 0x80000000u;

struct KvArgs {
  int B, Hq, Hkv, bits, tp, tw;
  int tps;               // packed tokens per split (a multiple of KV_TT)
  int ns;                // parts per (sequence, head): packed splits + 1 for the window
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

template <int G>
__global__ __launch_bounds__(256) void kv_packed_kernel(KvArgs a, const uint16_t *__restrict__ q,
                                                        const uint8_t *__restrict__ kc,
                                                        const uint16_t *__restrict__ ks,
                                                        const uint8_t *__restrict__ kz,
                                                        const uint8_t *__restrict__ vc,
                                                        const uint16_t *__restrict__ vs,
                                                        const uint8_t *__restrict__ vz,
                                                        uint32_t code_bytes, uint32_t groups,
                                                        float *__restrict__ part_o,
                                                        float *__restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) uint4 Kt0[KV_TILE / 16];
  __shared__ __attribute__((aligned(16))) uint4 Kt1[KV_TILE / 16];
  __shared__ __attribute__((aligned(16))) uint4 Vt0[KV_TILE / 16];
  __shared__ __attribute__((aligned(16))) uint4 Vt1[KV_TILE / 16];
  __shared__ uint32_t SZK[KV_HG][KV_TT][2];       // scale | zero << 16 per token and group
  __shared__ uint32_t SZV[KV_HG][KV_TT][2];
  __shared__ __attribute__((aligned(16))) float P[KV_HG][KV_TT][8];
  __shared__ float AL[KV_HG][8];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, b = blockIdx.y;
  const int kh0 = blockIdx.z * KV_HG;
  const int kh = kh0 + w;
  const bool active = kh < a.Hkv;
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

  // tile loads: instruction i of a tile carries 1 KB = 1024 / seg tokens,
  // lane l -> token i * (1024 / seg) + l / (seg / 16), 16-byte piece l % (seg / 16);
  // every offset goes in the per-lane (range-checked) offset
  const int lpt = (int)(seg / 16);                                // lanes per token
  const int ninst = (int)(KV_TT * seg / 1024);                    // >= 1
  auto dma_tile = [&](int tau, uint4 *kd, uint4 *vd) {
    for (int i = w; i < ninst; i += 4) {
      const int tok = i * (64 / lpt) + lane / lpt;
      const int t = t_begin + tau * KV_TT + tok;
      const uint32_t off = t < a.tp ? (uint32_t)((row0 + t) * a.row_bytes) + seg_off + 16u * (lane % lpt)
                                    : kOobKv;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kcr, (lds_void *)(kd + 64 * i), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vcr, (lds_void *)(vd + 64 * i), 16, off, 0, 0, 0);
    }
  };
  // scales and zero points of the wave's head for a tile: lane -> token
  // lane % 32, group lane / 32 (INT4 has one group per head)
  auto load_sz = [&](int tau, uint32_t &skv, uint32_t &zkv, uint32_t &svv, uint32_t &zvv) {
    const int tok = lane & 31, grp = (lane >> 5) & (gph - 1);
    const int t = t_begin + tau * KV_TT + tok;
    const bool ok = active && t < t_end;
    const uint32_t gi = ok ? (uint32_t)((row0 + t) * a.row_groups) + (uint32_t)(kh * gph + grp) : kOobKv;
    skv = ld16(ksr, ok ? 2u * gi : kOobKv);
    zkv = ld8(kzr, gi);
    svv = ld16(vsr, ok ? 2u * gi : kOobKv);
    zvv = ld8(vzr, gi);
  };
  auto store_sz = [&](uint32_t skv, uint32_t zkv, uint32_t svv, uint32_t zvv) {
    const int tok = lane & 31, grp = lane >> 5;
    SZK[w][tok][grp] = skv | (zkv << 16);
    SZV[w][tok][grp] = svv | (zvv << 16);
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
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[kb][2 * i] = qok ? bf16_bits_to_f32((uint16_t)(u[i] & 0xffffu)) : 0.f;
        qv[kb][2 * i + 1] = qok ? bf16_bits_to_f32((uint16_t)(u[i] >> 16)) : 0.f;
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

  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -__builtin_inff();
    l[i] = 0.f;
  }
  float o[G][8], Z[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Z[g] = 0.f;
#pragma unroll
    for (int f = 0; f < 8; ++f) o[g][f] = 0.f;
  }

  uint32_t skv, zkv, svv, zvv;
  if (ntiles > 0) {
    dma_tile(0, Kt0, Vt0);
    load_sz(0, skv, zkv, svv, zvv);
  }
  lds_barrier();
  for (int tau = 0; tau < ntiles; ++tau) {
    const uint4 *Kc = (tau & 1) ? Kt1 : Kt0;
    const uint4 *Vc = (tau & 1) ? Vt1 : Vt0;
    if (tau + 1 < ntiles) {
      if (tau & 1)
        dma_tile(tau + 1, Kt0, Vt0);
      else
        dma_tile(tau + 1, Kt1, Vt1);
    }
    store_sz(skv, zkv, svv, zvv);
    if (tau + 1 < ntiles) load_sz(tau + 1, skv, zkv, svv, zvv);
    if (active) {
      const uint8_t *kb8 = reinterpret_cast<const uint8_t *>(Kc);
      const uint8_t *vb8 = reinterpret_cast<const uint8_t *>(Vc);
      // ---- scores of the tile's two 16-token blocks
      float sv[2][4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int n = 16 * blk + r;                   // token of this lane's B column
        const uint32_t sz0 = SZK[w][n][0], sz1 = SZK[w][n][gph - 1];
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          half8 bv;
          const uint32_t base = (uint32_t)n * seg + (uint32_t)w * hbytes;
          uint32_t t4;
          uint32_t mask, shift;
          if (a.bits == 4) {
            t4 = *reinterpret_cast<const uint32_t *>(kb8 + base + (uint32_t)(16 * kb + 4 * kq));
            mask = 0x000f000fu;
            shift = 4;
          } else {
            const uint32_t u = *reinterpret_cast<const uint16_t *>(kb8 + base + (uint32_t)(8 * kb + 2 * kq));
            t4 = __builtin_amdgcn_perm(u, u, 0x0c010c00u);
            mask = 0x00030003u;
            shift = 2;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const half2v p = __builtin_bit_cast(half2v, and_or(t4 >> (shift * i), mask, 0x64006400u));
            bv[2 * i] = p.x;
            bv[2 * i + 1] = p.y;
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
        const bool valid = t_begin + tau * KV_TT + n < t_end;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float raw = a.bits == 4 ? s0 * acc0[i] : s0 * acc0[i] + s1 * acc1[i];
          sv[blk][i] = valid ? raw * fr[i] : -__builtin_inff();
        }
      }
      // ---- online softmax: rows 4 kq + i, the 16 lanes of a row group hold
      // the 16 columns (tokens) of each block
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = fmaxf(sv[0][i], sv[1][i]);
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
        const float mn = fmaxf(m[i], mx);
        const bool none = mn == -__builtin_inff();
        const float alpha = none ? 1.f : __expf(m[i] - mn);
        const float p0 = none ? 0.f : __expf(sv[0][i] - mn);
        const float p1 = none ? 0.f : __expf(sv[1][i] - mn);
        float ps = p0 + p1;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) ps += __shfl_xor(ps, d);
        l[i] = l[i] * alpha + ps;
        m[i] = mn;
        const int row = 4 * kq + i;
        if (row < G) {
          P[w][r][row] = p0;
          P[w][16 + r][row] = p1;
          if (r == 0) AL[w][row] = alpha;
        }
      }
      // ---- P . V: lane -> features 8 fs .. 8 fs + 7, tokens 4 j + kq
      const int fs = r;
      const int vg = a.bits == 4 ? 0 : (fs >> 3);      // group of these features
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float al = AL[w][g];
        Z[g] *= al;
#pragma unroll
        for (int f = 0; f < 8; ++f) o[g][f] *= al;
      }
#pragma unroll
      for (int jj = 0; jj < KV_TT / 4; ++jj) {
        const int t = 4 * jj + kq;
        const uint32_t base = (uint32_t)t * seg + (uint32_t)w * hbytes;
        uint32_t cw;
        if (a.bits == 4)
          cw = *reinterpret_cast<const uint32_t *>(vb8 + base + 4u * fs);
        else
          cw = *reinterpret_cast<const uint16_t *>(vb8 + base + 2u * fs);
        const uint32_t sz = SZV[w][t][vg];
        const float S = f16_bits_to_f32((uint16_t)(sz & 0xffffu));
        const float zf = (float)(sz >> 16);
        float c[8];
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          // the code under the mantissa of 2^23: exact, then minus 2^23
          const uint32_t bitsf = a.bits == 4 ? and_or(cw >> (4 * f), 0xfu, 0x4b000000u)
                                             : and_or(cw >> (2 * f), 0x3u, 0x4b000000u);
          c[f] = __uint_as_float(bitsf) - 8388608.f;
        }
        float pw[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pw[g] = P[w][t][g] * S;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          Z[g] = fmaf(pw[g], zf, Z[g]);
#pragma unroll
          for (int f = 0; f < 8; ++f) o[g][f] = fmaf(pw[g], c[f], o[g][f]);
        }
      }
    }
    // the next tile has landed in every wave's part, and no wave reads this one
    lds_barrier();
  }

  if (!active) return;
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
      float *dst = part_o + part_index(a, b, split, kh * G + g) * KV_D + 8 * r;
      float4 v0 = make_float4(o[g][0] - Z[g], o[g][1] - Z[g], o[g][2] - Z[g], o[g][3] - Z[g]);
      float4 v1 = make_float4(o[g][4] - Z[g], o[g][5] - Z[g], o[g][6] - Z[g], o[g][7] - Z[g]);
      *reinterpret_cast<float4 *>(dst) = v0;
      *reinterpret_cast<float4 *>(dst + 4) = v1;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * kq + i;
      if (row < G) {
        const size_t pi = part_index(a, b, split, kh * G + row);
        part_ml[2 * pi] = m[i];
        part_ml[2 * pi + 1] = l[i];
      }
    }
  }
}

// Window tokens (dense bf16 [B][tw][Hkv][D]), one workgroup per (sequence,
// key/value head): scores, softmax and P . V over the whole window, written
// as the last part.
constexpr int KV_TW_MAX = 1024;

template <int G>
__global__ __launch_bounds__(256) void kv_window_kernel(KvArgs a, const uint16_t *__restrict__ q,
                                                        const uint16_t *__restrict__ kw,
                                                        const uint16_t *__restrict__ vw,
                                                        float *__restrict__ part_o,
                                                        float *__restrict__ part_ml) {
  __shared__ float qs[G][KV_D];
  __shared__ float S[G][KV_TW_MAX];
  __shared__ float red[G][4];
  const int b = blockIdx.x, kh = blockIdx.y;
  const int tid = threadIdx.x;
  const int T = a.tw;
  for (int i = tid; i < G * KV_D; i += 256)
    qs[i / KV_D][i % KV_D] = bf16_bits_to_f32(q[((size_t)b * a.Hq + kh * G + i / KV_D) * KV_D + i % KV_D]);
  __syncthreads();
  const size_t tstride = (size_t)a.Hkv * KV_D;
  const uint16_t *kbase = kw + ((size_t)b * T * a.Hkv + kh) * KV_D;
  const uint16_t *vbase = vw + ((size_t)b * T * a.Hkv + kh) * KV_D;
  float mloc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mloc[g] = -__builtin_inff();
  for (int t = tid; t < T; t += 256) {
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    for (int d = 0; d < KV_D; d += 8) {
      const uint4 v = *reinterpret_cast<const uint4 *>(kbase + t * tstride + d);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float k0 = bf16_bits_to_f32((uint16_t)(u[i] & 0xffffu));
        const float k1 = bf16_bits_to_f32((uint16_t)(u[i] >> 16));
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = fmaf(qs[g][d + 2 * i + 1], k1, fmaf(qs[g][d + 2 * i], k0, acc[g]));
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      S[g][t] = acc[g] * a.scale;
      mloc[g] = fmaxf(mloc[g], acc[g] * a.scale);
    }
  }
  // block max and sum per head
  float mx[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = mloc[g];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
    if ((tid & 63) == 0) red[g][tid >> 6] = v;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = fmaxf(fmaxf(red[g][0], red[g][1]), fmaxf(red[g][2], red[g][3]));
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = 0.f;
    for (int t = tid; t < T; t += 256) {
      const float p = __expf(S[g][t] - mx[g]);
      S[g][t] = p;
      v += p;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    if ((tid & 63) == 0) red[g][tid >> 6] = v;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) sm[g] = red[g][0] + red[g][1] + red[g][2] + red[g][3];
  // P . V: thread -> (head g, feature d) pairs
  for (int i = tid; i < G * KV_D; i += 256) {
    const int g = i / KV_D, d = i % KV_D;
    float acc = 0.f;
    for (int t = 0; t < T; ++t) acc = fmaf(S[g][t], bf16_bits_to_f32(vbase[t * tstride + d]), acc);
    part_o[part_index(a, b, a.ns - 1, kh * G + g) * KV_D + d] = acc;
  }
  if (tid < G) {
    const size_t pi = part_index(a, b, a.ns - 1, kh * G + tid);
    part_ml[2 * pi] = mx[tid];
    part_ml[2 * pi + 1] = sm[tid];
  }
}

// out[b][h] = sum_s o_s e^(m_s - M) / sum_s l_s e^(m_s - M), M = max_s m_s,
// over the parts that saw tokens; bf16, round to nearest even.
__global__ __launch_bounds__(KV_D) void kv_combine_kernel(KvArgs a, const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml,
                                                          uint16_t *__restrict__ out) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int d = threadIdx.x;
  float M = -__builtin_inff();
  for (int s = 0; s < a.ns; ++s) {
    const size_t pi = part_index(a, b, s, h);
    if (part_ml[2 * pi + 1] > 0.f) M = fmaxf(M, part_ml[2 * pi]);
  }
  float num = 0.f, den = 0.f;
  for (int s = 0; s < a.ns; ++s) {
    const size_t pi = part_index(a, b, s, h);
    const float ls = part_ml[2 * pi + 1];
    if (!(ls > 0.f)) continue;
    const float e = __expf(part_ml[2 * pi] - M);
    num = fmaf(part_o[pi * KV_D + d], e, num);
    den = fmaf(ls, e, den);
  }
  out[((size_t)b * a.Hq + h) * KV_D + d] = f32_to_bf16_rne(num / den);
}

// The window part when there is no window: m = -inf, l = 0 (a fill kernel,
// not a memset, so that the call can be captured in a graph).
__global__ __launch_bounds__(256) void kv_empty_part_kernel(KvArgs a, float *__restrict__ part_ml) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.B * a.Hq) return;
  const size_t pi = part_index(a, i / a.Hq, a.ns - 1, i % a.Hq);
  part_ml[2 * pi] = -__builtin_inff();
  part_ml[2 * pi + 1] = 0.f;
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
  // about two workgroups per CU, at least 4 tiles per split
  int tps = KV_TT * 4;
  if (a.tp > 0) {
    const long want = (long)a.tp * a.B * p.ngroups / 512;
    if (want > tps) tps = (int)((want + KV_TT - 1) / KV_TT * KV_TT);
  }
  a.tps = tps;
  const int nsplit = a.tp > 0 ? (a.tp + tps - 1) / tps : 0;
  a.ns = nsplit + 1;
  p.o_bytes = round256((size_t)a.B * a.ns * a.Hq * KV_D * 4u);
  p.ml_bytes = round256((size_t)a.B * a.ns * a.Hq * 2 * 4u);
  return p;
}

template <int G>
hipError_t launch_kv_g(const KvPlan &p, const gq_kv_cache &c, const void *q, void *out, float *po,
                       float *pml, hipStream_t s) {
  const KvArgs &a = p.a;
  const uint16_t *qq = reinterpret_cast<const uint16_t *>(q);
  if (a.tp > 0) {
    const uint64_t code_bytes = (uint64_t)a.B * a.tp * a.row_bytes;
    const uint64_t groups = (uint64_t)a.B * a.tp * a.row_groups;
    hipLaunchKernelGGL((kv_packed_kernel<G>), dim3(a.ns - 1, a.B, p.ngroups), dim3(256), 0, s, a, qq,
                       reinterpret_cast<const uint8_t *>(c.k_codes), c.k_scales, c.k_zeros,
                       reinterpret_cast<const uint8_t *>(c.v_codes), c.v_scales, c.v_zeros,
                       (uint32_t)code_bytes, (uint32_t)groups, po, pml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.tw > 0) {
    hipLaunchKernelGGL((kv_window_kernel<G>), dim3(a.B, a.Hkv), dim3(256), 0, s, a, qq,
                       reinterpret_cast<const uint16_t *>(c.k_window),
                       reinterpret_cast<const uint16_t *>(c.v_window), po, pml);
  } else {
    hipLaunchKernelGGL(kv_empty_part_kernel, dim3((a.B * a.Hq + 255) / 256), dim3(256), 0, s, a, pml);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_combine_kernel, dim3(a.B * a.Hq), dim3(KV_D), 0, s, a, po, pml,
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
