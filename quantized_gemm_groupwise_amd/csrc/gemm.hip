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
#include "gq_internal.h"

namespace gq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));


// ---------------------------------------------------------------- pre-pass

// One workgroup per row of x: largest magnitude, exponent, rescale, convert,
// permute.  act 0: bf16 input (rescaled), act 1: fp16 input (copied).
template <int ACT>
__global__ __launch_bounds__(256) void prep_x_kernel(const uint16_t *__restrict__ x, int K,
                                                     uint16_t *__restrict__ xa,
                                                     int *__restrict__ rexp) {
  const int m = blockIdx.x;
  const uint16_t *row = x + (int64_t)m * K;
  uint16_t *out = xa + (int64_t)m * K;
  __shared__ float red[4];
  int e = 0;
  if (ACT == 0) {
    float amax = 0.f;
    for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
      const uint4 v = *reinterpret_cast<const uint4 *>(row + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
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
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4 *>(row + c);
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
    // chunk order (0,4,1,5,2,6,3,7)
    uint4 o;
    o.x = (uint32_t)h[0] | ((uint32_t)h[4] << 16);
    o.y = (uint32_t)h[1] | ((uint32_t)h[5] << 16);
    o.z = (uint32_t)h[2] | ((uint32_t)h[6] << 16);
    o.w = (uint32_t)h[3] | ((uint32_t)h[7] << 16);
    *reinterpret_cast<uint4 *>(out + c) = o;
  }
}

// ------------------------------------------------------------------- GEMM

// Unpack the 8 codes of one 8-k chunk into 4 packed fp16 pairs (q - z) * s,
// pair i holding chunk elements (i, i + 4).  `t` carries the chunk's codes
// with element i at bits [B*i, B*i + B) of its low half (elements 0..3) and
// element 4 + i at the same bits of its high half.
template <int B>
__device__ __forceinline__ void unpack_chunk(uint32_t t, half2v cz, half2v s2, half8 &out) {
  constexpr uint32_t MASK = B == 4 ? 0x000f000fu : 0x00030003u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = ((t >> (B * i)) & MASK) | 0x64006400u;   // 1024 + q, exact
    half2v v = __builtin_bit_cast(half2v, p);
    v = (v + cz) * s2;                                          // (q - z) exact, then * s
    out[2 * i] = v.x;
    out[2 * i + 1] = v.y;
  }
}

struct GemmArgs {
  int K, N, M, m0, nw;
  const uint16_t *xa;
  const int *rexp;
  uint16_t *y;
  int out_fp16;
};

// Main loop and epilogue of one wave; BITS is the bit-width of the wave's
// 64 columns (one Channel-mix block never splits a wave).  Every wave of the
// workgroup runs the same number of k steps and barriers, including waves
// whose columns lie beyond N (they only help load the x tile).
template <int BITS, int MB>
__device__ __forceinline__ void gemm_wave(const GemmArgs &g, uint16_t (*As)[32 * MB * 72],
                                          bool wave_active, const uint8_t *const *crow,
                                          const uint16_t *const *srow, const uint8_t *const *zrow,
                                          const bool *cvalid) {
  constexpr int LDA = 72;                 // halfs per LDS row: 64 + 8 padding
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h = lane >> 5;
  const int K = g.K;

  // A tile loads: thread -> (row = p*32 + tid/8, 16-byte chunk tid%8)
  const int arow = tid >> 3;
  const int achunk = tid & 7;
  uint4 areg[MB];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int p = 0; p < MB; ++p) {
      const int m = g.m0 + p * 32 + arow;
      if (m < g.M)
        areg[p] = *reinterpret_cast<const uint4 *>(g.xa + (int64_t)m * K + kt * 64 + achunk * 8);
      else
        areg[p] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int p = 0; p < MB; ++p)
      *reinterpret_cast<uint4 *>(&As[buf][(p * 32 + arow) * LDA + achunk * 8]) = areg[p];
  };
  // B code loads: lane half h takes chunks 4h..4h+3 of the 64-deep k step.
  uint4 bcur[2], bnext[2];
  auto load_b = [&](int kt, uint4 *dst) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if constexpr (BITS == 4) {
        dst[nb] = *reinterpret_cast<const uint4 *>(crow[nb] + kt * 32 + h * 16);
      } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(crow[nb] + kt * 16 + h * 8);
        dst[nb] = make_uint4(v.x, v.y, 0, 0);
      }
    }
  };
  half2v cz[2], s2[2];
  auto load_scale = [&](int kt) {
    const int gi = BITS == 4 ? (kt >> 1) : kt;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint16_t sb = cvalid[nb] ? srow[nb][gi] : (uint16_t)0;
      const float z = (float)zrow[nb][gi];
      const uint16_t zb = f32_to_f16_bits(-(1024.f + z));
      s2[nb] = __builtin_bit_cast(half2v, (uint32_t)sb | ((uint32_t)sb << 16));
      cz[nb] = __builtin_bit_cast(half2v, (uint32_t)zb | ((uint32_t)zb << 16));
    }
  };

  floatx16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;

  const int KT = K / 64;
  load_a(0);
  if (wave_active) load_b(0, bcur);
  store_a(0);
  __syncthreads();
  int cur = 0;
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      load_a(kt + 1);
      if (wave_active) load_b(kt + 1, bnext);
    }
    if (wave_active) {
      load_scale(kt);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        half8 bf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if constexpr (BITS == 4) {
            const uint32_t wv[4] = {bcur[nb].x, bcur[nb].y, bcur[nb].z, bcur[nb].w};
            unpack_chunk<4>(wv[t], cz[nb], s2[nb], bf[nb]);
          } else {
            const uint32_t wv = (t >> 1) ? bcur[nb].y : bcur[nb].x;
            // bytes (b0, b0, b1, b1) for the low chunk, (b2, b2, b3, b3) for the high one
            const uint32_t tc = __builtin_amdgcn_perm(wv, wv, (t & 1) ? 0x03030202u : 0x01010000u);
            unpack_chunk<2>(tc, cz[nb], s2[nb], bf[nb]);
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const half8 af =
              *reinterpret_cast<const half8 *>(&As[cur][(mb * 32 + j) * LDA + (4 * h + t) * 8]);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[nb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
    if (more) store_a(cur ^ 1);
    __syncthreads();
    cur ^= 1;
    if (more && wave_active) {
      bcur[0] = bnext[0];
      bcur[1] = bnext[1];
    }
  }

  if (!wave_active) return;
  // epilogue: lane (j, h) holds column nw + 32nb + j and rows 8(e/4) + 4h + e%4
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = g.m0 + mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (m >= g.M) continue;
      const int ex = g.rexp[m];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int n = g.nw + 32 * nb + j;
        if (n >= g.N) continue;
        const float v = ldexpf(acc[mb][nb][e], ex);
        g.y[(int64_t)m * g.N + n] = g.out_fp16 ? f32_to_f16_bits(v) : f32_to_bf16_rne(v);
      }
    }
  }
}

template <int MB>
__global__ __launch_bounds__(256) void gemm_kernel(LayoutDev L, int M, int m_tiles,
                                                   const uint16_t *__restrict__ xa,
                                                   const int *__restrict__ rexp,
                                                   const uint8_t *__restrict__ codes,
                                                   const uint16_t *__restrict__ scales,
                                                   const uint8_t *__restrict__ zeros,
                                                   uint16_t *__restrict__ y, int out_fp16) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][32 * MB * 72];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = threadIdx.x & 31;
  const int m_tile = (int)blockIdx.x % m_tiles;
  const int n_tile = (int)blockIdx.x / m_tiles;
  GemmArgs g;
  g.K = L.K; g.N = L.N; g.M = M;
  g.m0 = m_tile * 32 * MB;
  g.nw = n_tile * 256 + wave * 64;
  g.xa = xa; g.rexp = rexp; g.y = y; g.out_fp16 = out_fp16;
  const bool wave_active = g.nw < L.N;

  int bits = 4;
  const uint8_t *crow[2] = {codes, codes};
  const uint16_t *srow[2] = {scales, scales};
  const uint8_t *zrow[2] = {zeros, zeros};
  bool cvalid[2] = {false, false};
  if (wave_active) {
    const int blk = g.nw / L.block_n;
    const BlockInfo bi = block_info(L, blk);
    bits = __builtin_amdgcn_readfirstlane(bi.bits);
    const int RB = L.K * bits / 8;
    const int GPR = bits == 4 ? L.K / 128 : L.K / 64;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = g.nw + 32 * nb + j;
      cvalid[nb] = n < L.N;
      const int r = (cvalid[nb] ? n : g.nw) - blk * L.block_n;
      crow[nb] = codes + bi.code_off + (uint64_t)r * (uint64_t)RB;
      srow[nb] = scales + bi.grp_off + (uint64_t)r * (uint64_t)GPR;
      zrow[nb] = zeros + bi.grp_off + (uint64_t)r * (uint64_t)GPR;
    }
  }
  if (bits == 4)
    gemm_wave<4, MB>(g, As, wave_active, crow, srow, zrow, cvalid);
  else
    gemm_wave<2, MB>(g, As, wave_active, crow, srow, zrow, cvalid);
}

template <int MB>
hipError_t launch_tiles(const LayoutDev &L, int M, const uint16_t *xa, const int *rexp,
                        const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                        void *y, int out_fp16, hipStream_t s) {
  const int m_tiles = (M + 32 * MB - 1) / (32 * MB);
  const int n_tiles = (L.N + 255) / 256;
  hipLaunchKernelGGL(gemm_kernel<MB>, dim3(m_tiles * n_tiles), dim3(256), 0, s, L, M, m_tiles,
                     xa, rexp, reinterpret_cast<const uint8_t *>(codes), scales, zeros,
                     reinterpret_cast<uint16_t *>(y), out_fp16);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const LayoutDev &L, int M, gq_dtype act, const void *x,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       void *y, void *workspace, hipStream_t s) {
  const size_t a_bytes = ((size_t)M * (size_t)L.K * 2u + 255u) & ~(size_t)255u;
  uint16_t *xa = reinterpret_cast<uint16_t *>(workspace);
  int *rexp = reinterpret_cast<int *>(reinterpret_cast<char *>(workspace) + a_bytes);
  const uint16_t *xin = reinterpret_cast<const uint16_t *>(x);
  if (act == GQ_BF16)
    hipLaunchKernelGGL(prep_x_kernel<0>, dim3(M), dim3(256), 0, s, xin, L.K, xa, rexp);
  else
    hipLaunchKernelGGL(prep_x_kernel<1>, dim3(M), dim3(256), 0, s, xin, L.K, xa, rexp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int out_fp16 = act == GQ_FP16 ? 1 : 0;
  if (M <= 32) return launch_tiles<1>(L, M, xa, rexp, codes, scales, zeros, y, out_fp16, s);
  if (M <= 64) return launch_tiles<2>(L, M, xa, rexp, codes, scales, zeros, y, out_fp16, s);
  return launch_tiles<4>(L, M, xa, rexp, codes, scales, zeros, y, out_fp16, s);
}

}  // namespace gq
