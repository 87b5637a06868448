// Decode GEMV, one linear per launch (M <= 4): the kernel over a layout's
// row tiles and its launch configuration.  The arithmetic, the loads and
// the staging of x are in gemv_core.h, shared with the grouped decode.
#include "gemv_core.h"

namespace gq {
namespace {

// BITSEL: 4, 2 or 8 for a uniform (Layer-mix) linear; 0 for a Channel-mix
// layout of INT4 and INT2 blocks and 1 for one that also has 8-bit blocks,
// where the workgroup reads its block's width from the bit masks (the 4R
// rows of a workgroup never straddle two blocks).
template <int ACT, int M, int R, int NL, int BITSEL, int SS, bool ONE>
__global__ __launch_bounds__(kThreads) void gemv_kernel(LayoutDev L, const uint16_t *__restrict__ x,
                                                        const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        const uint8_t *__restrict__ zeros,
                                                        uint16_t *__restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int nb = (int)blockIdx.x * kWaves * R;
  const int n0 = nb + wave * R;
  const bool active = n0 < L.N;                // inactive waves still stage x
  // the launch picks SS so that a chunk holds at least one slice of every
  // bit-width in the layout; other combinations are never launched
  constexpr bool ok4 = chunk_slices(4, M, SS) >= 1, ok2 = chunk_slices(2, M, SS) >= 1;
  constexpr bool ok8 = chunk_slices(8, M, SS) >= 1;
  if constexpr (BITSEL == 4) {
    BlockInfo bi = {4, 0, 0};
    if constexpr (ok4)
      gemv_block<4, ACT, M, R, NL, SS, ONE>(L, bi, 0, n0, active, x, codes, scales, zeros, y, lds);
  } else if constexpr (BITSEL == 2) {
    BlockInfo bi = {2, 0, 0};
    if constexpr (ok2)
      gemv_block<2, ACT, M, R, NL, SS, ONE>(L, bi, 0, n0, active, x, codes, scales, zeros, y, lds);
  } else if constexpr (BITSEL == 8) {
    BlockInfo bi = {8, 0, 0};
    if constexpr (ok8)
      gemv_block<8, ACT, M, R, NL, SS, ONE>(L, bi, 0, n0, active, x, codes, scales, zeros, y, lds);
  } else if constexpr (ok4 && ok2 && (BITSEL == 0 || ok8)) {
    const int blk = nb / L.block_n;
    const BlockInfo bi = block_info(L, blk);
    const int bits = __builtin_amdgcn_readfirstlane(bi.bits);
    if (bits == 4)
      gemv_block<4, ACT, M, R, NL, SS, ONE>(L, bi, blk, n0, active, x, codes, scales, zeros, y, lds);
    else if (BITSEL == 1 && bits == 8)
      gemv_block<8, ACT, M, R, NL, SS, ONE>(L, bi, blk, n0, active, x, codes, scales, zeros, y, lds);
    else
      gemv_block<2, ACT, M, R, NL, SS, ONE>(L, bi, blk, n0, active, x, codes, scales, zeros, y, lds);
  }
}

template <int ACT, int M, int R, int NL, int SS>
hipError_t launch_rows(const LayoutDev &L, int bitsel, const void *x, const uint32_t *codes,
                       const uint16_t *scales, const uint8_t *zeros, void *y, hipStream_t s) {
  const int blocks = (L.N + kWaves * R - 1) / (kWaves * R);
  const uint16_t *xp = reinterpret_cast<const uint16_t *>(x);
  const uint8_t *cp = reinterpret_cast<const uint8_t *>(codes);
  uint16_t *yp = reinterpret_cast<uint16_t *>(y);
  const dim3 g(blocks), b(kThreads);
  const int ns4 = (L.K * 4 / 8 + 1023) / 1024, ns2 = (L.K * 2 / 8 + 1023) / 1024;
  const int ns8 = (L.K + 1023) / 1024;
  const int s4 = stage_bytes(4, M, ns4, SS), s2 = stage_bytes(2, M, ns2, SS);
  const int s8 = stage_bytes(8, M, ns8, SS);
  const bool one4 = ns4 <= NL && ns4 <= chunk_slices(4, M, SS);
  const bool one2 = ns2 <= NL && ns2 <= chunk_slices(2, M, SS);
  const bool one8 = ns8 <= NL && ns8 <= chunk_slices(8, M, SS);
  if (bitsel == 4) {
    if (one4)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 4, SS, true>), g, b, s4, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 4, SS, false>), g, b, s4, s, L, xp, cp, scales, zeros, yp);
  } else if (bitsel == 2) {
    if (one2)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 2, SS, true>), g, b, s2, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 2, SS, false>), g, b, s2, s, L, xp, cp, scales, zeros, yp);
  } else if (bitsel == 8) {
    if (one8)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 8, SS, true>), g, b, s8, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 8, SS, false>), g, b, s8, s, L, xp, cp, scales, zeros, yp);
  } else if (bitsel == 0) {
    const int sm = s4 > s2 ? s4 : s2;
    if (one4 && one2)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 0, SS, true>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 0, SS, false>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
  } else {
    // a map with 8-bit blocks: rows stream unless every width fits one group
    const int sm = s4 > s2 ? (s4 > s8 ? s4 : s8) : (s2 > s8 ? s2 : s8);
    if (one4 && one2 && one8)
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 1, SS, true>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
    else
      hipLaunchKernelGGL((gemv_kernel<ACT, M, R, NL, 1, SS, false>), g, b, sm, s, L, xp, cp, scales, zeros, yp);
  }
  return hipGetLastError();
}

// rows per wave: rsel 1 or 2; 4 for layouts with INT2 blocks at M >= 3,
// whose INT2 rows run on the matrix cores four rows per wave
template <int ACT, int M, int SS>
hipError_t launch_r(const LayoutDev &L, int bitsel, int rsel, int ns, const void *x,
                    const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros, void *y,
                    hipStream_t s) {
  if constexpr (M >= 3) {
    if (rsel == 4)
      return ns <= 1 ? launch_rows<ACT, M, 4, 1, SS>(L, bitsel, x, codes, scales, zeros, y, s)
                     : launch_rows<ACT, M, 4, 2, SS>(L, bitsel, x, codes, scales, zeros, y, s);
  }
  const bool two = rsel == 2;
  if (ns <= 1)
    return two ? launch_rows<ACT, M, 2, 1, SS>(L, bitsel, x, codes, scales, zeros, y, s)
               : launch_rows<ACT, M, 1, 1, SS>(L, bitsel, x, codes, scales, zeros, y, s);
  return two ? launch_rows<ACT, M, 2, 2, SS>(L, bitsel, x, codes, scales, zeros, y, s)
             : launch_rows<ACT, M, 1, 2, SS>(L, bitsel, x, codes, scales, zeros, y, s);
}

template <int ACT, int M>
hipError_t launch_m(const LayoutDev &L, const void *x, const uint32_t *codes,
                    const uint16_t *scales, const uint8_t *zeros, void *y, hipStream_t s) {
  int n4 = 0, n8 = 0;
  for (int i = 0; i < L.nblocks; ++i) {
    const int b = block_bits(L, i);
    n4 += b == 4;
    n8 += b == 8;
  }
  const int n2 = L.nblocks - n4 - n8;
  const int bitsel = n4 == L.nblocks ? 4 : n2 == L.nblocks ? 2 : n8 == L.nblocks ? 8 : (n8 ? 1 : 0);
  // Load groups of two 1 KB slices (one for rows of a single slice), issued
  // one group ahead; two rows per wave once N gives >= 2048 waves (four for
  // layouts with INT2 blocks at M >= 3: the matrix-core path).  Measured
  // on MI355X over the Llama-3-8B decode shapes: issuing a whole long row at
  // once, or more rows per wave, leaves fewer waves to cover HBM latency.
  const int widest = n8 ? 8 : (n4 ? 4 : 2);
  const int ns = (L.K * widest / 8 + 1023) / 1024;
  const bool two = L.N >= 4096;
  const int rsel = (M >= 3 && n2 > 0) ? 4 : two ? 2 : 1;
  // staging sub-units per thread that hold a whole row of x (an INT2 slice
  // carries twice the activations of an INT4 one, an 8-bit slice half)
  const int ns4 = (L.K * 4 / 8 + 1023) / 1024, ns2 = (L.K * 2 / 8 + 1023) / 1024;
  const int ns8 = (L.K + 1023) / 1024;
  const int u4 = n4 ? M * kLanes * 2 * ns4 : 0, u2 = n2 ? M * kLanes * 4 * ns2 : 0;
  const int u8 = n8 ? M * kLanes * ns8 : 0;
  const int um = u4 > u2 ? (u4 > u8 ? u4 : u8) : (u2 > u8 ? u2 : u8);
  const int need = (um + kThreads - 1) / kThreads;
  if (need <= 1) return launch_r<ACT, M, 1>(L, bitsel, rsel, ns, x, codes, scales, zeros, y, s);
  if (need <= 2) return launch_r<ACT, M, 2>(L, bitsel, rsel, ns, x, codes, scales, zeros, y, s);
  return launch_r<ACT, M, kStageSubMax>(L, bitsel, rsel, ns, x, codes, scales, zeros, y, s);
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
