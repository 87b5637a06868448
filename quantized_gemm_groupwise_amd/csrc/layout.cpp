// Host-side layout validation, packed sizes and workspace sizes.
// Pure host code: no HIP call is made here.
#include <string.h>

#include "gq_internal.h"

namespace gq {

gq_status make_layout(const gq_layout *in, LayoutDev *out) {
  if (!in || !out) return GQ_ERR_NULL_ARG;
  if (in->K <= 0 || in->N < 0 || in->block_n <= 0) return GQ_ERR_SHAPE;
  if (in->N % in->block_n != 0) return GQ_ERR_SHAPE;
  const int nblocks = in->N / in->block_n;
  if (nblocks > GQ_MAX_BLOCKS) return GQ_ERR_SHAPE;
  if (nblocks > 1 && in->block_n % 128 != 0) return GQ_ERR_SHAPE;
  if (nblocks > 0 && !in->bits) return GQ_ERR_NULL_ARG;
  memset(out, 0, sizeof(*out));
  out->K = in->K;
  out->N = in->N;
  out->block_n = in->block_n;
  out->nblocks = nblocks;
  for (int i = 0; i < nblocks; ++i) {
    const int b = in->bits[i];
    if (b != 4 && b != 2 && b != 8) return GQ_ERR_BITS;
    if (in->K % group_size(b) != 0) return GQ_ERR_SHAPE;
    if (b == 4) out->int4_mask[i >> 5] |= 1u << (i & 31);
    if (b == 8) {
      out->int8_mask[i >> 5] |= 1u << (i & 31);
      ++out->n8;
    }
  }
  // K * block_n bytes of codes per block must fit the 64-bit offsets; rows of
  // at most 2^31 weights keep the per-row index arithmetic in 32 bits.
  if ((int64_t)in->K * 8 > (int64_t)INT32_MAX) return GQ_ERR_SHAPE;
  return GQ_OK;
}

gq_status check_ptr16(const void *p) {
  if (!p) return GQ_ERR_NULL_ARG;
  return ((uintptr_t)p & 15u) ? GQ_ERR_ALIGNMENT : GQ_OK;
}

size_t linear_workspace_bytes(const LayoutDev &L, int M, gq_dtype act) {
  (void)act;
  if (M <= kGemvMaxM || L.N == 0) return 0;
  if (skinny_supported(L, M)) return skinny_workspace_bytes(L, M);
  return gemm_workspace_bytes(L, M);
}

}  // namespace gq
