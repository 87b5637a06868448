// C ABI of libgq (declared in include/gq.h): argument checks, then dispatch
// to the kernels.  Every check happens on the host before anything is
// enqueued; nothing here allocates, prints or aborts.
#include <stdlib.h>

#include <mutex>

#include "gq_internal.h"

using namespace gq;

// Scratch memory of gq_linear_noalloc: a static device array (each GPU the
// library runs on holds its own copy until the process ends).  Host code
// never uses this name as an address: the device address of the current
// GPU's copy comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[GQ_NOALLOC_SCRATCH_BYTES];

namespace {

gq_status launched(hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return GQ_ERR_HIP;
  static const bool debug_sync = [] {
    const char *v = getenv("GQ_DEBUG_SYNC");
    return v && v[0] == '1';
  }();
  if (debug_sync) {
    if (hipStreamSynchronize(s) != hipSuccess) return GQ_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return GQ_ERR_HIP;
  }
  return GQ_OK;
}

// Device address of the current GPU's scratch array, resolved once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];

gq_status scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GQ_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return GQ_OK;
}

// Argument checks of gq_linear that do not concern the workspace.  *done is
// set when there is no work (M == 0 or N == 0).
gq_status check_linear(const gq_layout *layout, int32_t M, gq_dtype act, const void *x,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       const void *y, LayoutDev *L, bool *done) {
  gq_status st = make_layout(layout, L);
  if (st != GQ_OK) return st;
  if (M < 0) return GQ_ERR_SHAPE;
  if (act != GQ_BF16 && act != GQ_FP16) return GQ_ERR_DTYPE;
  if (L->n8 > 0 && M > kGemvMaxM) return GQ_ERR_UNSUPPORTED;   // 8-bit rows: M <= 4 only
  *done = M == 0 || L->N == 0;
  if (*done) return GQ_OK;
  if ((st = check_ptr16(x)) != GQ_OK) return st;
  if ((st = check_ptr16(codes)) != GQ_OK) return st;
  if (!scales || !zeros || !y) return GQ_ERR_NULL_ARG;
  if (((uintptr_t)scales & 1u) || ((uintptr_t)y & 1u)) return GQ_ERR_ALIGNMENT;
  return GQ_OK;
}

// The kernels of gq_linear by M (workspace already checked).
gq_status dispatch_linear(const LayoutDev &L, int32_t M, gq_dtype act, const void *x,
                          const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                          void *y, void *workspace, hipStream_t s) {
  if (M <= kGemvMaxM)
    return launched(launch_gemv(L, M, act, x, codes, scales, zeros, y, s), s);
  if (skinny_supported(L, M))
    return launched(launch_skinny(L, M, act, x, codes, scales, zeros, y, workspace, s), s);
  return launched(launch_gemm(L, M, act, x, codes, scales, zeros, y, workspace, s), s);
}

}  // namespace

extern "C" {

gq_status gq_packed_bytes(const gq_layout *layout, size_t *codes_bytes, size_t *scales_bytes,
                          size_t *zeros_bytes) {
  if (!codes_bytes || !scales_bytes || !zeros_bytes) return GQ_ERR_NULL_ARG;
  LayoutDev L;
  const gq_status st = make_layout(layout, &L);
  if (st != GQ_OK) return st;
  size_t cb = 0, ng = 0;
  for (int i = 0; i < L.nblocks; ++i) {
    const int b = layout->bits[i];
    cb += (size_t)L.block_n * (size_t)L.K * (size_t)b / 8u;
    ng += (size_t)L.block_n * (size_t)L.K / (size_t)group_size(b);
  }
  *codes_bytes = cb;
  *scales_bytes = ng * 2u;
  *zeros_bytes = ng;
  return GQ_OK;
}

gq_status gq_quantize_pack(const gq_layout *layout, const float *w, uint32_t *codes,
                           uint16_t *scales, uint8_t *zeros, uint32_t *flags, void *stream) {
  LayoutDev L;
  gq_status st = make_layout(layout, &L);
  if (st != GQ_OK) return st;
  if (L.N == 0) return GQ_OK;
  if ((st = check_ptr16(w)) != GQ_OK) return st;
  if ((st = check_ptr16(codes)) != GQ_OK) return st;
  if (!scales || !zeros) return GQ_ERR_NULL_ARG;
  if ((uintptr_t)scales & 1u) return GQ_ERR_ALIGNMENT;
  if (flags && ((uintptr_t)flags & 3u)) return GQ_ERR_ALIGNMENT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return launched(launch_quantize_pack(L, w, codes, scales, zeros, flags, s), s);
}

gq_status gq_fake_quant(const gq_layout *layout, const float *w, gq_dtype out_dtype, void *w_out,
                        uint32_t *flags, void *stream) {
  LayoutDev L;
  gq_status st = make_layout(layout, &L);
  if (st != GQ_OK) return st;
  if (out_dtype != GQ_BF16 && out_dtype != GQ_FP16 && out_dtype != GQ_FP32) return GQ_ERR_DTYPE;
  if (L.N == 0) return GQ_OK;
  if ((st = check_ptr16(w)) != GQ_OK) return st;
  if ((st = check_ptr16(w_out)) != GQ_OK) return st;
  if (flags && ((uintptr_t)flags & 3u)) return GQ_ERR_ALIGNMENT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return launched(launch_fake_quant(L, w, out_dtype, w_out, flags, s), s);
}

gq_status gq_dequant(const gq_layout *layout, const uint32_t *codes, const uint16_t *scales,
                     const uint8_t *zeros, gq_dtype out_dtype, void *w_out, void *stream) {
  LayoutDev L;
  gq_status st = make_layout(layout, &L);
  if (st != GQ_OK) return st;
  if (out_dtype != GQ_BF16 && out_dtype != GQ_FP16 && out_dtype != GQ_FP32) return GQ_ERR_DTYPE;
  if (L.N == 0) return GQ_OK;
  if ((st = check_ptr16(codes)) != GQ_OK) return st;
  if ((st = check_ptr16(w_out)) != GQ_OK) return st;
  if (!scales || !zeros) return GQ_ERR_NULL_ARG;
  if ((uintptr_t)scales & 1u) return GQ_ERR_ALIGNMENT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return launched(launch_dequant(L, codes, scales, zeros, out_dtype, w_out, s), s);
}

gq_status gq_linear_workspace_bytes(const gq_layout *layout, int32_t M, gq_dtype act,
                                    size_t *bytes) {
  if (!bytes) return GQ_ERR_NULL_ARG;
  LayoutDev L;
  const gq_status st = make_layout(layout, &L);
  if (st != GQ_OK) return st;
  if (M < 0) return GQ_ERR_SHAPE;
  if (act != GQ_BF16 && act != GQ_FP16) return GQ_ERR_DTYPE;
  if (L.n8 > 0 && M > kGemvMaxM) return GQ_ERR_UNSUPPORTED;
  *bytes = linear_workspace_bytes(L, M, act);
  return GQ_OK;
}

gq_status gq_linear(const gq_layout *layout, int32_t M, gq_dtype act, const void *x,
                    const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                    void *y, void *workspace, size_t workspace_bytes, void *stream) {
  LayoutDev L;
  bool done = false;
  gq_status st = check_linear(layout, M, act, x, codes, scales, zeros, y, &L, &done);
  if (st != GQ_OK || done) return st;
  const size_t need = linear_workspace_bytes(L, M, act);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return GQ_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255u) return GQ_ERR_ALIGNMENT;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return dispatch_linear(L, M, act, x, codes, scales, zeros, y, workspace, s);
}

gq_status gq_linear_noalloc(const gq_layout *layout, int32_t M, gq_dtype act, const void *x,
                            const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                            void *y, void *stream) {
  LayoutDev L;
  bool done = false;
  gq_status st = check_linear(layout, M, act, x, codes, scales, zeros, y, &L, &done);
  if (st != GQ_OK || done) return st;
  const size_t need = linear_workspace_bytes(L, M, act);
  if (need > (size_t)GQ_NOALLOC_SCRATCH_BYTES) return GQ_ERR_TOO_LARGE;
  void *ws = nullptr;
  if (need > 0 && (st = scratch_address(&ws)) != GQ_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return dispatch_linear(L, M, act, x, codes, scales, zeros, y, ws, s);
}

gq_status gq_group_plan_bytes(int32_t count, const gq_group_item *items, int32_t M, gq_dtype act,
                              size_t *bytes) {
  if (!bytes) return GQ_ERR_NULL_ARG;
  return gemv_group_plan(count, items, M, act, nullptr, 0, bytes);
}

gq_status gq_group_plan(int32_t count, const gq_group_item *items, int32_t M, gq_dtype act,
                        void *plan, size_t plan_bytes) {
  if (!plan) return GQ_ERR_NULL_ARG;
  return gemv_group_plan(count, items, M, act, plan, plan_bytes, nullptr);
}

gq_status gq_linear_group(const void *plan, const void *plan_dev, void *stream) {
  gq_status st = gemv_group_check(plan);
  if (st != GQ_OK) return st;
  if ((st = check_ptr16(plan_dev)) != GQ_OK) return st;
  const GroupPlanHeader &H = *static_cast<const GroupPlanHeader *>(plan);
  if (H.nclass == 0) return GQ_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return launched(launch_gemv_group(H, plan_dev, s), s);
}

gq_status gq_linear_dx_workspace_bytes(const gq_layout *layout, int32_t M, gq_dtype act,
                                       size_t *bytes) {
  if (!bytes) return GQ_ERR_NULL_ARG;
  LayoutDev L;
  const gq_status st = make_layout(layout, &L);
  if (st != GQ_OK) return st;
  if (M < 0) return GQ_ERR_SHAPE;
  if (act != GQ_BF16 && act != GQ_FP16) return GQ_ERR_DTYPE;
  if (L.n8 > 0) return GQ_ERR_UNSUPPORTED;
  if (M > 0 && L.N > 0 && !dx_supported(L, M)) return GQ_ERR_SHAPE;
  *bytes = dx_workspace_bytes(L, M);
  return GQ_OK;
}

gq_status gq_linear_dx(const gq_layout *layout, int32_t M, gq_dtype act, const void *dy,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       void *dx, void *workspace, size_t workspace_bytes, void *stream) {
  LayoutDev L;
  gq_status st = make_layout(layout, &L);
  if (st != GQ_OK) return st;
  if (M < 0) return GQ_ERR_SHAPE;
  if (act != GQ_BF16 && act != GQ_FP16) return GQ_ERR_DTYPE;
  if (L.n8 > 0) return GQ_ERR_UNSUPPORTED;
  if (M == 0) return GQ_OK;
  if (L.N > 0 && !dx_supported(L, M)) return GQ_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!dx) return GQ_ERR_NULL_ARG;
  if ((uintptr_t)dx & 1u) return GQ_ERR_ALIGNMENT;
  if (L.N == 0)  // an empty sum: dX is zero
    return launched(launch_dx(L, M, act, nullptr, nullptr, nullptr, nullptr, dx, nullptr, s), s);
  if ((st = check_ptr16(dy)) != GQ_OK) return st;
  if ((st = check_ptr16(codes)) != GQ_OK) return st;
  if (!scales || !zeros) return GQ_ERR_NULL_ARG;
  if ((uintptr_t)scales & 1u) return GQ_ERR_ALIGNMENT;
  const size_t need = dx_workspace_bytes(L, M);
  if (!workspace || workspace_bytes < need) return GQ_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 255u) return GQ_ERR_ALIGNMENT;
  return launched(launch_dx(L, M, act, dy, codes, scales, zeros, dx, workspace, s), s);
}

gq_status gq_kv_attention_workspace_bytes(const gq_kv_cache *cache, size_t *bytes) {
  if (!cache || !bytes) return GQ_ERR_NULL_ARG;
  const gq_status st = kv_check(*cache);
  if (st != GQ_OK) return st;
  *bytes = kv_workspace_bytes(*cache);
  return GQ_OK;
}

gq_status gq_kv_attention(const gq_kv_cache *cache, const void *q, void *out, void *workspace,
                          size_t workspace_bytes, void *stream) {
  if (!cache) return GQ_ERR_NULL_ARG;
  gq_status st = kv_check(*cache);
  if (st != GQ_OK) return st;
  const gq_kv_cache &c = *cache;
  if ((st = check_ptr16(q)) != GQ_OK) return st;
  if (!out) return GQ_ERR_NULL_ARG;
  if ((uintptr_t)out & 1u) return GQ_ERR_ALIGNMENT;
  if (c.t_packed > 0) {
    if ((st = check_ptr16(c.k_codes)) != GQ_OK) return st;
    if ((st = check_ptr16(c.v_codes)) != GQ_OK) return st;
    if (!c.k_scales || !c.k_zeros || !c.v_scales || !c.v_zeros) return GQ_ERR_NULL_ARG;
    if (((uintptr_t)c.k_scales & 1u) || ((uintptr_t)c.v_scales & 1u)) return GQ_ERR_ALIGNMENT;
  }
  if (c.t_window > 0) {
    if ((st = check_ptr16(c.k_window)) != GQ_OK) return st;
    if ((st = check_ptr16(c.v_window)) != GQ_OK) return st;
  }
  const size_t need = kv_workspace_bytes(c);
  if (!workspace || workspace_bytes < need) return GQ_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 255u) return GQ_ERR_ALIGNMENT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return launched(launch_kv(c, q, out, workspace, s), s);
}

const char *gq_status_string(gq_status status) {
  switch (status) {
    case GQ_OK: return "GQ_OK: success";
    case GQ_ERR_NULL_ARG: return "GQ_ERR_NULL_ARG: a required pointer is NULL";
    case GQ_ERR_SHAPE: return "GQ_ERR_SHAPE: invalid K, N, M or block layout";
    case GQ_ERR_BITS: return "GQ_ERR_BITS: bit-widths must be 2, 4 or 8";
    case GQ_ERR_ALIGNMENT: return "GQ_ERR_ALIGNMENT: a device pointer is misaligned";
    case GQ_ERR_DTYPE: return "GQ_ERR_DTYPE: unsupported dtype";
    case GQ_ERR_WORKSPACE: return "GQ_ERR_WORKSPACE: workspace missing or too small";
    case GQ_ERR_HIP: return "GQ_ERR_HIP: the HIP runtime refused a launch";
    case GQ_ERR_TOO_LARGE:
      return "GQ_ERR_TOO_LARGE: the call needs more scratch than the library's static buffer holds";
    case GQ_ERR_UNSUPPORTED:
      return "GQ_ERR_UNSUPPORTED: this path has no kernel for the layout's 8-bit blocks";
  }
  return "unknown gq_status";
}

}  // extern "C"
