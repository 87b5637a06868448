// Host-side checks of libgq under AddressSanitizer and UndefinedBehavior-
// Sanitizer: every argument check, size query and plan encoding that runs on
// the host before anything is enqueued, on valid, edge and invalid inputs.
// No call here gets past its checks, so no kernel is launched and no GPU is
// needed.  Built host-only (kernels compiled out) by
// tests/test_host_sanitizers.py; exits non-zero on the first failed check
// (the sanitizers abort on their own findings).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "gq.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "host_checks: line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

static int group_size(int b) { return b == 2 ? 64 : 128; }

int main() {
  const uintptr_t A = 0x100000;            // 16-byte aligned, never dereferenced
  size_t c = 0, s = 0, z = 0;

  // ---- layouts and packed sizes
  std::vector<uint8_t> bits(GQ_MAX_BLOCKS + 1, 4);
  gq_layout L{4096, 14336, 14336, bits.data()};
  CHECK(gq_packed_bytes(&L, &c, &s, &z) == GQ_OK);
  CHECK(c == 14336ull * 4096 / 2 && s == 2 * (14336ull * 4096 / 128) && z == s / 2);
  for (int i = 0; i < GQ_MAX_BLOCKS; ++i) bits[i] = i % 3 == 0 ? 8 : (i % 3 == 1 ? 4 : 2);
  gq_layout Lc{1024, GQ_MAX_BLOCKS * 128, 128, bits.data()};
  CHECK(gq_packed_bytes(&Lc, &c, &s, &z) == GQ_OK);
  size_t ec = 0, eg = 0;
  for (int i = 0; i < GQ_MAX_BLOCKS; ++i) {
    ec += 128ull * 1024 * bits[i] / 8;
    eg += 128ull * 1024 / group_size(bits[i]);
  }
  CHECK(c == ec && s == 2 * eg && z == eg);
  gq_layout too_many{1024, (GQ_MAX_BLOCKS + 1) * 128, 128, bits.data()};
  CHECK(gq_packed_bytes(&too_many, &c, &s, &z) == GQ_ERR_SHAPE);
  uint8_t b3 = 3, b8 = 8, b2 = 2;
  gq_layout bad_bits{512, 512, 512, &b3};
  CHECK(gq_packed_bytes(&bad_bits, &c, &s, &z) == GQ_ERR_BITS);
  gq_layout bad_k8{192, 512, 512, &b8};
  CHECK(gq_packed_bytes(&bad_k8, &c, &s, &z) == GQ_ERR_SHAPE);
  gq_layout ok_k2{192, 512, 512, &b2};
  CHECK(gq_packed_bytes(&ok_k2, &c, &s, &z) == GQ_OK);
  gq_layout no_bits{512, 512, 512, nullptr};
  CHECK(gq_packed_bytes(&no_bits, &c, &s, &z) == GQ_ERR_NULL_ARG);
  gq_layout empty{512, 0, 1, nullptr};
  CHECK(gq_packed_bytes(&empty, &c, &s, &z) == GQ_OK && c == 0);
  gq_layout huge_k{INT32_MAX / 4, 1, 1, &b8};
  CHECK(gq_packed_bytes(&huge_k, &c, &s, &z) == GQ_ERR_SHAPE);
  CHECK(gq_packed_bytes(nullptr, &c, &s, &z) == GQ_ERR_NULL_ARG);
  CHECK(gq_packed_bytes(&L, nullptr, &s, &z) == GQ_ERR_NULL_ARG);

  // ---- workspace queries over M, widths and shapes
  std::vector<uint8_t> mix(64);
  for (int i = 0; i < 64; ++i) mix[i] = i % 2 ? 2 : 4;
  const gq_layout shapes[] = {
      {4096, 14336, 14336, bits.data() + 1},   // INT4 uniform (bits[1] == 4)
      {14336, 4096, 4096, bits.data() + 2},    // INT2 uniform (bits[2] == 2)
      {8192, 64 * 128, 128, mix.data()},       // Channel-mix INT4 / INT2
      {64, 5, 5, &b2}, {128, 3, 3, bits.data() + 1},
  };
  const int32_t Ms[] = {0, 1, 2, 4, 5, 16, 17, 32, 33, 64, 255, 256, 2048, 65536};
  for (const gq_layout &l : shapes)
    for (int32_t M : Ms)
      for (gq_dtype act : {GQ_BF16, GQ_FP16}) {
        size_t ws = 0;
        CHECK(gq_linear_workspace_bytes(&l, M, act, &ws) == GQ_OK);
        CHECK(M > 4 || ws == 0);
        const gq_status st = gq_linear_dx_workspace_bytes(&l, M, act, &ws);
        CHECK(st == GQ_OK || (st == GQ_ERR_SHAPE && l.N % 8 != 0));
      }
  size_t ws = 0;
  CHECK(gq_linear_workspace_bytes(&Lc, 5, GQ_BF16, &ws) == GQ_ERR_UNSUPPORTED);
  CHECK(gq_linear_workspace_bytes(&Lc, 4, GQ_BF16, &ws) == GQ_OK && ws == 0);
  CHECK(gq_linear_dx_workspace_bytes(&Lc, 8, GQ_BF16, &ws) == GQ_ERR_UNSUPPORTED);
  CHECK(gq_linear_workspace_bytes(&L, -1, GQ_BF16, &ws) == GQ_ERR_SHAPE);
  CHECK(gq_linear_workspace_bytes(&L, 1, GQ_FP32, &ws) == GQ_ERR_DTYPE);
  CHECK(gq_linear_workspace_bytes(&L, 1, GQ_BF16, nullptr) == GQ_ERR_NULL_ARG);

  // ---- refusals before any launch
  const gq_layout &L4 = shapes[0];
  CHECK(gq_quantize_pack(&L4, nullptr, (uint32_t *)fake(A), (uint16_t *)fake(A), (uint8_t *)fake(A),
                         nullptr, nullptr) == GQ_ERR_NULL_ARG);
  CHECK(gq_quantize_pack(&L4, (const float *)fake(A + 8), (uint32_t *)fake(A), (uint16_t *)fake(A),
                         (uint8_t *)fake(A), nullptr, nullptr) == GQ_ERR_ALIGNMENT);
  CHECK(gq_fake_quant(&L4, (const float *)fake(A), (gq_dtype)7, fake(A), nullptr, nullptr) == GQ_ERR_DTYPE);
  CHECK(gq_dequant(&L4, (const uint32_t *)fake(A), (const uint16_t *)fake(A), (const uint8_t *)fake(A),
                   GQ_FP32, fake(A + 4), nullptr) == GQ_ERR_ALIGNMENT);
  CHECK(gq_linear(&L4, 1, GQ_BF16, fake(A + 2), (const uint32_t *)fake(A), (const uint16_t *)fake(A),
                  (const uint8_t *)fake(A), fake(A), nullptr, 0, nullptr) == GQ_ERR_ALIGNMENT);
  CHECK(gq_linear(&L4, 64, GQ_BF16, fake(A), (const uint32_t *)fake(A), (const uint16_t *)fake(A),
                  (const uint8_t *)fake(A), fake(A), nullptr, 0, nullptr) == GQ_ERR_WORKSPACE);
  CHECK(gq_linear(&Lc, 8, GQ_BF16, fake(A), (const uint32_t *)fake(A), (const uint16_t *)fake(A),
                  (const uint8_t *)fake(A), fake(A), fake(A), 1 << 30, nullptr) == GQ_ERR_UNSUPPORTED);
  CHECK(gq_linear_noalloc(&Lc, 8, GQ_BF16, fake(A), (const uint32_t *)fake(A), (const uint16_t *)fake(A),
                          (const uint8_t *)fake(A), fake(A), nullptr) == GQ_ERR_UNSUPPORTED);
  CHECK(gq_linear_dx(&L4, 8, GQ_BF16, fake(A), (const uint32_t *)fake(A), (const uint16_t *)fake(A),
                     (const uint8_t *)fake(A), fake(A), nullptr, 0, nullptr) == GQ_ERR_WORKSPACE);

  // ---- KV cache checks
  gq_kv_cache kc;
  memset(&kc, 0, sizeof(kc));
  kc.batch = 2; kc.q_heads = 32; kc.kv_heads = 8; kc.head_dim = 128; kc.bits = 4;
  kc.t_packed = 4096; kc.t_window = 64;
  CHECK(gq_kv_attention_workspace_bytes(&kc, &ws) == GQ_OK && ws > 0);
  kc.head_dim = 64;
  CHECK(gq_kv_attention_workspace_bytes(&kc, &ws) != GQ_OK);
  kc.head_dim = 128; kc.bits = 8;
  CHECK(gq_kv_attention_workspace_bytes(&kc, &ws) != GQ_OK);
  kc.bits = 2; kc.q_heads = 24;               // 3 query heads per key/value head
  CHECK(gq_kv_attention_workspace_bytes(&kc, &ws) != GQ_OK);
  CHECK(gq_kv_attention_workspace_bytes(nullptr, &ws) == GQ_ERR_NULL_ARG);

  // ---- grouped decode plans: 300 linears of mixed widths and layouts
  std::vector<gq_group_item> items;
  std::vector<std::vector<uint8_t>> maps;
  for (int i = 0; i < 300; ++i) {
    const int kind = i % 5;
    const int32_t K = kind == 1 ? 14336 : (kind == 4 ? 1024 : 4096);
    const int32_t N = kind == 2 ? 384 : (kind == 3 ? 1000 : 4096);
    const int32_t bn = kind == 2 ? 128 : N;
    maps.emplace_back(N / bn);
    for (size_t j = 0; j < maps.back().size(); ++j) maps.back()[j] = (i + j) % 3 == 0 ? 8 : ((i + j) % 3 == 1 ? 4 : 2);
    gq_group_item it;
    it.layout = {K, N, bn, maps.back().data()};
    it.x = fake(A); it.codes = (const uint32_t *)fake(A); it.scales = (const uint16_t *)fake(A);
    it.zeros = (const uint8_t *)fake(A); it.y = fake(A);
    items.push_back(it);
  }
  for (int32_t M = 1; M <= 4; ++M) {
    size_t need = 0;
    CHECK(gq_group_plan_bytes((int32_t)items.size(), items.data(), M, GQ_BF16, &need) == GQ_OK && need > 0);
    std::vector<uint8_t> plan(need + 64);
    CHECK(gq_group_plan((int32_t)items.size(), items.data(), M, GQ_BF16, plan.data(), need - 1) == GQ_ERR_WORKSPACE);
    CHECK(gq_group_plan((int32_t)items.size(), items.data(), M, GQ_BF16, plan.data(), need) == GQ_OK);
    // the launch checks the host plan, then refuses a misaligned device copy
    CHECK(gq_linear_group(plan.data(), fake(A + 8), nullptr) == GQ_ERR_ALIGNMENT);
    std::vector<uint8_t> junk(need, 0x5a);
    CHECK(gq_linear_group(junk.data(), fake(A), nullptr) == GQ_ERR_SHAPE);
  }
  size_t need = 0;
  CHECK(gq_group_plan_bytes(0, items.data(), 1, GQ_BF16, &need) == GQ_ERR_SHAPE);
  CHECK(gq_group_plan_bytes(1, items.data(), 5, GQ_BF16, &need) == GQ_ERR_SHAPE);
  CHECK(gq_group_plan_bytes(1, items.data(), 1, GQ_FP32, &need) == GQ_ERR_DTYPE);
  items[7].x = fake(A + 4);
  CHECK(gq_group_plan_bytes((int32_t)items.size(), items.data(), 1, GQ_BF16, &need) == GQ_ERR_ALIGNMENT);
  CHECK(gq_linear_group(nullptr, fake(A), nullptr) == GQ_ERR_NULL_ARG);

  // ---- status strings
  for (int st = 0; st <= 9; ++st) CHECK(strncmp(gq_status_string((gq_status)st), "GQ_", 3) == 0);
  CHECK(strncmp(gq_status_string((gq_status)99), "unknown", 7) == 0);
  printf("host_checks: all checks passed\n");
  return 0;
}
