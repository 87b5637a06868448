// Streaming-read probe: the measured ceiling the decode kernels are set
// against.  It reads a device buffer once with the loads the decode kernels
// use for codes (128-bit, nontemporal, coalesced) and no arithmetic beyond a
// running XOR, so its time is what the memory system gives a kernel that
// moves the same bytes in one launch: the ramp of the first loads, the
// transfer and the drain of the last ones.  It is measurement
// infrastructure, built as its own library (libgq_probe.so) and called only
// by the benchmark.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLoads = 4;   // 16-byte loads per thread: a workgroup reads 16 KB

// Workgroup b reads the 16-byte words [b * 1024, (b + 1) * 1024), each lane
// every 256th one, so every load instruction of a wave covers 1 KB of
// consecutive bytes.  The XOR of everything read is stored only if it equals
// a value the caller cannot make it equal by chance in practice; the store
// keeps the loads from being removed.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                               uint32_t *__restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * kThreads * kLoads + threadIdx.x;
  u32x4 v[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const size_t i = base + (size_t)u * kThreads;
    if (i < n16) v[u] = __builtin_nontemporal_load(p + i);
    else v[u] = u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kLoads; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

// Read `bytes` bytes at device address `buf` (16-byte aligned, bytes a
// multiple of 16) on `stream` (a hipStream_t; null for the default stream).
// `sink` is one device uint32 the kernel may write.  Returns 0, or -1 for a
// bad argument (nothing enqueued), or the HIP error of the launch.
extern "C" int gqprobe_stream_read(const void *buf, size_t bytes, void *sink, void *stream) {
  if (!buf || !sink || bytes == 0 || (bytes & 15u) != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return -1;
  const size_t n16 = bytes / 16;
  const size_t per = (size_t)kThreads * kLoads;
  const size_t grid = (n16 + per - 1) / per;
  if (grid > 0x7fffffffu) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf), n16,
                     static_cast<uint32_t *>(sink));
  return (int)hipGetLastError();
}
