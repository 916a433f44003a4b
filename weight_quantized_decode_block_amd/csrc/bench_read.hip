// Measurement helper for bench.py (not part of the product C ABI): a plain
// coalesced read of a device buffer, the single-launch HBM read ceiling for a
// weight matrix of the same size on the same cold ring.
//
// Each thread reads four 16-byte chunks (consecutive threads, consecutive
// addresses), XORs them and stores nothing unless the result equals a value
// that the caller makes impossible (*sink is written only for a fixed
// pattern), so the compiler keeps the loads and the kernel writes no bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kPerThread = 4;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4_t *__restrict__ p, uint64_t chunks,
                                                        uint32_t *__restrict__ sink) {
  const uint64_t base = (uint64_t)blockIdx.x * kThreads * kPerThread + threadIdx.x;
  u32x4_t v[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const uint64_t c = base + (uint64_t)u * kThreads;
    v[u] = c < chunks ? p[c] : (u32x4_t){0u, 0u, 0u, 0u};
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (x == 0x9E3779B9u && threadIdx.x == 0u) *sink = x;
}

}  // namespace

// Reads `bytes` (a multiple of 16) starting at the 16-byte aligned device
// pointer `p` on `stream`.  `sink` is a device word the kernel writes only in
// the (data-dependent, practically never met) case above.  Returns a
// hipError_t value.
extern "C" int wqd_bench_read(const void *p, uint64_t bytes, uint32_t *sink, hipStream_t stream) {
  if (p == nullptr || sink == nullptr || (bytes & 15u) != 0u || ((uintptr_t)p & 15u) != 0u)
    return (int)hipErrorInvalidValue;
  const uint64_t chunks = bytes / 16u;
  if (chunks == 0u) return 0;
  const uint64_t grid = (chunks + kThreads * kPerThread - 1) / (kThreads * kPerThread);
  hipLaunchKernelGGL(read_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t *>(p), chunks, sink);
  return (int)hipGetLastError();
}
