// Streaming probes of the HBM (measurement only; kamera_stream_probe in include/kamera.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kamera_desc.h"

namespace kamera {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ============================================================================
// Streaming probes (not part of the operator): plain nontemporal copies, reads and
// writes of 16-byte words, each workgroup over a contiguous 16 KB block, four words per
// thread in flight. They measure the HBM's practical rates for the access kinds the
// operator mixes, so its own rate can be read against them.
// ============================================================================
constexpr int64_t kProbeWords = 1024;   // 16-byte words per workgroup (16 KB)

__global__ __launch_bounds__(kBlockThreads) void probe_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * kProbeWords;
  const int64_t end = min(base + kProbeWords, n16);
  u32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = base + threadIdx.x + kBlockThreads * u;
    if (j < end) v[u] = __builtin_nontemporal_load(src + j);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = base + threadIdx.x + kBlockThreads * u;
    if (j < end) __builtin_nontemporal_store(v[u], dst + j);
  }
}

// reads every word; writes one word per thread to `sink` only if the XOR of what it read
// equals a value no caller's data is built to produce, so the loads cannot be dropped
__global__ __launch_bounds__(kBlockThreads) void probe_read(const u32x4* __restrict__ src, u32x4* __restrict__ sink,
                                                            int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * kProbeWords;
  const int64_t end = min(base + kProbeWords, n16);
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = base + threadIdx.x + kBlockThreads * u;
    if (j < end) acc ^= __builtin_nontemporal_load(src + j);
  }
  if (acc.x == 0x6b616d65u && acc.y == 0x72612d70u && acc.z == 0x726f6265u && acc.w == 0x21212121u)
    sink[threadIdx.x] = acc;
}

__global__ __launch_bounds__(kBlockThreads) void probe_write(u32x4* __restrict__ dst, int64_t n16, uint32_t value) {
  const int64_t base = (int64_t)blockIdx.x * kProbeWords;
  const int64_t end = min(base + kProbeWords, n16);
  const u32x4 v = {value, value, value, value};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = base + threadIdx.x + kBlockThreads * u;
    if (j < end) __builtin_nontemporal_store(v, dst + j);
  }
}

// kind 0: copy src -> dst; 1: read src (dst: a sink of kBlockThreads words); 2: write dst
hipError_t launch_stream_probe(int kind, const void* src, void* dst, int64_t n16, uint32_t value, hipStream_t stream) {
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = (n16 + kProbeWords - 1) / kProbeWords;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kBlockThreads);
  if (kind == 0) hipLaunchKernelGGL(probe_copy, grid, block, 0, stream, (const u32x4*)src, (u32x4*)dst, n16);
  else if (kind == 1) hipLaunchKernelGGL(probe_read, grid, block, 0, stream, (const u32x4*)src, (u32x4*)dst, n16);
  else hipLaunchKernelGGL(probe_write, grid, block, 0, stream, (u32x4*)dst, n16, value);
  return hipGetLastError();
}

}  // namespace kamera
