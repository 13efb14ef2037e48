// Read-bandwidth reference for the HBM-bound kernels' rooflines: one streaming pass
// over a buffer, the plainest access pattern the chip serves (every workgroup reads
// one contiguous chunk, 16 independent 16-byte loads per lane in flight, nothing
// written but one checksum word per workgroup).  Timing it on the same buffer, box
// and cache state as a decode-shape GEMM shows how much of the nominal 8 TB/s a read
// of that size can reach at all.  The checksum (XOR of the chunk's 32-bit words)
// keeps the loads live and lets a test confirm that every byte was read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fgemm.h"

namespace fgemm {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 16;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src,
                                                                   int64_t n16, int64_t per_group,
                                                                   uint32_t* __restrict__ out) {
  const int64_t start = (int64_t)blockIdx.x * per_group;
  const int64_t end = start + per_group < n16 ? start + per_group : n16;
  uint32_t acc = 0;
  for (int64_t base = start; base < end; base += kProbeThreads * kProbeUnroll) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) {
      const int64_t i = base + j * kProbeThreads + threadIdx.x;
      v[j] = i < end ? src[i] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // XOR across the wave, then across the workgroup's four waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) x ^= part[w];
    out[blockIdx.x] = x;
  }
}

}  // namespace
}  // namespace fgemm

extern "C" fgemm_status_t fgemm_read_probe(const void* src, int64_t bytes, uint32_t* out,
                                           void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || !out) return FGEMM_ERR_INVALID_VALUE;
  if (bytes > 0 && (!src || reinterpret_cast<uintptr_t>(src) % 16 != 0))
    return FGEMM_ERR_INVALID_VALUE;
  const int64_t n16 = bytes / 16;
  const int64_t per_group = (n16 + FGEMM_READ_PROBE_GROUPS - 1) / FGEMM_READ_PROBE_GROUPS;
  // every group writes its word, so an empty buffer still leaves out[] defined (zeros)
  hipLaunchKernelGGL(fgemm::read_probe_kernel, dim3(FGEMM_READ_PROBE_GROUPS),
                     dim3(fgemm::kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), n16, per_group, out);
  return hipGetLastError() == hipSuccess ? FGEMM_OK : FGEMM_ERR_HIP;
}
