// Read-bandwidth probe (a measurement helper, not part of the layer): the
// second denominator next to the HBM peak.  Every workgroup streams one
// contiguous slab with 16-byte non-temporal loads (the cache policy the
// expert-weight loads use; 6.2 TB/s without it, 7.0 TB/s with it on the
// MI355X), eight per thread in flight, and folds
// the data into one word so the loads stay live; the word is stored only if
// it equals a value the data never produces in practice.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kProbeBlocks = 2048;
constexpr int kProbeDepth = 8;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

__global__ __launch_bounds__(256) void k_stream_read(const char* __restrict__ src, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b = static_cast<size_t>(blockIdx.x) * per;
  const size_t e = min(n16, b + per);
  uint32_t acc = 0;
  for (size_t i = b + threadIdx.x; i < e; i += 256 * kProbeDepth) {
    u32x4_t v[kProbeDepth];
#pragma unroll
    for (int j = 0; j < kProbeDepth; ++j) {
      const size_t idx = i + static_cast<size_t>(j) * 256;
      v[j] = idx < e ? ld16_stream(src + idx * 16) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kProbeDepth; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  if (acc == kProbeMagic) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(k_stream_read, dim3(kProbeBlocks), dim3(256), 0, st,
                     static_cast<const char*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
