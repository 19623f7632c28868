// Staging of the active experts' records into device memory ("Agent Field
// Notes -- full corpus", AFN-019, section "Hypothesis H5: prefill and decode
// need different streaming modes": a block reads the deduplicated union of
// its routes; section "Why overlap alone cannot defeat the byte roofline":
// exact bytes first).  The GPU reads the source records directly (host
// memory over PCIe, or device memory), so the active set never has to reach
// the host.  Pure byte copies.
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kStageChunk = 256 * 16 * 16;   // bytes per workgroup and piece

// grid (chunks of the largest piece, E); workgroup (c, a) copies chunk c of
// every piece of the a-th active expert.
__global__ __launch_bounds__(256) void k_stage_experts(StagePieces pc, const int32_t* __restrict__ active,
                                                       const int32_t* __restrict__ n_active, int E) {
  const int a = static_cast<int>(blockIdx.y);
  if (a >= min(max(n_active[0], 0), E)) return;
  const int e = active[a];
  if (e < 0 || e >= E) return;
  const size_t c0 = static_cast<size_t>(blockIdx.x) * kStageChunk;
#pragma unroll 1
  for (int m = 0; m < kStagePieces; ++m) {
    const size_t n = pc.bytes[m];
    if (!pc.src[m] || c0 >= n) continue;
    const char* s = pc.src[m] + static_cast<size_t>(e) * n;
    char* d = pc.dst[m] + static_cast<size_t>(e) * n;
    const size_t end = min(n, c0 + kStageChunk);
    u32x4_t v[16];
    // 16 loads in flight per thread, then the stores
    for (size_t o = c0 + threadIdx.x * 16; o < end; o += 256 * 16 * 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const size_t p = o + static_cast<size_t>(i) * 256 * 16;
        if (p < end) v[i] = ld16(s + p);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const size_t p = o + static_cast<size_t>(i) * 256 * 16;
        if (p < end) *reinterpret_cast<u32x4_t*>(d + p) = v[i];
      }
    }
  }
}

hipError_t launch_stage_experts(const moe_shape& s, const StagePieces& pc, const int32_t* active,
                                const int32_t* n_active, hipStream_t st) {
  size_t mx = 0;
  for (int m = 0; m < kStagePieces; ++m)
    if (pc.src[m]) mx = std::max(mx, pc.bytes[m]);
  const unsigned chunks = static_cast<unsigned>((mx + kStageChunk - 1) / kStageChunk);
  hipLaunchKernelGGL(k_stage_experts, dim3(chunks, s.E), dim3(256), 0, st, pc, active, n_active, s.E);
  return hipGetLastError();
}

}  // namespace moe
