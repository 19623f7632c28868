// Device-side finiteness checks for MOE_F_CHECK_FINITE (non-finite
// rejection before publication: "Agent Field Notes -- full corpus", AFN-010,
// section "The publication model").  A status word in the workspace collects
// one bit per checked tensor; the host reads it after synchronizing.
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(64) void k_zero_u32(uint32_t* __restrict__ p) {
  if (threadIdx.x == 0) p[0] = 0u;
}

// Sets `bit` in *status when any of the n values is NaN or +-infinity (an
// all-ones exponent field).  bf16: n halfwords; float32: n words.  Each
// thread reads 16 bytes per step; a wave that found one sets the bit once.
template <bool BF16>
__global__ __launch_bounds__(256) void k_check_finite(const void* __restrict__ src, size_t n,
                                                      uint32_t bit, uint32_t* __restrict__ status) {
  const size_t per = BF16 ? 8 : 4;                       // elements per 16 bytes
  const size_t chunks = n / per;
  bool bad = false;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t c = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks; c += stride) {
    const u32x4_t v = ld16(static_cast<const char*>(src) + c * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (BF16) {
        bad |= (v[j] & 0x7F80u) == 0x7F80u || (v[j] & 0x7F800000u) == 0x7F800000u;
      } else {
        bad |= (v[j] & 0x7F800000u) == 0x7F800000u;
      }
    }
  }
  // tail (n not a multiple of 16 bytes)
  const size_t t = chunks * per + static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < n) {
    if constexpr (BF16) {
      const uint16_t u = static_cast<const uint16_t*>(src)[t];
      bad |= (u & 0x7F80u) == 0x7F80u;
    } else {
      const uint32_t u = static_cast<const uint32_t*>(src)[t];
      bad |= (u & 0x7F800000u) == 0x7F800000u;
    }
  }
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) atomicOr(status, bit);
}

hipError_t launch_zero_status(uint32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, st, status);
  return hipGetLastError();
}

hipError_t launch_check_finite(const void* src, size_t n, bool bf16, uint32_t bit,
                               uint32_t* status, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t per = bf16 ? 8 : 4;
  const size_t chunks = n / per;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>(std::max<size_t>((chunks + 255) / 256, 1), 1024));
  if (bf16)
    hipLaunchKernelGGL(k_check_finite<true>, dim3(blocks), dim3(256), 0, st, src, n, bit, status);
  else
    hipLaunchKernelGGL(k_check_finite<false>, dim3(blocks), dim3(256), 0, st, src, n, bit, status);
  return hipGetLastError();
}

}  // namespace moe
