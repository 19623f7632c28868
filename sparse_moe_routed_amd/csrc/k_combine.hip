// Route-rank-order weighted combine (+ residual).
//
// Reference: "Agent Field Notes -- full corpus", AFN-019 "Hide SSD misses
// before the router knows they exist", section "Hypothesis H4: ExpertMajor
// should stream as a wavefront, not a barrier": experts write separate result
// slots and the final weighted sum follows a deterministic route-rank order.
//
// out[t][n] = residual[t][n] + sum_{j=0}^{k-1} w[t][j] * y[pair_row[t*k+j]][n]
// The sum runs in float32 with j ascending, then the residual is added and
// the result rounded once to the activation type.  One thread per 8 (bf16)
// or 4 (float32) consecutive features; loads are 16 bytes.
#include "combine_device.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// One thread per token and 16-byte chunk: combine_chunk_bf16 with the rows
// of the token's slots taken from pair_row, or (PAIRY: y already in pair
// order) rows t*k .. t*k + k-1.
template <int KB, bool PAIRY>
__global__ __launch_bounds__(256) void k_combine_bf16(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ res,
                                                      uint16_t* __restrict__ out, int T, int H,
                                                      int k) {
  const int chunks = H >> 3;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * chunks) return;
  const int t = static_cast<int>(idx / chunks), c = static_cast<int>(idx % chunks);
  const int P = T * k;
  const int32_t* pr = PAIRY ? nullptr : pair_row + static_cast<size_t>(t) * k;
  combine_chunk_bf16<KB>([&](int row, int cc) { return ld16(y + static_cast<size_t>(row) * H + cc * 8); },
                         [&](int j) { return PAIRY ? t * k + j : min(max(pr[j], 0), P - 1); }, w,
                         res, out, t, c, H, k);
}

__global__ __launch_bounds__(256) void k_combine_f32(const float* __restrict__ y,
                                                     const int32_t* __restrict__ pair_row,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ res,
                                                     float* __restrict__ out, int T, int H, int k) {
  const int chunks = H >> 2;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * chunks) return;
  const int t = static_cast<int>(idx / chunks), c = static_cast<int>(idx % chunks);
  const int P = T * k;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int row = min(max(pair_row[static_cast<size_t>(t) * k + j], 0), P - 1);
    const float wj = w[static_cast<size_t>(t) * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + static_cast<size_t>(row) * H + c * 4);
    acc[0] = fmaf(wj, v.x, acc[0]);
    acc[1] = fmaf(wj, v.y, acc[1]);
    acc[2] = fmaf(wj, v.z, acc[2]);
    acc[3] = fmaf(wj, v.w, acc[3]);
  }
  if (res) {
    const float4 v = *reinterpret_cast<const float4*>(res + static_cast<size_t>(t) * H + c * 4);
    acc[0] += v.x;
    acc[1] += v.y;
    acc[2] += v.z;
    acc[3] += v.w;
  }
  *reinterpret_cast<float4*>(out + static_cast<size_t>(t) * H + c * 4) =
      make_float4(acc[0], acc[1], acc[2], acc[3]);
}

hipError_t launch_combine(const moe_shape& s, const void* y, const int32_t* pair_row,
                          const float* w, const void* residual, void* out, hipStream_t st) {
  if (s.act == MOE_DT_BF16) {
    const size_t n = static_cast<size_t>(s.T) * (s.H / 8);
    // pair_row == nullptr: y rows are in pair order
    auto kern = s.top_k <= 16 ? (pair_row ? k_combine_bf16<16, false> : k_combine_bf16<16, true>)
                              : (pair_row ? k_combine_bf16<8, false> : k_combine_bf16<8, true>);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       st, static_cast<const uint16_t*>(y), pair_row, w,
                       static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out), s.T,
                       s.H, s.top_k);
  } else {
    const size_t n = static_cast<size_t>(s.T) * (s.H / 4);
    hipLaunchKernelGGL(k_combine_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       st, static_cast<const float*>(y), pair_row, w,
                       static_cast<const float*>(residual), static_cast<float*>(out), s.T, s.H,
                       s.top_k);
  }
  return hipGetLastError();
}

}  // namespace moe
