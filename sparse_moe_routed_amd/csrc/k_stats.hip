// Route locality of one call's token sequence ("Agent Field Notes -- full
// corpus", AFN-019, section "Hypothesis H7: DFlash block size must follow
// I/O cost" and the trace-only locality gate: overlap with the previous
// token, unions of consecutive blocks of 2-5 tokens).  Integer counts,
// exact.  Values of topk_ids are only
// compared, never used as addresses.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// One wave per output value: overlap of token t (outputs 0..T-1), then the
// block unions (B = 1..5 in turn).  The wave copies the ids it needs (tokens
// t-1 and t, or the block's tokens: at most 5 top_k values) into LDS, each
// lane tests some of them, and a wave sum gives the count.
__global__ __launch_bounds__(64) void k_route_locality(const int32_t* __restrict__ ids, int T, int k,
                                                       int32_t* __restrict__ overlap,
                                                       int32_t* __restrict__ block_unique) {
  extern __shared__ int32_t sids[];
  const int i = static_cast<int>(blockIdx.x), lane = static_cast<int>(threadIdx.x);
  int t0, t1, j = 0, o = 0;
  if (i < T) {
    if (i == 0) {
      if (lane == 0) overlap[0] = 0;
      return;
    }
    t0 = i - 1;
    t1 = i + 1;
  } else {
    j = i - T;
    int B = 1;
    for (; B <= kMaxLocalityBlock; ++B) {
      const int nb = (T + B - 1) / B;
      if (j < nb) break;
      j -= nb;
      o += nb;
    }
    if (B > kMaxLocalityBlock) return;        // past the last output
    t0 = j * B;
    t1 = min(T, t0 + B);
  }
  const int n = (t1 - t0) * k;
  for (int p = lane; p < n; p += 64) sids[p] = ids[static_cast<size_t>(t0) * k + p];
  __syncthreads();
  int c = 0;
  if (i < T) {
    // ids of token i that token i-1 also selects
    for (int a = lane; a < k; a += 64) {
      const int32_t e = sids[k + a];
      for (int b = 0; b < k; ++b)
        if (sids[b] == e) {
          ++c;
          break;
        }
    }
  } else {
    // an expert counts at its first token in the block (one token's ids
    // are distinct)
    for (int p = lane; p < n; p += 64) {
      const int32_t e = sids[p];
      const int before = (p / k) * k;
      bool seen = false;
      for (int q = 0; q < before; ++q)
        if (sids[q] == e) {
          seen = true;
          break;
        }
      c += seen ? 0 : 1;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, 64);
  if (lane == 0) {
    if (i < T) overlap[i] = c;
    else block_unique[o + j] = c;
  }
}

hipError_t launch_route_locality(const moe_shape& s, const int32_t* ids, int32_t* overlap,
                                 int32_t* block_unique, hipStream_t st) {
  const int n = s.T + locality_blocks(s.T);
  const size_t lds = static_cast<size_t>(kMaxLocalityBlock) * s.top_k * sizeof(int32_t);
  hipLaunchKernelGGL(k_route_locality, dim3(n), dim3(64), lds, st, ids, s.T, s.top_k, overlap,
                     block_unique);
  return hipGetLastError();
}

}  // namespace moe
