// Device code of the routing kernels: the part sums of small-batch router
// logits and the exact top-k of one token.
//
// Reference: "Agent Field Notes -- full corpus", AFN-001, section "Phase 1:
// separate math from acceleration" (float32 router softmax and normalized
// top-10 selection); AFN-017, section "Tie handling belongs to membership"
// (equal scores: the smaller index is chosen).
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kRouterBatch = 8;

// One part of a 16-token x 16-expert logit tile, by one wave: float32
// chunk sums from MFMA, added in float64 in k order.  slot[lane][j]
// receives the part sum of expert e0 + 4q + j, token t0 + r (lane = r + 16 q).
__device__ __forceinline__ void router_part(const uint16_t* __restrict__ x,
                                            const uint16_t* __restrict__ wr, int T, int H, int E,
                                            int nparts, int t0, int e0, int part,
                                            double (*slot)[4]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int cpp = H / 32 / nparts;
  const int kbeg = part * cpp * 32;
  const int tt = min(t0 + r, T - 1);
  const int ee = min(e0 + r, E - 1);
  const uint16_t* xp = x + static_cast<size_t>(tt) * H + kbeg + q * 8;
  const uint16_t* wp = wr + static_cast<size_t>(ee) * H + kbeg + q * 8;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < cpp; c += kRouterBatch) {
    u32x4_t a[kRouterBatch], b[kRouterBatch];
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      if (c + u < cpp) {
        a[u] = ld16_stream(wp + (c + u) * 32);
        b[u] = ld16(xp + (c + u) * 32);
      }
    }
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      if (c + u < cpp) {
        const f32x4_t f = mfma_bf16(a[u], b[u], zero);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += static_cast<double>(f[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) slot[lane][j] = acc[j];
}

// Wave 0 after a barrier: the `np` part sums of one group added in part
// order (float64) and stored to gsum[t][e] (the group's slice [T][E]).
__device__ __forceinline__ void router_group_store(const double (*red)[64][4], int np, int T,
                                                   int E, int t0, int e0,
                                                   double* __restrict__ gsum) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int t = t0 + r;
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 4 * q + j;
    if (e < E) {
      double s = red[0][lane][j];
      for (int w = 1; w < np; ++w) s += red[w][lane][j];
      gsum[static_cast<size_t>(t) * E + e] = s;
    }
  }
}

// Exact top-k of one token by one wave; lane l holds the logits v[j] of
// experts j*64 + l (NV slots, E <= 64 NV; slots at or past E are ignored).
// Each of the k rounds takes the wave maximum m of the remaining logits,
// then the smallest expert index whose logit equals m -- the total order
// (logit descending, index ascending) -- with DPP row reductions and
// readlanes (no LDS round trips).  -0.0 and +0.0 compare equal.  Weights:
// exp(l_j - l_0) / sum over the selected, in float32 (the full softmax
// renormalized over the selection).  `sel` is this wave's LDS scratch of k
// floats.  DEV: the ids are stored device-coherent (another workgroup of the
// same launch reads them).
template <int NV, bool DEV = false>
__device__ __forceinline__ void topk_select(const float (&v)[NV], int E, int k, float* sel,
                                            int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  uint32_t live = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j)
    if (j * 64 + lane < E) live |= 1u << j;
  for (int rnk = 0; rnk < k; ++rnk) {
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if ((live >> j) & 1u) lm = fmaxf(lm, v[j]);
    const float m = wave_max_f32(lm);
    uint32_t li = 0xffffffffu;
#pragma unroll
    for (int j = NV - 1; j >= 0; --j)
      if (((live >> j) & 1u) && v[j] == m) li = static_cast<uint32_t>(j * 64 + lane);
    const uint32_t e = wave_min_u32(li);
    if (static_cast<int>(e & 63u) == lane) live &= ~(1u << (e >> 6));
    if (lane == 0) {
      if constexpr (DEV)
        store_dev_i32(ids + rnk, static_cast<int32_t>(e));
      else
        ids[rnk] = static_cast<int32_t>(e);
      sel[rnk] = m;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float m0 = sel[0];
  float part = 0.f;
  for (int rnk = lane; rnk < k; rnk += 64) {
    const float ex = expf(sel[rnk] - m0);
    sel[rnk] = ex;
    part += ex;
  }
  const float sum = wave_sum_f32(part);
  for (int rnk = lane; rnk < k; rnk += 64) w[rnk] = sel[rnk] / sum;
}

}  // namespace moe
