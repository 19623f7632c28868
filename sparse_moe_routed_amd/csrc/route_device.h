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
// The router rows are read with the default cache policy, not as a
// non-temporal stream like the expert records: they are a few MB that every
// call reads again (measured: decode step 1.5 us and the 48-layer verifier
// step 1.4% faster than with non-temporal loads).
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
        a[u] = ld16(wp + (c + u) * 32);
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

// Order-preserving integer key of a logit: a > b (as floats) exactly when
// key(a) > key(b); -0.0 keys as +0.0 (the two compare equal), NaN keys as 0,
// below every other value, and every other value keys above 0.
__device__ __forceinline__ uint32_t logit_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  const uint32_t kk = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return f != f ? 0u : kk;
}
__device__ __forceinline__ float logit_of_key(uint32_t kk) {
  return __uint_as_float((kk & 0x80000000u) ? (kk & 0x7fffffffu) : ~kk);
}

// LDS written by lanes of this wave is visible to its other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The selection of topk_select by k rounds (any k; the fallback of
// topk_threshold): each round takes the wave maximum m of the remaining
// logits, then the smallest expert index whose logit equals m -- the total
// order (logit descending, index ascending) -- with DPP row reductions and
// readlanes (no LDS round trips).  -0.0 and +0.0 compare equal.  Writes
// ids[r] and sel[r] (the logit) for every rank r < k.
template <int NV, bool DEV>
__device__ __forceinline__ void topk_rounds(const float (&v)[NV], int E, int k, float* sel,
                                            int32_t* __restrict__ ids) {
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
}

// The selection of topk_select for k <= 64 without k dependent rounds.  With
// integer keys (logit_key; ignored slots key as 0) and lane maxima m_l:
// tau = the k-th largest m_l (each lane counts the maxima >= its own from
// LDS; tau is the largest m_l whose count reaches k).  The k lanes holding
// the k largest maxima give k distinct logits >= tau, so the k-th largest
// logit is >= tau and every logit of the top k has key >= tau.  The keys >=
// tau (the candidates, each with its expert index) are packed into LDS in
// lane order, and every candidate's rank is the number of candidates
// before it in the total order (key descending, index ascending) -- the
// rank it has among all logits, since everything before it is a
// candidate too.  Ranks below k give ids[r] and sel[r].  Returns false,
// having written no id, when fewer than k logits are selectable (tau = 0)
// or more than 64 keys reach tau (massive ties); sel[0 .. 191] is scratch.
template <int NV, bool DEV>
__device__ __forceinline__ bool topk_threshold(const float (&v)[NV], int E, int k, float* sel,
                                               int32_t* __restrict__ ids) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NV];
  uint32_t lm = 0u;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    key[j] = (j * 64 + lane < E) ? logit_key(v[j]) : 0u;
    lm = max(lm, key[j]);
  }
  uint32_t* S = reinterpret_cast<uint32_t*>(sel);
  S[lane] = lm;
  wave_lds_sync();
  uint32_t cc[4] = {0u, 0u, 0u, 0u};   // four independent count chains
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const u32x4_t a = reinterpret_cast<const u32x4_t*>(S)[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) cc[i] += a[i] >= lm ? 1u : 0u;
  }
  const uint32_t c = (cc[0] + cc[1]) + (cc[2] + cc[3]);
  const uint32_t tau = wave_max_u32(c >= static_cast<uint32_t>(k) ? lm : 0u);
  if (tau == 0u) return false;
  uint32_t bits = 0u;
#pragma unroll
  for (int j = 0; j < NV; ++j) bits |= (key[j] >= tau ? 1u : 0u) << j;
  const uint32_t cnt = __popc(bits);
  // exclusive prefix of the per-lane counts (<= 16: five bit planes)
  uint32_t pre = 0u, C = 0u;
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    const uint64_t m = __ballot((cnt >> b) & 1u);
    pre += __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u))
           << b;
    C += static_cast<uint32_t>(__popcll(m)) << b;
  }
  if (C > 64u) return false;
  uint32_t* ck = S + 64;    // candidate keys
  uint32_t* ci = S + 128;   // candidate expert indices
  uint32_t pos = pre;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    if ((bits >> j) & 1u) {
      ck[pos] = key[j];
      ci[pos] = static_cast<uint32_t>(j * 64 + lane);
      ++pos;
    }
  }
  wave_lds_sync();
  if (static_cast<uint32_t>(lane) < C) {
    const uint32_t kl = ck[lane], il = ci[lane];
    uint32_t rank = 0u;
    for (uint32_t q = 0; q < (C + 3u) / 4u; ++q) {
      const u32x4_t a = reinterpret_cast<const u32x4_t*>(ck)[q];
      const u32x4_t b = reinterpret_cast<const u32x4_t*>(ci)[q];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rank += (4u * q + i < C && (a[i] > kl || (a[i] == kl && b[i] < il))) ? 1u : 0u;
    }
    if (rank < static_cast<uint32_t>(k)) {
      if constexpr (DEV)
        store_dev_i32(ids + rank, static_cast<int32_t>(il));
      else
        ids[rank] = static_cast<int32_t>(il);
      sel[rank] = logit_of_key(kl);   // over the lane maxima, no longer read
    }
  }
  return true;
}

// Exact top-k of one token by one wave; lane l holds the logits v[j] of
// experts j*64 + l (NV slots, E <= 64 NV; slots at or past E are ignored),
// in the total order (logit descending, index ascending; -0.0 and +0.0
// compare equal): topk_threshold for k <= 64, else (or when it cannot
// decide) topk_rounds.  Weights: exp(l_j - l_0) / sum over the selected, in
// float32 (the full softmax renormalized over the selection).  `sel` is this
// wave's LDS scratch of max(k, 192) floats.  DEV: the ids are stored
// device-coherent (another workgroup of the same launch reads them).
template <int NV, bool DEV = false>
__device__ __forceinline__ void topk_select(const float (&v)[NV], int E, int k, float* sel,
                                            int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  if (!(k <= 64 && topk_threshold<NV, DEV>(v, E, k, sel, ids))) {
    wave_lds_sync();
    topk_rounds<NV, DEV>(v, E, k, sel, ids);
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
