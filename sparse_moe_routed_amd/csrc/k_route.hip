// Router logits and exact top-k selection.
//
// Reference: "Agent Field Notes -- full corpus", AFN-001 "Porting
// Qwen3.8-Flash-Next to Hebrus: evidence before execution", section "Phase 1:
// separate math from acceleration" (float32 router softmax and normalized
// top-10 selection); AFN-021 "Replay decode as prefill", section "The key
// equivalence -- and where it breaks" (exact IDs in rank order); AFN-017 "Top-k
// chooses the set; time chooses the order", section "Tie handling belongs to
// membership" (equal scores: the smaller index is chosen during membership).
#include <climits>

#include "moe_device.h"
#include "moe_internal.h"
#include "perm_device.h"
#include "route_device.h"

namespace moe {

// bf16 router.  The dot product over H is cut into `nparts` parts of
// `cpp` chunks of 32 (nparts = the largest divisor of H/32 that is <= 16, so
// the cut depends on H alone), and the parts into groups of kRouterGroup
// consecutive parts (the last group may be shorter).  Each
// v_mfma_f32_16x16x32_bf16 sums the 32 exact bf16 products of a chunk in
// float32; the chunk sums of a part are added in float64 in k order, the
// part sums of a group in part order, the group sums in group order, then
// the bias is added and the total is rounded once to float32.  Every path
// below uses exactly this association, so a token's logits are
// bit-identical whatever the batch size or the kernels that computed them.

// Small batches: one workgroup per (16-token x 16-expert tile, group of
// parts), one wave per part; the group's part sums are added through LDS and
// stored in float64 to gsum[group][T][E] (the top-k kernel finishes the
// logits).  `arrive` (route + permute in one call): the top-k kernel's
// arrival counter, zeroed here.  grid (ceil(T/16), ceil(E/16), ngroups),
// block 64 * kRouterGroup.
__global__ __launch_bounds__(64 * kRouterGroup) void k_router_parts(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E,
    int nparts, double* __restrict__ gsum, int32_t* __restrict__ arrive) {
  __shared__ double red[kRouterGroup][64][4];
  const int wave = threadIdx.x >> 6;
  if (arrive != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
    *arrive = 0;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16, g = blockIdx.z;
  const int p0 = g * kRouterGroup, np = min(kRouterGroup, nparts - p0);
  if (wave < np) router_part(x, wr, T, H, E, nparts, t0, e0, p0 + wave, red[wave]);
  __syncthreads();
  if (wave == 0) router_group_store(red, np, T, E, t0, e0, gsum + static_cast<size_t>(g) * T * E);
}

// Larger batches: workgroup tile of 32 A tokens x 32 A experts, four waves
// in 2 x 2, each (16 A) x (16 A).  Token rows and router rows are staged in
// LDS once per workgroup and 128-wide k unit (in MFMA fragment order), and
// each wave walks the 32-wide chunks in k order, keeping float64 part,
// group and total sums per output (the association above).  Two LDS
// buffers: the next unit is loaded while the current one is multiplied.
// GS: one workgroup per (tile, group of parts) covering only that group's
// units, storing the float64 group sums to gsum[group][T][E] (the top-k
// kernel finishes the logits); otherwise the whole H and the finished
// logits.  A group spans whole 128-k units: H/32 = nparts * cpp is a
// multiple of 4, and so is every group's chunk count.
// grid (ceil(T / 32 A), ceil(E / 32 A), GS ? groups : 1), block 256.
template <int A, bool GS>
__global__ __launch_bounds__(256) void k_router_lds(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wr,
                                                    const float* __restrict__ bias, int T, int H,
                                                    int E, int nparts,
                                                    float* __restrict__ logits,
                                                    double* __restrict__ gsum) {
  constexpr int NB = 2 * A;   // 16-row blocks per staged tile
  __shared__ __align__(16) char xs[2][NB * 4096];
  __shared__ __align__(16) char wsm[2][NB * 4096];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int tb = blockIdx.x * 32 * A, eb = blockIdx.y * 32 * A;
  const int tblk = (wave & 1) * A, eblk = (wave >> 1) * A;
  const int cpp = H / 32 / nparts;
  const int g = GS ? static_cast<int>(blockIdx.z) : 0;
  const int ubeg = GS ? g * cpp : 0;                                   // 4 cpp chunks per group
  const int units = GS ? min(kRouterGroup * (g + 1), nparts) * cpp / 4 - ubeg : H / 128;

  XUnit<NB> xu, wu;
  xu.init(x, [&](int R) { return static_cast<size_t>(min(tb + R, T - 1)) * H; });
  wu.init(wr, [&](int R) { return static_cast<size_t>(min(eb + R, E - 1)) * H; });

  double part[A][A][4], grp[A][A][4], tot[A][A][4];
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[a][i][j] = grp[a][i][j] = tot[a][i][j] = 0.0;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

  xu.load(ubeg);
  wu.load(ubeg);
  xu.store(xs[0]);
  wu.store(wsm[0]);
  __syncthreads();
  for (int u = 0; u < units; ++u) {
    if (u + 1 < units) {
      xu.load(ubeg + u + 1);
      wu.load(ubeg + u + 1);
    }
    const char* bx = xs[u & 1];
    const char* bw = wsm[u & 1];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4_t xa[A], wa[A];
#pragma unroll
      for (int i = 0; i < A; ++i) xa[i] = xfrag<NB>(bx, st, tblk + i, lane);
#pragma unroll
      for (int a = 0; a < A; ++a) wa[a] = xfrag<NB>(bw, st, eblk + a, lane);
#pragma unroll
      for (int a = 0; a < A; ++a)
#pragma unroll
        for (int i = 0; i < A; ++i) {
          const f32x4_t f = mfma_bf16(wa[a], xa[i], zero);
#pragma unroll
          for (int j = 0; j < 4; ++j) part[a][i][j] += static_cast<double>(f[j]);
        }
      const int c = 4 * (ubeg + u) + st;            // chunk index in H
      if ((c + 1) % cpp == 0) {                       // a part ends
        const int p = c / cpp;
        const bool gend = (p + 1) % kRouterGroup == 0 || p + 1 == nparts;
#pragma unroll
        for (int a = 0; a < A; ++a)
#pragma unroll
          for (int i = 0; i < A; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              grp[a][i][j] += part[a][i][j];
              part[a][i][j] = 0.0;
              if (gend) {
                tot[a][i][j] += grp[a][i][j];
                grp[a][i][j] = 0.0;
              }
            }
      }
    }
    if (u + 1 < units) {
      xu.store(xs[(u + 1) & 1]);
      wu.store(wsm[(u + 1) & 1]);
    }
    __syncthreads();
  }
  // lane holds experts eb + 16 (eblk + a) + 4 q + j of token tb + 16 (tblk + i) + r
#pragma unroll
  for (int i = 0; i < A; ++i) {
    const int t = tb + 16 * (tblk + i) + r;
    if (t >= T) continue;
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = eb + 16 * (eblk + a) + 4 * q + j;
        if (e >= E) continue;
        if constexpr (GS) {
          gsum[(static_cast<size_t>(g) * T + t) * E + e] = tot[a][i][j];
        } else {
          double sum = tot[a][i][j];
          if (bias) sum += static_cast<double>(bias[e]);
          logits[static_cast<size_t>(t) * E + e] = static_cast<float>(sum);
        }
      }
  }
}

// float32 router: one thread per (token, expert), products and sums in
// float64 in ascending h, bias added, rounded once to float32.
__global__ __launch_bounds__(256) void k_router_f32(const float* __restrict__ x,
                                                    const float* __restrict__ wr,
                                                    const float* __restrict__ bias, int T, int H,
                                                    int E, float* __restrict__ logits) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * E) return;
  const int t = static_cast<int>(idx / E), e = static_cast<int>(idx % E);
  const float* xp = x + static_cast<size_t>(t) * H;
  const float* wp = wr + static_cast<size_t>(e) * H;
  double s = 0.0;
  for (int h = 0; h < H; ++h) s += static_cast<double>(xp[h]) * static_cast<double>(wp[h]);
  if (bias) s += static_cast<double>(bias[e]);
  logits[idx] = static_cast<float>(s);
}

// Exact top-k of logits already finished (f32 router, LDS router): one wave
// per token (topk_select).  grid ceil(T/4), block 256.
template <int NV>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float sel[4][1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;   // whole wave leaves; no workgroup barrier below
  const float* lt = logits + static_cast<size_t>(t) * E;
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = lt[min(j * 64 + lane, E - 1)];
  const size_t o = static_cast<size_t>(t) * k;
  topk_select<NV>(v, E, k, sel[wave], ids + o, w + o);
}

// Permutation outputs of the fused route + permute launch.
struct PermArgs {
  PermPtrs pp;
  int rt, max_tiles;
  int32_t* tiles;
  int32_t* arrive;   // zeroed by the router kernel of the same call
};

// Small bf16 batches: finish the logits of one token from the router's
// group sums, then its exact top-k.  Workgroup per token; wave w finishes
// the experts of slots w, w+4, ... (the ngroups float64 group sums, all
// loaded before any is added, summed in group order, bias added, rounded
// once to float32) into LDS and `logits`; after a barrier wave 0 selects.
// PERM (up to 32 tokens): every workgroup then publishes its token's routes
// (device-coherent stores, arrival counter); the last one to arrive reads
// them all and builds the permutation and the tile plan (permute_w1_body),
// so routing and grouping take one launch.  grid T, block 256.
template <int NV, bool PERM>
__global__ __launch_bounds__(256) void k_topk_groups(const double* __restrict__ gsum, int ngroups,
                                                     const float* __restrict__ bias,
                                                     float* __restrict__ logits, int T, int E, int k,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ w, PermArgs pa) {
  constexpr int NJ = (NV + 3) / 4;   // slots per wave
  __shared__ float lv[NV * 64];
  __shared__ float sel[1024];
  __shared__ PermW1Lds plds;   // PERM only (unused LDS is not allocated)
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const size_t slice = static_cast<size_t>(T) * E;
  const double* gt = gsum + static_cast<size_t>(t) * E;
  double gv[kRouterMaxGroups][NJ];
  float bv[NJ];
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int e = min((wave + 4 * i) * 64 + lane, E - 1);
#pragma unroll
    for (int g = 0; g < kRouterMaxGroups; ++g) gv[g][i] = g < ngroups ? gt[g * slice + e] : 0.0;
    bv[i] = bias ? bias[e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int j = wave + 4 * i;
    if (j >= NV) break;
    double sv = gv[0][i];
#pragma unroll
    for (int g = 1; g < kRouterMaxGroups; ++g)
      if (g < ngroups) sv += gv[g][i];
    if (bias) sv += static_cast<double>(bv[i]);
    const float f = static_cast<float>(sv);
    lv[j * 64 + lane] = f;
    if (j * 64 + lane < E) logits[static_cast<size_t>(t) * E + j * 64 + lane] = f;
  }
  __syncthreads();
  if (wave == 0) {
    float v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = lv[j * 64 + lane];
    const size_t o = static_cast<size_t>(t) * k;
    topk_select<NV, PERM>(v, E, k, sel, ids + o, w + o);
  }
  if constexpr (PERM) {
    // the ids went out device-coherent (no device-scope fence: it would
    // write back and invalidate the XCD's whole L2); wait for them, count
    // this token done, and let the last token's workgroup group the pairs
    wait_memory_done();
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(pa.arrive, 1) == T - 1;
    __syncthreads();
    if (!s_last) return;
    permute_w1_body<true>(ids, T, k, E, pa.pp.counts, pa.pp.offsets, pa.pp.sorted_pair,
                          pa.pp.pair_row, pa.pp.active, pa.pp.n_active, pa.rt, pa.max_tiles,
                          pa.tiles, plds);
    if (threadIdx.x == 0) store_dev_i32(pa.arrive, 0);
  }
}

template <int NV>
static void launch_topk(const moe_shape& s, const double* gsum, int ngroups, const float* bias,
                        float* lg, int32_t* ids, float* w, const PermArgs* pa, hipStream_t st) {
  if (gsum && pa)
    hipLaunchKernelGGL((k_topk_groups<NV, true>), dim3(s.T), dim3(256), 0, st, gsum, ngroups, bias,
                       lg, s.T, s.E, s.top_k, ids, w, *pa);
  else if (gsum)
    hipLaunchKernelGGL((k_topk_groups<NV, false>), dim3(s.T), dim3(256), 0, st, gsum, ngroups, bias,
                       lg, s.T, s.E, s.top_k, ids, w, PermArgs{});
  else
    hipLaunchKernelGGL((k_topk<NV>), dim3((s.T + 3) / 4), dim3(256), 0, st, lg, s.T, s.E, s.top_k,
                       ids, w);
}

// The router logits, or (bf16 batches up to 1024 tokens) their group sums
// in `gsum`.
static hipError_t launch_router(const moe_shape& s, const void* x, const void* w_router,
                                const float* bias, float* lg, double* gsum, int32_t* arrive,
                                hipStream_t st) {
  if (s.act == MOE_DT_BF16) {
    const int np = router_parts(s.H);
    const unsigned ng = gsum ? static_cast<unsigned>(router_groups(s.H)) : 1u;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* wb = static_cast<const uint16_t*>(w_router);
    if (s.T <= 64) {
      dim3 grid((s.T + 15) / 16, (s.E + 15) / 16, ng);
      hipLaunchKernelGGL(k_router_parts, grid, dim3(64 * kRouterGroup), 0, st, xb, wb, s.T, s.H,
                         s.E, np, gsum, arrive);
    } else if (s.T <= 1024) {
      dim3 grid((s.T + 31) / 32, (s.E + 31) / 32, ng);
      auto kern = gsum ? k_router_lds<1, true> : k_router_lds<1, false>;
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, xb, wb, bias, s.T, s.H, s.E, np, lg, gsum);
    } else {
      dim3 grid((s.T + 63) / 64, (s.E + 63) / 64);
      hipLaunchKernelGGL((k_router_lds<2, false>), grid, dim3(256), 0, st, xb, wb, bias, s.T, s.H,
                         s.E, np, lg, gsum);
    }
  } else {
    const size_t n = static_cast<size_t>(s.T) * s.E;
    hipLaunchKernelGGL(k_router_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(w_router), bias, s.T,
                       s.H, s.E, lg);
  }
  return hipGetLastError();
}

// The routing of one call; with `pp` (route + permute in one launch) the
// permutation and tile plan too.
static hipError_t route_impl(const moe_shape& s, const Plan& pl, const void* x,
                             const void* w_router, const float* bias, int32_t* ids, float* w,
                             float* logits, void* ws, const PermPtrs* pp, int32_t* tiles,
                             hipStream_t st) {
  float* lg = logits ? logits : reinterpret_cast<float*>(static_cast<char*>(ws) + pl.logits_off);
  double* gsum = router_gsum(s) ? reinterpret_cast<double*>(static_cast<char*>(ws) + pl.gsum_off)
                                : nullptr;
  PermArgs pa{};
  const PermArgs* pap = nullptr;
  if (pp) {
    pa.pp = *pp;
    pa.rt = 16 * pl.nb;
    pa.max_tiles = pl.max_tiles;
    pa.tiles = tiles;
    pa.arrive = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + pl.tiles_off) +
                3 * pl.max_tiles + 1;
    pap = &pa;
  }
  hipError_t e = launch_router(s, x, w_router, bias, lg, gsum, pap ? pa.arrive : nullptr, st);
  if (e != hipSuccess) return e;
  const int nv = (s.E + 63) / 64, ng = router_groups(s.H);
  const float* fb = gsum ? bias : nullptr;   // the other paths added the bias already
  if (nv <= 1) launch_topk<1>(s, gsum, ng, fb, lg, ids, w, pap, st);
  else if (nv <= 2) launch_topk<2>(s, gsum, ng, fb, lg, ids, w, pap, st);
  else if (nv <= 4) launch_topk<4>(s, gsum, ng, fb, lg, ids, w, pap, st);
  else if (nv <= 8) launch_topk<8>(s, gsum, ng, fb, lg, ids, w, pap, st);
  else launch_topk<16>(s, gsum, ng, fb, lg, ids, w, pap, st);
  return hipGetLastError();
}

hipError_t launch_route(const moe_shape& s, const Plan& pl, const void* x, const void* w_router,
                        const float* bias, int32_t* ids, float* w, float* logits, void* ws,
                        hipStream_t st) {
  return route_impl(s, pl, x, w_router, bias, ids, w, logits, ws, nullptr, nullptr, st);
}

bool route_permute_fused(const moe_shape& s) {
  return s.act == MOE_DT_BF16 && router_gsum(s) && s.T <= 64 && permute_w1_ok(s);
}

hipError_t launch_route_permute(const moe_shape& s, const Plan& pl, const void* x,
                                const void* w_router, const float* bias, int32_t* ids, float* w,
                                float* logits, const PermPtrs& pp, int32_t* tiles, void* ws,
                                hipStream_t st) {
  if (route_permute_fused(s))
    return route_impl(s, pl, x, w_router, bias, ids, w, logits, ws, &pp, tiles, st);
  hipError_t e = route_impl(s, pl, x, w_router, bias, ids, w, logits, ws, nullptr, nullptr, st);
  if (e == hipSuccess) e = launch_permute(s, pl, ids, pp, tiles, ws, st);
  return e;
}

}  // namespace moe
