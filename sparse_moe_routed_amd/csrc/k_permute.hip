// Per-expert permutation of (token, slot) pairs and the FFN tile plan.
//
// Reference: "Agent Field Notes -- full corpus", AFN-019 "Hide SSD misses
// before the router knows they exist", section "Why overlap alone cannot
// defeat the byte roofline" (grouping token rows by expert; deduplicating
// repeated routes across a verifier block) and section "Hypothesis H5"
// (a verify block reads the deduplicated union).
//
// Determinism: a row's place inside its expert segment is the number of
// pairs of the same expert with a smaller token, computed as a popcount over
// a per-expert token bitmap built with LDS atomic OR (OR is order-free), so
// the result is bit-identical on every run and equals a stable counting sort.
// Small batches use one workgroup with the whole bitmap in LDS; large batches
// split the tokens into 256-token chunks (per-chunk counts, a scan that gives
// each chunk its base row per expert, then a per-chunk bitmap placement).
#include "moe_device.h"
#include "moe_internal.h"
#include "perm_device.h"

namespace moe {

// Exclusive scan over a 1024-thread block; every thread must call it.
__device__ int block_excl_scan(int v, int* s_tot, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int inc = wave_incl_scan_i32(v);
  if (lane == 63) s_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int tv = lane < 16 ? s_tot[lane] : 0;
    const int ti = wave_incl_scan_i32(tv);
    if (lane < 16) s_tot[lane] = ti - tv;
    if (lane == 15) s_tot[16] = ti;
  }
  __syncthreads();
  const int res = s_tot[wave] + inc - v;
  *total = s_tot[16];
  __syncthreads();
  return res;
}

// Zero the bitmap of experts [c0, c1) and set bit t of row e for every pair
// (t, j) with ids[t*k+j] == e.  Invalid ids are skipped.
__device__ void build_bits(const int32_t* __restrict__ ids, int P, int k, int W, int c0, int c1,
                           uint32_t* bits) {
  const int n = (c1 - c0) * W;
  for (int i = threadIdx.x; i < n; i += blockDim.x) bits[i] = 0u;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = ids[p];
    if (e >= c0 && e < c1) {
      const int t = p / k;
      atomicOr(&bits[(e - c0) * W + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();
}

// Word-exclusive popcount prefixes of rows [c0, c1); one thread per expert
// (rows are at most a few words long on this path).
__device__ void build_prefix(int W, int c0, int c1, const uint32_t* bits, uint32_t* pre,
                             int* s_cnt) {
  for (int e = c0 + static_cast<int>(threadIdx.x); e < c1; e += blockDim.x) {
    int count = 0;
    for (int wi = 0; wi < W; ++wi) {
      pre[(e - c0) * W + wi] = static_cast<uint32_t>(count);
      count += __popc(bits[(e - c0) * W + wi]);
    }
    s_cnt[e] = count;
  }
  __syncthreads();
}

// Tiles of at most `rt` rows for each active expert, in active order.
// Thread a < nact owns active slot a.  Writes tiles[3*i .. 3*i+2] =
// (expert, first row, rows) and tiles[3*max_tiles] = number of tiles.
__device__ void emit_tiles(int nact, const int* s_act, const int* s_cnt, const int* s_off, int P,
                           int rt, int max_tiles, int32_t* tiles, int* s_tot) {
  int e = -1, nt = 0;
  if (static_cast<int>(threadIdx.x) < nact) {
    e = s_act[threadIdx.x];
    if (e >= 0) nt = (s_cnt[e] + rt - 1) / rt;
  }
  int total = 0;
  const int tpos = block_excl_scan(nt, s_tot, &total);
  for (int j = 0; j < nt; ++j) {
    const int ti = tpos + j;
    if (ti >= max_tiles) break;
    const int r0 = s_off[e] + j * rt;
    tiles[3 * ti] = e;
    tiles[3 * ti + 1] = r0;
    tiles[3 * ti + 2] = min(min(rt, s_cnt[e] - j * rt), P - r0);
  }
  if (threadIdx.x == 0) tiles[3 * max_tiles] = min(total, max_tiles);
}

// Small batches: everything in one 1024-thread workgroup, one pass.  `ids`
// may point to global memory or LDS; bits/pre hold E*W words each.
__device__ void permute_small_body(const int32_t* ids, int T, int k, int E, int W,
                                   int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row,
                                   int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                   int rt, int max_tiles, int32_t* __restrict__ tiles,
                                   uint32_t* bits, uint32_t* pre, int* s_cnt,
                                   int* s_off, int* s_act, int* s_tot) {
  const int tid = threadIdx.x;
  const int P = T * k;

  build_bits(ids, P, k, W, 0, E, bits);
  build_prefix(W, 0, E, bits, pre, s_cnt);

  const int c = tid < E ? s_cnt[tid] : 0;
  int total = 0;
  const int ex = block_excl_scan(c, s_tot, &total);
  if (tid < E) {
    s_off[tid] = ex;
    counts[tid] = c;
    offsets[tid] = ex;
    if (tid == E - 1) offsets[E] = ex + c;
  }
  const int flag = (tid < E && c > 0) ? 1 : 0;
  int nact = 0;
  const int apos = block_excl_scan(flag, s_tot, &nact);
  if (flag) {
    active[apos] = tid;
    s_act[apos] = tid;
  }
  if (tid < E && tid >= nact) active[tid] = -1;
  if (tid == 0) n_active[0] = nact;
  __syncthreads();
  if (tiles != nullptr) emit_tiles(nact, s_act, s_cnt, s_off, P, rt, max_tiles, tiles, s_tot);
  for (int p = tid; p < P; p += blockDim.x) {
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    const int t = p / k;
    const int wi = t >> 5;
    const uint32_t b = bits[e * W + wi];
    const int row = s_off[e] + static_cast<int>(pre[e * W + wi]) + __popc(b & ((1u << (t & 31)) - 1u));
    sorted_pair[row] = p;
    pair_row[p] = row;
  }
}

__global__ __launch_bounds__(1024) void k_permute_small(
    const int32_t* __restrict__ ids, int T, int k, int E, int W, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_row, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int rt, int max_tiles, int32_t* __restrict__ tiles) {
  extern __shared__ uint32_t dyn[];
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ int s_act[1024];
  __shared__ int s_tot[17];
  permute_small_body(ids, T, k, E, W, counts, offsets, sorted_pair, pair_row, active, n_active, rt,
                     max_tiles, tiles, dyn, dyn + E * W, s_cnt, s_off, s_act, s_tot);
}

// Up to 32 tokens: permute_w1_body (perm_device.h) in one 256-thread
// workgroup, 4 barriers (against 13 barriers of 16 waves in the general
// single-workgroup kernel).
__global__ __launch_bounds__(256) void k_permute_w1(
    const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_row, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int rt, int max_tiles, int32_t* __restrict__ tiles) {
  __shared__ PermW1Lds lds;
  permute_w1_body(ids, T, k, E, counts, offsets, sorted_pair, pair_row, active, n_active, rt,
                  max_tiles, tiles, lds);
}

// Large batches: chunks of kChunkTok tokens.
//   1) k_perm_count : per-chunk expert counts          (grid = chunks)
//   2) k_perm_scan  : chunk bases within each expert segment, offsets,
//                     active, tiles (one workgroup)
//   3) k_perm_place : stable rows (offset + chunk base + rank in chunk)
//                     (grid = chunks)
constexpr int kChunkWords = kChunkTok / 32;

__global__ __launch_bounds__(1024) void k_perm_count(const int32_t* __restrict__ ids, int T, int k,
                                                     int E, int32_t* __restrict__ chunk_cnt) {
  __shared__ int s_cnt[1024];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int p0 = c * kChunkTok * k, p1 = min(T, (c + 1) * kChunkTok) * k;
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_cnt[static_cast<size_t>(c) * E + e] = s_cnt[e];
}

__global__ __launch_bounds__(1024) void k_perm_scan(const int32_t* __restrict__ chunk_cnt, int nchunks,
                                                    int T, int k, int E,
                                                    int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ active,
                                                    int32_t* __restrict__ n_active, int rt,
                                                    int max_tiles, int32_t* __restrict__ tiles) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ int s_act[1024];
  __shared__ int s_tot[17];
  const int tid = threadIdx.x;
  const int P = T * k;
  // per expert: each chunk's first row relative to the expert's segment;
  // the counts of a batch of chunks are loaded before any is added
  constexpr int kScanBatch = 16;
  int run = 0;
  if (tid < E) {
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        v[u] = c0 + u < nchunks ? chunk_cnt[static_cast<size_t>(c0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (c0 + u < nchunks) chunk_base[static_cast<size_t>(c0 + u) * E + tid] = run;
        run += v[u];
      }
    }
    s_cnt[tid] = run;
  }
  int total = 0;
  const int ex = block_excl_scan(tid < E ? run : 0, s_tot, &total);
  if (tid < E) {
    s_off[tid] = ex;
    counts[tid] = run;
    offsets[tid] = ex;
    if (tid == E - 1) offsets[E] = ex + run;
  }
  const int flag = (tid < E && run > 0) ? 1 : 0;
  int nact = 0;
  const int apos = block_excl_scan(flag, s_tot, &nact);
  if (flag) {
    active[apos] = tid;
    s_act[apos] = tid;
  }
  if (tid < E && tid >= nact) active[tid] = -1;
  if (tid == 0) n_active[0] = nact;
  __syncthreads();
  if (tiles != nullptr) emit_tiles(nact, s_act, s_cnt, s_off, P, rt, max_tiles, tiles, s_tot);
}

__global__ __launch_bounds__(1024) void k_perm_place(const int32_t* __restrict__ ids, int T, int k,
                                                     int E, const int32_t* __restrict__ chunk_base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_pair,
                                                     int32_t* __restrict__ pair_row) {
  __shared__ uint32_t bits[1024 * kChunkWords];
  const int c = blockIdx.x;
  const int t0 = c * kChunkTok;
  for (int i = threadIdx.x; i < E * kChunkWords; i += blockDim.x) bits[i] = 0u;
  __syncthreads();
  const int p0 = t0 * k, p1 = min(T, t0 + kChunkTok) * k;
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      const int t = p / k - t0;
      atomicOr(&bits[e * kChunkWords + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    const int t = p / k - t0;
    const int wi = t >> 5;
    int row = offsets[e] + chunk_base[static_cast<size_t>(c) * E + e] +
              __popc(bits[e * kChunkWords + wi] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < wi; ++w) row += __popc(bits[e * kChunkWords + w]);
    sorted_pair[row] = p;
    pair_row[p] = row;
  }
}

// Scan and placement in one launch for up to kScanPlaceChunks chunks (4096
// tokens): every workgroup forms the expert counts of all pairs, and of the
// pairs of the chunks before its own, itself, instead of reading bases that
// a single-workgroup scan launch wrote; workgroup 0 also publishes the
// counts, offsets, active list and tile plan.  COUNT (up to kCountChunks
// chunks): the counts come from a histogram of all pairs' ids in LDS, so
// the count launch goes too; otherwise from k_perm_count's per-chunk counts
// (one round of E x C loads).  Same rows as k_perm_count + k_perm_scan +
// k_perm_place (integer sums, chunk and token order).  Measured: 512
// tokens (2 chunks) step -1.3% with COUNT; 4096 tokens (16 chunks) -0.3%
// without it and +0.8% with it.
constexpr int kScanPlaceChunks = 16;
constexpr int kCountChunks = 4;
template <bool COUNT>
__global__ __launch_bounds__(1024) void k_perm_scan_place(
    const int32_t* __restrict__ ids, int T, int k, int E, const int32_t* __restrict__ chunk_cnt,
    int nchunks, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, int rt, int max_tiles,
    int32_t* __restrict__ tiles, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ int s_base[1024];
  __shared__ int s_act[1024];
  __shared__ int s_tot[17];
  __shared__ uint32_t bits[1024 * kChunkWords];
  const int tid = threadIdx.x, c = blockIdx.x;
  const int P = T * k;
  const int t0 = c * kChunkTok;
  const int p0 = t0 * k, p1 = min(T, t0 + kChunkTok) * k;
  for (int i = tid; i < E * kChunkWords; i += blockDim.x) bits[i] = 0u;
  if constexpr (COUNT) {
    for (int e = tid; e < E; e += blockDim.x) {
      s_cnt[e] = 0;
      s_base[e] = 0;
    }
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x) {
      const int e = ids[p];
      if (e >= 0 && e < E) {
        atomicAdd(&s_cnt[e], 1);
        if (p < p0) atomicAdd(&s_base[e], 1);
      }
    }
  } else if (tid < E) {
    int v[kScanPlaceChunks];
#pragma unroll
    for (int u = 0; u < kScanPlaceChunks; ++u)
      v[u] = u < nchunks ? chunk_cnt[static_cast<size_t>(u) * E + tid] : 0;
    int run = 0, base = 0;
#pragma unroll
    for (int u = 0; u < kScanPlaceChunks; ++u) {
      if (u == c) base = run;
      run += v[u];
    }
    s_cnt[tid] = run;
    s_base[tid] = base;
  }
  __syncthreads();
  const int run = tid < E ? s_cnt[tid] : 0;
  int total = 0;
  const int ex = block_excl_scan(run, s_tot, &total);
  if (tid < E) s_off[tid] = ex;
  if (c == 0) {
    if (tid < E) {
      counts[tid] = run;
      offsets[tid] = ex;
      if (tid == E - 1) offsets[E] = ex + run;
    }
    const int flag = (tid < E && run > 0) ? 1 : 0;
    int nact = 0;
    const int apos = block_excl_scan(flag, s_tot, &nact);
    if (flag) {
      active[apos] = tid;
      s_act[apos] = tid;
    }
    if (tid < E && tid >= nact) active[tid] = -1;
    if (tid == 0) n_active[0] = nact;
    __syncthreads();
    if (tiles != nullptr) emit_tiles(nact, s_act, s_cnt, s_off, P, rt, max_tiles, tiles, s_tot);
  }
  // placement of this chunk's pairs (as k_perm_place)
  for (int p = p0 + tid; p < p1; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      const int t = p / k - t0;
      atomicOr(&bits[e * kChunkWords + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();
  for (int p = p0 + tid; p < p1; p += blockDim.x) {
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    const int t = p / k - t0;
    const int wi = t >> 5;
    int row = s_off[e] + s_base[e] + __popc(bits[e * kChunkWords + wi] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < wi; ++w) row += __popc(bits[e * kChunkWords + w]);
    sorted_pair[row] = p;
    pair_row[p] = row;
  }
}

// Tile plan from an existing permutation (for moe_grouped_ffn, whose caller
// may supply any permutation).  Values are clamped so that tiles never
// address rows outside [0, P).
__global__ __launch_bounds__(1024) void k_plan_tiles(const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ active,
                                                     const int32_t* __restrict__ n_active, int E,
                                                     int P, int rt, int max_tiles,
                                                     int32_t* __restrict__ tiles) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ int s_act[1024];
  __shared__ int s_tot[17];
  const int tid = threadIdx.x;
  const int nact = min(max(n_active[0], 0), E);
  if (tid < E) {
    const int o = min(max(offsets[tid], 0), P);
    s_off[tid] = o;
    s_cnt[tid] = min(max(counts[tid], 0), P - o);
  }
  if (tid < nact) {
    const int e = active[tid];
    s_act[tid] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  emit_tiles(nact, s_act, s_cnt, s_off, P, rt, max_tiles, tiles, s_tot);
}

hipError_t launch_permute(const moe_shape& s, const Plan& pl, const int32_t* ids,
                          const PermPtrs& pp, int32_t* tiles, void* ws, hipStream_t st) {
  const int rt = 16 * pl.nb;
  if (permute_w1_ok(s)) {
    hipLaunchKernelGGL(k_permute_w1, dim3(1), dim3(256), 0, st, ids, s.T, s.top_k, s.E,
                       pp.counts, pp.offsets, pp.sorted_pair, pp.pair_row, pp.active,
                       pp.n_active, rt, pl.max_tiles, tiles);
  } else if (permute_single_pass(s)) {
    const int W = (s.T + 31) / 32;
    const size_t lds = static_cast<size_t>(s.E) * W * 2 * sizeof(uint32_t);
    hipLaunchKernelGGL(k_permute_small, dim3(1), dim3(1024), lds, st, ids, s.T, s.top_k, s.E, W,
                       pp.counts, pp.offsets, pp.sorted_pair, pp.pair_row, pp.active, pp.n_active,
                       rt, pl.max_tiles, tiles);
  } else {
    const int C = permute_chunks(s);
    int32_t* chunk_cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + pl.chunk_off);
    int32_t* chunk_base = chunk_cnt + static_cast<size_t>(C) * s.E;
    if (C <= kCountChunks) {
      hipLaunchKernelGGL(k_perm_scan_place<true>, dim3(C), dim3(1024), 0, st, ids, s.T, s.top_k,
                         s.E, nullptr, C, pp.counts, pp.offsets, pp.active, pp.n_active, rt,
                         pl.max_tiles, tiles, pp.sorted_pair, pp.pair_row);
    } else if (C <= kScanPlaceChunks) {
      hipLaunchKernelGGL(k_perm_count, dim3(C), dim3(1024), 0, st, ids, s.T, s.top_k, s.E,
                         chunk_cnt);
      hipLaunchKernelGGL(k_perm_scan_place<false>, dim3(C), dim3(1024), 0, st, ids, s.T, s.top_k,
                         s.E, chunk_cnt, C, pp.counts, pp.offsets, pp.active, pp.n_active, rt,
                         pl.max_tiles, tiles, pp.sorted_pair, pp.pair_row);
    } else {
      hipLaunchKernelGGL(k_perm_count, dim3(C), dim3(1024), 0, st, ids, s.T, s.top_k, s.E,
                         chunk_cnt);
      hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, st, chunk_cnt, C, s.T, s.top_k, s.E,
                         chunk_base, pp.counts, pp.offsets, pp.active, pp.n_active, rt,
                         pl.max_tiles, tiles);
      hipLaunchKernelGGL(k_perm_place, dim3(C), dim3(1024), 0, st, ids, s.T, s.top_k, s.E,
                         chunk_base, pp.offsets, pp.sorted_pair, pp.pair_row);
    }
  }
  return hipGetLastError();
}

hipError_t launch_plan_tiles(const moe_shape& s, const Plan& pl, const PermPtrs& pp,
                             int32_t* tiles, hipStream_t st) {
  hipLaunchKernelGGL(k_plan_tiles, dim3(1), dim3(1024), 0, st, pp.counts, pp.offsets, pp.active,
                     pp.n_active, s.E, s.T * s.top_k, 16 * pl.nb, pl.max_tiles, tiles);
  return hipGetLastError();
}

}  // namespace moe
