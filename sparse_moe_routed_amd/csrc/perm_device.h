// Device code of the small-batch permutation, shared by the permutation
// kernel and the top-k kernel that builds the permutation in its last
// workgroup (route + permute in one launch).
//
// Reference: "Agent Field Notes -- full corpus", AFN-019 "Hide SSD misses
// before the router knows they exist", section "Why overlap alone cannot
// defeat the byte roofline" (token rows grouped by expert, repeated routes
// deduplicated) and section "Hypothesis H5" (a verifier block reads the
// deduplicated union of its routes).
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// The arrival counter of the single-launch route + permute sits after the
// FFN tile plan in the workspace (tiles[3 max_tiles] is the tile count,
// tiles[3 max_tiles + 1] the counter).  It is zeroed by the router kernel of
// the same call and reset by the last workgroup that arrives, so a
// workspace needs no initialisation.

// LDS of permute_w1_body.
constexpr int kPermW1KeepPairs = 2048;   // routes kept in LDS between the two passes
struct PermW1Lds {
  uint32_t bits[1024];                // token bitmap per expert (T <= 32)
  int off[1024];                      // first row of each expert
  int wtot[4][3];                     // per-wave totals of (rows, active experts, tiles)
  int32_t ids[kPermW1KeepPairs];      // the routes, when P <= kPermW1KeepPairs
};

// Up to 32 tokens (one bitmap word per expert; decode and verifier blocks),
// E <= 1024, one 256-thread workgroup, each thread owning up to 4
// consecutive experts, one combined scan of (rows, active flag, tiles) per
// expert in expert order.  Writes the stable counting sort of the pairs by
// expert (rows of an expert in ascending token order), the active experts
// ascending (-1 after the last), their count, and (tiles != nullptr) the
// tile plan of at most `rt` rows per tile.
// DEV: `ids` were written by other workgroups of the same launch with
// device-coherent stores that have completed; they are read the same way.
template <bool DEV = false>
__device__ __forceinline__ void permute_w1_body(const int32_t* ids, int T, int k, int E,
                                                int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ sorted_pair,
                                                int32_t* __restrict__ pair_row,
                                                int32_t* __restrict__ active,
                                                int32_t* __restrict__ n_active, int rt,
                                                int max_tiles, int32_t* __restrict__ tiles,
                                                PermW1Lds& L) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int P = T * k;
  const int ept = (E + 255) / 256;   // experts per thread (<= 4)
  const int e0 = tid * ept;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < ept && e0 + i < E) L.bits[e0 + i] = 0u;
  __syncthreads();
  const bool keep = P <= kPermW1KeepPairs;   // the second pass reads the routes from LDS
  for (int p = tid; p < P; p += 256) {
    const int e = DEV ? load_dev_i32(ids + p) : ids[p];
    if (keep) L.ids[p] = e;
    if (e >= 0 && e < E) atomicOr(&L.bits[e], 1u << (p / k));
  }
  __syncthreads();
  // rows per tile are 16 nb (a power of two): a shift instead of a division
  const bool pow2 = (rt & (rt - 1)) == 0;
  const int rsh = __ffs(rt) - 1;
  int c[4], n[4], C = 0, F = 0, N = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = (i < ept && e0 + i < E) ? __popc(L.bits[e0 + i]) : 0;
    n[i] = pow2 ? (c[i] + rt - 1) >> rsh : (c[i] + rt - 1) / rt;
    C += c[i];
    F += c[i] > 0 ? 1 : 0;
    N += n[i];
  }
  // inclusive wave scans of the three per-thread sums, then wave offsets
  const int iC = wave_incl_scan_i32(C), iF = wave_incl_scan_i32(F), iN = wave_incl_scan_i32(N);
  if (lane == 63) {
    L.wtot[wave][0] = iC;
    L.wtot[wave][1] = iF;
    L.wtot[wave][2] = iN;
  }
  __syncthreads();
  int bC = 0, bF = 0, bN = 0, tF = 0, tN = 0;   // this wave's base; totals
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) {
      bC += L.wtot[w][0];
      bF += L.wtot[w][1];
      bN += L.wtot[w][2];
    }
    tF += L.wtot[w][1];
    tN += L.wtot[w][2];
  }
  int off = bC + iC - C, apos = bF + iF - F, tpos = bN + iN - N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + i;
    if (i >= ept || e >= E) break;
    counts[e] = c[i];
    offsets[e] = off;
    L.off[e] = off;
    if (e == E - 1) offsets[E] = off + c[i];
    if (c[i] > 0) active[apos++] = e;
    if (e >= tF) active[e] = -1;
    if (tiles != nullptr) {
      for (int j = 0; j < n[i]; ++j) {
        const int ti = tpos + j;
        if (ti >= max_tiles) break;
        const int r0 = off + j * rt;
        tiles[3 * ti] = e;
        tiles[3 * ti + 1] = r0;
        tiles[3 * ti + 2] = min(min(rt, c[i] - j * rt), P - r0);
      }
    }
    off += c[i];
    tpos += n[i];
  }
  if (tid == 0) {
    n_active[0] = tF;
    if (tiles != nullptr) tiles[3 * max_tiles] = min(tN, max_tiles);
  }
  __syncthreads();
  for (int p = tid; p < P; p += 256) {
    const int e = keep ? L.ids[p] : (DEV ? load_dev_i32(ids + p) : ids[p]);
    if (e < 0 || e >= E) continue;
    const int t = p / k;
    const int row = L.off[e] + __popc(L.bits[e] & ((1u << t) - 1u));
    sorted_pair[row] = p;
    pair_row[p] = row;
  }
}

}  // namespace moe
