// Internal interface between the C-ABI layer (moe_abi.cpp) and the kernel
// launchers.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Sizes shared by the host planning code (plan.cpp) and the kernels.
constexpr int kChunkTok = 256;          // tokens per chunk of the large-batch permutation
constexpr int kRouterGroup = 4;         // consecutive H parts whose sums are added first
constexpr int kRouterMaxParts = 16;     // parts of the router's H reduction, at most
constexpr int kRouterMaxGroups = kRouterMaxParts / kRouterGroup;
constexpr int kRouterGsumMaxT = 1024;   // group sums finished by the top-k kernel up to here
constexpr int kFusedCols = 64;          // intermediate columns per fused-FFN work item
constexpr int kMaxLocalityBlock = 5;    // route-locality block sizes 1..5

// Launch geometry and workspace layout for one shape.  Every region is
// 256-byte aligned; moe_workspace_size() returns `total`.
struct Plan {
  // router
  size_t logits_off;      // float [T][E] (when the caller passes no logits buffer)
  size_t gsum_off;        // double [router groups][T][E] (bf16 batches up to 1024 tokens)
  // permutation
  int chunks;             // 256-token chunks of the large-batch path (0: one pass)
  size_t chunk_off;       // int32 chunk counts [chunks][E] + chunk bases [chunks][E]
  size_t perm_off;        // int32 counts[E], offsets[E+1], sorted_pair[P],
                          // pair_row[P], active[E], n_active[1]
  // grouped FFN
  int nb;                 // 16-row token groups per tile (rows per tile = 16*nb)
  int max_tiles;          // upper bound on tiles: P/(16 nb) + min(E, P)
  size_t tiles_off;       // int32 [3*max_tiles] (expert, row0, rows) + n_tiles + the
                          // route + permute arrival counter
  size_t h_off;           // act [P][I] SwiGLU intermediate
  size_t y_off;           // act [P][H] expert outputs (moe_layer only)
  // MOE_F_CHECK_FINITE: private results until the status word is clean
  size_t ids_off;         // int32 [P]
  size_t w_off;           // float [P]
  size_t out_off;         // act [T][H] (moe_layer)
  size_t status_off;      // uint32 status word
  // MOE_F_FUSED_FFN: float [I/64][P][H] partial expert outputs
  size_t part_off;
  size_t total;
};

bool make_plan(const moe_shape& s, Plan* p);

// Supplies the workspace of a validated moe_layer call that received none:
// `need` is the plan's size; on MOE_OK *ws / *ws_bytes describe device
// memory of at least `need` bytes usable on `st`'s device.
typedef int (*ScratchFn)(size_t need, hipStream_t st, void** ws, size_t* ws_bytes);

// moe_layer with an optional scratch supplier (nullptr: the caller's
// workspace); every validation step runs before `scratch` is called.
int layer_call(const moe_shape* shape, const void* x, const void* w_router, const float* router_bias,
               const moe_experts* experts, const void* residual, void* out, int32_t* topk_ids,
               float* topk_w, const moe_perm* perm, void* workspace, size_t workspace_bytes,
               hipStream_t stream, ScratchFn scratch);

struct PermPtrs {
  int32_t *counts, *offsets, *sorted_pair, *pair_row, *active, *n_active;
};

// Launchers: enqueue only, return hipGetLastError().
int router_parts(int H);        // parts of the H reduction (largest divisor of H/32 <= 16)
int router_groups(int H);       // groups of consecutive parts
bool router_gsum(const moe_shape& s);   // router group sums finished by the top-k kernel
hipError_t launch_route(const moe_shape& s, const Plan& pl, const void* x, const void* w_router,
                        const float* bias, int32_t* ids, float* w, float* logits, void* ws,
                        hipStream_t st);
// route + permute in one call: fused (the top-k kernel's last workgroup
// builds the permutation) for bf16 batches of up to 32 tokens, else the two
// launches back to back
bool route_permute_fused(const moe_shape& s);
hipError_t launch_route_permute(const moe_shape& s, const Plan& pl, const void* x,
                                const void* w_router, const float* bias, int32_t* ids, float* w,
                                float* logits, const PermPtrs& pp, int32_t* tiles, void* ws,
                                hipStream_t st);
bool permute_single_pass(const moe_shape& s);
bool permute_w1_ok(const moe_shape& s);   // the 32-token permutation (one bitmap word per expert)
int permute_chunks(const moe_shape& s);
hipError_t launch_permute(const moe_shape& s, const Plan& pl, const int32_t* ids,
                          const PermPtrs& pp, int32_t* tiles /* may be null */, void* ws,
                          hipStream_t st);
hipError_t launch_plan_tiles(const moe_shape& s, const Plan& pl, const PermPtrs& pp,
                             int32_t* tiles, hipStream_t st);
hipError_t launch_gateup(const moe_shape& s, const Plan& pl, const void* x, const moe_experts& ex,
                         const int32_t* sorted_pair, const int32_t* tiles, void* h,
                         hipStream_t st);
hipError_t launch_down(const moe_shape& s, const Plan& pl, const void* h, const moe_experts& ex,
                       const int32_t* tiles, void* y, hipStream_t st);
// 128-row tiles (nb = 8) are planned only for bf16 tiled weights
bool tiles128_ok(const moe_shape& s);
hipError_t launch_ffn(const moe_shape& s, const Plan& pl, const void* x, const moe_experts& ex,
                      const int32_t* sorted_pair, const int32_t* tiles, void* h, void* y,
                      hipStream_t st);
// down then combine (y in `y`): with 16-row tiles of tiled bf16-activation
// weights y goes to pair slots and the combine reads them directly
bool down_pair_order(const moe_shape& s, const Plan& pl);
hipError_t launch_down_combine(const moe_shape& s, const Plan& pl, const void* h,
                               const moe_experts& ex, const int32_t* tiles,
                               const int32_t* sorted_pair, const int32_t* pair_row, const float* w,
                               const void* residual, void* out, void* y, hipStream_t st);
int fused_slices(const moe_shape& s);   // I / 64
hipError_t launch_ffn_fused(const moe_shape& s, const Plan& pl, const void* x,
                            const moe_experts& ex, const int32_t* sorted_pair,
                            const int32_t* tiles, float* part, int wave_tiles, uint64_t* clock,
                            hipStream_t st);
hipError_t launch_reduce_parts(const moe_shape& s, const float* part, void* y, hipStream_t st);
hipError_t launch_combine_parts(const moe_shape& s, const float* part, const int32_t* pair_row,
                                const float* w, const void* residual, void* out, hipStream_t st);
hipError_t launch_tile_experts(const moe_shape& s, const moe_experts& src, const moe_experts& dst,
                               hipStream_t st);
int locality_blocks(int T);   // sum over B = 1..5 of ceil(T / B)
hipError_t launch_route_locality(const moe_shape& s, const int32_t* ids, int32_t* overlap,
                                 int32_t* block_unique, hipStream_t st);
// Per-expert byte pieces of one expert record set (gate, up, down and their
// scales): source and destination bases (device-usable addresses) and bytes
// per expert; a null source skips the piece.
constexpr int kStagePieces = 6;
struct StagePieces {
  const char* src[kStagePieces];
  char* dst[kStagePieces];
  size_t bytes[kStagePieces];
};
hipError_t launch_stage_experts(const moe_shape& s, const StagePieces& pc, const int32_t* active,
                                const int32_t* n_active, hipStream_t st);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_zero_status(uint32_t* status, hipStream_t st);
// sets `bit` in *status if any of the n values (bf16 or float32) is NaN/inf
hipError_t launch_check_finite(const void* src, size_t n, bool bf16, uint32_t bit,
                               uint32_t* status, hipStream_t st);
// pair_row == nullptr: y rows in pair order (row t*k + j)
hipError_t launch_combine(const moe_shape& s, const void* y, const int32_t* pair_row,
                          const float* w, const void* residual, void* out, hipStream_t st);

}  // namespace moe
