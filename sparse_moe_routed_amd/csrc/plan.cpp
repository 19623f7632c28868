// Host-side launch planning shared by the C-ABI layer and the launchers:
// which permutation path a shape takes, how the router's H reduction is cut,
// how many fused-FFN slices and route-locality values a shape has.  Plain
// C++ with no device code, so the validation layer builds and runs without
// a GPU.
#include <cstddef>
#include <cstdint>

#include "moe_internal.h"

namespace moe {

// The single-workgroup permutation keeps a token bitmap and its prefix
// counts per expert in LDS (2 words per expert and 32 tokens).
bool permute_single_pass(const moe_shape& s) {
  return static_cast<size_t>(s.E) * ((s.T + 31) / 32) * 2 * sizeof(uint32_t) <= 48 * 1024;
}

int permute_chunks(const moe_shape& s) { return (s.T + kChunkTok - 1) / kChunkTok; }

bool permute_w1_ok(const moe_shape& s) { return s.T <= 32 && s.E <= 1024; }

int router_parts(int H) {
  const int chunks = H / 32;
  int best = 1;
  for (int d = 1; d <= kRouterMaxParts; ++d)
    if (chunks % d == 0) best = d;
  return best;
}

int router_groups(int H) { return (router_parts(H) + kRouterGroup - 1) / kRouterGroup; }

// One workgroup per group of parts multiplies the parallelism of the router
// by the group count (512 tokens: 3.7 us less per layer); at 4096 tokens the
// float64 group sums (groups * T * E * 8 bytes = 64 MB) cost more than the
// parallelism saves (+13 us), so larger batches let the LDS kernel finish
// the sums.
bool router_gsum(const moe_shape& s) { return s.act == MOE_DT_BF16 && s.T <= kRouterGsumMaxT; }

int fused_slices(const moe_shape& s) { return s.I / kFusedCols; }

// 128-row tiles: the bf16 LDS-staged gate/up kernel at 8 token blocks (two
// 16-row blocks of gate and of up per wave; 256 VGPRs with the token
// fragments read one at a time), down on the tiles' two 64-row halves.  At
// 32768 tokens gate/up went 2530 -> 2200 us against 64-row tiles.
bool tiles128_ok(const moe_shape& s) {
  return s.act == MOE_DT_BF16 && s.wfmt == MOE_WF_DENSE && (s.flags & MOE_F_TILED_WEIGHTS) &&
         s.I % 128 == 0;
}

int locality_blocks(int T) {
  int n = 0;
  for (int B = 1; B <= kMaxLocalityBlock; ++B) n += (T + B - 1) / B;
  return n;
}

}  // namespace moe
