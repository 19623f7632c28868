// Test double for the kernel launchers: the validation battery only makes
// calls the C ABI must reject, so reaching any launcher is a failure (the
// entry point would have enqueued work for an invalid call).
#include <cstdio>
#include <cstdlib>

#include "../../sparse_moe_routed_amd/csrc/moe_internal.h"

namespace moe {

[[noreturn]] static void reached(const char* name) {
  std::fprintf(stderr, "FAIL: %s was reached by a call that must be rejected\n", name);
  std::abort();
}

hipError_t launch_route(const moe_shape&, const Plan&, const void*, const void*, const float*,
                        int32_t*, float*, float*, void*, hipStream_t) { reached("launch_route"); }
hipError_t launch_permute(const moe_shape&, const Plan&, const int32_t*, const PermPtrs&, int32_t*,
                          void*, hipStream_t) { reached("launch_permute"); }
hipError_t launch_plan_tiles(const moe_shape&, const Plan&, const PermPtrs&, int32_t*, hipStream_t) {
  reached("launch_plan_tiles");
}
hipError_t launch_gateup(const moe_shape&, const Plan&, const void*, const moe_experts&,
                         const int32_t*, const int32_t*, void*, hipStream_t) { reached("launch_gateup"); }
hipError_t launch_down(const moe_shape&, const Plan&, const void*, const moe_experts&, const int32_t*,
                       void*, hipStream_t) { reached("launch_down"); }
hipError_t launch_ffn(const moe_shape&, const Plan&, const void*, const moe_experts&, const int32_t*,
                      const int32_t*, void*, void*, hipStream_t) { reached("launch_ffn"); }
hipError_t launch_ffn_fused(const moe_shape&, const Plan&, const void*, const moe_experts&,
                            const int32_t*, const int32_t*, float*, int, uint64_t*, hipStream_t) {
  reached("launch_ffn_fused");
}
hipError_t launch_reduce_parts(const moe_shape&, const float*, void*, hipStream_t) {
  reached("launch_reduce_parts");
}
hipError_t launch_combine_parts(const moe_shape&, const float*, const int32_t*, const float*,
                                const void*, void*, hipStream_t) { reached("launch_combine_parts"); }
hipError_t launch_tile_experts(const moe_shape&, const moe_experts&, const moe_experts&, hipStream_t) {
  reached("launch_tile_experts");
}
hipError_t launch_route_locality(const moe_shape&, const int32_t*, int32_t*, int32_t*, hipStream_t) {
  reached("launch_route_locality");
}
hipError_t launch_stage_experts(const moe_shape&, const StagePieces&, const int32_t*, const int32_t*,
                                hipStream_t) { reached("launch_stage_experts"); }
hipError_t launch_stream_read(const void*, size_t, uint32_t*, hipStream_t) { reached("launch_stream_read"); }
hipError_t launch_zero_status(uint32_t*, hipStream_t) { reached("launch_zero_status"); }
hipError_t launch_check_finite(const void*, size_t, bool, uint32_t, uint32_t*, hipStream_t) {
  reached("launch_check_finite");
}
hipError_t launch_combine(const moe_shape&, const void*, const int32_t*, const float*, const void*,
                          void*, hipStream_t) { reached("launch_combine"); }
hipError_t launch_route_permute(const moe_shape&, const Plan&, const void*, const void*, const float*,
                                int32_t*, float*, float*, const PermPtrs&, int32_t*, void*,
                                hipStream_t) { reached("launch_route_permute"); }
hipError_t launch_down_combine(const moe_shape&, const Plan&, const void*, const moe_experts&,
                               const int32_t*, const int32_t*, const int32_t*, const float*,
                               const void*, void*, void*, hipStream_t) {
  reached("launch_down_combine");
}

}  // namespace moe
