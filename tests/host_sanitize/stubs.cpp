// Host-only stand-ins for the kernel launchers, for the sanitizer build of the
// C-ABI layer (api.cpp, contract.cpp) with g++. The driver only makes calls
// that validation rejects or that are empty, so no launcher may ever run:
// every stand-in reports a failure, which the entry point turns into
// INV_E_HIP and the driver into a test failure.
#include <hip/hip_runtime_api.h>

#include <cstdio>

#include "../../split_invariant_deterministic_amd/csrc/launch.h"

namespace {
hipError_t reached(const char* what) {
  std::fprintf(stderr, "launcher reached in a host-only test: %s\n", what);
  return hipErrorInvalidValue;
}
}  // namespace

namespace inv {
hipError_t launch_gemm(const GemmLaunch&, hipStream_t) { return reached("gemm"); }
hipError_t launch_tree_combine(const float*, int, int64_t, void*, bool, bool, hipStream_t) { return reached("tree"); }
hipError_t launch_cast_bf16(const float*, uint16_t*, int64_t, hipStream_t) { return reached("cast"); }
hipError_t launch_rmsnorm(const void*, const void*, void*, int64_t, int64_t, float, hipStream_t) {
  return reached("rmsnorm");
}
hipError_t launch_logprob(const float*, int64_t, const int32_t*, float*, float*, float*, int64_t, int64_t, int, int,
                          int, bool, bool, hipStream_t) {
  return reached("logprob");
}
hipError_t launch_block16_merge(const float*, const float*, const int32_t*, float*, int64_t, int64_t, bool,
                                hipStream_t) {
  return reached("block16 merge");
}
hipError_t launch_block16_stats(const float*, int64_t, const int32_t*, float*, float*, int64_t, int64_t, hipStream_t) {
  return reached("block16 stats");
}
hipError_t launch_logprob_combine(const float*, const float*, const int32_t*, float*, int64_t, int64_t, int, bool,
                                  hipStream_t) {
  return reached("logprob combine");
}
hipError_t launch_attn_splits(const AttnLaunch&, hipStream_t) { return reached("attn splits"); }
hipError_t launch_attn_combine(const float*, void*, int64_t, int, int, int, bool, hipStream_t) {
  return reached("attn combine");
}
hipError_t launch_gdn_prefill(const GdnArgs&, int, bool, hipStream_t) { return reached("gdn prefill"); }
hipError_t launch_gdn_decode(const GdnDecodeArgs&, int, bool, hipStream_t) { return reached("gdn decode"); }
hipError_t launch_mfma_loop(int64_t, int, uint64_t*, float*, hipStream_t) { return reached("mfma loop"); }
hipError_t scratch_device_ptr(void**) { return reached("scratch"); }
hipError_t launch_moe_route(const float*, int32_t*, float*, int64_t, int, int, hipStream_t) { return reached("route"); }
hipError_t launch_moe_permute(const int32_t*, int32_t*, int32_t*, int32_t*, int64_t, int, int, hipStream_t) {
  return reached("permute");
}
hipError_t launch_swiglu(const void*, void*, int64_t, int64_t, hipStream_t) { return reached("swiglu"); }
hipError_t launch_moe_combine(const float*, const float*, const int32_t*, int64_t, void*, int64_t, int64_t, int, bool,
                              hipStream_t) {
  return reached("moe combine");
}
}  // namespace inv
