// Launch entry points for a CPU-only build of the C ABI's host code
// (argument validation, policy descriptor, workspace queries) under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every launch reports an
// error instead of running: the host tests never reach one with real
// buffers.  Test infrastructure only; not part of libtig.so.
#include "tig_internal.h"

namespace tig {
hipError_t launch_tree_gemm(const TreeGemmLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_logprob(const LogprobLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_moe(const MoeLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_group_gemm(const GroupLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fp8_gemm(const Fp8GemmLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fp8_group_gemm(const Fp8GroupLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fp8_quantize(const uint16_t*, int64_t, uint8_t*, int64_t, uint8_t*, int64_t, int64_t, int,
                               hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fp8_dequant(const uint8_t*, const uint8_t*, int64_t, int64_t, int, uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_silu_mul_fp8(const float*, int64_t, uint8_t*, int64_t, uint8_t*, int64_t, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_silu_mul(const float*, int64_t, uint16_t*, int64_t, int64_t, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_topk_positions(const float*, int64_t, const int32_t*, int64_t, int, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_router_logits(const void*, const void*, float*, int64_t, int64_t, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_moe_route(const float*, int64_t, int, int, int32_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t noalloc_scratch(void**) { return hipErrorNotSupported; }
}  // namespace tig

extern "C" const char* hipGetErrorString(hipError_t) { return "launch stubbed in the sanitizer build"; }
