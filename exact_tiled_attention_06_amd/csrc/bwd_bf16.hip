// Backward attention (placeholder until the MFMA backward lands).
#include "common.hpp"
#include "launch.hpp"

namespace fa2 {
hipError_t launch_bwd_bf16(const BwdParams&, int, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fa2
