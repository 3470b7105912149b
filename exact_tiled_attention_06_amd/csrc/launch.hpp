// Host-side launchers implemented next to their kernels; called by the C ABI
// layer after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace fa2 {

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t stream);
// Backward: delta/zeroing pass, the K/V-block pass and the dQ conversion.
hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool deterministic, hipStream_t stream);

}  // namespace fa2
