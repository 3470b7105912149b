// Host-side launchers implemented next to their kernels; called by the C ABI
// layer after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace fa2 {

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t stream);
// Backward. split_dq: the dQ pass with the D pass folded in (fuse_stats), then the
// dK/dV pass (no atomics); else D pass with accumulator zeroing, key-block pass with
// atomic dQ, dQ conversion.
hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool split_dq, hipStream_t stream);
// The passes of the split backward, launched one at a time (the dQ pass forms D
// itself when p.fuse_stats is set, else it reads what the D pass wrote).
hipError_t launch_bwd_prep(const BwdParams& p, int d, bool zero_acc, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, int d, hipStream_t stream);

}  // namespace fa2
