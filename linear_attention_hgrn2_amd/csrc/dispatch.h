// Internal dispatch table between the C ABI and the kernel templates.
#pragma once

#include <hip/hip_runtime.h>

#include "bwd.h"
#include "decode.h"
#include "fwd.h"

namespace hgrn2 {

// Each returns hipErrorNotSupported (without launching) when no kernel
// exists for the combination, else the launch status.
hipError_t dispatch_fwd(int dtype, int D, int C, const FwdArgs &a, hipStream_t s);
hipError_t dispatch_bwd(int dtype, int D, int C, const BwdArgs &a, hipStream_t s);
hipError_t dispatch_decode(int dtype, int D, const DecodeArgs &a, hipStream_t s);
bool fwd_exists(int dtype, int D, int C);
bool bwd_exists(int dtype, int D, int C);

}  // namespace hgrn2
