// Internal dispatch between the C ABI and the kernel templates.
#pragma once

#include <hip/hip_runtime.h>

#include "cbwd.h"
#include "cfwd.h"
#include "decode.h"
#include "scan.h"

namespace hgrn2 {

// Runs Op<T, D, C>::run(args...) for the runtime (dtype, D, chunk), or
// returns hipErrorNotSupported when the combination has no instance.
template <template <typename, int, int> class Op, typename T, int D, typename... A>
hipError_t run_c(int C, A... args) {
  switch (C) {
    case 16: return Op<T, D, 16>::run(args...);
    case 32: return Op<T, D, 32>::run(args...);
    case 64: return Op<T, D, 64>::run(args...);
  }
  return hipErrorNotSupported;
}
template <template <typename, int, int> class Op, typename T, typename... A>
hipError_t run_d(int D, int C, A... args) {
  switch (D) {
    case 16: return run_c<Op, T, 16>(C, args...);
    case 32: return run_c<Op, T, 32>(C, args...);
    case 64: return run_c<Op, T, 64>(C, args...);
    case 128: return run_c<Op, T, 128>(C, args...);
  }
  return hipErrorNotSupported;
}
template <template <typename, int, int> class Op, typename... A>
hipError_t run_config(int dtype, int D, int C, A... args) {
  if (dtype == 0) return run_d<Op, float>(D, C, args...);
  if (dtype == 1) return run_d<Op, bf16_t>(D, C, args...);
  return hipErrorNotSupported;
}

// Each returns hipErrorNotSupported (without launching) when no kernel
// exists for the combination, else the launch status.  A null args pointer
// only asks whether the kernel exists.
// `tied`: k = 1 - exp(log f) is formed in the kernel (k pointers unused) and
// the backward writes the total dlog f and no dk.
hipError_t dispatch_scan(int dtype, int D, int C, bool reverse, bool tied, const ScanArgs *a, hipStream_t s);
hipError_t dispatch_chunk_fwd(int dtype, int D, int C, bool tied, const ChunkFwdArgs *a, hipStream_t s);
hipError_t dispatch_chunk_bwd(int dtype, int D, int C, bool tied, const ChunkBwdArgs *a, hipStream_t s);
hipError_t dispatch_decode(int dtype, int D, bool tied, const DecodeArgs &a, hipStream_t s);

}  // namespace hgrn2
