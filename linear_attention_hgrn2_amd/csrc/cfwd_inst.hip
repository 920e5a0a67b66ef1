// Instantiations of the per-chunk forward outputs.
#include "dispatch.h"

namespace hgrn2 {

template <typename T, int D, int C> struct ChunkFwdOp {
  static hipError_t run(int gm, const ChunkFwdArgs *a, hipStream_t s) {
    static_assert(sizeof(typename CfwdCfg<T, D, C>::Smem) <= 160 * 1024, "LDS");
    if (gm < kUntied || gm > kScalar) return hipErrorNotSupported;
    if (!a) return hipSuccess;
    if (gm == kTied) return launch_chunk_fwd<T, D, C, kTied>(*a, s);
    if (gm == kGate) return launch_chunk_fwd<T, D, C, kGate>(*a, s);
    if (gm == kScalar) return launch_chunk_fwd<T, D, C, kScalar>(*a, s);
    return launch_chunk_fwd<T, D, C, kUntied>(*a, s);
  }
};

hipError_t dispatch_chunk_fwd(int dtype, int D, int C, int gm, const ChunkFwdArgs *a, hipStream_t s) {
  return run_config<ChunkFwdOp>(dtype, D, C, gm, a, s);
}

}  // namespace hgrn2
