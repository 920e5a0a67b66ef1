// Instantiations of the per-chunk forward outputs.
#include "dispatch.h"

namespace hgrn2 {

template <typename T, int D, int C> struct ChunkFwdOp {
  static hipError_t run(bool tied, const ChunkFwdArgs *a, hipStream_t s) {
    static_assert(sizeof(typename CfwdCfg<T, D, C>::Smem) <= 160 * 1024, "LDS");
    if (!a) return hipSuccess;
    return tied ? launch_chunk_fwd<T, D, C, true>(*a, s) : launch_chunk_fwd<T, D, C, false>(*a, s);
  }
};

hipError_t dispatch_chunk_fwd(int dtype, int D, int C, bool tied, const ChunkFwdArgs *a, hipStream_t s) {
  return run_config<ChunkFwdOp>(dtype, D, C, tied, a, s);
}

}  // namespace hgrn2
