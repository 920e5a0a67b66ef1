// Instantiations of the per-chunk gradients.
#include "dispatch.h"

namespace hgrn2 {

template <typename T, int D, int C> struct ChunkBwdOp {
  static hipError_t run(const ChunkBwdArgs *a, hipStream_t s) {
    static_assert(sizeof(typename CbwdCfg<T, D, C>::Smem) <= 160 * 1024, "LDS");
    if (!a) return hipSuccess;
    return launch_chunk_bwd<T, D, C>(*a, s);
  }
};

hipError_t dispatch_chunk_bwd(int dtype, int D, int C, const ChunkBwdArgs *a, hipStream_t s) {
  return run_config<ChunkBwdOp>(dtype, D, C, a, s);
}

}  // namespace hgrn2
