// Instantiations of the per-chunk gradients.
#include "dispatch.h"
#include "cbwd_res.h"

#include <type_traits>

namespace hgrn2 {

template <typename T, int D, int C> struct ChunkBwdOp {
  static hipError_t run(bool tied, const ChunkBwdArgs *a, hipStream_t s) {
    static_assert(sizeof(typename CbwdCfg<T, D, C>::Smem) <= 160 * 1024, "LDS");
    if (!a) return hipSuccess;
    if constexpr (std::is_same<T, bf16_t>::value && D == 128 && C == 64) {
      static_assert(sizeof(CbwdResCfg::Smem) <= 160 * 1024, "LDS");
      return tied ? launch_chunk_bwd_res<true>(*a, s) : launch_chunk_bwd_res<false>(*a, s);
    } else {
      return tied ? launch_chunk_bwd<T, D, C, true>(*a, s) : launch_chunk_bwd<T, D, C, false>(*a, s);
    }
  }
};

hipError_t dispatch_chunk_bwd(int dtype, int D, int C, bool tied, const ChunkBwdArgs *a, hipStream_t s) {
  return run_config<ChunkBwdOp>(dtype, D, C, tied, a, s);
}

}  // namespace hgrn2
