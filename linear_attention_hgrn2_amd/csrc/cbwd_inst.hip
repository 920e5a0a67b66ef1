// Instantiations of the per-chunk gradients.
#include "dispatch.h"
#include "cbwd_res.h"

#include <type_traits>

namespace hgrn2 {

template <typename T, int D, int C> struct ChunkBwdOp {
  template <int GM> static hipError_t go(const ChunkBwdArgs &a, hipStream_t s) {
    if constexpr (std::is_same<T, bf16_t>::value && D == 128 && C == 64) {
      static_assert(sizeof(CbwdResCfg::Smem) <= 160 * 1024, "LDS");
      return launch_chunk_bwd_res<GM>(a, s);
    } else {
      return launch_chunk_bwd<T, D, C, GM>(a, s);
    }
  }
  static hipError_t run(int gm, const ChunkBwdArgs *a, hipStream_t s) {
    // tiles too large for the 160 KB LDS (float32 at D = 128, chunk 128): no kernel
    if constexpr (sizeof(typename CbwdCfg<T, D, C>::Smem) > 160 * 1024) {
      return hipErrorNotSupported;
    } else {
      if (gm < kUntied || gm > kScalar) return hipErrorNotSupported;
      if (!a) return hipSuccess;
      if (gm == kTied) return go<kTied>(*a, s);
      if (gm == kGate) return go<kGate>(*a, s);
      if (gm == kScalar) return go<kScalar>(*a, s);
      return go<kUntied>(*a, s);
    }
  }
};

hipError_t dispatch_chunk_bwd(int dtype, int D, int C, int gm, const ChunkBwdArgs *a, hipStream_t s) {
  return run_config<ChunkBwdOp>(dtype, D, C, gm, a, s);
}

}  // namespace hgrn2
