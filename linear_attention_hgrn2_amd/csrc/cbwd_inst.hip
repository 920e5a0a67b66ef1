// Instantiations of the per-chunk gradients, written in the input dtype.
#include "cbwd_op.h"

namespace hgrn2 {

template <typename T, int D, int C> struct ChunkBwdOp {
  static hipError_t run(int gm, const ChunkBwdArgs *a, hipStream_t s) {
    if constexpr (!chunk_bwd_fits<T, D, C>()) {
      return hipErrorNotSupported;
    } else {
      if (gm < kUntied || gm > kScalar) return hipErrorNotSupported;
      if (!a) return hipSuccess;
      // float32 gradients for bfloat16 inputs (float32 inputs write float32 anyway)
      if constexpr (std::is_same<T, bf16_t>::value) {
        if (a->out_f32) return chunk_bwd_f32out(D, C, gm, *a, s);
      }
      return ChunkBwdLaunch<T, D, C, T>::run(gm, *a, s);
    }
  }
};

hipError_t dispatch_chunk_bwd(int dtype, int D, int C, int gm, const ChunkBwdArgs *a, hipStream_t s) {
  return run_config<ChunkBwdOp>(dtype, D, C, gm, a, s);
}

}  // namespace hgrn2
