// Instantiations of the per-chunk gradients for bfloat16 inputs with float32
// gradients (compiled apart from the input-dtype ones so the two build in
// parallel).
#include "cbwd_op.h"

namespace hgrn2 {

template <typename T, int D, int C> struct ChunkBwdF32Op {
  static hipError_t run(int gm, const ChunkBwdArgs *a, hipStream_t s) {
    if constexpr (!chunk_bwd_fits<T, D, C>()) {
      return hipErrorNotSupported;
    } else {
      return ChunkBwdLaunch<T, D, C, float>::run(gm, *a, s);
    }
  }
};

hipError_t chunk_bwd_f32out(int D, int C, int gm, const ChunkBwdArgs &a, hipStream_t s) {
  return run_d<ChunkBwdF32Op, bf16_t>(D, C, gm, &a, s);
}

}  // namespace hgrn2
