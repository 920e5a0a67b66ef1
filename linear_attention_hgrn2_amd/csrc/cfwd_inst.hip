// Instantiations of the per-chunk forward outputs.
#include "dispatch.h"

namespace hgrn2 {

template <typename T, int D, int C> struct ChunkFwdOp {
  template <typename TO> static hipError_t go(int gm, const ChunkFwdArgs &a, hipStream_t s) {
    if (gm == kTied) return launch_chunk_fwd<T, D, C, kTied, TO>(a, s);
    if (gm == kGate) return launch_chunk_fwd<T, D, C, kGate, TO>(a, s);
    if (gm == kScalar) return launch_chunk_fwd<T, D, C, kScalar, TO>(a, s);
    return launch_chunk_fwd<T, D, C, kUntied, TO>(a, s);
  }
  static hipError_t run(int gm, const ChunkFwdArgs *a, hipStream_t s) {
    // tiles too large for the 160 KB LDS (float32 at D = 128, chunk 128): no kernel
    if constexpr (sizeof(typename CfwdCfg<T, D, C>::Smem) > 160 * 1024) {
      return hipErrorNotSupported;
    } else {
      if (gm < kUntied || gm > kScalar) return hipErrorNotSupported;
      if (!a) return hipSuccess;
      // float32 y for bfloat16 inputs (float32 inputs write float32 anyway)
      if constexpr (std::is_same<T, bf16_t>::value) {
        if (a->out_f32) return go<float>(gm, *a, s);
      }
      return go<T>(gm, *a, s);
    }
  }
};

hipError_t dispatch_chunk_fwd(int dtype, int D, int C, int gm, const ChunkFwdArgs *a, hipStream_t s) {
  return run_config<ChunkFwdOp>(dtype, D, C, gm, a, s);
}

// one workgroup of 4 C work-items per chunk (the chunk forward and the
// non-resident chunk backward alike; the resident backward launches at most
// one workgroup per compute unit)
long long chunk_items_per_chunk(int C) { return 4LL * C; }

}  // namespace hgrn2
