// The per-chunk gradients of one (T, D, C), gradients written as TO: the
// resident kernel for bfloat16 at D = 128, chunk 64 (instantiated apart, in
// cbwd_res_inst.hip), else the generic one, instantiated by cbwd_inst.hip
// (TO = T) and cbwd_f32out_inst.hip (bfloat16 inputs, float32 gradients).
#pragma once

#include <type_traits>

#include "dispatch.h"

namespace hgrn2 {

// the resident kernel (cbwd_res_inst.hip): gradients in bfloat16 or float32
hipError_t chunk_bwd_res(int gm, bool out_f32, const ChunkBwdArgs &a, hipStream_t s);

template <typename T, int D, int C, typename TO> struct ChunkBwdLaunch {
  template <int GM> static hipError_t go(const ChunkBwdArgs &a, hipStream_t s) {
    if constexpr (std::is_same<T, bf16_t>::value && D == 128 && C == 64) {
      return chunk_bwd_res(GM, std::is_same<TO, float>::value, a, s);
    } else {
      return launch_chunk_bwd<T, D, C, GM, TO>(a, s);
    }
  }
  static hipError_t run(int gm, const ChunkBwdArgs &a, hipStream_t s) {
    if (gm == kTied) return go<kTied>(a, s);
    if (gm == kGate) return go<kGate>(a, s);
    if (gm == kScalar) return go<kScalar>(a, s);
    return go<kUntied>(a, s);
  }
};

// tiles too large for the 160 KB LDS (float32 at D = 128, chunk 128): no kernel
template <typename T, int D, int C> constexpr bool chunk_bwd_fits() {
  return sizeof(typename CbwdCfg<T, D, C>::Smem) <= 160 * 1024;
}

// bfloat16 inputs, float32 gradients (cbwd_f32out_inst.hip)
hipError_t chunk_bwd_f32out(int D, int C, int gm, const ChunkBwdArgs &a, hipStream_t s);

}  // namespace hgrn2
