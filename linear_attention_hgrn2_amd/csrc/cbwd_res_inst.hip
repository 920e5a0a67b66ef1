// Instantiations of the resident per-chunk gradients (bfloat16 inputs, d =
// 128, chunk 64; gradients in bfloat16 or float32), compiled apart from the
// generic kernels so that their build options can differ (build.py).
#include "cbwd_res.h"

namespace hgrn2 {

static_assert(sizeof(CbwdResCfg::Smem) <= 160 * 1024, "LDS");

hipError_t chunk_bwd_res(int gm, bool out_f32, const ChunkBwdArgs &a, hipStream_t s) {
  if (out_f32) {
    if (gm == kTied) return launch_chunk_bwd_res<kTied, float>(a, s);
    if (gm == kGate) return launch_chunk_bwd_res<kGate, float>(a, s);
    if (gm == kScalar) return launch_chunk_bwd_res<kScalar, float>(a, s);
    return launch_chunk_bwd_res<kUntied, float>(a, s);
  }
  if (gm == kTied) return launch_chunk_bwd_res<kTied, bf16_t>(a, s);
  if (gm == kGate) return launch_chunk_bwd_res<kGate, bf16_t>(a, s);
  if (gm == kScalar) return launch_chunk_bwd_res<kScalar, bf16_t>(a, s);
  return launch_chunk_bwd_res<kUntied, bf16_t>(a, s);
}

}  // namespace hgrn2
