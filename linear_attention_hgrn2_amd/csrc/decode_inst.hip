// Instantiations of the recurrent decode step for every supported (dtype, D).
#include "dispatch.h"

namespace hgrn2 {

template <typename TIn, bool TIED>
static hipError_t decode_d(int D, const DecodeArgs &a, hipStream_t s) {
  switch (D) {
    case 16: return launch_decode<TIn, 16, TIED>(a, s);
    case 32: return launch_decode<TIn, 32, TIED>(a, s);
    case 64: return launch_decode<TIn, 64, TIED>(a, s);
    case 128: return launch_decode<TIn, 128, TIED>(a, s);
  }
  return hipErrorNotSupported;
}

hipError_t dispatch_decode(int dtype, int D, bool tied, const DecodeArgs &a, hipStream_t s) {
  if (dtype == 0) return tied ? decode_d<float, true>(D, a, s) : decode_d<float, false>(D, a, s);
  if (dtype == 1) return tied ? decode_d<bf16_t, true>(D, a, s) : decode_d<bf16_t, false>(D, a, s);
  return hipErrorNotSupported;
}

}  // namespace hgrn2
