// Instantiations of the recurrent decode step for every supported (dtype, D).
#include "dispatch.h"

namespace hgrn2 {

template <typename TIn>
static hipError_t decode_d(int D, const DecodeArgs &a, hipStream_t s) {
  switch (D) {
    case 16: return launch_decode<TIn, 16>(a, s);
    case 32: return launch_decode<TIn, 32>(a, s);
    case 64: return launch_decode<TIn, 64>(a, s);
    case 128: return launch_decode<TIn, 128>(a, s);
  }
  return hipErrorNotSupported;
}

hipError_t dispatch_decode(int dtype, int D, const DecodeArgs &a, hipStream_t s) {
  if (dtype == 0) return decode_d<float>(D, a, s);
  if (dtype == 1) return decode_d<bf16_t>(D, a, s);
  return hipErrorNotSupported;
}

}  // namespace hgrn2
