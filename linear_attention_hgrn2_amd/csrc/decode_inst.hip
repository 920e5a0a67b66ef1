// Instantiations of the recurrent decode step for every supported (dtype, D),
// and of the lower-bound gradient reduction.
#include "dispatch.h"
#include "dlb.h"

namespace hgrn2 {

template <typename TIn, int GM, typename TO>
static hipError_t decode_d(int D, const DecodeArgs &a, hipStream_t s) {
  switch (D) {
    case 16: return launch_decode<TIn, 16, GM, TO>(a, s);
    case 32: return launch_decode<TIn, 32, GM, TO>(a, s);
    case 64: return launch_decode<TIn, 64, GM, TO>(a, s);
    case 128: return launch_decode<TIn, 128, GM, TO>(a, s);
  }
  return hipErrorNotSupported;
}

template <typename TIn, typename TO>
static hipError_t decode_t(int D, int gm, const DecodeArgs &a, hipStream_t s) {
  if (gm == kTied) return decode_d<TIn, kTied, TO>(D, a, s);
  if (gm == kGate) return decode_d<TIn, kGate, TO>(D, a, s);
  if (gm == kScalar) return decode_d<TIn, kScalar, TO>(D, a, s);
  if (gm == kUntied) return decode_d<TIn, kUntied, TO>(D, a, s);
  return hipErrorNotSupported;
}

hipError_t dispatch_decode(int dtype, int D, int gm, const DecodeArgs &a, hipStream_t s) {
  if (dtype == 0) return decode_t<float, float>(D, gm, a, s);
  if (dtype == 1) return a.out_f32 ? decode_t<bf16_t, float>(D, gm, a, s) : decode_t<bf16_t, bf16_t>(D, gm, a, s);
  return hipErrorNotSupported;
}

long long decode_items_per_bh(int D) {
  switch (D) {
    case 16: return DecodeCfg<16>::NT;
    case 32: return DecodeCfg<32>::NT;
    case 64: return DecodeCfg<64>::NT;
    case 128: return DecodeCfg<128>::NT;
  }
  return 0;
}

hipError_t dispatch_dlb_reduce(int B, int H, int N, int D, const float *part, float *dlb, hipStream_t s) {
  switch (D) {
    case 16: return launch_dlb_reduce<16>(B, H, N, part, dlb, s);
    case 32: return launch_dlb_reduce<32>(B, H, N, part, dlb, s);
    case 64: return launch_dlb_reduce<64>(B, H, N, part, dlb, s);
    case 128: return launch_dlb_reduce<128>(B, H, N, part, dlb, s);
  }
  return hipErrorNotSupported;
}

}  // namespace hgrn2
