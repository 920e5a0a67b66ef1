// Instantiations of the chunked backward for every supported (dtype, D, chunk).
#include "dispatch.h"

namespace hgrn2 {

template <typename TIn, int D, int C>
static hipError_t bwd_one(const BwdArgs *a, hipStream_t s) {
  if constexpr (BwdCfg<TIn, D, C>::fits) {
    if (a) return launch_bwd<TIn, D, C>(*a, s);
    return hipSuccess;
  } else {
    return hipErrorNotSupported;
  }
}

template <typename TIn, int D>
static hipError_t bwd_c(int C, const BwdArgs *a, hipStream_t s) {
  switch (C) {
    case 16: return bwd_one<TIn, D, 16>(a, s);
    case 32: return bwd_one<TIn, D, 32>(a, s);
    case 64: return bwd_one<TIn, D, 64>(a, s);
  }
  return hipErrorNotSupported;
}

template <typename TIn>
static hipError_t bwd_d(int D, int C, const BwdArgs *a, hipStream_t s) {
  switch (D) {
    case 16: return bwd_c<TIn, 16>(C, a, s);
    case 32: return bwd_c<TIn, 32>(C, a, s);
    case 64: return bwd_c<TIn, 64>(C, a, s);
    case 128: return bwd_c<TIn, 128>(C, a, s);
  }
  return hipErrorNotSupported;
}

static hipError_t bwd_any(int dtype, int D, int C, const BwdArgs *a, hipStream_t s) {
  if (dtype == 0) return bwd_d<float>(D, C, a, s);
  if (dtype == 1) return bwd_d<bf16_t>(D, C, a, s);
  return hipErrorNotSupported;
}

hipError_t dispatch_bwd(int dtype, int D, int C, const BwdArgs &a, hipStream_t s) {
  return bwd_any(dtype, D, C, &a, s);
}
bool bwd_exists(int dtype, int D, int C) { return bwd_any(dtype, D, C, nullptr, nullptr) == hipSuccess; }

}  // namespace hgrn2
