// Instantiations of the chunked forward for every supported (dtype, D, chunk).
#include "dispatch.h"

namespace hgrn2 {

template <typename TIn, int D, int C>
static hipError_t fwd_one(const FwdArgs *a, hipStream_t s) {
  constexpr int DVT = D < 64 ? D : 64;
  if constexpr (FwdCfg<TIn, D, C, DVT>::fits) {
    if (a) return launch_fwd<TIn, D, C, DVT>(*a, s);
    return hipSuccess;
  } else {
    return hipErrorNotSupported;
  }
}

template <typename TIn, int D>
static hipError_t fwd_c(int C, const FwdArgs *a, hipStream_t s) {
  switch (C) {
    case 16: return fwd_one<TIn, D, 16>(a, s);
    case 32: return fwd_one<TIn, D, 32>(a, s);
    case 64: return fwd_one<TIn, D, 64>(a, s);
  }
  return hipErrorNotSupported;
}

template <typename TIn>
static hipError_t fwd_d(int D, int C, const FwdArgs *a, hipStream_t s) {
  switch (D) {
    case 16: return fwd_c<TIn, 16>(C, a, s);
    case 32: return fwd_c<TIn, 32>(C, a, s);
    case 64: return fwd_c<TIn, 64>(C, a, s);
    case 128: return fwd_c<TIn, 128>(C, a, s);
  }
  return hipErrorNotSupported;
}

static hipError_t fwd_any(int dtype, int D, int C, const FwdArgs *a, hipStream_t s) {
  if (dtype == 0) return fwd_d<float>(D, C, a, s);
  if (dtype == 1) return fwd_d<bf16_t>(D, C, a, s);
  return hipErrorNotSupported;
}

hipError_t dispatch_fwd(int dtype, int D, int C, const FwdArgs &a, hipStream_t s) {
  return fwd_any(dtype, D, C, &a, s);
}
bool fwd_exists(int dtype, int D, int C) { return fwd_any(dtype, D, C, nullptr, nullptr) == hipSuccess; }

}  // namespace hgrn2
