// Instantiations of the HGRN1 elementwise scan (both dtypes, untied and tied).
#include "dispatch.h"
#include "hgrn1.h"

namespace hgrn2 {

template <typename T, int GM, typename TO> static hipError_t h1_run(int op, const H1Args &a, hipStream_t s) {
  switch (op) {
    case kH1SummaryFwd:
      hipLaunchKernelGGL((hgrn1_summary_kernel<T, GM, false>), h1_sum_grid(a), dim3(64 * kH1Grp), 0, s, a);
      break;
    case kH1SummaryRev:
      hipLaunchKernelGGL((hgrn1_summary_kernel<T, kUntied, true>), h1_sum_grid(a), dim3(64 * kH1Grp), 0, s, a);
      break;
    case kH1CarryFwd:
      hipLaunchKernelGGL((hgrn1_carry_kernel<false>), h1_chan_grid(a), dim3(256), 0, s, a);
      break;
    case kH1CarryRev:
      hipLaunchKernelGGL((hgrn1_carry_kernel<true>), h1_chan_grid(a), dim3(256), 0, s, a);
      break;
    case kH1FinalFwd:
      hipLaunchKernelGGL((hgrn1_final_fwd_kernel<T, GM, TO>), h1_seg_grid(a), dim3(kH1Pairs), 0, s, a);
      break;
    case kH1FinalBwd:
      hipLaunchKernelGGL((hgrn1_final_bwd_kernel<T, GM, TO>), h1_seg_grid(a), dim3(kH1Pairs), 0, s, a);
      break;
    default:
      return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t dispatch_hgrn1(int op, int dtype, int gm, const H1Args &a, hipStream_t s) {
  if (gm != kUntied && gm != kTied) return hipErrorNotSupported;
  if (dtype == 0) return gm == kTied ? h1_run<float, kTied, float>(op, a, s) : h1_run<float, kUntied, float>(op, a, s);
  if (dtype == 1 && a.out_f32)  // float32 y and gradients for bfloat16 inputs
    return gm == kTied ? h1_run<bf16_t, kTied, float>(op, a, s) : h1_run<bf16_t, kUntied, float>(op, a, s);
  if (dtype == 1) return gm == kTied ? h1_run<bf16_t, kTied, bf16_t>(op, a, s) : h1_run<bf16_t, kUntied, bf16_t>(op, a, s);
  return hipErrorNotSupported;
}

}  // namespace hgrn2
