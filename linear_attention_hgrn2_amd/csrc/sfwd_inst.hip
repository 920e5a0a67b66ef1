// Instantiations of the forward without stored chunk-boundary states: the
// state scan in segment mode, the carry of the segment summaries and the
// segment walk (chunk 64; bf16 at D = 32, 64, 128 and float32 at D = 32, 64,
// whose tiles fit the LDS).
#include "dispatch.h"
#include "sfwd.h"

namespace hgrn2 {

namespace {

template <typename T, int D, int GM> hipError_t seg_t(int op, const void *a, hipStream_t s) {
  if (op == 0) return launch_scan<T, D, 64, false, GM, true>(*(const ScanArgs *)a, s);
  const SegFwdArgs &fa = *(const SegFwdArgs *)a;
  // float32 y for bfloat16 inputs (float32 inputs write float32 anyway)
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (fa.out_f32) return launch_seg_fwd<T, D, 64, GM, float>(fa, s);
  }
  return launch_seg_fwd<T, D, 64, GM>(fa, s);
}

template <typename T, int D> hipError_t seg_g(int gm, int op, const void *a, hipStream_t s) {
  if (!a) return hipSuccess;
  switch (gm) {
    case kUntied: return seg_t<T, D, kUntied>(op, a, s);
    case kTied: return seg_t<T, D, kTied>(op, a, s);
    case kGate: return seg_t<T, D, kGate>(op, a, s);
    case kScalar: return seg_t<T, D, kScalar>(op, a, s);
  }
  return hipErrorNotSupported;
}

hipError_t seg_any(int dtype, int D, int C, int gm, int op, const void *a, hipStream_t s) {
  if (C != 64 || gm < kUntied || gm > kScalar) return hipErrorNotSupported;
  if (dtype == 1) {
    if (D == 32) return seg_g<bf16_t, 32>(gm, op, a, s);
    if (D == 64) return seg_g<bf16_t, 64>(gm, op, a, s);
    if (D == 128) return seg_g<bf16_t, 128>(gm, op, a, s);
  } else if (dtype == 0) {
    if (D == 32) return seg_g<float, 32>(gm, op, a, s);
    if (D == 64) return seg_g<float, 64>(gm, op, a, s);
  }
  return hipErrorNotSupported;
}

}  // namespace

hipError_t dispatch_seg_scan(int dtype, int D, int C, int gm, const ScanArgs *a, hipStream_t s) {
  return seg_any(dtype, D, C, gm, 0, a, s);
}

hipError_t dispatch_seg_fwd(int dtype, int D, int C, int gm, const SegFwdArgs *a, hipStream_t s) {
  return seg_any(dtype, D, C, gm, 1, a, s);
}

hipError_t dispatch_seg_carry(int D, int BH, int NSEG, const float *h0, float *sin, const float *asum, float *ht,
                              hipStream_t s) {
  switch (D) {
    case 32: return launch_seg_carry<32>(BH, NSEG, h0, sin, asum, ht, s);
    case 64: return launch_seg_carry<64>(BH, NSEG, h0, sin, asum, ht, s);
    case 128: return launch_seg_carry<128>(BH, NSEG, h0, sin, asum, ht, s);
  }
  return hipErrorNotSupported;
}

}  // namespace hgrn2
