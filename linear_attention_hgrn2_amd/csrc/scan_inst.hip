// Instantiations of the chunk-boundary state scan (both directions).
#include "dispatch.h"

namespace hgrn2 {

template <typename T, int D, int C> struct ScanOp {
  static hipError_t run(bool reverse, bool tied, const ScanArgs *a, hipStream_t s) {
    if (!a) return reverse && tied ? hipErrorNotSupported : hipSuccess;
    if (reverse) return tied ? hipErrorNotSupported : launch_scan<T, D, C, true>(*a, s);
    return tied ? launch_scan<T, D, C, false, true>(*a, s) : launch_scan<T, D, C, false>(*a, s);
  }
};

hipError_t dispatch_scan(int dtype, int D, int C, bool reverse, bool tied, const ScanArgs *a, hipStream_t s) {
  return run_config<ScanOp>(dtype, D, C, reverse, tied, a, s);
}

}  // namespace hgrn2
