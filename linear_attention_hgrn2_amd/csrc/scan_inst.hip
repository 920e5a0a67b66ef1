// Instantiations of the chunk-boundary state scan (both directions).
#include "dispatch.h"

namespace hgrn2 {

template <typename T, int D, int C> struct ScanOp {
  // the adjoint scan never reads k: it runs in the untied form or, when log f
  // is formed from the gate pre-activation or read per head, in that mode
  static hipError_t run(bool reverse, int gm, const ScanArgs *a, hipStream_t s) {
    // tiles too large for the 160 KB LDS (float32 at D = 128, chunk 128): no kernel
    if constexpr (sizeof(typename ScanCfg<T, D, C, false>::Smem) > 160 * 1024) {
      return hipErrorNotSupported;
    } else {
      if (gm < kUntied || gm > kScalar || (reverse && gm == kTied)) return hipErrorNotSupported;
      if (!a) return hipSuccess;
      if (reverse) {
        if (gm == kGate) return launch_scan<T, D, C, true, kGate>(*a, s);
        if (gm == kScalar) return launch_scan<T, D, C, true, kScalar>(*a, s);
        return launch_scan<T, D, C, true>(*a, s);
      }
      if (gm == kTied) return launch_scan<T, D, C, false, kTied>(*a, s);
      if (gm == kGate) return launch_scan<T, D, C, false, kGate>(*a, s);
      if (gm == kScalar) return launch_scan<T, D, C, false, kScalar>(*a, s);
      return launch_scan<T, D, C, false>(*a, s);
    }
  }
};

hipError_t dispatch_scan(int dtype, int D, int C, bool reverse, int gm, const ScanArgs *a, hipStream_t s) {
  return run_config<ScanOp>(dtype, D, C, reverse, gm, a, s);
}

template <typename T, int D, int C> struct ScanItemsOp {
  static hipError_t run(long long *n) {
    using Cfg = ScanCfg<T, D, C, false>;
    if constexpr (sizeof(typename Cfg::Smem) > 160 * 1024) {
      return hipErrorNotSupported;
    } else {
      *n = (long long)Cfg::NS * Cfg::NT;
      return hipSuccess;
    }
  }
};

long long scan_items_per_bh(int dtype, int D, int C) {
  long long n = 0;
  return run_config<ScanItemsOp>(dtype, D, C, &n) == hipSuccess ? n : 0;
}

}  // namespace hgrn2
