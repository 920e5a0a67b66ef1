// Internal dispatch between the C ABI and the kernel templates.
#pragma once

#include <hip/hip_runtime.h>

#include "cbwd.h"
#include "cfwd.h"
#include "decode.h"
#include "hgrn1.h"
#include "scan.h"
#include "sfwd.h"

namespace hgrn2 {

// Runs Op<T, D, C>::run(args...) for the runtime (dtype, D, chunk), or
// returns hipErrorNotSupported when the combination has no instance.
template <template <typename, int, int> class Op, typename T, int D, typename... A>
hipError_t run_c(int C, A... args) {
  switch (C) {
    case 16: return Op<T, D, 16>::run(args...);
    case 32: return Op<T, D, 32>::run(args...);
    case 64: return Op<T, D, 64>::run(args...);
    case 128: return Op<T, D, 128>::run(args...);
  }
  return hipErrorNotSupported;
}
template <template <typename, int, int> class Op, typename T, typename... A>
hipError_t run_d(int D, int C, A... args) {
  switch (D) {
    case 16: return run_c<Op, T, 16>(C, args...);
    case 32: return run_c<Op, T, 32>(C, args...);
    case 64: return run_c<Op, T, 64>(C, args...);
    case 128: return run_c<Op, T, 128>(C, args...);
  }
  return hipErrorNotSupported;
}
template <template <typename, int, int> class Op, typename... A>
hipError_t run_config(int dtype, int D, int C, A... args) {
  if (dtype == 0) return run_d<Op, float>(D, C, args...);
  if (dtype == 1) return run_d<Op, bf16_t>(D, C, args...);
  return hipErrorNotSupported;
}

// Each returns hipErrorNotSupported (without launching) when no kernel
// exists for the combination, else the launch status.  A null args pointer
// only asks whether the kernel exists.
// `gm` is a GateMode: kUntied (k and log f are inputs), kTied (k = 1 - f
// formed from log f; the backward writes the total dlog f and no dk) or kGate
// (log f and k formed from the pre-activation and the lower bound; the
// backward writes dz and per-chunk sums of dlb, and no dk).
hipError_t dispatch_scan(int dtype, int D, int C, bool reverse, int gm, const ScanArgs *a, hipStream_t s);
hipError_t dispatch_chunk_fwd(int dtype, int D, int C, int gm, const ChunkFwdArgs *a, hipStream_t s);
hipError_t dispatch_chunk_bwd(int dtype, int D, int C, int gm, const ChunkBwdArgs *a, hipStream_t s);
hipError_t dispatch_decode(int dtype, int D, int gm, const DecodeArgs &a, hipStream_t s);
// dlb[h][c] = sum over b and chunks n of part[(b H + h) N + n][c], in a fixed order
hipError_t dispatch_dlb_reduce(int B, int H, int N, int D, const float *part, float *dlb, hipStream_t s);
// one pass of the HGRN1 elementwise scan (gm: kUntied or kTied)
enum H1Op : int { kH1SummaryFwd, kH1SummaryRev, kH1CarryFwd, kH1CarryRev, kH1FinalFwd, kH1FinalBwd };
hipError_t dispatch_hgrn1(int op, int dtype, int gm, const H1Args &a, hipStream_t s);

// The forward without stored chunk-boundary states (sfwd.h): the state scan
// in segment mode (segment summaries), their carry, and the segment walk.
// A null args pointer only asks whether the kernel exists.
hipError_t dispatch_seg_scan(int dtype, int D, int C, int gm, const ScanArgs *a, hipStream_t s);
hipError_t dispatch_seg_fwd(int dtype, int D, int C, int gm, const SegFwdArgs *a, hipStream_t s);
hipError_t dispatch_seg_carry(int D, int BH, int NSEG, const float *h0, float *sin, const float *asum, float *ht,
                              hipStream_t s);

// Launch geometry, for the size checks that run before anything is launched:
// work-items per (b, h) of the state scan (its workgroups for one (b, h) are
// padded to groups of eight (b, h)), per chunk of the chunk kernels, and per
// (b, h) of the decode step; 0 when no kernel exists.
long long scan_items_per_bh(int dtype, int D, int C);
long long chunk_items_per_chunk(int C);
long long decode_items_per_bh(int D);

}  // namespace hgrn2
