// Sum of the per-chunk lower-bound gradients over batch and chunks (gate
// mode): dlb[h][c] = sum_{b, n} part[(b H + h) N + n][c].  The lower bound of
// a head channel is shared by every token, so its gradient sums the
// per-token terms (HGRN2 summary, paperlayer.ai, §2.2: per-layer lower
// bounds).  Small and HBM-bound (one read of B H N D floats); the order of
// the additions is fixed, so repeated runs agree bit for bit.
#pragma once

#include "common.h"

namespace hgrn2 {

// One workgroup of 1024 threads per (head, group of CG channels): RG row
// groups split the B N rows of that head in a fixed interleave, each thread
// issuing sixteen loads at a time into eight partial sums (the sum is bound by
// load latency, not bytes), and the row groups are combined in LDS in a fixed
// order.
template <int D>
__global__ __launch_bounds__(1024) void hgrn2_dlb_reduce_kernel(int B, int H, int N, const float *part, float *dlb) {
  constexpr int CG = D < 64 ? D : 64, RG = 1024 / CG, U = 16;
  __shared__ float acc[RG][CG];
  const int h = blockIdx.x / (D / CG), c = (blockIdx.x % (D / CG)) * CG + threadIdx.x % CG;
  const int rg = threadIdx.x / CG;
  const int rows = B * N;
  auto at = [&](int r) { return part[(((size_t)(r / N) * H + h) * N + (r % N)) * D + c]; };
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int r = rg;
  for (; r + (U - 1) * RG < rows; r += U * RG) {
    float x[U];
#pragma unroll
    for (int i = 0; i < U; ++i) x[i] = at(r + i * RG);
#pragma unroll
    for (int i = 0; i < U; ++i) s[i % 8] += x[i];
  }
  for (; r < rows; r += RG) s[0] += at(r);
  acc[rg][threadIdx.x % CG] = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  __syncthreads();
  if (rg == 0) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) t += acc[i][threadIdx.x];
    dlb[h * D + c] = t;
  }
}

template <int D>
hipError_t launch_dlb_reduce(int B, int H, int N, const float *part, float *dlb, hipStream_t stream) {
  hipLaunchKernelGGL(hgrn2_dlb_reduce_kernel<D>, dim3(H * (D / (D < 64 ? D : 64))), dim3(1024), 0, stream, B, H, N,
                     part, dlb);
  return hipGetLastError();
}

}  // namespace hgrn2
