// Recurrent decode step (HGRN2 summary, paperlayer.ai, §1: recurrent
// inference with linear cost; §3.2: state update and readout):
//   S <- Diag(exp(log_f)) S + k^T v   (in place),   y = q S
// (k = 1 - exp(log_f) with tied gates; log f and k from the pre-activation z
// and the lower bound lb in gate mode, f = lb + (1 - lb) sigmoid(z)).
// Pure HBM streaming: each (b, h) state (D*D float32) is read once and written
// once.  One workgroup per (b, h); a thread owns a 4-column group (16-byte
// accesses, consecutive threads on consecutive columns, so every wavefront
// instruction covers whole rows) and a strided set of rows; all of its row
// loads are issued before any of them is used.  The column sums of q S are
// reduced through LDS.  State stores are non-temporal (streamed past the
// caches), which lifts the write rate of this read-once/write-once pattern.
#pragma once

#include "common.h"

namespace hgrn2 {

struct DecodeArgs {
  int B, H;
  const void *q, *k, *v, *log_f;  // log_f holds z in gate mode
  const float *lb;                // gate mode: lower bound of f, [H,D]
  float *state;
  void *y;          // [B,H,D], the input dtype or (out_f32) float32
  int out_f32 = 0;  // bfloat16 inputs: write y as float32
};

template <int D> struct DecodeCfg {
  static constexpr int CG = D / 4;                         // 4-column groups per row
  static constexpr int NT = (D * D / 4 < 256) ? D * D / 4 : 256;
  static constexpr int RG = NT / CG;                       // rows handled per pass
  static constexpr int PASSES = D / RG;
  static_assert(D % RG == 0, "row split");
};

// TO: the element type of y (TIn, or float32 for bfloat16 inputs)
template <typename TIn, int D, int GM, typename TO = TIn>
__global__ __launch_bounds__(256) void hgrn2_decode_kernel(DecodeArgs a) {
  using Cfg = DecodeCfg<D>;
  constexpr int CG = Cfg::CG, RG = Cfg::RG, PASSES = Cfg::PASSES;
  __shared__ float s_q[D], s_k[D], s_f[D];
  __shared__ float4 s_part[RG][CG];

  const int bh = blockIdx.x;
  if (bh >= a.B * a.H) return;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;

  const TIn *gq = (const TIn *)a.q + (size_t)bh * D;
  const TIn *gk = (const TIn *)a.k + (size_t)bh * D;
  const TIn *gv = (const TIn *)a.v + (size_t)bh * D;
  const TIn *gl = (const TIn *)a.log_f + (size_t)bh * D;  // per channel (not kScalar)
  float4 *S = (float4 *)(a.state + (size_t)bh * D * D);

  // issue the state loads first: they are the whole cost of the step
  float4 st[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) st[p] = S[(size_t)(p * RG + rg) * CG + cg];

  for (int c = tid; c < D; c += Cfg::NT) {
    const float lbc = GM == kGate ? a.lb[(bh % a.H) * D + c] : 0.f;
    // the gate input of channel c (one per head with kScalar)
    const TIn x = GM == kScalar ? ((const TIn *)a.log_f)[bh] : gl[c];
    s_q[c] = to_f32(gq[c]);
    s_k[c] = k_of<GM>(reads_k(GM) ? gk[c] : x, x, lbc);
    s_f[c] = __expf(lf_of<GM>(to_f32(x), lbc));
  }
  const float v0 = to_f32(gv[4 * cg + 0]), v1 = to_f32(gv[4 * cg + 1]),
              v2 = to_f32(gv[4 * cg + 2]), v3 = to_f32(gv[4 * cg + 3]);
  __syncthreads();

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int c = p * RG + rg;
    const float f = s_f[c], kc = s_k[c], qc = s_q[c];
    float4 x = st[p];
    x.x = f * x.x + kc * v0;
    x.y = f * x.y + kc * v1;
    x.z = f * x.z + kc * v2;
    x.w = f * x.w + kc * v3;
    // non-temporal: the state is written once per step and not read back here
    __builtin_nontemporal_store(f32x4_t{x.x, x.y, x.z, x.w}, (f32x4_t *)&S[(size_t)c * CG + cg]);
    acc.x += qc * x.x;
    acc.y += qc * x.y;
    acc.z += qc * x.z;
    acc.w += qc * x.w;
  }
  s_part[rg][cg] = acc;
  __syncthreads();
  if (tid < CG) {
    float4 r = s_part[0][tid];
    for (int i = 1; i < RG; ++i) {
      const float4 u = s_part[i][tid];
      r.x += u.x;
      r.y += u.y;
      r.z += u.z;
      r.w += u.w;
    }
    TO *gy = (TO *)a.y + (size_t)bh * D + 4 * tid;
    gy[0] = from_f32<TO>(r.x);
    gy[1] = from_f32<TO>(r.y);
    gy[2] = from_f32<TO>(r.z);
    gy[3] = from_f32<TO>(r.w);
  }
}

template <typename TIn, int D, int GM, typename TO = TIn>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((hgrn2_decode_kernel<TIn, D, GM, TO>), dim3(a.B * a.H), dim3(DecodeCfg<D>::NT), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace hgrn2
