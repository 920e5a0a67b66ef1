// Chunk-boundary state scan of the HGRN2 recurrence (gfx950).
//
// HGRN2 summary (paperlayer.ai) §3.2: per head a d x d state whose rows (the
// d_k channels) are scaled by the forget gate and which receives an outer
// product write each step.  Over one chunk of C tokens with in-chunk
// inclusive prefix b_t of log f and total Gamma = b_C, the state advances as
//   S <- Diag(e^Gamma) S + sum_t Diag(e^{Gamma - b_t}) x_t^T z_t
// with (x, z) = (k, v).  Walked backwards with (x, z) = (q, dy) and weights
// e^{b_t}, the same pass carries the state adjoint Lambda (the gradient of the
// loss with respect to the state at a chunk end):
//   Lambda <- Diag(e^Gamma) Lambda + sum_t Diag(e^{b_t}) q_t^T dy_t.
// Every chunk's state is written out (forward: the state after n chunks, n =
// 0..N; backward: the adjoint at the end of chunk n, n = 0..N-1) so that the
// chunk kernels can run all chunks in parallel.
//
// One workgroup owns one (batch, head, DJ-wide slice of the d_v columns) and
// holds that slice of the state transposed, S^T[j][c], in float32 matrix-core
// accumulators.  Waves own the chunk's 16-token sub-blocks while they build
// the decayed x rows (lane = CPL channels, sixteen tokens in registers), and
// 16 x 16 tiles of S^T while they multiply.
#pragma once

#include "tile.h"

namespace hgrn2 {

struct ScanArgs {
  int B, T, H, N;
  const void *x, *z, *log_f;  // [B,T,H,D]
  const float *s_in;          // initial state (h0 or dht), [B,H,D,D] float32, or null
  void *states;               // forward: [B,H,N+1,D,D]; backward: [B,H,N,D,D]; input dtype
  float *s_out;               // final state (ht or dh0), or null
};

template <typename T, int D, int C, bool REV> struct ScanCfg {
  static constexpr int NW = C / 16, NT = 64 * NW;
  static constexpr int DJ = D < 32 ? D : 32;            // state columns per workgroup
  static constexpr int NJ = D / DJ;
  static constexpr int CPL = D > 64 ? D / 64 : 1;       // channels per lane in the prep layout
  static constexpr int LANES = D / CPL;                 // prep lanes with channels
  static constexpr int JB = DJ / 16, CB = D / 16;
  static constexpr int NTILE = JB * CB;
  static constexpr int TPW = (NTILE + NW - 1) / NW;     // state tiles per wave
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int VZ = C * DJ / EPV;               // 16-byte vectors of one z slice
  static constexpr int NVZ = (VZ + NT - 1) / NT;
  struct Smem {
    T x[C * RowTile<T, D>::LD];      // decayed x, RowTile<T, D>
    T z[2][C * RowTile<T, DJ>::LD];  // z slice, RowTile<T, DJ>, double-buffered
    float Lb[NW][D]; // sub-block totals of log f
    float eG[D];     // e^Gamma
  };
};

template <typename T, int D, int C, bool REV>
__global__ __launch_bounds__(4 * C) void hgrn2_scan_kernel(ScanArgs a) {
  using Cfg = ScanCfg<T, D, C, REV>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, DJ = Cfg::DJ, NJ = Cfg::NJ, CPL = Cfg::CPL, JB = Cfg::JB,
                EPV = Cfg::EPV;
  using XT = RowTile<T, D>;
  using ZT = RowTile<T, DJ>;
  __shared__ typename Cfg::Smem sm;

  // slices of one (b, h) get ids equal mod 8: they run on one XCD and share its L2
  const int bid = blockIdx.x;
  const int grp = bid / (8 * NJ), rem = bid % (8 * NJ);
  const int slice = rem / 8;
  const int bh = grp * 8 + (rem % 8);
  if (bh >= a.B * a.H) return;
  const int b = bh / a.H, h = bh % a.H;
  const int j0 = slice * DJ;
  const int T_ = a.T, H = a.H, N = a.N;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
  const bool has_ch = lane < Cfg::LANES;
  const int c0 = (has_ch ? lane : 0) * CPL;

  const T *gx = (const T *)a.x;
  const T *gz = (const T *)a.z;
  const T *gl = (const T *)a.log_f;
  T *gst = (T *)a.states;
  const size_t SS = (size_t)D * D;
  auto tok = [&](int t) { return (((size_t)b * T_ + t) * H + h) * D; };

  // ---- state tiles: tile q = w + NW * i (q < NTILE) covers S^T rows (j) 16 jb.. and columns (c) 16 cb..
  f32x4_t S[Cfg::TPW];
#pragma unroll
  for (int i = 0; i < Cfg::TPW; ++i) {
    const int q = w + NW * i;
    const int jb = q % JB, cb = q / JB;
    const int c = cb * 16 + n16, j = j0 + jb * 16 + 4 * g;
    if (q < Cfg::NTILE && a.s_in) {
      const float4 v = *(const float4 *)(a.s_in + (size_t)bh * SS + (size_t)c * D + j);
      S[i] = f32x4_t{v.x, v.y, v.z, v.w};
    } else {
      acc_zero(S[i]);
    }
  }
  auto store_tiles = [&](int slot) {
    const int nst = REV ? N : N + 1;
    T *st = gst + ((size_t)bh * nst + slot) * SS;
#pragma unroll
    for (int i = 0; i < Cfg::TPW; ++i) {
      const int q = w + NW * i;
      if (q < Cfg::NTILE) {
        const int jb = q % JB, cb = q / JB;
        const int c = cb * 16 + n16, j = j0 + jb * 16 + 4 * g;
        Pack<T, 4> p;
#pragma unroll
        for (int r = 0; r < 4; ++r) p.v[r] = from_f32<T>(S[i][r]);
        stpack<T, 4>(st + (size_t)c * D + j, p);
      }
    }
  };
  if (!REV) store_tiles(0);

  // ---- register prefetch, two chunks ahead in two register sets: x, log f
  // in the prep layout; the z slice
  using XP = Pack<T, CPL>[16];
  using ZP = uint4[Cfg::NVZ];
  auto prefetch = [&](XP &px, XP &pl, ZP &pz, int n) {
    const int t0 = n * C, len = min(C, T_ - t0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int tt = 16 * w + t;
      Pack<T, CPL> zx, zl;
#pragma unroll
      for (int e = 0; e < CPL; ++e) zx.v[e] = zl.v[e] = from_f32<T>(0.f);
      if (tt < len && has_ch) {
        zx = ldpack<T, CPL>(gx + tok(t0 + tt) + c0);
        zl = ldpack<T, CPL>(gl + tok(t0 + tt) + c0);
      }
      px[t] = zx;
      pl[t] = zl;
    }
#pragma unroll
    for (int i = 0; i < Cfg::NVZ; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / (DJ / EPV), col = (idx % (DJ / EPV)) * EPV;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (idx < Cfg::VZ && row < len) v = *(const uint4 *)(gz + tok(t0 + row) + j0 + col);
      pz[i] = v;
    }
  };

  // one chunk: consumes (px, pl, pz), then refills them with the chunk two steps on
  auto step = [&](XP &px, XP &pl, ZP &pz, int it) {
    const int n = REV ? N - 1 - it : it;
    T *zs = sm.z[it & 1];
    // ---- block-local prefix of the floored log f (registers), sub-block totals
    float l[16][CPL];
    {
      float acc[CPL];
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          acc[e] += floor_logf(to_f32(pl[t].v[e]));
          l[t][e] = acc[e];
        }
      if (has_ch)
#pragma unroll
        for (int e = 0; e < CPL; ++e) sm.Lb[w][c0 + e] = acc[e];
    }
#pragma unroll
    for (int i = 0; i < Cfg::NVZ; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / (DJ / EPV), col = (idx % (DJ / EPV)) * EPV;
      if (idx < Cfg::VZ) *(uint4 *)&zs[ZT::at(row, col)] = pz[i];
    }
    __syncthreads();
    // ---- decayed x rows: forward x e^{Gamma - b_t}, backward x e^{b_t}
    if (has_ch) {
      float P[CPL], G[CPL];
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        float p = 0.f, s = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          const float L = sm.Lb[i][c0 + e];
          p += (i < w) ? L : 0.f;
          s += L;
        }
        P[e] = p;
        G[e] = s;
        if (w == 0) sm.eG[c0 + e] = __expf(s);
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        Pack<T, CPL> o;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const float ex = REV ? (P[e] + l[t][e]) : fminf(G[e] - P[e] - l[t][e], 0.f);
          o.v[e] = from_f32<T>(to_f32(px[t].v[e]) * __expf(ex));
        }
        stpack<T, CPL>(&sm.x[XT::at(16 * w + t, c0)], o);
      }
    }
    // this register set is consumed: fetch the chunk two steps on into it
    if (it + 2 < N) prefetch(px, pl, pz, REV ? n - 2 : n + 2);
    __syncthreads();
    // ---- the adjoint at the end of chunk n is the value before its update
    if (REV) store_tiles(n);
    // ---- S^T <- S^T Diag(e^Gamma) + z^T xd
#pragma unroll
    for (int i = 0; i < Cfg::TPW; ++i) {
      const int q = w + NW * i;
      if (q < Cfg::NTILE) {
        const int jb = q % JB, cb = q / JB;
        const float eg = sm.eG[cb * 16 + n16];
#pragma unroll
        for (int r = 0; r < 4; ++r) S[i][r] *= eg;
        if constexpr (C % 32 == 0) {
#pragma unroll
          for (int ks = 0; ks < C / 32; ++ks)
            mma(S[i], tr8<DJ>(zs, 32 * ks, 16 * jb), tr8<D>(sm.x, 32 * ks, 16 * cb));
        } else {
          mma16(S[i], tr4<DJ>(zs, 0, 16 * jb), tr4<D>(sm.x, 0, 16 * cb));
        }
      }
    }
    if (!REV) store_tiles(n + 1);
  };

  Pack<T, CPL> px0[16], pl0[16], px1[16], pl1[16];
  uint4 pz0[Cfg::NVZ], pz1[Cfg::NVZ];
  prefetch(px0, pl0, pz0, REV ? N - 1 : 0);
  if (N > 1) prefetch(px1, pl1, pz1, REV ? N - 2 : 1);
  for (int it = 0; it < N; it += 2) {
    step(px0, pl0, pz0, it);
    if (it + 1 < N) step(px1, pl1, pz1, it + 1);
  }
  if (a.s_out) {
#pragma unroll
    for (int i = 0; i < Cfg::TPW; ++i) {
      const int q = w + NW * i;
      if (q < Cfg::NTILE) {
        const int jb = q % JB, cb = q / JB;
        const int c = cb * 16 + n16, j = j0 + jb * 16 + 4 * g;
        *(float4 *)(a.s_out + (size_t)bh * SS + (size_t)c * D + j) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
      }
    }
  }
}

template <typename T, int D, int C, bool REV>
hipError_t launch_scan(const ScanArgs &a, hipStream_t stream) {
  using Cfg = ScanCfg<T, D, C, REV>;
  const int groups = (a.B * a.H + 7) / 8;
  hipLaunchKernelGGL((hgrn2_scan_kernel<T, D, C, REV>), dim3(groups * 8 * Cfg::NJ), dim3(Cfg::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hgrn2
