// Chunked forward of the HGRN2 recurrence on CDNA4 matrix cores.
//
// HGRN2 summary (paperlayer.ai) §3.2: per head a d x d state, rows scaled by
// the forget gate, outer-product write, matrix-vector readout; §3.2 p.5: the
// recurrence is GLA's, so it is evaluated chunk by chunk in linear-attention
// form (q = output gate, k = input gate, v = input).
//
// One workgroup owns one (batch, head, 16*NW-wide slice of the d_v columns)
// and walks the chunks in order, holding its d_k x DVT slice of the state in
// float32 matrix-core accumulators.  Per chunk of C tokens (prefix b_t of
// log f from the chunk start, Gamma = b at the chunk end):
//   A     = tril( sum_c q_t k_s e^{b_t - b_s} )        (C x C, shared by all slices)
//   Y     = A V + (q e^b) S                           (intra + inter chunk)
//   S    <- e^Gamma S + (k e^{Gamma - b})^T V         (state passing, float32)
// Every exponent is a partial sum of log f anchored inside the span it
// covers, so it is <= 0: sub-blocks of 16 tokens carry block-local prefixes
// ell, the off-diagonal blocks of A use anchors at sub-block boundaries, and
// diagonal blocks whose in-block decay exceeds kDiagLimit nats are evaluated
// directly instead of through the factorised product.
#pragma once

#include "common.h"

namespace hgrn2 {

struct FwdArgs {
  int B, T, H;
  const void *q, *k, *v, *log_f;
  const float *h0;
  void *y;
  float *ht;
  float *states;  // [B,H,N+1,D,D] or null
  int N;          // number of chunks
};

template <typename TIn, int D, int C, int DVT>
struct FwdCfg {
  static constexpr int NW = DVT / 16;             // waves; wave w owns state columns [16w, 16w+16)
  static constexpr int NT = NW * 64;
  static constexpr int NB = C / 16;               // 16-token sub-blocks per chunk
  static constexpr int CB = D / 16;               // 16-channel blocks of d_k
  static constexpr int KSD = (D + 31) / 32;       // 32-wide k steps over channels
  static constexpr int KSC = (C + 31) / 32;       // 32-wide k steps over tokens
  static constexpr int EPV = 16 / (int)sizeof(TIn);
  static constexpr int LDQ = D + EPV;             // q, k rows (16-byte pad)
  static constexpr int LDL = D + 4;               // ell rows (float)
  static constexpr int LDV = DVT + EPV;
  static constexpr int LDKT = C + EPV;            // (k e^{Gamma-b})^T rows
  static constexpr int LDA = C + EPV;             // A rows
  static constexpr int VQ = C * D / EPV;          // 16-byte vectors per [C x D] tile
  static constexpr int VV = C * DVT / EPV;        // ... per [C x DVT] tile
  static constexpr int NVQ = (VQ + NT - 1) / NT;
  static constexpr int NVV = (VV + NT - 1) / NT;
  struct Smem {
    TIn q[C][LDQ];
    TIn k[C][LDQ];
    float l[C][LDL];          // block-local inclusive prefix of floored log f
    TIn v[C][LDV];
    TIn khT[D][LDKT];         // (k e^{Gamma - b})^T, operand of the state update
    TIn a[C][LDA];            // causal scores A[t][s]
    float Lb[NB][D];          // sub-block totals
    float Pb[NB + 1][D];      // chunk-relative sub-block starts; Pb[NB] = Gamma
    int flags;                // bit i: diagonal block i evaluated directly
  };
  static constexpr bool fits = sizeof(Smem) <= 160 * 1024;  // LDS per workgroup on gfx950
  static_assert(D % DVT == 0 && DVT % 16 == 0 && C % 16 == 0, "tile shape");
};

template <typename TIn, int D, int C, int DVT>
__global__ __launch_bounds__(4 * DVT) void hgrn2_fwd_kernel(FwdArgs args) {
  using Cfg = FwdCfg<TIn, D, C, DVT>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, NB = Cfg::NB, CB = Cfg::CB, KSD = Cfg::KSD,
                KSC = Cfg::KSC, EPV = Cfg::EPV;
  __shared__ typename Cfg::Smem sm;

  const int B = args.B, T = args.T, H = args.H;
  constexpr int ntile = D / DVT;
  // Work-group id -> (b, h, column slice).  Workgroups are dealt round-robin
  // to the 8 XCDs, so the slices of one (b, h) get ids that are equal mod 8
  // and therefore share one XCD's L2 for the q, k, log f tiles they all read.
  const int bid = blockIdx.x;
  const int grp = bid / (8 * ntile), rem = bid % (8 * ntile);
  const int tile = rem / 8;
  const int bh = grp * 8 + (rem % 8);
  if (bh >= B * H) return;
  const int b = bh / H, h = bh % H;
  const int j0 = tile * DVT;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
  const int N = args.N;

  const TIn *gq = (const TIn *)args.q;
  const TIn *gk = (const TIn *)args.k;
  const TIn *gv = (const TIn *)args.v;
  const TIn *gl = (const TIn *)args.log_f;
  TIn *gy = (TIn *)args.y;
  const size_t SS = (size_t)D * D;
  const size_t state_base = (size_t)bh * SS;

  // ---- state slice: S[cb] holds rows [16cb, 16cb+16) x columns j0 + 16w + [0,16)
  f32x4_t S[CB];
  const int jcol = j0 + w * 16 + n16;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = cb * 16 + 4 * g + r;
      S[cb][r] = args.h0 ? args.h0[state_base + (size_t)c * D + jcol] : 0.f;
    }
  }
  if (args.states) {
    float *st = args.states + (size_t)bh * (N + 1) * SS;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[(size_t)(cb * 16 + 4 * g + r) * D + jcol] = S[cb][r];
  }

  // ---- register prefetch of one chunk's tiles
  uint4 pq[Cfg::NVQ], pk[Cfg::NVQ], pl[Cfg::NVQ], pv[Cfg::NVV];
  auto prefetch = [&](int n) {
    const int t0 = n * C;
    const int len = min(C, T - t0);
#pragma unroll
    for (int it = 0; it < Cfg::NVQ; ++it) {
      const int idx = tid + it * NT;
      const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
      uint4 zq = make_uint4(0, 0, 0, 0), zk = zq, zl = zq;
      if (idx < Cfg::VQ && row < len) {
        const size_t off = (((size_t)b * T + t0 + row) * H + h) * D + col;
        zq = *(const uint4 *)(gq + off);
        zk = *(const uint4 *)(gk + off);
        zl = *(const uint4 *)(gl + off);
      }
      pq[it] = zq;
      pk[it] = zk;
      pl[it] = zl;
    }
#pragma unroll
    for (int it = 0; it < Cfg::NVV; ++it) {
      const int idx = tid + it * NT;
      const int row = idx / (DVT / EPV), col = (idx % (DVT / EPV)) * EPV;
      uint4 zv = make_uint4(0, 0, 0, 0);
      if (idx < Cfg::VV && row < len) {
        const size_t off = (((size_t)b * T + t0 + row) * H + h) * D + j0 + col;
        zv = *(const uint4 *)(gv + off);
      }
      pv[it] = zv;
    }
  };
  prefetch(0);

  for (int n = 0; n < N; ++n) {
    const int t0 = n * C;
    const int len = min(C, T - t0);
    __syncthreads();  // previous chunk's readers of LDS are done
    // ---- registers -> LDS
#pragma unroll
    for (int it = 0; it < Cfg::NVQ; ++it) {
      const int idx = tid + it * NT;
      if (idx < Cfg::VQ) {
        const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
        *(uint4 *)&sm.q[row][col] = pq[it];
        *(uint4 *)&sm.k[row][col] = pk[it];
        float f[EPV];
        Vec<TIn>::unpack(pl[it], f);
#pragma unroll
        for (int e = 0; e < EPV; ++e) sm.l[row][col + e] = floor_logf(f[e]);
      }
    }
#pragma unroll
    for (int it = 0; it < Cfg::NVV; ++it) {
      const int idx = tid + it * NT;
      if (idx < Cfg::VV) {
        const int row = idx / (DVT / EPV), col = (idx % (DVT / EPV)) * EPV;
        *(uint4 *)&sm.v[row][col] = pv[it];
      }
    }
    if (tid == 0) sm.flags = 0;
    __syncthreads();
    if (n + 1 < N) prefetch(n + 1);  // in flight while this chunk computes

    // ---- block-local prefixes of log f, block totals, diagonal-range flags
    {
      int fl = 0;
      for (int p = tid; p < NB * D; p += NT) {
        const int i = p / D, c = p % D;
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc += sm.l[i * 16 + r][c];
          sm.l[i * 16 + r][c] = acc;
        }
        sm.Lb[i][c] = acc;
        if (-acc > kDiagLimit) fl |= 1 << i;
      }
      if (fl) atomicOr(&sm.flags, fl);
    }
    __syncthreads();
    for (int c = tid; c < D; c += NT) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        sm.Pb[i][c] = s;
        s += sm.Lb[i][c];
      }
      sm.Pb[NB][c] = s;
    }
    __syncthreads();
    const int flags = sm.flags;

    // ---- (k e^{Gamma - b})^T: exponent (Gamma - P_{j+1}) + (L_j - ell_s) <= 0
    for (int e = tid; e < C * D; e += NT) {
      const int s = e % C, c = e / C, jb = s / 16;
      const float ex = (sm.Pb[NB][c] - sm.Pb[jb + 1][c]) + (sm.Lb[jb][c] - sm.l[s][c]);
      sm.khT[c][s] = from_f32<TIn>(to_f32(sm.k[s][c]) * __expf(ex));
    }

    // ---- causal scores, as transposed tiles (rows s in block jb, columns t in block ib)
    for (int pi = w; pi < NB * (NB + 1) / 2; pi += NW) {
      int ib = 0, jb = pi;
      while (jb > ib) {  // pair index -> (ib, jb), jb <= ib
        jb -= ib + 1;
        ++ib;
      }
      const int s_row = jb * 16 + n16;   // A-operand row (token s)
      const int t_col = ib * 16 + n16;   // B-operand column (token t)
      f32x4_t acc;
      acc_zero(acc);
      const bool direct = (jb == ib) && ((flags >> ib) & 1);
      if (!direct) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int c0 = ks * 32 + 8 * g;
          Frag fa, fb;
          if (c0 < D) {
#pragma unroll
            for (int x = 0; x < 8; ++x) {
              const int c = c0 + x;
              const float eK = (jb < ib) ? (sm.Lb[jb][c] - sm.l[s_row][c]) + (sm.Pb[ib][c] - sm.Pb[jb + 1][c])
                                         : -sm.l[s_row][c];
              fa.v[x] = to_f32(sm.k[s_row][c]) * __expf(eK);
              fb.v[x] = to_f32(sm.q[t_col][c]) * __expf(sm.l[t_col][c]);
            }
          } else {
            frag_zero(fa);
            frag_zero(fb);
          }
          Mma<TIn>::run(acc, fa, fb);
        }
      } else {
        // wide in-block decay: A[t][s] = sum_c q_t k_s e^{ell_t - ell_s}, every exponent <= 0
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = jb * 16 + 4 * g + r;
          float a = 0.f;
          if (s <= t_col)
            for (int c = 0; c < D; ++c)
              a += to_f32(sm.q[t_col][c]) * to_f32(sm.k[s][c]) * __expf(sm.l[t_col][c] - sm.l[s][c]);
          acc[r] = a;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = jb * 16 + 4 * g + r;
        sm.a[t_col][s] = from_f32<TIn>((jb < ib || s <= t_col) ? acc[r] : 0.f);
      }
    }
    __syncthreads();

    // ---- V fragments (k = token), reused by the intra product and the state update
    Frag fv[KSC];
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int s = ks * 32 + 8 * g + x;
        fv[ks].v[x] = (s < C) ? to_f32(sm.v[s][w * 16 + n16]) : 0.f;
      }
    }

    // ---- Y = A V + (q e^b) S_prev  for this wave's 16 columns
    f32x4_t Y[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      acc_zero(Y[tb]);
      const int t = tb * 16 + n16;
      // intra: s < 16 (tb + 1)
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        if (ks * 32 < 16 * (tb + 1)) {
          Frag fa;
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int s = ks * 32 + 8 * g + x;
            fa.v[x] = (s < 16 * (tb + 1) && s < C) ? to_f32(sm.a[t][s]) : 0.f;
          }
          Mma<TIn>::run(Y[tb], fa, fv[ks]);
        }
      }
      // inter: channels in the accumulator order of S (slots 0-3: block 2ks, 4-7: block 2ks+1)
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        Frag fa, fb;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int cb = 2 * ks + (x >> 2);
          const int c = cb * 16 + 4 * g + (x & 3);
          if (cb < CB) {
            fa.v[x] = to_f32(sm.q[t][c]) * __expf(sm.Pb[tb][c] + sm.l[t][c]);
            fb.v[x] = S[cb][x & 3];
          } else {
            fa.v[x] = 0.f;
            fb.v[x] = 0.f;
          }
        }
        Mma<TIn>::run(Y[tb], fa, fb);
      }
    }

    // ---- S <- e^Gamma S + (k e^{Gamma-b})^T V
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[cb][r] *= __expf(sm.Pb[NB][cb * 16 + 4 * g + r]);
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        Frag fa;
        const int c = cb * 16 + n16;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int s = ks * 32 + 8 * g + x;
          fa.v[x] = (s < C) ? to_f32(sm.khT[c][s]) : 0.f;
        }
        Mma<TIn>::run(S[cb], fa, fv[ks]);
      }
    }

    // ---- outputs
    if (gy) {
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tb * 16 + 4 * g + r;
          if (t < len) gy[(((size_t)b * T + t0 + t) * H + h) * D + jcol] = from_f32<TIn>(Y[tb][r]);
        }
    }
    if (args.states) {
      float *st = args.states + ((size_t)bh * (N + 1) + n + 1) * SS;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[(size_t)(cb * 16 + 4 * g + r) * D + jcol] = S[cb][r];
    }
  }
  if (args.ht) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        args.ht[state_base + (size_t)(cb * 16 + 4 * g + r) * D + jcol] = S[cb][r];
  }
}

template <typename TIn, int D, int C, int DVT>
hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
  using Cfg = FwdCfg<TIn, D, C, DVT>;
  const int ntile = D / DVT;
  const int groups = (a.B * a.H + 7) / 8;
  dim3 grid(groups * 8 * ntile), block(Cfg::NT);
  hipLaunchKernelGGL((hgrn2_fwd_kernel<TIn, D, C, DVT>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace hgrn2
