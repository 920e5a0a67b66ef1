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
//
// A preparation pass evaluates each decayed operand once per chunk, with
// exponents anchored inside the span they cover so that they are <= 0:
// 16-token sub-blocks carry block-local prefixes ell (totals L_j, starts P_j),
//   qo = q e^{ell}, ko = k e^{L_j - ell}, kh = ko e^{Gamma - P_{j+1}} = k e^{Gamma - b}.
// Block (t in i, s in j) of A is qo_t . (ko_s * gap_ij) with
// gap_ij = e^{P_i - P_{j+1}} (<= 1) off the diagonal and e^{-L_i} on it; a
// diagonal block whose in-block decay exceeds kDiagLimit nats is evaluated
// directly.  The inter-chunk readout uses qo against S scaled by e^{P_i}.
#pragma once

#include "common.h"

namespace hgrn2 {

struct FwdArgs {
  int B, T, H;
  const void *q, *k, *v, *log_f;
  const float *h0;
  void *y;
  float *ht;
  void *states;  // [B,H,N+1,D,D] in the input dtype, or null
  int N;         // number of chunks
};

template <typename TIn, int D, int C, int DVT>
struct FwdCfg {
  static constexpr int NW = DVT / 16;             // waves; wave w owns state columns [16w, 16w+16)
  static constexpr int NT = NW * 64;
  static constexpr int NB = C / 16;               // 16-token sub-blocks per chunk
  static constexpr int NPAIR = NB * (NB + 1) / 2;
  static constexpr int CB = D / 16;               // 16-channel blocks of d_k
  static constexpr int KSD = (D + 31) / 32;       // 32-wide k steps over channels
  static constexpr int KSC = (C + 31) / 32;       // 32-wide k steps over tokens
  static constexpr int EPV = 16 / (int)sizeof(TIn);
  static constexpr int LDN = D + EPV;             // natural [token][channel] rows (16-byte pad)
  static constexpr int LDL = D + 4;
  static constexpr int LDV = DVT + EPV;
  static constexpr int LDKT = C + EPV;
  static constexpr int LDA = C + EPV;
  static constexpr int VQ = C * D / EPV;          // 16-byte vectors per [C x D] tile
  static constexpr int VV = C * DVT / EPV;        // ... per [C x DVT] tile
  static constexpr int NVQ = (VQ + NT - 1) / NT;
  static constexpr int NVV = (VV + NT - 1) / NT;
  struct Smem {
    union {
      float l[C][LDL];        // block-local inclusive prefix of floored log f
      struct {                // after the score tiles: output staging
        TIn ys[C][LDV];       // y slice
        TIn ss[D][LDV];       // chunk-boundary state slice
      };
    };
    TIn qo[C][LDN];           // q e^{ell}
    TIn ko[C][LDN];           // k e^{L_j - ell}
    TIn khT[D * TTile<TIn, C>::LD];  // (k e^{Gamma - b})^T (TTile layout)
    TIn v[C][LDV];
    TIn a[C][LDA];            // causal scores A[t][s]
    float Lb[NB][D];          // sub-block totals L_j
    float Pb[NB + 1][D];      // sub-block starts P_j; Pb[NB] = Gamma
    float ePb[NB][D];         // e^{P_i}
    float eG[D];              // e^{Gamma}
    float gp[NPAIR][D];       // gap factors of the score blocks
    int flags;                // bit i: diagonal block i evaluated directly
  };
  static constexpr bool fits = sizeof(Smem) <= 160 * 1024;  // LDS per workgroup on gfx950
  static_assert(D % DVT == 0 && DVT % 16 == 0 && C % 16 == 0, "tile shape");
};

// pair index of score block (i, j), j <= i
__host__ __device__ constexpr int pair_index(int i, int j) { return i * (i + 1) / 2 + j; }

template <typename TIn, int D, int C, int DVT>
__global__ __launch_bounds__(4 * DVT) void hgrn2_fwd_kernel(FwdArgs args) {
  using Cfg = FwdCfg<TIn, D, C, DVT>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, NB = Cfg::NB, CB = Cfg::CB, KSD = Cfg::KSD,
                KSC = Cfg::KSC, EPV = Cfg::EPV, NPAIR = Cfg::NPAIR;
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
  TIn *gst = (TIn *)args.states;
  const size_t SS = (size_t)D * D;
  const size_t state_base = (size_t)bh * SS;
  auto tok = [&](int t) { return (((size_t)b * T + t) * H + h) * D; };

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
  auto store_state = [&](int n) {
    TIn *st = gst + ((size_t)bh * (N + 1) + n) * SS;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[(size_t)(cb * 16 + 4 * g + r) * D + jcol] = from_f32<TIn>(S[cb][r]);
  };
  if (gst) store_state(0);

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
        const size_t off = tok(t0 + row) + col;
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
      if (idx < Cfg::VV && row < len) zv = *(const uint4 *)(gv + tok(t0 + row) + j0 + col);
      pv[it] = zv;
    }
  };
  prefetch(0);

  for (int n = 0; n < N; ++n) {
    const int t0 = n * C;
    const int len = min(C, T - t0);
    // ================= preparation =================
    __syncthreads();  // previous chunk's readers of LDS are done
    {
    const int tid = opaque(threadIdx.x);
#pragma unroll
    for (int it = 0; it < Cfg::NVQ; ++it) {
      const int idx = tid + it * NT;
      if (idx < Cfg::VQ) {
        const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
        float f[EPV];
        Vec<TIn>::unpack(pl[it], f);
#pragma unroll
        for (int e = 0; e < EPV; e += 4)
          *(float4 *)&sm.l[row][col + e] =
              make_float4(floor_logf(f[e]), floor_logf(f[e + 1]), floor_logf(f[e + 2]), floor_logf(f[e + 3]));
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
    {  // block-local prefixes of log f, block totals, diagonal-range flags
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
        sm.ePb[i][c] = __expf(s);
        s += sm.Lb[i][c];
      }
      sm.Pb[NB][c] = s;
      sm.eG[c] = __expf(s);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j)
          sm.gp[pair_index(i, j)][c] = (j < i) ? __expf(sm.Pb[i][c] - sm.Pb[j + 1][c]) : __expf(-sm.Lb[i][c]);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < Cfg::NVQ; ++it) {
      const int idx = tid + it * NT;
      if (idx < Cfg::VQ) {
        const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
        const int jb = row >> 4;
        float fq[EPV], fk[EPV];
        Vec<TIn>::unpack(pq[it], fq);
        Vec<TIn>::unpack(pk[it], fk);
        TIn oq[EPV], ok[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int c = col + e;
          const float l = sm.l[row][c];
          const float kown = fk[e] * __expf(sm.Lb[jb][c] - l);
          oq[e] = from_f32<TIn>(fq[e] * __expf(l));
          ok[e] = from_f32<TIn>(kown);
          sm.khT[TTile<TIn, C>::at(c, row)] = from_f32<TIn>(kown * __expf(sm.Pb[NB][c] - sm.Pb[jb + 1][c]));
        }
        *(uint4 *)&sm.qo[row][col] = *(const uint4 *)oq;
        *(uint4 *)&sm.ko[row][col] = *(const uint4 *)ok;
      }
    }
    }
    const int flags = sm.flags;  // final since the barrier after the prefix pass
    __syncthreads();
    if (n + 1 < N) prefetch(n + 1);  // in flight while this chunk computes

    // ================= causal scores, as transposed tiles =================
    for (int pi = w; pi < NPAIR; pi += NW) {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4;
      int ib = 0, jb = pi;  // rows s in block jb, columns t in block ib, jb <= ib
      while (jb > ib) {
        jb -= ib + 1;
        ++ib;
      }
      const int s_row = jb * 16 + n16;
      const int t_col = ib * 16 + n16;
      f32x4_t acc;
      acc_zero(acc);
      const bool direct = (jb == ib) && ((flags >> ib) & 1);
      if (!direct) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int c0 = ks * 32 + 8 * g;
          const bool ok = c0 < D;  // D = 16: lanes past the channels feed zeros
          const int cc = ok ? c0 : 0;
          float kv[8];
          Vec<TIn>::unpack(*(const uint4 *)&sm.ko[s_row][cc], kv);
          if constexpr (EPV == 4) Vec<TIn>::unpack(*(const uint4 *)&sm.ko[s_row][cc + 4], kv + 4);
          const float4 g0 = ldf4(&sm.gp[pi][cc]);
          const float4 g1 = ldf4(&sm.gp[pi][cc + 4]);
          Frag fa;
          fa.v[0] = kv[0] * g0.x; fa.v[1] = kv[1] * g0.y; fa.v[2] = kv[2] * g0.z; fa.v[3] = kv[3] * g0.w;
          fa.v[4] = kv[4] * g1.x; fa.v[5] = kv[5] * g1.y; fa.v[6] = kv[6] * g1.z; fa.v[7] = kv[7] * g1.w;
          mma(acc, to_pfrag<TIn>(fa), masked(ld8(&sm.qo[t_col][cc]), ok));
        }
      } else {
        // wide in-block decay: A[t][s] = sum_c q_t k_s e^{ell_t - ell_s}, every exponent <= 0
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = jb * 16 + 4 * g + r;
          float a = 0.f;
          if (s <= t_col && t_col < len)
            for (int c = 0; c < D; ++c)
              a += to_f32(gq[tok(t0 + t_col) + c]) * to_f32(gk[tok(t0 + s) + c]) *
                   __expf(sm.l[t_col][c] - sm.l[s][c]);
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

    {
    const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4;
    // ---- V fragments (k = token), reused by the intra product and the state update
    PFrag<TIn> fv[KSC];
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      const int s0 = ks * 32 + 8 * g;
      fv[ks] = ldcol8(&sm.v[s0 < C ? s0 : 0][w * 16 + n16], Cfg::LDV, s0 < C);
    }

    // ---- Y = A V + qo (e^{P_i} S_prev)  for this wave's 16 columns
    f32x4_t Y[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      acc_zero(Y[tb]);
      const int t = tb * 16 + n16;
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        if (ks * 32 < 16 * (tb + 1)) {
          const int s0 = ks * 32 + 8 * g;
          const bool ok = s0 < 16 * (tb + 1) && s0 < C;
          mma(Y[tb], masked(ld8(&sm.a[t][ok ? s0 : 0]), ok), fv[ks]);
        }
      }
      // channels in the accumulator order of S (slots 0-3: block 2ks, 4-7: block 2ks+1)
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        Frag fb;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int cb = 2 * ks + hf;
          if (cb < CB) {
            const float4 e4 = ldf4(&sm.ePb[tb][cb * 16 + 4 * g]);
            fb.v[4 * hf + 0] = S[cb][0] * e4.x;
            fb.v[4 * hf + 1] = S[cb][1] * e4.y;
            fb.v[4 * hf + 2] = S[cb][2] * e4.z;
            fb.v[4 * hf + 3] = S[cb][3] * e4.w;
          } else {
#pragma unroll
            for (int x = 0; x < 4; ++x) fb.v[4 * hf + x] = 0.f;
          }
        }
        const int c0 = 2 * ks * 16 + 4 * g;
        const int c1 = (2 * ks + 1 < CB) ? c0 + 16 : c0;  // D = 16: slots 4-7 meet zeros
        mma(Y[tb], ld4x2(&sm.qo[t][c0], &sm.qo[t][c1]), to_pfrag<TIn>(fb));
      }
    }

    // ---- S <- e^Gamma S + (k e^{Gamma-b})^T V
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float4 e4 = ldf4(&sm.eG[cb * 16 + 4 * g]);
      S[cb][0] *= e4.x;
      S[cb][1] *= e4.y;
      S[cb][2] *= e4.z;
      S[cb][3] *= e4.w;
      const int c = cb * 16 + n16;
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        const int s0 = ks * 32 + 8 * g;
        const bool ok = s0 < C;
        mma(S[cb], masked(ldT8<C>(sm.khT, c, ok ? s0 : 0), ok), fv[ks]);
      }
    }

    // ---- outputs, staged in the dead prefix tile and stored as whole rows
    // (the accumulators hold one column per lane, so direct stores would be
    // scattered 2-byte writes)
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.ys[tb * 16 + 4 * g + r][w * 16 + n16] = from_f32<TIn>(Y[tb][r]);
    if (gst) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.ss[cb * 16 + 4 * g + r][w * 16 + n16] = from_f32<TIn>(S[cb][r]);
    }
    }
    __syncthreads();
    {
      const int tid = opaque(threadIdx.x);
      if (gy) {
#pragma unroll
        for (int it = 0; it < Cfg::NVV; ++it) {
          const int idx = tid + it * NT;
          const int row = idx / (DVT / EPV), col = (idx % (DVT / EPV)) * EPV;
          if (idx < Cfg::VV && row < len) *(uint4 *)(gy + tok(t0 + row) + j0 + col) = *(const uint4 *)&sm.ys[row][col];
        }
      }
      if (gst) {
        TIn *st = gst + ((size_t)bh * (N + 1) + n + 1) * SS;
        constexpr int VS = D * DVT / EPV;
#pragma unroll
        for (int it = 0; it < (VS + NT - 1) / NT; ++it) {
          const int idx = tid + it * NT;
          const int row = idx / (DVT / EPV), col = (idx % (DVT / EPV)) * EPV;
          if (idx < VS) *(uint4 *)(st + (size_t)row * D + j0 + col) = *(const uint4 *)&sm.ss[row][col];
        }
      }
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
