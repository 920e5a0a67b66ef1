// Per-chunk outputs of the HGRN2 forward (gfx950), all chunks in parallel.
//
// HGRN2 summary (paperlayer.ai) §3.2: y_t = q_t S_t with S_t the gated
// outer-product state; §3.2 p.5: evaluated chunk by chunk in the linear-
// attention form (q = output gate, k = input gate, v = input).  Given the
// state S at the start of chunk n (written by the state scan), the chunk's
// outputs are
//   y_t = sum_{s <= t} (sum_c q_t[c] k_s[c] e^{b_t[c] - b_s[c]}) v_s + (q_t e^{b_t}) S
// with b the in-chunk inclusive prefix of log f.
//
// One workgroup per (batch, head, chunk); wave w owns the chunk's 16-token
// sub-block w.  Exponents are anchored inside the span they cover so that
// they are <= 0: with block-local prefixes ell (totals L_j, starts P_j)
//   qo = q e^{ell},  ko = k e^{L_j - ell},
// score block (t in i, s in j) = qo_t . (ko_s * gap_ij) where gap_ij =
// e^{P_i - P_{j+1}} off the diagonal and e^{-L_i} on it.  A diagonal block
// whose decay exceeds kDiagLimit nats is summed directly instead.  The inter-
// chunk term uses (qo e^{P_i}) against S.
#pragma once

#include "tile.h"

namespace hgrn2 {

struct ChunkFwdArgs {
  int B, T, H, N;
  const void *q, *k, *v, *log_f;  // [B,T,H,D]; log_f holds the gate pre-activation in gate mode
  const float *lb;                // gate mode: lower bound of f, [H,D]
  const void *states;             // [B,H,N+1,D,D] input dtype; entry n = state before chunk n
  void *y;                        // [B,T,H,D], the input dtype or (out_f32) float32
  int out_f32 = 0;                // bfloat16 inputs: write y as float32
};

template <typename T, int D, int C> struct CfwdCfg {
  static constexpr int NW = C / 16, NT = 64 * NW, NB = NW;
  static constexpr int CPL = D > 64 ? D / 64 : 1;
  static constexpr int LANES = D / CPL;
  static constexpr int CB = D / 16;
  static constexpr int KSD = (D + 31) / 32;  // 32-deep steps over channels
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int NPAIR = NB * (NB + 1) / 2;
  static constexpr int VV = C * D / EPV, NVV = (VV + NT - 1) / NT;
  static constexpr int VS = D * D / EPV, NVS = (VS + NT - 1) / NT;
  static constexpr int LD = RowTile<T, D>::LD;
  struct KV {
    T ko[C * LD];
    T v[C * LD];
  };
  struct Smem {
    T qo[C * LD];  // RowTile<T, D>; later the y staging of each wave's rows
    union {
      KV kv;        // scores and the intra-chunk product
      T S[D * LD];  // then the chunk's initial state
    } u;
    float Lb[NB][D];
    float gp[NPAIR][D];
    float eP[NB][D];
  };
};

__host__ __device__ constexpr int pair_ij(int i, int j) { return i * (i + 1) / 2 + j; }

// Sixteen tokens of one lane's CPL channels: the block-local inclusive prefix
// of the floored log f, in registers.  Tokens from `nvalid` on lie past the
// end of the sequence (they matter only in gate mode, where log f is formed).
// kk receives k of every token (loaded, or formed with log f).
template <int GM, typename T, int CPL>
__device__ __forceinline__ void block_prefix(const Pack<T, CPL> *pk, const Pack<T, CPL> *pl, float (*l)[CPL],
                                             float *L, float (*kk)[CPL], const float *lb, int nvalid) {
#pragma unroll
  for (int e = 0; e < CPL; ++e) L[e] = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      float lf;
      lf_k<GM>(pk[t].v[e], lfe<GM>(pl[t], e), lb[e], t < nvalid, lf, kk[t][e]);
      L[e] += lf;
      l[t][e] = L[e];
    }
}

// TO: the element type of y (T, or float32 for bfloat16 inputs)
template <typename T, int D, int C, int GM, typename TO = T>
__global__ __launch_bounds__(4 * C) void hgrn2_chunk_fwd_kernel(ChunkFwdArgs a) {
  using Cfg = CfwdCfg<T, D, C>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, NB = Cfg::NB, CPL = Cfg::CPL, CB = Cfg::CB, KSD = Cfg::KSD,
                EPV = Cfg::EPV;
  using XT = RowTile<T, D>;
  __shared__ typename Cfg::Smem sm;

  const int N = a.N, T_ = a.T, H = a.H;
  const int bh = blockIdx.x / N, n = blockIdx.x % N;
  if (bh >= a.B * H) return;
  const int b = bh / H, h = bh % H;
  const int t0 = n * C, len = min(C, T_ - t0);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
  const bool has_ch = lane < Cfg::LANES;
  const int c0 = (has_ch ? lane : 0) * CPL;
  float lbv[CPL];  // gate mode: lower bounds of this lane's channels
#pragma unroll
  for (int e = 0; e < CPL; ++e) lbv[e] = GM == kGate ? a.lb[h * D + c0 + e] : 0.f;

  const T *gq = (const T *)a.q;
  const T *gk = (const T *)a.k;
  const T *gv = (const T *)a.v;
  const T *gl = (const T *)a.log_f;
  // one decay per head (kScalar): log a [B,T,H] of this chunk, token stride H
  const T *gls = (const T *)a.log_f + (((size_t)b * T_ + t0) * H + h);
  const T *gs = (const T *)a.states + ((size_t)bh * (N + 1) + n) * D * D;
  T *gy = (T *)a.y;
  // chunk-uniform base pointers; per-lane 32-bit element offsets within the chunk
  const size_t cbase = (((size_t)b * T_ + t0) * H + h) * D;
  const uint32_t HD = (uint32_t)H * D;
  gq += cbase;
  gk += cbase;
  gv += cbase;
  gl += cbase;
  gy += cbase;
  auto tok = [&](int t) { return (uint32_t)t * HD; };  // token t of the chunk
  // kScalar: lane j holds log a of this wave's token 16 w + (j & 15) (0 past the end)
  T las = from_f32<T>(0.f);
  if constexpr (GM == kScalar) {
    const int tj = 16 * w + (lane & 15);
    if (tj < len) las = gls[(size_t)tj * H];
  }
  // this lane's CPL log decays of token tt (kScalar: the head's value, element 0,
  // read through lfe; tt is a token of this wave, the same on every lane)
  auto ldlf = [&](int tt) {
    if constexpr (GM == kScalar) {
      Pack<T, CPL> p;
      p.v[0] = readlane(las, tt - 16 * w);
      return p;
    } else {
      return ldpack<T, CPL>(gl + (tok(tt) + c0));
    }
  };

  // ---- loads: v, then this wave's q, k, log f, all issued before any is
  // used (the v tile goes to LDS after them); the state tile, used last, once
  // the prefix is done.  v rows past the end of the sequence read as zero.
  const GBuf bvw((const char *)gv, (uint32_t)len * HD * sizeof(T));
  uint4 pvv[Cfg::NVV];
#pragma unroll
  for (int i = 0; i < Cfg::NVV; ++i) {
    const int idx = tid + i * NT;
    const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
    pvv[i] = idx < Cfg::VV ? bvw.ld16((tok(row) + col) * (uint32_t)sizeof(T)) : make_uint4(0, 0, 0, 0);
  }
  float l[16][CPL], L[CPL];
  bool wide = false;
  {
    Pack<T, CPL> pq[16], pk[16], pl[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int tt = 16 * w + t;
#pragma unroll
      for (int e = 0; e < CPL; ++e) pq[t].v[e] = pk[t].v[e] = pl[t].v[e] = from_f32<T>(0.f);
      if (tt < len && has_ch) {
        pq[t] = ldpack<T, CPL>(gq + (tok(tt) + c0));
        if constexpr (reads_k(GM)) pk[t] = ldpack<T, CPL>(gk + (tok(tt) + c0));
        if constexpr (GM != kScalar) pl[t] = ldlf(tt);
      }
    }
    if constexpr (GM == kScalar) {
      // the broadcasts wait for the one log a load: only after every load is issued
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (16 * w + t < len && has_ch) pl[t] = ldlf(16 * w + t);
    }
#pragma unroll
    for (int i = 0; i < Cfg::NVV; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
      if (idx < Cfg::VV) *(uint4 *)&sm.u.kv.v[XT::at(row, col)] = pvv[i];
    }
    float kk[16][CPL];
    block_prefix<GM, T, CPL>(pk, pl, l, L, kk, lbv, len - 16 * w);
    if (has_ch) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        Pack<T, CPL> oq, ok;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          oq.v[e] = from_f32<T>(to_f32(pq[t].v[e]) * __expf(l[t][e]));
          ok.v[e] = from_f32<T>(kk[t][e] * __expf(L[e] - l[t][e]));
        }
        stpack<T, CPL>(&sm.qo[XT::at(16 * w + t, c0)], oq);
        stpack<T, CPL>(&sm.u.kv.ko[XT::at(16 * w + t, c0)], ok);
      }
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        sm.Lb[w][c0 + e] = L[e];
        wide |= -L[e] > kDiagLimit;
      }
    }
  }
  wide = __ballot(wide) != 0;  // wave-uniform: this wave's diagonal block is summed directly
  __syncthreads();

  // the chunk's initial state, used last
  uint4 ps[Cfg::NVS];
#pragma unroll
  for (int i = 0; i < Cfg::NVS; ++i) {
    const int idx = tid + i * NT;
    ps[i] = (idx < Cfg::VS) ? *(const uint4 *)(gs + (size_t)idx * EPV) : make_uint4(0, 0, 0, 0);
  }

  // ---- this wave's gap factors (pairs (w, j <= w)) and e^{P_w}
  if (has_ch) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int c = c0 + e;
      // P_i = sum_{m < i} L_m; the index w is a runtime value, so P_w is accumulated separately
      float P[NB + 1], Pw = 0.f;
      P[0] = 0.f;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const float Li = sm.Lb[i][c];
        P[i + 1] = P[i] + Li;
        Pw += (i < w) ? Li : 0.f;
      }
      const float Lw = sm.Lb[w][c];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (j <= w) sm.gp[pair_ij(w, j)][c] = (j < w) ? __expf(Pw - P[j + 1]) : __expf(fminf(-Lw, 80.f));
      sm.eP[w][c] = __expf(Pw);
    }
  }
  wave_lds_sync();

  // ---- scores, as transposed tiles: A[j] holds A[t = 16w + n][s = 16j + 4g + r]
  f32x4_t A[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    acc_zero(A[j]);
    if (j > w) continue;  // wave-uniform
    if (j == w && wide) {
      // wide in-block decay: A[t][s] = sum_c q_t k_s e^{ell_t - ell_s}, summed
      // directly; for each t the exponent grows as s walks back from t, so
      // every factor is e^{<= 0}.  Rare, so reloads from global memory.
      for (int t = 0; t < 16; ++t) {
        const bool tv = (16 * w + t < len) && has_ch;
        float qt[CPL], ex[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          qt[e] = 0.f;
          ex[e] = 0.f;
        }
        if (tv) {
          const Pack<T, CPL> pq = ldpack<T, CPL>(gq + (tok(16 * w + t) + c0));
#pragma unroll
          for (int e = 0; e < CPL; ++e) qt[e] = to_f32(pq.v[e]);
        }
        for (int s = t; s >= 0; --s) {
          float part = 0.f;
          if (tv) {
            Pack<T, CPL> pk;
            if constexpr (reads_k(GM)) pk = ldpack<T, CPL>(gk + (tok(16 * w + s) + c0));
            const Pack<T, CPL> pl = ldlf(16 * w + s);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
              float lf, kv;
              lf_k<GM>(pk.v[e], lfe<GM>(pl, e), lbv[e], true, lf, kv);
              part += qt[e] * kv * __expf(ex[e]);
              ex[e] += lf;  // the factor of s - 1 includes f_s
            }
          }
          const float tot = wave_sum(part);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n16 == t && 4 * g + r == s) A[j][r] = tot;
        }
      }
      continue;
    }
    const int pi = pair_ij(w, j);
    if (j == w - 1) {
      // adjacent blocks: the gap factor is e^{P_w - P_w} = 1 exactly
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const int cc = 32 * ks + 8 * g;
        const bool ok = cc < D;
        const int c = ok ? cc : 0;
        mma(A[j], masked(row8<D>(sm.u.kv.ko, 16 * j + n16, c), ok), masked(row8<D>(sm.qo, 16 * w + n16, c), ok));
      }
      continue;
    }
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      const int cc = 32 * ks + 8 * g;
      const bool ok = cc < D;  // D = 16: groups past the channels feed zeros
      const int c = ok ? cc : 0;
      float kv[8];
      unpack8(row8<D>(sm.u.kv.ko, 16 * j + n16, c), kv);
      const float4 g0 = ldf4(&sm.gp[pi][c]), g1 = ldf4(&sm.gp[pi][c + 4]);
      Frag fa;
      fa.v[0] = kv[0] * g0.x; fa.v[1] = kv[1] * g0.y; fa.v[2] = kv[2] * g0.z; fa.v[3] = kv[3] * g0.w;
      fa.v[4] = kv[4] * g1.x; fa.v[5] = kv[5] * g1.y; fa.v[6] = kv[6] * g1.z; fa.v[7] = kv[7] * g1.w;
      masked(fa, ok);
      mma(A[j], to_pfrag<T>(fa), masked(row8<D>(sm.qo, 16 * w + n16, c), ok));
    }
    if (j == w) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g + r > n16) A[j][r] = 0.f;
    }
  }

  // ---- intra-chunk product Y = A V (two 16-token blocks of s per 32-deep step)
  f32x4_t Y[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc_zero(Y[cb]);
#pragma unroll
  for (int j1 = 0; j1 < NB; j1 += 2) {
    if (j1 > w) continue;
    const int j2 = j1 + 1;
    const bool has2 = (j2 <= w);
    const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const PFrag<T> fa = accs_to_frag<T>(A[j1], has2 ? A[j2 < NB ? j2 : j1] : zero);
    const int rb = 16 * (j2 < NB ? j2 : j1);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) mma(Y[cb], fa, tr8acc<D>(sm.u.kv.v, 16 * j1, rb, 16 * cb));
  }
  // the inter-chunk operand qb = qo e^{P_w} (rows of this wave)
  PFrag<T> qb[KSD];
#pragma unroll
  for (int ks = 0; ks < KSD; ++ks) {
    const int cc = 32 * ks + 8 * g;
    const bool ok = cc < D;
    const int c = ok ? cc : 0;
    float qv[8];
    unpack8(row8<D>(sm.qo, 16 * w + n16, c), qv);
    const float4 e0 = ldf4(&sm.eP[w][c]), e1 = ldf4(&sm.eP[w][c + 4]);
    Frag f;
    f.v[0] = qv[0] * e0.x; f.v[1] = qv[1] * e0.y; f.v[2] = qv[2] * e0.z; f.v[3] = qv[3] * e0.w;
    f.v[4] = qv[4] * e1.x; f.v[5] = qv[5] * e1.y; f.v[6] = qv[6] * e1.z; f.v[7] = qv[7] * e1.w;
    masked(f, ok);
    qb[ks] = to_pfrag<T>(f);
  }
  __syncthreads();  // every wave is done with ko and v

  // ---- the chunk's initial state into LDS (row c, column j)
#pragma unroll
  for (int i = 0; i < Cfg::NVS; ++i) {
    const int idx = tid + i * NT;
    const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
    if (idx < Cfg::VS) *(uint4 *)&sm.u.S[XT::at(row, col)] = ps[i];
  }
  __syncthreads();

  // ---- inter-chunk term: Y += qb S
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      if constexpr (D >= 32) {
        mma(Y[cb], qb[ks], tr8<D>(sm.u.S, 32 * ks, 16 * cb));
      } else {
        // D = 16: rows 8g + i exist for g < 2 only (qb is zero for g >= 2)
        mma(Y[cb], qb[ks], masked(tr8<D>(sm.u.S, (g < 2) ? 0 : -8 * g, 16 * cb), g < 2));
      }
    }

  if constexpr (std::is_same<TO, T>::value) {
    // ---- y: stage this wave's rows in its own qo rows, store whole rows
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.qo[XT::at(16 * w + 4 * g + r, 16 * cb + n16)] = from_f32<T>(Y[cb][r]);
    wave_lds_sync();
    constexpr int RV = 16 * D / EPV;  // 16-byte vectors in this wave's 16 rows
#pragma unroll
    for (int i = 0; i < (RV + 63) / 64; ++i) {
      const int idx = lane + 64 * i;
      const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
      const int t = 16 * w + row;
      if (idx < RV && t < len) {
        const uint4 u = *(const uint4 *)&sm.qo[XT::at(t, col)];
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, u), (u32x4_t *)(gy + (tok(t) + col)));
      }
    }
  } else {
    // ---- float32 y straight from the accumulators (no rounding to T): each
    // 16 lanes of a group write 64 contiguous bytes of one row
    TO *gyo = (TO *)a.y + cbase;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * w + 4 * g + r;
        if (t < len) __builtin_nontemporal_store(Y[cb][r], gyo + (tok(t) + 16 * cb + n16));
      }
  }
}

template <typename T, int D, int C, int GM, typename TO = T>
hipError_t launch_chunk_fwd(const ChunkFwdArgs &a, hipStream_t stream) {
  using Cfg = CfwdCfg<T, D, C>;
  hipLaunchKernelGGL((hgrn2_chunk_fwd_kernel<T, D, C, GM, TO>), dim3(a.B * a.H * a.N), dim3(Cfg::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hgrn2
