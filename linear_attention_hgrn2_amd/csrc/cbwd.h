// Per-chunk gradients of the HGRN2 recurrence (gfx950), all chunks in parallel.
//
// HGRN2 summary (paperlayer.ai) §3.2: S_t = Diag(f_t) S_{t-1} + k_t^T v_t,
// y_t = q_t S_t, evaluated chunkwise (§3.2 p.5).  Given the state S at the
// start of chunk n and the state adjoint Lam at its end (both written by the
// state scans), with b the in-chunk inclusive prefix of log f and Gamma = b_C:
//   dA[t][s] = dy_t . v_s                              (s <= t in the chunk)
//   dq_t = sum_{s<=t} dA[t][s] k_s e^{b_t-b_s} + e^{b_t} (S dy_t^T)
//   dk_s = sum_{t>=s} dA[t][s] q_t e^{b_t-b_s} + e^{Gamma-b_s} (Lam v_s^T)
//   dv_s = sum_{t>=s} A[t][s] dy_t + (k_s e^{Gamma-b_s}) Lam
//   dlog f_r = sum_{t>=r in chunk} (q_t dq_t - k_t dk_t) + rowsum(S_end * Lam)
// where rowsum(S_end * Lam) = e^Gamma rowsum(S * Lam) + sum_s k_s dk_s^inter
// carries every later token's contribution.  Exponents are anchored as in the
// forward: qo = q e^{ell}, ko = k e^{L_j - ell}, gap factors between 16-token
// sub-blocks; dq = e^{ell} dq', dk = e^{L - ell} dk' with dq', dk' formed from
// qo, ko and the gaps.  dlog f uses qo dq' - ko dk' with the same rounded qo,
// ko that entered the products, so the terms that cancel in exact arithmetic
// cancel here too.  A diagonal block whose decay exceeds kDiagLimit nats is
// summed directly.  With tied gates (k = 1 - f) k is formed from log f,
// dk is not written, and dlog f is the total derivative G = dlog f - f dk.
// With the gate pre-activation z as input (f = lb + (1 - lb) sigmoid(z)), log
// f and k are formed from z, the output is dz = G dlog f/dz, and each chunk
// writes its sums over tokens of G dlog f/dlb (reduced over chunks later).
//
// One workgroup per (batch, head, chunk); wave w owns 16-token sub-block w and
// produces all its outputs.  Phases: products from LDS tiles of qo, ko, v, dy
// (S and Lam fragments straight from memory); then per-token epilogues in the
// prep layout (lane = CPL channels, sixteen tokens in registers) through an
// LDS staging area; then the dv term that needs Lam with its rows as k.
#pragma once

#include "cfwd.h"

namespace hgrn2 {

struct ChunkBwdArgs {
  int B, T, H, N;
  const void *q, *k, *v, *log_f, *dy;  // [B,T,H,D]; log_f holds z in gate mode
  const void *states;                  // [B,H,N+1,D,D]; entry n = state before chunk n
  const void *lam;                     // [B,H,N,D,D]; entry n = adjoint at the end of chunk n
  void *dq, *dk, *dv, *dlog_f;         // [B,T,H,D]; dlog_f receives dz in gate mode; the input
                                       // dtype or (out_f32) float32
  const float *lb;                     // gate mode: lower bound of f, [H,D]
  float *dlb;                          // gate mode: per-chunk sums [B,H,N,D]
  int out_f32 = 0;                     // bfloat16 inputs: write the gradients as float32
};

template <typename T, int D, int C> struct CbwdCfg {
  static constexpr int NW = C / 16, NT = 64 * NW, NB = NW;
  static constexpr int CPL = D > 64 ? D / 64 : 1;
  static constexpr int LANES = D / CPL;
  static constexpr int CB = D / 16;
  static constexpr int KSD = (D + 31) / 32;
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int VT = C * D / EPV, NVT = (VT + NT - 1) / NT;  // 16-byte vectors of a token tile
  static constexpr int VS = D * D / EPV, NVS = (VS + NT - 1) / NT;
  static constexpr int LDG = D + 4;  // staging row stride (floats)
  static constexpr int LD = RowTile<T, D>::LD;
  // the gap factors are tabulated where the table fits the LDS beside the
  // tiles (chunk 64 and below); at chunk 128 they are formed where used
  static constexpr size_t kTileBytes = 4 * (size_t)C * LD * sizeof(T) + (size_t)NB * D * 4 + 16;
  static constexpr size_t kOutBytes = (2 * (size_t)NW * 16 * LDG + 2 * (size_t)NW * D + D) * 4;
  static constexpr size_t kFixed = ((size_t)NW * 2 * D + D) * 4;
  static constexpr bool GPT =
      kFixed + (kTileBytes + (size_t)NW * NB * D * sizeof(T) > kOutBytes ? kTileBytes + (size_t)NW * NB * D * sizeof(T)
                                                                         : kOutBytes) <=
      160 * 1024;
  struct In {
    float Lb[NB][D];  // sub-block totals of log f
    T gp[GPT ? NW : 1][GPT ? NB : 1][GPT ? D : 1];  // wave w: gap factor of its pair with block m
                                                   // (the same rounded value on both sides of a pair)
    float Pp[GPT ? 1 : NB + 1][GPT ? 1 : D];        // without the table: prefix sums P_i of the totals
    // RowTile<T, D> tiles, read and written 16 bytes at a time
    alignas(16) T qo[C * LD];
    alignas(16) T ko[C * LD];
    alignas(16) T v[C * LD];
    alignas(16) T dy[C * LD];
  };
  struct SL {
    T S[D * LD];  // RowTile<T, D>: the chunk's initial state (row c, column j)
    T L[D * LD];  // RowTile<T, D>: the adjoint at the chunk end
  };
  struct Out {
    float stg[2][NW][16 * LDG];  // per-wave staging of dq' and dk'
    float tot[NW][D];            // per-block sums of q dq - k dk
    float cpart[NW][D];          // per-block sums of ko dk'_inter
    float rs[D];                 // rowsum(S * Lam)
  };
  struct Smem {
    float fac[NW][2][D];  // wave w: e^{P_w}, e^{Gamma - P_{w+1}}
    float eG[D];          // e^Gamma
    union {
      In in;            // scores and intra-chunk products
      SL sl;            // then the inter-chunk products
      T dvs[C * LD];    // then the dv staging (RowTile<T, D>)
      Out out;          // then the epilogues
    } u;
  };
};

// TO: the element type of the gradients (T, or float32 for bfloat16 inputs)
template <typename T, int D, int C, int GM, typename TO = T>
__global__ __launch_bounds__(4 * C) __attribute__((amdgpu_waves_per_eu(2))) void hgrn2_chunk_bwd_kernel(ChunkBwdArgs a) {
  using Cfg = CbwdCfg<T, D, C>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, NB = Cfg::NB, CPL = Cfg::CPL, CB = Cfg::CB, KSD = Cfg::KSD,
                EPV = Cfg::EPV, LDG = Cfg::LDG;
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

  // buffer windows over this chunk's rows: offsets are 32-bit byte offsets
  // from the chunk's first row; rows past the end of the sequence read as zero
  // and their stores are dropped
  const size_t cbase = (((size_t)b * T_ + t0) * H + h) * D * sizeof(T);
  const uint32_t HDB = (uint32_t)H * D * sizeof(T);
  const uint32_t rows = (uint32_t)len * HDB;
  const GBuf bq((const char *)a.q + cbase, rows), bk((const char *)a.k + cbase, rows);
  const GBuf bv((const char *)a.v + cbase, rows), bl((const char *)a.log_f + cbase, rows);
  const GBuf bdy((const char *)a.dy + cbase, rows);
  // the gradients' rows, of TO elements
  const size_t cbaseo = cbase / sizeof(T) * sizeof(TO);
  const uint32_t HDBO = (uint32_t)H * D * sizeof(TO), rowso = (uint32_t)len * HDBO;
  const GBuf bdq((char *)a.dq + cbaseo, rowso), bdk((char *)a.dk + cbaseo, rowso);
  const GBuf bdv((char *)a.dv + cbaseo, rowso), bdl((char *)a.dlog_f + cbaseo, rowso);
  const GBuf bS((const char *)a.states + ((size_t)bh * (N + 1) + n) * D * D * sizeof(T), D * D * sizeof(T));
  const GBuf bL((const char *)a.lam + ((size_t)bh * N + n) * D * D * sizeof(T), D * D * sizeof(T));
  const uint32_t c0b = (uint32_t)c0 * sizeof(T), c0bo = (uint32_t)c0 * sizeof(TO);
  auto tok = [&](int t) { return (uint32_t)t * HDB; };    // byte offset of token t of the chunk
  auto toko = [&](int t) { return (uint32_t)t * HDBO; };  // the same in the gradients' rows
  // the chunk's log decays: per channel, or one per head broadcast (kScalar)
  const LfRows<GM> lr = lf_rows<GM, T>(a.log_f, b, T_, H, h, D, t0, len);
  // this lane's CPL elements of token t of the chunk (0 past the end)
  auto ldtok = [&](const GBuf &buf, int t) {
    Pack<T, CPL> p = buf.template ldpack<T, CPL>(tok(t) + c0b);
    if (!has_ch) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) p.v[e] = from_f32<T>(0.f);
    }
    return p;
  };
  auto ldlf = [&](int t) {
    Pack<T, CPL> p = lr.template ld<T, CPL>(t, c0b);
    if (!has_ch) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) p.v[e] = from_f32<T>(0.f);
    }
    return p;
  };

  // =============== phase 0: tiles of v and dy; qo, ko in the prep layout
#pragma unroll
  for (int i = 0; i < Cfg::NVT; ++i) {
    const int idx = tid + i * NT;
    const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
    const uint32_t off = tok(row) + (uint32_t)col * sizeof(T);
    const uint4 x = bv.ld16(off), y = bdy.ld16(off);
    if (idx < Cfg::VT) {
      *(uint4 *)&sm.u.in.v[XT::at(row, col)] = x;
      *(uint4 *)&sm.u.in.dy[XT::at(row, col)] = y;
    }
  }
  bool wide = false;
  {
    Pack<T, CPL> pq[16], pk[16], pl[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      pq[t] = ldtok(bq, 16 * w + t);
      if constexpr (reads_k(GM)) pk[t] = ldtok(bk, 16 * w + t);
      pl[t] = ldlf(16 * w + t);
    }
    float l[16][CPL], L[CPL], kk[16][CPL];
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
        stpack<T, CPL>(&sm.u.in.qo[XT::at(16 * w + t, c0)], oq);
        stpack<T, CPL>(&sm.u.in.ko[XT::at(16 * w + t, c0)], ok);
      }
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        sm.u.in.Lb[w][c0 + e] = L[e];
        wide |= -L[e] > kDiagLimit;
      }
    }
  }
  wide = __ballot(wide) != 0;
  __syncthreads();  // B1

  // =============== phase 1a: this wave's gap factors and exponential factors
  if (has_ch) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int c = c0 + e;
      float P[NB + 1], Pw = 0.f, Pw1 = 0.f;
      P[0] = 0.f;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const float Li = sm.u.in.Lb[i][c];
        P[i + 1] = P[i] + Li;
        Pw += (i < w) ? Li : 0.f;
        Pw1 += (i <= w) ? Li : 0.f;
      }
      const float G = P[NB], Lw = sm.u.in.Lb[w][c];
      if constexpr (Cfg::GPT) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
          float x;
          if (m < w) x = Pw - P[m + 1];
          else if (m == w) x = fminf(-Lw, 80.f);
          else x = P[m] - Pw1;
          sm.u.in.gp[w][m][c] = from_f32<T>(__expf(x));
        }
      } else {
        // every wave forms the same prefix sums; wave 0 keeps them
        if (w == 0) {
#pragma unroll
          for (int i = 0; i <= NB; ++i) sm.u.in.Pp[i][c] = P[i];
        }
      }
      sm.fac[w][0][c] = __expf(Pw);
      sm.fac[w][1][c] = __expf(G - Pw1);
      if (w == 0) sm.eG[c] = __expf(G);
    }
  }
  // the table is per wave; the prefix sums are read by every wave
  if constexpr (Cfg::GPT) {
    wave_lds_sync();
  } else {
    __syncthreads();
  }

  // the gap factor of block w's pair with block m at channel c, rounded to T:
  // from the table, or formed again from the prefix sums with the table's
  // arithmetic (the same sums, so the same bits on both sides of a pair)
  auto gap = [&](int m, int c) -> float {
    if constexpr (Cfg::GPT) {
      return to_f32(sm.u.in.gp[w][m][c]);
    } else {
      const float x = m < w    ? sm.u.in.Pp[w][c] - sm.u.in.Pp[m + 1][c]
                      : m == w ? fminf(-sm.u.in.Lb[w][c], 80.f)
                               : sm.u.in.Pp[m][c] - sm.u.in.Pp[w + 1][c];
      return to_f32(from_f32<T>(__expf(x)));
    }
  };

  // =============== phase 1b: products
  f32x4_t DQ[CB], DK[CB], DV[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    acc_zero(DQ[cb]);
    acc_zero(DK[cb]);
    acc_zero(DV[cb]);
  }
  const T *qo = sm.u.in.qo, *ko = sm.u.in.ko, *tv = sm.u.in.v, *tdy = sm.u.in.dy;

  // (a) dq' intra: pairs (w, m <= w).  dA^T tile: rows s in m, columns t in w.
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    if (m > w || (m == w && wide)) continue;  // wave-uniform
    f32x4_t X;
    acc_zero(X);
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      const int jj = 32 * ks + 8 * g;
      const bool ok = jj < D;
      const int j = ok ? jj : 0;
      mma(X, masked(row8<D>(tv, 16 * m + n16, j), ok), masked(row8<D>(tdy, 16 * w + n16, j), ok));
    }
    if (m == w) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g + r > n16) X[r] = 0.f;  // s > t
    }
    const PFrag4<T> fa = acc_to_frag4<T>(X);  // lane (g, t): k-slots s = 16m + 4g + r
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      f32x4_t tmp;
      acc_zero(tmp);
      mma16(tmp, fa, tr4<D>(ko, 16 * m, 16 * cb));
      const float gpf = gap(m, 16 * cb + n16);
#pragma unroll
      for (int r = 0; r < 4; ++r) DQ[cb][r] += gpf * tmp[r];
    }
  }

  // (b) dk' intra and (c) scores for dv: pairs (m >= w, w).  Tiles: rows t in m, columns s in w.
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    if (m < w) continue;
    const bool direct = (m == w) && wide;
    if (!direct) {
      f32x4_t X;
      acc_zero(X);
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const int jj = 32 * ks + 8 * g;
        const bool ok = jj < D;
        const int j = ok ? jj : 0;
        mma(X, masked(row8<D>(tdy, 16 * m + n16, j), ok), masked(row8<D>(tv, 16 * w + n16, j), ok));
      }
      if (m == w) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r < n16) X[r] = 0.f;  // t < s
      }
      const PFrag4<T> fa = acc_to_frag4<T>(X);  // lane (g, s): k-slots t = 16m + 4g + r
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        f32x4_t tmp;
        acc_zero(tmp);
        mma16(tmp, fa, tr4<D>(qo, 16 * m, 16 * cb));
        const float gpf = gap(m, 16 * cb + n16);
#pragma unroll
        for (int r = 0; r < 4; ++r) DK[cb][r] += gpf * tmp[r];
      }
    }
    // scores A[t][s] = sum_c qo_t (ko_s gap), lane (g, s) holds t = 16m + 4g + r
    f32x4_t A;
    acc_zero(A);
    if (!direct) {
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const int cc = 32 * ks + 8 * g;
        const bool ok = cc < D;
        const int c = ok ? cc : 0;
        float kv[8];
        unpack8(row8<D>(ko, 16 * w + n16, c), kv);
        float gv[8];
        if constexpr (Cfg::GPT) {
          unpack8(ld8(&sm.u.in.gp[w][m][c]), gv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) gv[e] = gap(m, c + e);
        }
        Frag fb;
#pragma unroll
        for (int i = 0; i < 8; ++i) fb.v[i] = kv[i] * gv[i];
        masked(fb, ok);
        mma(A, masked(row8<D>(qo, 16 * m + n16, c), ok), to_pfrag<T>(fb));
      }
      if (m == w) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r < n16) A[r] = 0.f;
      }
    } else {
      // wide in-block decay: A[t][s] summed directly (every exponent <= 0)
      for (int t = 0; t < 16; ++t) {
        const bool tv_ = (16 * w + t < len) && has_ch;
        float qt[CPL], ex[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          qt[e] = 0.f;
          ex[e] = 0.f;
        }
        if (tv_) {
          const Pack<T, CPL> p = bq.template ldpack<T, CPL>(tok(16 * w + t) + c0b);
#pragma unroll
          for (int e = 0; e < CPL; ++e) qt[e] = to_f32(p.v[e]);
        }
        for (int s = t; s >= 0; --s) {
          float part = 0.f;
          if (tv_) {
            Pack<T, CPL> pk;
            if constexpr (reads_k(GM)) pk = bk.template ldpack<T, CPL>(tok(16 * w + s) + c0b);
            const Pack<T, CPL> pl = lr.template ld<T, CPL>(16 * w + s, c0b);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
              float lf, kv;
              lf_k<GM>(pk.v[e], lfe<GM>(pl, e), lbv[e], true, lf, kv);
              part += qt[e] * kv * __expf(ex[e]);
              ex[e] += lf;
            }
          }
          const float tot = wave_sum(part);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n16 == s && 4 * g + r == t) A[r] = tot;
        }
      }
    }
    // dv intra += A^T dy over this block of t
    const PFrag4<T> fa = acc_to_frag4<T>(A);
#pragma unroll
    for (int jb = 0; jb < CB; ++jb) mma16(DV[jb], fa, tr4<D>(tdy, 16 * m, 16 * jb));
  }

  // (d) inter-chunk terms.  This wave's rows of dy, v and kh = ko e^{Gamma - P_{w+1}}
  // and its ko in the accumulator arrangement stay in registers while S and Lam
  // replace the tiles in LDS.
  PFrag<T> dyA[KSD], vA[KSD], khA[KSD];
#pragma unroll
  for (int ks = 0; ks < KSD; ++ks) {
    const int jj = 32 * ks + 8 * g;
    const bool ok = jj < D;
    const int j = ok ? jj : 0;
    dyA[ks] = masked(row8<D>(tdy, 16 * w + n16, j), ok);
    vA[ks] = masked(row8<D>(tv, 16 * w + n16, j), ok);
    float kv[8];
    unpack8(row8<D>(ko, 16 * w + n16, j), kv);
    const float4 e0 = ldf4(&sm.fac[w][1][j]), e1 = ldf4(&sm.fac[w][1][j + 4]);
    Frag f;
    f.v[0] = kv[0] * e0.x; f.v[1] = kv[1] * e0.y; f.v[2] = kv[2] * e0.z; f.v[3] = kv[3] * e0.w;
    f.v[4] = kv[4] * e1.x; f.v[5] = kv[5] * e1.y; f.v[6] = kv[6] * e1.z; f.v[7] = kv[7] * e1.w;
    masked(f, ok);
    khA[ks] = to_pfrag<T>(f);
  }
  Quad<T> kq[CB];  // ko[16w + 4g + r][16 cb + n], as it entered the products
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) kq[cb].set(r, ko[XT::at(16 * w + 4 * g + r, 16 * cb + n16)]);
  __syncthreads();  // B2: the tiles are dead
  T *sS = sm.u.sl.S, *sL = sm.u.sl.L;
#pragma unroll
  for (int i = 0; i < Cfg::NVS; ++i) {
    const int idx = tid + i * NT;
    const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
    if (idx < Cfg::VS) {
      const uint32_t off = (uint32_t)(row * D + col) * sizeof(T);
      *(uint4 *)&sS[XT::at(row, col)] = bS.ld16(off);
      *(uint4 *)&sL[XT::at(row, col)] = bL.ld16(off);
    }
    if (i % 4 == 3) asm volatile("" ::: "memory");  // bounds the loads in flight
  }
  __syncthreads();  // B3

  // rowsum(S * Lam) of this wave's channel blocks cb = w + NW i: the diagonal of
  // the 16 x 16 block S Lam^T, on lane (n >> 2, n)
  constexpr int RSN = (CB + NW - 1) / NW;
  float rsv[RSN];
  float cp[CB];  // sum over this block of ko dk'_inter, channel 16 cb + n
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = 16 * cb + n16;
    f32x4_t tq, tk, dg;
    acc_zero(tq);
    acc_zero(tk);
    acc_zero(dg);
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      const int jj = 32 * ks + 8 * g;
      const bool ok = jj < D;
      const int j = ok ? jj : 0;
      const PFrag<T> sf = masked(row8<D>(sS, c, j), ok), lf = masked(row8<D>(sL, c, j), ok);
      mma(tq, dyA[ks], sf);
      mma(tk, vA[ks], lf);
      if (cb % NW == w) mma(dg, sf, lf);
    }
    if (cb % NW == w) {
      const int r = n16 & 3;
      rsv[cb / NW] = (r == 0) ? dg[0] : (r == 1) ? dg[1] : (r == 2) ? dg[2] : dg[3];
    }
    const float eP = sm.fac[w][0][c], eK = sm.fac[w][1][c];
    float ckp = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      DQ[cb][r] += eP * tq[r];
      const float x = eK * tk[r];
      DK[cb][r] += x;
      ckp += kq[cb].get(r) * x;
    }
    cp[cb] = group_sum(ckp);
  }
  // dv += kh Lam (Lam rows as k)
#pragma unroll
  for (int jb = 0; jb < CB; ++jb)
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      if constexpr (D >= 32) {
        mma(DV[jb], khA[ks], tr8<D>(sL, 32 * ks, 16 * jb));
      } else {
        mma(DV[jb], khA[ks], masked(tr8<D>(sL, (g < 2) ? 0 : -8 * g, 16 * jb), g < 2));
      }
    }
  __syncthreads();  // B4: S and Lam are dead

  // =============== phase 2: dv out, then the epilogues of dq, dk and dlog f
  if constexpr (std::is_same<TO, T>::value) {
    T *dvs = sm.u.dvs;
#pragma unroll
    for (int jb = 0; jb < CB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dvs[XT::at(16 * w + 4 * g + r, 16 * jb + n16)] = from_f32<T>(DV[jb][r]);
    wave_lds_sync();
    constexpr int RV = 16 * D / EPV;
#pragma unroll
    for (int i = 0; i < (RV + 63) / 64; ++i) {
      const int idx = lane + 64 * i;
      const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
      const int t = 16 * w + row;
      if (idx < RV) bdv.st16(tok(t) + (uint32_t)col * sizeof(T), *(const uint4 *)&dvs[XT::at(t, col)]);
    }
  } else {
    // float32 dv straight from the accumulators: each 16 lanes of a group
    // write 64 contiguous bytes of one row (rows past the end are dropped)
#pragma unroll
    for (int jb = 0; jb < CB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Pack<TO, 1> o;
        o.v[0] = DV[jb][r];
        bdv.stpack<TO, 1>(toko(16 * w + 4 * g + r) + (uint32_t)(16 * jb + n16) * sizeof(TO), o);
      }
  }
  __syncthreads();  // B5: the dv staging is dead

  auto &out = sm.u.out;
  if (g == 0) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) out.cpart[w][16 * cb + n16] = cp[cb];

  }
  if (g == (n16 >> 2)) {
#pragma unroll
    for (int i = 0; i < RSN; ++i)
      if (w + NW * i < CB) out.rs[16 * (w + NW * i) + n16] = rsv[i];
  }
  float *sq = out.stg[0][w], *sk = out.stg[1][w];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sq[(4 * g + r) * LDG + 16 * cb + n16] = DQ[cb][r];
      sk[(4 * g + r) * LDG + 16 * cb + n16] = DK[cb][r];
    }
  wave_lds_sync();
  // per token (prep layout): dq = e^{ell} dq', dk = e^{L - ell} dk', and
  // X = q dq - k dk formed with qo, ko exactly as they entered the products.
  // A wave whose diagonal block is summed directly takes a slow path that
  // keeps X in its staging rows instead of registers.
  float X[16][CPL];
  if (!wide) {
    Pack<T, CPL> pl[16];
    float L[CPL], ell[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) L[e] = ell[e] = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      pl[t] = ldlf(16 * w + t);
#pragma unroll
      for (int e = 0; e < CPL; ++e) L[e] += lf_of<GM>(to_f32(lfe<GM>(pl[t], e)), lbv[e], 16 * w + t < len);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int tt = 16 * w + t;
      const Pack<T, CPL> pq = ldtok(bq, tt);
      Pack<T, CPL> pk;
      if constexpr (reads_k(GM)) pk = ldtok(bk, tt);
      Pack<TO, CPL> oq, ok;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        float lft, kv;
        lf_k<GM>(pk.v[e], lfe<GM>(pl[t], e), lbv[e], tt < len, lft, kv);
        ell[e] += lft;
        const float el = __expf(ell[e]), ek = __expf(L[e] - ell[e]);
        const float qor = to_f32(from_f32<T>(to_f32(pq.v[e]) * el));
        const float kor = to_f32(from_f32<T>(kv * ek));
        const float d1 = sq[t * LDG + c0 + e], d2 = sk[t * LDG + c0 + e];
        oq.v[e] = from_f32<TO>(el * d1);
        ok.v[e] = from_f32<TO>(ek * d2);
        X[t][e] = qor * d1 - kor * d2;
        // k tied to f: f dk, subtracted from dlog f below (replaces the consumed dk'_t)
        if (ties_k(GM) && has_ch) sk[t * LDG + c0 + e] = __expf(lft) * (ek * d2);
      }
      if (has_ch) {
        bdq.stpack<TO, CPL>(toko(tt) + c0bo, oq);
        if constexpr (reads_k(GM)) bdk.stpack<TO, CPL>(toko(tt) + c0bo, ok);
      }
    }
    if (has_ch) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        float s_ = 0.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) s_ += X[t][e];
        out.tot[w][c0 + e] = s_;
      }
    }
  } else {
    // diagonal block summed directly: dq_t adds sum_{s <= t} dA[t][s] k_s e^{ell_t - ell_s},
    // dk_t adds sum_{u >= t} dA[u][t] q_u e^{ell_u - ell_t} (every exponent <= 0)
    float L[CPL], ell[CPL], tot[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) L[e] = ell[e] = tot[e] = 0.f;
    for (int t = 0; t < 16; ++t) {
      const Pack<T, CPL> p = ldlf(16 * w + t);
#pragma unroll
      for (int e = 0; e < CPL; ++e) L[e] += lf_of<GM>(to_f32(lfe<GM>(p, e)), lbv[e], 16 * w + t < len);
    }
    for (int t = 0; t < 16; ++t) {
      const int tt = 16 * w + t;
      const Pack<T, CPL> pq = ldtok(bq, tt), plt = ldlf(tt);
      Pack<T, CPL> pk;
      if constexpr (reads_k(GM)) pk = ldtok(bk, tt);
      const Pack<T, CPL> pdy = ldtok(bdy, tt), pv = ldtok(bv, tt);
      float dqd[CPL], dkd[CPL], ex[CPL];
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        ell[e] += lf_of<GM>(to_f32(lfe<GM>(plt, e)), lbv[e], tt < len);
        dqd[e] = dkd[e] = ex[e] = 0.f;
      }
      for (int s_ = t; s_ >= 0; --s_) {
        const Pack<T, CPL> pvs = ldtok(bv, 16 * w + s_), pls = ldlf(16 * w + s_);
        Pack<T, CPL> pks;
        if constexpr (reads_k(GM)) pks = ldtok(bk, 16 * w + s_);
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) part += to_f32(pdy.v[e]) * to_f32(pvs.v[e]);
        const float dA = wave_sum(part);
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          dqd[e] += dA * k_of<GM>(pks.v[e], lfe<GM>(pls, e), lbv[e]) * __expf(ex[e]);
          ex[e] += lf_of<GM>(to_f32(lfe<GM>(pls, e)), lbv[e], 16 * w + s_ < len);
        }
      }
#pragma unroll
      for (int e = 0; e < CPL; ++e) ex[e] = 0.f;
      for (int u = t; u < 16; ++u) {
        const Pack<T, CPL> pdu = ldtok(bdy, 16 * w + u), pqu = ldtok(bq, 16 * w + u);
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) part += to_f32(pdu.v[e]) * to_f32(pv.v[e]);
        const float dA = wave_sum(part);
        if (u > t) {
          const Pack<T, CPL> plu = ldlf(16 * w + u);
#pragma unroll
          for (int e = 0; e < CPL; ++e) ex[e] += lf_of<GM>(to_f32(lfe<GM>(plu, e)), lbv[e], 16 * w + u < len);
        }
#pragma unroll
        for (int e = 0; e < CPL; ++e) dkd[e] += dA * to_f32(pqu.v[e]) * __expf(ex[e]);
      }
      Pack<TO, CPL> oq, ok;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const float el = __expf(ell[e]), ek = __expf(L[e] - ell[e]);
        const float qv = to_f32(pq.v[e]), kv = k_of<GM>(pk.v[e], lfe<GM>(plt, e), lbv[e]);
        const float qor = to_f32(from_f32<T>(qv * el)), kor = to_f32(from_f32<T>(kv * ek));
        const float d1 = sq[t * LDG + c0 + e], d2 = sk[t * LDG + c0 + e];
        oq.v[e] = from_f32<TO>(el * d1 + dqd[e]);
        ok.v[e] = from_f32<TO>(ek * d2 + dkd[e]);
        const float x = (qor * d1 + qv * dqd[e]) - (kor * d2 + kv * dkd[e]);
        if (has_ch) sq[t * LDG + c0 + e] = x;  // X_t replaces the consumed dq'_t
        if (ties_k(GM) && has_ch)
          sk[t * LDG + c0 + e] = __expf(lf_of<GM>(to_f32(lfe<GM>(plt, e)), lbv[e], tt < len)) * (ek * d2 + dkd[e]);
        tot[e] += x;
      }
      if (has_ch) {
        bdq.stpack<TO, CPL>(toko(tt) + c0bo, oq);
        if constexpr (reads_k(GM)) bdk.stpack<TO, CPL>(toko(tt) + c0bo, ok);
      }
    }
    if (has_ch)
#pragma unroll
      for (int e = 0; e < CPL; ++e) out.tot[w][c0 + e] = tot[e];
  }
  __syncthreads();  // B6: tot, cpart, rs complete
  // dlog f = reverse in-chunk sum of X plus the carry; k tied to f subtracts
  // f dk; gate mode turns that total G into dz and sums G dlog f/dlb over the
  // chunk's tokens
  float dlbs[CPL], ssum[16];  // ssum: per-head decay, this lane's part of each token's dlog a
#pragma unroll
  for (int e = 0; e < CPL; ++e) dlbs[e] = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t) ssum[t] = 0.f;
  if (has_ch) {
    float carry[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int c = c0 + e;
      carry[e] = sm.eG[c] * out.rs[c];
#pragma unroll
      for (int i = 0; i < NW; ++i) carry[e] += out.cpart[i][c] + ((i > w) ? out.tot[i][c] : 0.f);
    }
    auto emit = [&](int t, const float *cr) {
      const int tt = 16 * w + t;
      Pack<TO, CPL> o;
      Pack<T, CPL> pz;
      if constexpr (GM == kGate) pz = ldtok(bl, tt);
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        float G = ties_k(GM) ? cr[e] - sk[t * LDG + c0 + e] : cr[e];
        if constexpr (GM == kGate) {
          const GateGrad gg = gate_grad(to_f32(pz.v[e]), lbv[e]);
          if (tt < len) dlbs[e] += G * gg.dlb;
          G *= gg.dz;
        }
        o.v[e] = from_f32<TO>(G);
        if constexpr (GM == kScalar) ssum[t] += G;
      }
      if constexpr (GM != kScalar) bdl.stpack<TO, CPL>(toko(tt) + c0bo, o);
    };
    if (!wide) {
#pragma unroll
      for (int t = 15; t >= 0; --t) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) carry[e] += X[t][e];
        emit(t, carry);
      }
    } else {
#pragma unroll
      for (int t = 15; t >= 0; --t) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) carry[e] += sq[t * LDG + c0 + e];
        emit(t, carry);
      }
    }
  }
  if constexpr (GM == kScalar) {
    // dlog a of each token: the sum over the head's channels, across the wave
    const GBuf bda((char *)a.dlog_f + (((size_t)b * T_ + t0) * H + h) * sizeof(TO), (uint32_t)(len * H * sizeof(TO)));
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float tot = wave_sum(ssum[t]);
      if (lane == 0) {
        Pack<TO, 1> o;
        o.v[0] = from_f32<TO>(tot);
        bda.stpack<TO, 1>((uint32_t)(16 * w + t) * H * sizeof(TO), o);
      }
    }
  }
  if constexpr (GM == kGate) {
    // per-wave sums into row 0 of the wave's (consumed) dq' staging, then one
    // fixed-order sum over the waves per channel
    if (has_ch) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) sq[c0 + e] = dlbs[e];
    }
    __syncthreads();
    for (int c = tid; c < D; c += NT) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) acc += out.stg[0][i][c];
      a.dlb[((size_t)bh * N + n) * D + c] = acc;
    }
  }
}

template <typename T, int D, int C, int GM, typename TO = T>
hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, hipStream_t stream) {
  using Cfg = CbwdCfg<T, D, C>;
  hipLaunchKernelGGL((hgrn2_chunk_bwd_kernel<T, D, C, GM, TO>), dim3(a.B * a.H * a.N), dim3(Cfg::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hgrn2
