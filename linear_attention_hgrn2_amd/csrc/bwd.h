// Chunked backward of the HGRN2 recurrence: reverse chunk scan of the state
// adjoint on CDNA4 matrix cores.
//
// Loss L = sum(y * dy) + sum(S_T * dht).  Lam denotes the adjoint of the
// state at the end of the current chunk (Lam = dht after the last chunk).  For
// one chunk, with b, Gamma, A as in the forward and dA = tril(dY V^T):
//   dq       = dA (k e^{b_t - b_s}) + e^b * (dY S_prev^T)
//   dk       = dA^T (q e^{b_t - b_s}) + e^{Gamma - b} * (V Lam^T)
//   dv       = A^T dY + (k e^{Gamma - b}) Lam
//   dlog_f_t = sum_{t' >= t in chunk} (q dq - k dk)_{t'} + rowsum(S_end * Lam)
//   Lam     <- e^Gamma * Lam + (q e^b)^T dY          (carried to the previous chunk)
// and dh0 = Lam after the first chunk.  The dlog_f form follows from every
// path through token t picking up log f_t once: the gradient of log f_t is
// the part of <dL/dS, S> that flows through steps >= t, which reduces to the
// chunk-local reverse sum plus the carry rowsum(S_end * Lam) from the right.
//
// Each (batch, head) is handled by two workgroups that walk the chunks in
// reverse side by side, each carrying the full D x D adjoint in float32
// accumulators in the layout its products need:
//   channel side: Lam^T, wave w owning channels [16w, 16w+16); computes dA,
//                 dq, dk, dlog_f (everything contracted against channels);
//   value side  : Lam, wave w owning value columns [16w, 16w+16); computes A
//                 and dv.
// Both update their copy of the adjoint from the same operands, so the two
// never communicate.  S_prev comes from the chunk-boundary states saved by
// the forward.
//
// Per chunk a preparation pass evaluates every decayed operand once (the
// channel-major tiles use the bank-spreading TT32/TT16 layouts), with
// exponents anchored inside the span they cover (<= 0 except on diagonal
// sub-blocks; those are evaluated directly when their decay range exceeds
// kDiagLimit).  16-token sub-blocks carry block-local prefixes ell (totals
// L_j, starts P_j); the operands are
//   qo = q e^{ell}, ko = k e^{L_j - ell}, kh = k e^{Gamma - b}, qh = q e^b,
// and the remaining per-block factors e^{P_i - P_{j+1}} (gap), e^{-L_j}
// (diagonal) are per-channel scalars applied to whole fragments.
//
// Precision: dlog_f is a reverse sum of q dq - k dk, whose intra-chunk parts
// cancel pair by pair (only token pairs straddling t survive).  Rounding the
// decayed k and q operands of dq and dk independently to bf16 would destroy
// that cancellation, so the channel side keeps qo, ko in float32 and feeds
// them to the MFMA as bf16 hi + lo pairs, and forms q dq, k dk in float32.
#pragma once

#include "common.h"
#include "fwd.h"

namespace hgrn2 {

struct BwdArgs {
  int B, T, H;
  const void *q, *k, *v, *log_f, *dy;
  const void *states;  // [B,H,N+1,D,D], input dtype
  const float *dht;
  void *dq, *dk, *dv, *dlog_f;
  float *dh0;
  int N;
};

template <typename TIn, int D, int C>
struct BwdCfg {
  static constexpr int NW = D / 16;
  static constexpr int NT = NW * 64;
  static constexpr int NB = C / 16;
  static constexpr int NPAIR = NB * (NB + 1) / 2;
  static constexpr int CB = D / 16;
  static constexpr int KSD = (D + 31) / 32;
  static constexpr int KSC = (C + 31) / 32;
  static constexpr int EPV = 16 / (int)sizeof(TIn);
  static constexpr int LDN = D + EPV;   // [token][channel] rows
  static constexpr int LDA = C + EPV;   // [token][token] rows
  static constexpr int LDL = D + 4;     // float32 [token][channel] rows
  static constexpr int VQ = C * D / EPV;
  static constexpr int NVQ = (VQ + NT - 1) / NT;
  struct SmemC {                 // channel side
    union {
      struct {
        float lT[D * TT32<C>::LD];   // ell, channel-major (TT32 layout)
        float koT[D * TT32<C>::LD];  // k e^{L_j - ell}
      };
      struct {                       // once dq and dk are done: output staging
        TIn sq[C][LDN];              // dq
        TIn sl[C][LDN];              // dlog_f
      };
    };
    float qoT[D * TT32<C>::LD];  // q e^{ell}
    TIn v[C][LDN];               // V; once dk is done: dk staging
    TIn dy[C][LDN];
    TIn dA[C][LDA];              // dA[t][s], causal
    float Lb[NB][D];
    float Pb[NB + 1][D];
    int flags;
  };
  struct SmemV {                 // value side
    float l[C][LDL];             // ell, token-major
    TIn qo[C][LDN];              // q e^{ell}
    TIn ko[C][LDN];              // k e^{L_j - ell}; once the score tiles are done: dv staging
    TIn kh[C][LDN];              // k e^{Gamma - b}
    TIn qhT[D * TTile<TIn, C>::LD];  // (q e^b)^T (TTile layout)
    TIn dy[C][LDN];
    TIn At[C][LDA];              // A^T[s][t], causal
    float Lb[NB][D];
    float Pb[NB + 1][D];
    float gp[NPAIR][D];          // gap factors of the score blocks
    int flags;
  };
  union Smem {
    SmemC c;
    SmemV v;
  };
  static constexpr bool fits = sizeof(Smem) <= 160 * 1024;  // LDS per workgroup on gfx950
};

// ---------------------------------------------------------------- channel side
template <typename TIn, int D, int C>
__device__ __forceinline__ void bwd_channel_side(const BwdArgs &args, typename BwdCfg<TIn, D, C>::SmemC &sm,
                                                 int b, int h) {
  using Cfg = BwdCfg<TIn, D, C>;
  constexpr int NT = Cfg::NT, NB = Cfg::NB, CB = Cfg::CB, KSD = Cfg::KSD, KSC = Cfg::KSC,
                EPV = Cfg::EPV, NW = Cfg::NW, NPAIR = Cfg::NPAIR;
  const int T = args.T, H = args.H, N = args.N;
  const int bh = b * H + h;
  const int tid = threadIdx.x;
  const int w = tid >> 6;

  const TIn *gq = (const TIn *)args.q;
  const TIn *gk = (const TIn *)args.k;
  const TIn *gv = (const TIn *)args.v;
  const TIn *gl = (const TIn *)args.log_f;
  const TIn *gdy = (const TIn *)args.dy;
  TIn *gdq = (TIn *)args.dq;
  TIn *gdk = (TIn *)args.dk;
  TIn *gdl = (TIn *)args.dlog_f;
  const size_t SS = (size_t)D * D;
  const TIn *st_base = (const TIn *)args.states + (size_t)bh * (N + 1) * SS;
  auto tok = [&](int t) { return (((size_t)b * T + t) * H + h) * D; };

  // Row cw of a state, in the value-column order of the Lam^T accumulators:
  // slot x of k step ks is column j = 16(2ks + x/4) + 4g + x%4.
  auto load_state_frag = [&](const TIn *St, Frag *f) {
    const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int jb = 2 * ks + half;
#pragma unroll
        for (int x = 0; x < 4; ++x)
          f[ks].v[4 * half + x] = (jb < CB) ? to_f32(St[(size_t)cw * D + jb * 16 + 4 * g + x]) : 0.f;
      }
  };

  // Lam^T: tile jb holds rows j = 16jb + 4g + r, column c = cw.
  f32x4_t LamT[CB];
  {
    const int lane = tid & 63, n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
#pragma unroll
    for (int jb = 0; jb < CB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        LamT[jb][r] = args.dht ? args.dht[(size_t)bh * SS + (size_t)cw * D + jb * 16 + 4 * g + r] : 0.f;
  }
  auto rowsum = [&](const Frag *Sf) {  // sum_j S[cw][j] Lam[cw][j]
    float a = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int jb = 2 * ks + (x >> 2);
        if (jb < CB) a += Sf[ks].v[x] * LamT[jb][x & 3];
      }
    a += __shfl_xor(a, 16);
    a += __shfl_xor(a, 32);
    return a;
  };
  float carry;
  {
    Frag Send[KSD];
    load_state_frag(st_base + (size_t)N * SS, Send);
    carry = rowsum(Send);
  }

  uint4 pq[Cfg::NVQ], pk[Cfg::NVQ], pv[Cfg::NVQ], pd[Cfg::NVQ], pl[Cfg::NVQ];
  auto prefetch = [&](int n) {
    const int t0 = n * C;
    const int len = min(C, T - t0);
#pragma unroll
    for (int it = 0; it < Cfg::NVQ; ++it) {
      const int idx = tid + it * NT;
      const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
      uint4 z = make_uint4(0, 0, 0, 0);
      pq[it] = pk[it] = pv[it] = pd[it] = pl[it] = z;
      if (idx < Cfg::VQ && row < len) {
        const size_t off = tok(t0 + row) + col;
        pq[it] = *(const uint4 *)(gq + off);
        pk[it] = *(const uint4 *)(gk + off);
        pv[it] = *(const uint4 *)(gv + off);
        pd[it] = *(const uint4 *)(gdy + off);
        pl[it] = *(const uint4 *)(gl + off);
      }
    }
  };
  prefetch(N - 1);

  for (int n = N - 1; n >= 0; --n) {
    const int t0 = n * C;
    const int len = min(C, T - t0);
    Frag Sprev[KSD];  // S at the start of this chunk (boundary state n)
    load_state_frag(st_base + (size_t)n * SS, Sprev);

    // ================= preparation =================
    __syncthreads();
    {
      const int tid = opaque(threadIdx.x);
#pragma unroll
      for (int it = 0; it < Cfg::NVQ; ++it) {
        const int idx = tid + it * NT;
        if (idx < Cfg::VQ) {
          const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
          *(uint4 *)&sm.v[row][col] = pv[it];
          *(uint4 *)&sm.dy[row][col] = pd[it];
          float f[EPV];
          Vec<TIn>::unpack(pl[it], f);
#pragma unroll
          for (int e = 0; e < EPV; ++e) sm.lT[TT32<C>::at(col + e, row)] = floor_logf(f[e]);
        }
      }
      if (tid == 0) sm.flags = 0;
      __syncthreads();
      {  // block-local inclusive prefixes along tokens, block totals, flags
        int fl = 0;
        for (int p = tid; p < NB * D; p += NT) {
          const int i = p / D, c = p % D;
          float acc = 0.f;
#pragma unroll
          for (int u4 = 0; u4 < 4; ++u4) {
            float4 *pp = (float4 *)&sm.lT[TT32<C>::at(c, i * 16 + 4 * u4)];
            float4 x = *pp;
            acc += x.x;
            x.x = acc;
            acc += x.y;
            x.y = acc;
            acc += x.z;
            x.z = acc;
            acc += x.w;
            x.w = acc;
            *pp = x;
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
#pragma unroll
      for (int it = 0; it < Cfg::NVQ; ++it) {
        const int idx = tid + it * NT;
        if (idx < Cfg::VQ) {
          const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
          const int jb = row >> 4;
          float fq[EPV], fk[EPV];
          Vec<TIn>::unpack(pq[it], fq);
          Vec<TIn>::unpack(pk[it], fk);
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const int c = col + e;
            const int o = TT32<C>::at(c, row);
            const float l = sm.lT[o];
            sm.qoT[o] = fq[e] * __expf(l);
            sm.koT[o] = fk[e] * __expf(sm.Lb[jb][c] - l);
          }
        }
      }
    }
    const int flags = sm.flags;  // final since the barrier after the prefix pass
    __syncthreads();
    if (n > 0) prefetch(n - 1);  // in flight while this chunk computes

    // ================= dA tiles (from dA^T = V dY^T) =================
    for (int pi = w; pi < NPAIR; pi += NW) {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4;
      int ib = 0, jb = pi;  // t block ib >= s block jb
      while (jb > ib) {
        jb -= ib + 1;
        ++ib;
      }
      const int s_row = jb * 16 + n16, t_col = ib * 16 + n16;
      f32x4_t acc;
      acc_zero(acc);
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const int c0 = ks * 32 + 8 * g;  // D = 16: lanes with c0 >= D feed zeros (the MFMA runs on the whole wave)
        const bool ok = c0 < D;
        mma(acc, masked(ld8(&sm.v[s_row][ok ? c0 : 0]), ok), ld8(&sm.dy[t_col][ok ? c0 : 0]));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = jb * 16 + 4 * g + r;
        sm.dA[t_col][s] = from_f32<TIn>((jb < ib || s <= t_col) ? acc[r] : 0.f);
      }
    }
    __syncthreads();

    // ================= dk, dq, dlog_f for channel cw =================
    // Results are staged in LDS regions whose contents are dead by then and
    // written out as whole rows (16-byte stores): the accumulator layout puts
    // one channel per lane, so direct stores would be scattered 2-byte writes.
    float u[NB][4];   // q dq - k dk at tokens 16i + 4g + r
    float vk[NB][4];  // dk
    float vq[NB][4];  // dq, then dlog_f
    {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
      PFrag<TIn> LP[KSD];  // Lam^T as B operand, j in accumulator order
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        Frag f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int jb = 2 * ks + (x >> 2);
          f.v[x] = (jb < CB) ? LamT[jb][x & 3] : 0.f;
        }
        LP[ks] = to_pfrag<TIn>(f);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f32x4_t dk;
        acc_zero(dk);
        const int s = j * 16 + n16;
        // inter: V[s][j'] Lam[cw][j']
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int j0 = 2 * ks * 16 + 4 * g;
          const int j1 = (2 * ks + 1 < CB) ? j0 + 16 : j0;
          mma(dk, ld4x2(&sm.v[s][j0], &sm.v[s][j1]), LP[ks]);
        }
        const float eG = __expf(sm.Pb[NB][cw] - sm.Pb[j + 1][cw]);
#pragma unroll
        for (int r = 0; r < 4; ++r) dk[r] *= eG;
        // intra: sum_{t >= 16j} dA^T[s][t] q_t e^{b_t - E_j}; the lane's 8 tokens lie
        // in block tb with factor e^{P_tb - P_{j+1}} (tb > j) or e^{-L_j} (tb == j)
        const bool direct = (flags >> j) & 1;
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
          if (ks * 32 + 32 > 16 * j) {
            const int tq0 = ks * 32 + 8 * g;
            const int tb = tq0 >> 4;
            const bool ok = tb >= j && tq0 < C && !(direct && tb == j);
            const int tbc = tb < NB ? tb : NB - 1;
            const float ex = (tb > j) ? sm.Pb[tbc][cw] - sm.Pb[j + 1][cw] : -sm.Lb[j][cw];
            const float gap = __expf(ok ? ex : 0.f);
            const int tqc = tbc * 16 + (tq0 & 15);
            const float4 q0 = ldf4(&sm.qoT[TT32<C>::at(cw, tqc)]);
            const float4 q1 = ldf4(&sm.qoT[TT32<C>::at(cw, tqc + 4)]);
            Frag fb;
            fb.v[0] = q0.x * gap; fb.v[1] = q0.y * gap; fb.v[2] = q0.z * gap; fb.v[3] = q0.w * gap;
            fb.v[4] = q1.x * gap; fb.v[5] = q1.y * gap; fb.v[6] = q1.z * gap; fb.v[7] = q1.w * gap;
            masked(fb, ok);
            mma_split(dk, ldcol8(&sm.dA[tqc][s], Cfg::LDA, ok), fb);
          }
        }
        const float4 l4 = ldf4(&sm.lT[TT32<C>::at(cw, j * 16 + 4 * g)]);
        const float4 k4 = ldf4(&sm.koT[TT32<C>::at(cw, j * 16 + 4 * g)]);
        const float ll[4] = {l4.x, l4.y, l4.z, l4.w};
        const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
        const float Lj = sm.Lb[j][cw];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ss = j * 16 + 4 * g + r;
          u[j][r] = -kk[r] * dk[r];  // k dk = (k e^{L_j - ell}) Z
          float val = dk[r] * __expf(Lj - ll[r]);
          if (direct && ss < len) {
            float a = 0.f;
            for (int t = ss; t < j * 16 + 16; ++t)
              a += to_f32(sm.dA[t][ss]) * to_f32(gq[tok(t0 + t) + cw]) * __expf(sm.lT[TT32<C>::at(cw, t)] - ll[r]);
            val += a;
            u[j][r] -= to_f32(gk[tok(t0 + ss) + cw]) * a;
          }
          vk[j][r] = val;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // every wave is done with V
    {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.v[j * 16 + 4 * g + r][cw] = from_f32<TIn>(vk[j][r]);
    }
    {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
      PFrag<TIn> SP[KSD];
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) SP[ks] = to_pfrag<TIn>(Sprev[ks]);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        f32x4_t dq;
        acc_zero(dq);
        const int t = i * 16 + n16;
        // inter: dY[t][j] S_prev[cw][j], j in the accumulator order of S_prev's fragment
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int j0 = 2 * ks * 16 + 4 * g;
          const int j1 = (2 * ks + 1 < CB) ? j0 + 16 : j0;  // D = 16: slots 4-7 meet zeros of S_prev
          mma(dq, ld4x2(&sm.dy[t][j0], &sm.dy[t][j1]), SP[ks]);
        }
        const float eP = __expf(sm.Pb[i][cw]);
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[r] *= eP;
        // intra: sum_s dA[t][s] k_s e^{P_i - b_s}, s < 16(i+1).  The 8 tokens of a
        // lane's slots lie in one 16-block sb; its factor is e^{P_i - P_{sb+1}}
        // (sb < i) or e^{-L_i} (sb == i).  Branch-free: invalid lanes are masked.
        const bool direct = (flags >> i) & 1;
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
          if (ks * 32 < 16 * (i + 1)) {
            const int s0 = ks * 32 + 8 * g;  // 8 tokens of one 16-block
            const int sb = s0 >> 4;
            const bool ok = sb <= i && !(direct && sb == i);
            const int sbc = sb < NB ? sb : NB - 1;
            const float ex = (sb < i) ? sm.Pb[i][cw] - sm.Pb[sbc + 1][cw] : -sm.Lb[i][cw];
            const float gap = __expf(ok ? ex : 0.f);
            const int s0c = sbc * 16 + (s0 & 15);
            const float4 k0 = ldf4(&sm.koT[TT32<C>::at(cw, s0c)]);
            const float4 k1 = ldf4(&sm.koT[TT32<C>::at(cw, s0c + 4)]);
            Frag fb;
            fb.v[0] = k0.x * gap; fb.v[1] = k0.y * gap; fb.v[2] = k0.z * gap; fb.v[3] = k0.w * gap;
            fb.v[4] = k1.x * gap; fb.v[5] = k1.y * gap; fb.v[6] = k1.z * gap; fb.v[7] = k1.w * gap;
            masked(fb, ok);
            mma_split(dq, ld8(&sm.dA[t][s0c]), fb);
          }
        }
        const float4 l4 = ldf4(&sm.lT[TT32<C>::at(cw, i * 16 + 4 * g)]);
        const float4 q4 = ldf4(&sm.qoT[TT32<C>::at(cw, i * 16 + 4 * g)]);
        const float ll[4] = {l4.x, l4.y, l4.z, l4.w};
        const float qq[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tt = i * 16 + 4 * g + r;
          u[i][r] += qq[r] * dq[r];  // q dq = (q e^{ell}) X
          float val = dq[r] * __expf(ll[r]);
          if (direct && tt < len) {
            float a = 0.f;
            for (int s = i * 16; s <= tt; ++s)
              a += to_f32(sm.dA[tt][s]) * to_f32(gk[tok(t0 + s) + cw]) * __expf(ll[r] - sm.lT[TT32<C>::at(cw, s)]);
            val += a;
            u[i][r] += to_f32(gq[tok(t0 + tt) + cw]) * a;
          }
          vq[i][r] = val;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // every wave is done with dA, lT, koT
    {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.sq[i * 16 + 4 * g + r][cw] = from_f32<TIn>(vq[i][r]);
    }
    {  // dlog_f: reverse cumulative sum of u inside the chunk, plus the carry
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
      float suf[NB][4], tot[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        float run = 0.f;
#pragma unroll
        for (int r = 3; r >= 0; --r) {
          run += u[i][r];
          suf[i][r] = run;
        }
        tot[i] = run;
      }
      float rest = carry;
#pragma unroll
      for (int i = NB - 1; i >= 0; --i) {
        float above = 0.f, blk = 0.f;
#pragma unroll
        for (int gp = 0; gp < 4; ++gp) {
          const float x = __shfl(tot[i], n16 + 16 * gp);
          blk += x;
          if (gp > g) above += x;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = i * 16 + 4 * g + r;
          vq[i][r] = suf[i][r] + above + rest;  // dq already staged: reuse its registers
        }
        rest += blk;
      }
    }

    {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.sl[i * 16 + 4 * g + r][cw] = from_f32<TIn>(vq[i][r]);
    }
    __syncthreads();
    {  // whole-row stores of dk, dq, dlog_f
      const int tid = opaque(threadIdx.x);
#pragma unroll
      for (int it = 0; it < Cfg::NVQ; ++it) {
        const int idx = tid + it * NT;
        const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
        if (idx < Cfg::VQ && row < len) {
          const size_t off = tok(t0 + row) + col;
          *(uint4 *)(gdk + off) = *(const uint4 *)&sm.v[row][col];
          *(uint4 *)(gdq + off) = *(const uint4 *)&sm.sq[row][col];
          *(uint4 *)(gdl + off) = *(const uint4 *)&sm.sl[row][col];
        }
      }
    }

    // ================= Lam^T <- e^{Gamma} Lam^T + dY^T (q e^b) =================
    {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
      const float eG = __expf(sm.Pb[NB][cw]);
      PFrag<TIn> fqh[KSC];  // (q e^b)^T fragments: column cw, k = token
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        const int tq0 = ks * 32 + 8 * g;
        const bool ok = tq0 < C;
        const int tqc = ok ? tq0 : 0;
        const float eP = __expf(sm.Pb[tqc >> 4][cw]);
        const float4 q0 = ldf4(&sm.qoT[TT32<C>::at(cw, tqc)]);
        const float4 q1 = ldf4(&sm.qoT[TT32<C>::at(cw, tqc + 4)]);
        Frag f;
        f.v[0] = q0.x * eP; f.v[1] = q0.y * eP; f.v[2] = q0.z * eP; f.v[3] = q0.w * eP;
        f.v[4] = q1.x * eP; f.v[5] = q1.y * eP; f.v[6] = q1.z * eP; f.v[7] = q1.w * eP;
        masked(f, ok);
        fqh[ks] = to_pfrag<TIn>(f);
      }
#pragma unroll
      for (int jb = 0; jb < CB; ++jb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) LamT[jb][r] *= eG;
        const int jrow = jb * 16 + n16;
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
          const int tq0 = ks * 32 + 8 * g;
          mma(LamT[jb], ldcol8(&sm.dy[tq0 < C ? tq0 : 0][jrow], Cfg::LDN, tq0 < C), fqh[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (n > 0) carry = rowsum(Sprev);
  }
  if (args.dh0) {
    const int lane = tid & 63, n16 = lane & 15, g = lane >> 4, cw = w * 16 + n16;
#pragma unroll
    for (int jb = 0; jb < CB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        args.dh0[(size_t)bh * SS + (size_t)cw * D + jb * 16 + 4 * g + r] = LamT[jb][r];
  }
}

// ------------------------------------------------------------------ value side
template <typename TIn, int D, int C>
__device__ __forceinline__ void bwd_value_side(const BwdArgs &args, typename BwdCfg<TIn, D, C>::SmemV &sm,
                                               int b, int h) {
  using Cfg = BwdCfg<TIn, D, C>;
  constexpr int NT = Cfg::NT, NB = Cfg::NB, CB = Cfg::CB, KSD = Cfg::KSD, KSC = Cfg::KSC,
                EPV = Cfg::EPV, NW = Cfg::NW, NPAIR = Cfg::NPAIR;
  const int T = args.T, H = args.H, N = args.N;
  const int bh = b * H + h;
  const int tid = threadIdx.x;
  const int w = tid >> 6;

  const TIn *gq = (const TIn *)args.q;
  const TIn *gk = (const TIn *)args.k;
  const TIn *gl = (const TIn *)args.log_f;
  const TIn *gdy = (const TIn *)args.dy;
  TIn *gdv = (TIn *)args.dv;
  const size_t SS = (size_t)D * D;
  auto tok = [&](int t) { return (((size_t)b * T + t) * H + h) * D; };

  // Lam: tile cb holds rows c = 16cb + 4g + r, column j = jw.
  f32x4_t Lam[CB];
  {
    const int lane = tid & 63, n16 = lane & 15, g = lane >> 4, jw = w * 16 + n16;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Lam[cb][r] = args.dht ? args.dht[(size_t)bh * SS + (size_t)(cb * 16 + 4 * g + r) * D + jw] : 0.f;
  }

  uint4 pq[Cfg::NVQ], pk[Cfg::NVQ], pd[Cfg::NVQ], pl[Cfg::NVQ];
  auto prefetch = [&](int n) {
    const int t0 = n * C;
    const int len = min(C, T - t0);
#pragma unroll
    for (int it = 0; it < Cfg::NVQ; ++it) {
      const int idx = tid + it * NT;
      const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
      uint4 z = make_uint4(0, 0, 0, 0);
      pq[it] = pk[it] = pd[it] = pl[it] = z;
      if (idx < Cfg::VQ && row < len) {
        const size_t off = tok(t0 + row) + col;
        pq[it] = *(const uint4 *)(gq + off);
        pk[it] = *(const uint4 *)(gk + off);
        pd[it] = *(const uint4 *)(gdy + off);
        pl[it] = *(const uint4 *)(gl + off);
      }
    }
  };
  prefetch(N - 1);

  for (int n = N - 1; n >= 0; --n) {
    const int t0 = n * C;
    const int len = min(C, T - t0);

    // ================= preparation =================
    __syncthreads();
    {
      const int tid = opaque(threadIdx.x);
#pragma unroll
      for (int it = 0; it < Cfg::NVQ; ++it) {
        const int idx = tid + it * NT;
        if (idx < Cfg::VQ) {
          const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
          *(uint4 *)&sm.dy[row][col] = pd[it];
          float f[EPV];
          Vec<TIn>::unpack(pl[it], f);
#pragma unroll
          for (int e = 0; e < EPV; e += 4)
            *(float4 *)&sm.l[row][col + e] =
                make_float4(floor_logf(f[e]), floor_logf(f[e + 1]), floor_logf(f[e + 2]), floor_logf(f[e + 3]));
        }
      }
      if (tid == 0) sm.flags = 0;
      __syncthreads();
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
          TIn oq[EPV], ok[EPV], oh[EPV];
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const int c = col + e;
            const float l = sm.l[row][c];
            const float ko = fk[e] * __expf(sm.Lb[jb][c] - l);
            const float qo = fq[e] * __expf(l);
            oq[e] = from_f32<TIn>(qo);
            ok[e] = from_f32<TIn>(ko);
            oh[e] = from_f32<TIn>(ko * __expf(sm.Pb[NB][c] - sm.Pb[jb + 1][c]));
            sm.qhT[TTile<TIn, C>::at(c, row)] = from_f32<TIn>(qo * __expf(sm.Pb[jb][c]));
          }
          *(uint4 *)&sm.qo[row][col] = *(const uint4 *)oq;
          *(uint4 *)&sm.ko[row][col] = *(const uint4 *)ok;
          *(uint4 *)&sm.kh[row][col] = *(const uint4 *)oh;
        }
      }
    }
    const int flags = sm.flags;  // final since the barrier after the prefix pass
    __syncthreads();
    if (n > 0) prefetch(n - 1);

    // ================= A tiles -> A^T =================
    for (int pi = w; pi < NPAIR; pi += NW) {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4;
      int ib = 0, jb = pi;  // t block ib >= s block jb
      while (jb > ib) {
        jb -= ib + 1;
        ++ib;
      }
      const int t_row = ib * 16 + n16, s_col = jb * 16 + n16;
      f32x4_t acc;
      acc_zero(acc);
      const bool direct = (jb == ib) && ((flags >> ib) & 1);
      if (!direct) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int c0 = ks * 32 + 8 * g;  // D = 16: lanes with c0 >= D feed zeros
          const bool ok = c0 < D;
          const int cc = ok ? c0 : 0;
          float kv[8];
          Vec<TIn>::unpack(*(const uint4 *)&sm.ko[s_col][cc], kv);
          if constexpr (EPV == 4) Vec<TIn>::unpack(*(const uint4 *)&sm.ko[s_col][cc + 4], kv + 4);
          const float4 g0 = ldf4(&sm.gp[pi][cc]);
          const float4 g1 = ldf4(&sm.gp[pi][cc + 4]);
          Frag fb;
          fb.v[0] = kv[0] * g0.x; fb.v[1] = kv[1] * g0.y; fb.v[2] = kv[2] * g0.z; fb.v[3] = kv[3] * g0.w;
          fb.v[4] = kv[4] * g1.x; fb.v[5] = kv[5] * g1.y; fb.v[6] = kv[6] * g1.z; fb.v[7] = kv[7] * g1.w;
          mma(acc, masked(ld8(&sm.qo[t_row][cc]), ok), to_pfrag<TIn>(fb));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = ib * 16 + 4 * g + r;
          float a = 0.f;
          if (s_col <= t && t < len)
            for (int c = 0; c < D; ++c)
              a += to_f32(gq[tok(t0 + t) + c]) * to_f32(gk[tok(t0 + s_col) + c]) *
                   __expf(sm.l[t][c] - sm.l[s_col][c]);
          acc[r] = a;
        }
      }
      // lane holds A[t = 16ib + 4g + r][s = s_col] -> A^T[s][t..t+3]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = ib * 16 + 4 * g + r;
        sm.At[s_col][t] = from_f32<TIn>((jb < ib || s_col <= t) ? acc[r] : 0.f);
      }
    }
    __syncthreads();

    // ================= dv for value column jw, then Lam update =================
    {
      const int lane = opaque(tid & 63), n16 = lane & 15, g = lane >> 4, jw = w * 16 + n16;
      PFrag<TIn> fdyT[KSC];  // dY^T fragments: column jw, k = token
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        const int tq0 = ks * 32 + 8 * g;
        fdyT[ks] = ldcol8(&sm.dy[tq0 < C ? tq0 : 0][jw], Cfg::LDN, tq0 < C);
      }
      PFrag<TIn> LP[KSD];  // Lam as B operand, channels in accumulator order
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        Frag f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int cb = 2 * ks + (x >> 2);
          f.v[x] = (cb < CB) ? Lam[cb][x & 3] : 0.f;
        }
        LP[ks] = to_pfrag<TIn>(f);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f32x4_t acc;
        acc_zero(acc);
        const int s = j * 16 + n16;
        // inter: (k e^{Gamma - b})[s][c] Lam[c][jw]
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int c0 = 2 * ks * 16 + 4 * g;
          const int c1 = (2 * ks + 1 < CB) ? c0 + 16 : c0;  // D = 16: slots 4-7 meet zeros of Lam
          mma(acc, ld4x2(&sm.kh[s][c0], &sm.kh[s][c1]), LP[ks]);
        }
        // intra: A^T[s][t] dY[t][jw], t >= 16j
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
          if (ks * 32 + 32 > 16 * j) {
            const int t0f = ks * 32 + 8 * g;
            const bool ok = t0f >= 16 * j && t0f < C;
            mma(acc, masked(ld8(&sm.At[s][ok ? t0f : 0]), ok), fdyT[ks]);
          }
        }
        // staged in ko (dead since the score tiles) and stored as whole rows below
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.ko[j * 16 + 4 * g + r][jw] = from_f32<TIn>(acc[r]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      {
        const int tid = opaque(threadIdx.x);
#pragma unroll
        for (int it = 0; it < Cfg::NVQ; ++it) {
          const int idx = tid + it * NT;
          const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
          if (idx < Cfg::VQ && row < len) *(uint4 *)(gdv + tok(t0 + row) + col) = *(const uint4 *)&sm.ko[row][col];
        }
      }
      // Lam[c][jw] <- e^{Gamma} Lam + sum_t (q e^b)[t][c] dY[t][jw]
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float4 g4 = ldf4(&sm.Pb[NB][cb * 16 + 4 * g]);
        Lam[cb][0] *= __expf(g4.x);
        Lam[cb][1] *= __expf(g4.y);
        Lam[cb][2] *= __expf(g4.z);
        Lam[cb][3] *= __expf(g4.w);
        const int crow = cb * 16 + n16;
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
          const int tq0 = ks * 32 + 8 * g;
          const bool ok = tq0 < C;
          mma(Lam[cb], masked(ldT8<C>(sm.qhT, crow, ok ? tq0 : 0), ok), fdyT[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <typename TIn, int D, int C>
__global__ __launch_bounds__(4 * D) void hgrn2_bwd_kernel(BwdArgs args) {
  using Cfg = BwdCfg<TIn, D, C>;
  __shared__ typename Cfg::Smem sm;
  // Work-group id -> (b, h, side).  The two sides of one (b, h) get ids that
  // differ by 8, so they land on the same XCD (workgroups are dealt to the
  // 8 XCDs round-robin) and share its L2 for the chunk tiles both read.
  const int bid = blockIdx.x;
  const int grp = bid >> 4, rem = bid & 15;
  const int side = rem >> 3;
  const int bh = grp * 8 + (rem & 7);
  if (bh >= args.B * args.H) return;
  const int b = bh / args.H, h = bh % args.H;
  if (side == 0)
    bwd_channel_side<TIn, D, C>(args, sm.c, b, h);
  else
    bwd_value_side<TIn, D, C>(args, sm.v, b, h);
}

template <typename TIn, int D, int C>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
  using Cfg = BwdCfg<TIn, D, C>;
  const int groups = (a.B * a.H + 7) / 8;
  hipLaunchKernelGGL((hgrn2_bwd_kernel<TIn, D, C>), dim3(groups * 16), dim3(Cfg::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hgrn2
