// Per-chunk gradients of the HGRN2 recurrence, resident variant for bfloat16
// at d = 128 and chunk 64 (gfx950).
//
// Computes exactly what cbwd.h computes (HGRN2 summary, paperlayer.ai, §3.2:
// the gated outer-product recurrence evaluated chunkwise, §3.2 p.5), with the
// same anchored exponents and the same consistently rounded dlog f, but lays
// the work out for a whole CU:
//   - one persistent 8-wave workgroup per CU walks chunks; the next chunk's
//     token rows are prefetched into registers while the current one computes,
//     in three groups spread over the chunk's phases (a single burst of every
//     load fills the CU's memory queues and stalls the waves that issue it);
//   - the chunk's token tiles (qo, ko, v, dy) and its initial state S and end
//     adjoint Lam are all resident in LDS at once.  S and Lam arrive by
//     asynchronous copies straight into LDS, issued when the chunk starts and
//     waited for only when the inter-chunk products need them;
//   - the 30 intra-chunk score tiles (dA and its transpose, and the decayed
//     scores A, for the 10 block pairs) are formed once, by whichever wave is
//     free, and shared through LDS as ready-made matrix-core operands;
//   - wave (w, hh) then owns the outputs of token block w for channel half hh
//     (products), and tokens 16 w + 8 hh .. + 7 for all channels (prefix and
//     epilogue).
// S and Lam are stored unpadded with each row's 16-byte chunks permuted by
// XOR with (row & 15), which the copy realises by permuting its source
// addresses; reads of 16 consecutive rows then never share a bank.  With tied
// gates (k = 1 - f) k is formed from log f, dk is not written, and dlog f is
// the total derivative G = dlog f - f dk; with the gate pre-activation as input
// the output is dz = G dlog f/dz and each chunk writes its token sums of
// G dlog f/dlb, f being recovered from the block-local prefix of log f.
#pragma once

#include "cbwd.h"

namespace hgrn2 {

struct CbwdResCfg {
  using T = bf16_t;
  static constexpr int D = 128, C = 64, NB = 4, NWV = 8, NT = 64 * NWV;
  static constexpr int LD = RowTile<T, D>::LD;
  static constexpr int LDG = D + 4;  // staging row stride (floats)
  static constexpr int NPAIR = NB * (NB + 1) / 2, NTILE = 3 * NPAIR;
  struct A {  // during the products
    T S[D * D];  // swizzled rows (see above)
    T L[D * D];
    union {
      uint2 sc[NTILE][64];  // score tiles, lane order: kind 0 dA^T, 1 dA, 2 A, then pair
      float Lh[NB][2][D];   // (before them) log f totals of each half block
    } x;
  };
  struct E {  // during the epilogues
    float stg[2][C][LDG];  // dq', dk'
    float tot[NWV][D];     // per-wave sums of q dq - k dk
    float cpart[NB][D];    // per-block sums of ko dk'_inter
    float rs[D];           // rowsum(S * Lam)
  };
  struct Smem {
    T qo[C * LD], ko[C * LD], v[C * LD], dy[C * LD];  // RowTile<T, D>
    union {
      A a;
      E e;
    } u;
    float Lb[NB][D];      // block totals of log f
    T gp[NB][NB][D];      // gap factor of a block pair (symmetric)
    float fac[NB][2][D];  // block w: e^{P_w}, e^{Gamma - P_{w+1}}
    float eG[D];          // e^Gamma
    float lbc[2][D];      // gate mode: lower bounds of this chunk and the next (by parity)
  };
};

// the swizzled position (in elements) of element col of row r of S or Lam
__device__ __forceinline__ int res_sw(int r, int col) {
  return r * 128 + ((((col >> 3) ^ (r & 15))) << 3) + (col & 7);
}

// 8 consecutive elements col0..col0+7 (col0 % 8 == 0) of row r as an operand fragment
__device__ __forceinline__ PFrag<bf16_t> res_row8(const bf16_t *m, int r, int col0) {
  return ld8(m + res_sw(r, col0));
}

// tr8 of a swizzled matrix: slots i <-> rows r0 + 8g + i, column n0 + n (r0 % 16 == 0)
__device__ __forceinline__ PFrag<bf16_t> res_tr8(const bf16_t *m, int r0, int n0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  union {
    v4s_t h[2];
    bf16x8_t v;
  } u;
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    const int r = r0 + 8 * g + 4 * hp + (i >> 2), col = n0 + 4 * (i & 3);
    u.h[hp] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s_t *)(m + res_sw(r, col)));
  }
  PFrag<bf16_t> f;
  f.x = u.v;
  return f;
}

__device__ __forceinline__ int res_pair_i(int p) { return p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0; }

// TO: the element type of the gradients (bfloat16, or float32)
template <int GM, typename TO = bf16_t>
__global__ __launch_bounds__(512) void hgrn2_chunk_bwd_res_kernel(ChunkBwdArgs a) {
  using Cfg = CbwdResCfg;
  using T = bf16_t;
  constexpr int D = Cfg::D, C = Cfg::C, NB = Cfg::NB, NWV = Cfg::NWV, NT = Cfg::NT, LDG = Cfg::LDG;
  using XT = RowTile<T, D>;
  __shared__ Cfg::Smem sm;

  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = wv >> 1, hh = wv & 1;
  const int H = a.H, T_ = a.T, N = a.N;
  const int NC = a.B * H * N;
  const uint32_t HDB = (uint32_t)H * D * sizeof(T);
  auto tok = [&](int t) { return (uint32_t)t * HDB; };

  struct Chunk {
    int bh, n, len;
    size_t cbase;
  };
  auto chunk_of = [&](int ci) {
    Chunk k;
    k.bh = ci / N;
    k.n = ci % N;
    const int b = k.bh / H, h = k.bh % H, t0 = k.n * C;
    k.len = min(C, T_ - t0);
    k.cbase = (((size_t)b * T_ + t0) * H + h) * D * sizeof(T);
    return k;
  };
  // the chunk's log decays: per channel, or one per head broadcast (kScalar)
  auto lfr = [&](const Chunk &k) {
    return lf_rows<GM, T>(a.log_f, k.bh / H, T_, H, k.bh % H, D, k.n * C, k.len);
  };
  auto win = [&](const void *base, const Chunk &k) {
    return GBuf((const char *)base + k.cbase, (uint32_t)k.len * HDB);
  };
  // the gradients' rows, of TO elements
  const uint32_t HDBO = (uint32_t)H * D * sizeof(TO);
  auto toko = [&](int t) { return (uint32_t)t * HDBO; };
  auto wino = [&](void *base, const Chunk &k) {
    return GBuf((char *)base + k.cbase / sizeof(T) * sizeof(TO), (uint32_t)k.len * HDBO);
  };

  // ---- register prefetch of a chunk's token rows, in groups: kPfTiles (v and
  // dy tiles; gate mode: the lower bounds), kPfK (k), kPfQL (q and log f)
  constexpr int kPfTiles = 1, kPfK = 2, kPfQL = 4, kPfAll = 7;
  // vector-memory loads a kPfTiles group and a kPfK group issue, at least
  constexpr int kPfLoads = 4 + (GM == kGate ? 1 : 0) + (reads_k(GM) ? 8 : 0);
  uint4 pv[2], pdy[2];               // tile vectors idx = tid + NT i: row idx >> 4, column 8 (idx & 15)
  Pack<T, 2> pq[8], pk[8], pl[8];    // tokens 16 w + 8 hh + t, channels c0, c0 + 1
  T pla;                             // kScalar: log a of token 16 w + 8 hh + (lane & 7)
  float plb[2];                      // gate mode: lower bounds of channels c0, c0 + 1
  auto prefetch = [&](int ci, int part) {
    // lane-dependent offsets are recomputed per use (never kept live across the loop)
    const int tid = opaque((int)threadIdx.x), c0 = 2 * (tid & 63);
    const Chunk k = chunk_of(ci);
    const GBuf bq = win(a.q, k), bv = win(a.v, k), bdy = win(a.dy, k);
    const LfRows<GM> bl = lfr(k);
    if (part & kPfTiles) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int idx = tid + NT * i;
        const uint32_t off = tok(idx >> 4) + (uint32_t)(idx & 15) * 16;
        pv[i] = bv.ld16(off);
        pdy[i] = bdy.ld16(off);
      }
      if constexpr (GM == kGate) {
        plb[0] = a.lb[(k.bh % H) * D + c0];
        plb[1] = a.lb[(k.bh % H) * D + c0 + 1];
      }
    }
    if constexpr (reads_k(GM)) {
      if (part & kPfK) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          pk[t] = win(a.k, k).template ldpack<T, 2>(tok(16 * w + 8 * hh + t) + (uint32_t)c0 * sizeof(T));
      }
    }
    if (part & kPfQL) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t off = tok(16 * w + 8 * hh + t) + (uint32_t)c0 * sizeof(T);
        pq[t] = bq.ldpack<T, 2>(off);
        if constexpr (GM != kScalar) pl[t] = bl.template ld<T, 2>(16 * w + 8 * hh + t, (uint32_t)c0 * sizeof(T));
      }
      if constexpr (GM == kScalar) pla = bl.template ld<T, 1>(16 * w + 8 * hh + (tid & 7), 0).v[0];
    }
  };

  const int G = gridDim.x;
  int ci = blockIdx.x;
  if (ci < NC) prefetch(ci, kPfAll);
  if constexpr (GM == kGate) {
    // the first chunk's lower bounds (later chunks': staged in P3 of the chunk before)
    if (ci < NC && wv == 0) {
      const int cc = 2 * (int)(threadIdx.x & 63);
      sm.lbc[0][cc] = plb[0];
      sm.lbc[0][cc + 1] = plb[1];
    }
  }
  // gate mode: a chunk's token sums of G dlog f/dlb, per wave in the dq'
  // staging rows 0..7 (written at the chunk's end), summed over the waves in
  // a fixed order by the first D threads once a barrier has passed: after the
  // next chunk's B0 (beside that chunk's prefix work, before its B1, after
  // which the copies into S may land there), and after the walk for the last
  auto dlb_out = [&](int cprev) {
    const int t = (int)threadIdx.x;
    if (t < D) {
      const Chunk kp = chunk_of(cprev);
      float acc = 0.f;
#pragma unroll
      for (int o = 0; o < NWV; ++o) acc += sm.u.e.stg[0][o][t];
      a.dlb[((size_t)kp.bh * N + kp.n) * D + t] = acc;
    }
  };
  int par = 0;  // parity of this workgroup's chunk count: the lbc slot of the current chunk
  for (; ci < NC; ci += G, par ^= 1) {
    const Chunk k = chunk_of(ci);
    __syncthreads();  // B0: the previous chunk's LDS reads are done
    // lane-dependent values are derived anew each chunk so that the compiler
    // does not hoist every address of the body out of the loop
    const int tid = opaque((int)threadIdx.x), lane = tid & 63, n16 = lane & 15, g = lane >> 4;
    const int c0 = 2 * lane;  // prep / epilogue channels c0, c0 + 1
    // gate mode: lower bounds of channels c0, c0 + 1 (prefetched with the
    // token rows and staged in LDS; read where they are used)
    auto lbs = [&](float *o) {
      const int cc = 2 * (opaque((int)threadIdx.x) & 63);
#pragma unroll
      for (int e = 0; e < 2; ++e) o[e] = GM == kGate ? sm.lbc[par][cc + e] : 0.f;
    };
    float lb2[2];
    lbs(lb2);
    if constexpr (GM == kGate) {
      if (ci != (int)blockIdx.x) dlb_out(ci - G);
    }

    // ---- P0a: v, dy tiles; half-block totals of log f
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + NT * i, row = idx >> 4, col = (idx & 15) * 8;
      *(uint4 *)&sm.v[XT::at(row, col)] = pv[i];
      *(uint4 *)&sm.dy[XT::at(row, col)] = pdy[i];
    }
    float l[8][2], Lw[2], hoff[2] = {0.f, 0.f};  // hoff: prefix before this wave's first token
    float kf[8][2];                                 // k of the tokens (loaded, or formed with log f)
    {
      float run[2] = {0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float lf;
          lf_k<GM>(pk[t].v[e], GM == kScalar ? readlane(pla, t) : pl[t].v[e], lb2[e],
                   16 * w + 8 * hh + t < k.len, lf, kf[t][e]);
          run[e] += lf;
          l[t][e] = run[e];
        }
      sm.u.a.x.Lh[w][hh][c0] = run[0];
      sm.u.a.x.Lh[w][hh][c0 + 1] = run[1];
    }
    __syncthreads();  // B1

    // ---- P0b: block-local prefix, qo and ko, block totals
    bool wide;
    {
      bool wd = false;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float first = sm.u.a.x.Lh[w][0][c0 + e];
        Lw[e] = first + sm.u.a.x.Lh[w][1][c0 + e];
        if (hh == 1) {
          hoff[e] = first;
#pragma unroll
          for (int t = 0; t < 8; ++t) l[t][e] += first;
        }
        wd |= -Lw[e] > kDiagLimit;
      }
      wide = __ballot(wd) != 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int tt = 16 * w + 8 * hh + t;
        Pack<T, 2> oq, ok;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          oq.v[e] = from_f32<T>(to_f32(pq[t].v[e]) * __expf(l[t][e]));
          ok.v[e] = from_f32<T>(kf[t][e] * __expf(Lw[e] - l[t][e]));
        }
        *(Pack<T, 2> *)&sm.qo[XT::at(tt, c0)] = oq;
        *(Pack<T, 2> *)&sm.ko[XT::at(tt, c0)] = ok;
      }
      if (hh == 0) {
        sm.Lb[w][c0] = Lw[0];
        sm.Lb[w][c0 + 1] = Lw[1];
      }
    }
    // ---- S and Lam: asynchronous copies straight into LDS (issued after the
    // prefetched registers are consumed, before the next prefetch, so that no
    // wait of the compiler's for a register load also waits for them, and the
    // wait for the copies need not wait for the prefetch).  Wave wv copies
    // rows 32 (wv % 4) .. + 31 of S (wv < 4) or Lam (wv >= 4), four rows of
    // 256 bytes per instruction; lane i lands in chunk i % 16 of row 4 j + i / 16
    // and fetches the logical chunk that the swizzle puts there.
    {
      const bool isL = wv >= 4;
      const T *src = isL ? (const T *)a.lam + ((size_t)k.bh * N + k.n) * D * D
                         : (const T *)a.states + ((size_t)k.bh * (N + 1) + k.n) * D * D;
      const GBuf bs(src, D * D * sizeof(T));
      T *dst = isL ? sm.u.a.L : sm.u.a.S;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 32 * (wv & 3) + 4 * j + (lane >> 4);
        const int q = (lane & 15) ^ (r & 15);
        lds_dma16(bs, (uint32_t)(r * D + 8 * q) * sizeof(T), dst + (32 * (wv & 3) + 4 * j) * D);
      }
    }
    __syncthreads();  // B2

    // ---- P0c: gap factors of block w with blocks 2 hh, 2 hh + 1; e^{P_w} (hh = 0)
    // or e^{Gamma - P_{w+1}} (hh = 1); e^Gamma
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = c0 + e;
      float P[NB + 1];
      P[0] = 0.f;
#pragma unroll
      for (int i = 0; i < NB; ++i) P[i + 1] = P[i] + sm.Lb[i][c];
      float Pw = 0.f, Pw1 = 0.f;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        Pw = (i == w) ? P[i] : Pw;
        Pw1 = (i == w) ? P[i + 1] : Pw1;
      }
      const float G_ = P[NB];
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int m = 2 * hh + mm;
        float x;
        if (m < w) x = Pw - P[m + 1];
        else if (m == w) x = fminf(-(Pw1 - Pw), 80.f);
        else x = P[m] - Pw1;
        sm.gp[w][m][c] = from_f32<T>(__expf(x));
      }
      sm.fac[w][hh][c] = __expf(hh == 0 ? Pw : G_ - Pw1);
      if (wv == 0) sm.eG[c] = __expf(G_);
    }
    __syncthreads();  // B3
    // the registers are free: the next chunk's v and dy tiles (and lower bounds)
    if (ci + G < NC) prefetch(ci + G, kPfTiles);

    const T *qo = sm.qo, *ko = sm.ko, *tv = sm.v, *tdy = sm.dy;
    // ---- P1: the score tiles, tile id = wv + 8 s
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int tau = wv + NWV * s4;
      if (tau >= Cfg::NTILE) break;
      const int kind = tau / Cfg::NPAIR, p = tau % Cfg::NPAIR;
      const int i = res_pair_i(p), j = p - i * (i + 1) / 2;  // block i >= block j
      f32x4_t X;
      acc_zero(X);
      if (kind == 0) {  // dA^T: rows s in j, columns t in i
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          mma(X, row8<D>(tv, 16 * j + n16, 32 * ks + 8 * g), row8<D>(tdy, 16 * i + n16, 32 * ks + 8 * g));
        if (i == j) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g + r > n16) X[r] = 0.f;  // s > t
        }
      } else if (kind == 1) {  // dA: rows t in i, columns s in j
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          mma(X, row8<D>(tdy, 16 * i + n16, 32 * ks + 8 * g), row8<D>(tv, 16 * j + n16, 32 * ks + 8 * g));
        if (i == j) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g + r < n16) X[r] = 0.f;  // t < s
        }
      } else {  // A = qo_i (ko_j gap)^T: rows t in i, columns s in j
        bool wide_i = false;
        if (i == j) wide_i = __ballot(-sm.Lb[i][c0] > kDiagLimit || -sm.Lb[i][c0 + 1] > kDiagLimit) != 0;
        if (i == j + 1) {
          // adjacent blocks: the gap factor is e^{P_i - P_i} = 1 exactly
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            mma(X, row8<D>(qo, 16 * i + n16, 32 * ks + 8 * g), row8<D>(ko, 16 * j + n16, 32 * ks + 8 * g));
        } else if (!wide_i) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int cc = 32 * ks + 8 * g;
            float kv[8], gv[8];
            unpack8(row8<D>(ko, 16 * j + n16, cc), kv);
            unpack8(ld8(&sm.gp[i][j][cc]), gv);
            Frag fb;
#pragma unroll
            for (int e = 0; e < 8; ++e) fb.v[e] = kv[e] * gv[e];
            mma(X, row8<D>(qo, 16 * i + n16, cc), to_pfrag<T>(fb));
          }
          if (i == j) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (4 * g + r < n16) X[r] = 0.f;
          }
        } else {
          // wide in-block decay: A[t][s] summed directly (every exponent <= 0)
          const GBuf bq = win(a.q, k);
          const LfRows<GM> bl = lfr(k);
          float lb2[2];
          lbs(lb2);
          for (int t = 0; t < 16; ++t) {
            const Pack<T, 2> pt = bq.ldpack<T, 2>(tok(16 * i + t) + (uint32_t)c0 * sizeof(T));
            float ex[2] = {0.f, 0.f};
            for (int s = t; s >= 0; --s) {
              const uint32_t off = tok(16 * i + s) + (uint32_t)c0 * sizeof(T);
              const Pack<T, 2> pls = bl.template ld<T, 2>(16 * i + s, (uint32_t)c0 * sizeof(T));
              Pack<T, 2> pks;
              if constexpr (reads_k(GM)) pks = win(a.k, k).template ldpack<T, 2>(off);
              float part = 0.f;
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                part += to_f32(pt.v[e]) * k_of<GM>(pks.v[e], lfe<GM>(pls, e), lb2[e]) * __expf(ex[e]);
                ex[e] += lf_of<GM>(to_f32(lfe<GM>(pls, e)), lb2[e], 16 * i + s < k.len);
              }
              const float tot = wave_sum(part);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n16 == s && 4 * g + r == t) X[r] = tot;
            }
          }
        }
      }
      sm.u.a.x.sc[tau][lane] = __builtin_bit_cast(uint2, acc_to_frag4<T>(X).x);
    }
    __syncthreads();  // B4
    if (ci + G < NC) prefetch(ci + G, kPfK);

    // ---- P2: intra-chunk products of block w, channel half hh
    auto sc_frag = [&](int kind, int i, int j) {
      PFrag4<T> f;
      f.x = __builtin_bit_cast(v4s_t, sm.u.a.x.sc[kind * Cfg::NPAIR + i * (i + 1) / 2 + j][lane]);
      return f;
    };
    f32x4_t DQ[4], DK[4], DV[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      acc_zero(DQ[cb]);
      acc_zero(DK[cb]);
      acc_zero(DV[cb]);
    }
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      if (m <= w && !(m == w && wide)) {  // dq' += gap (dA ko) over pair (w, m)
        const PFrag4<T> fa = sc_frag(0, w, m);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int cc = 64 * hh + 16 * cb;
          f32x4_t tmp;
          acc_zero(tmp);
          mma16(tmp, fa, tr4<D>(ko, 16 * m, cc, lane));
          const float gpf = to_f32(sm.gp[w][m][cc + n16]);
#pragma unroll
          for (int r = 0; r < 4; ++r) DQ[cb][r] += gpf * tmp[r];
        }
      }
      if (m >= w) {
        if (!(m == w && wide)) {  // dk' += gap (dA^T qo) over pair (m, w)
          const PFrag4<T> fa = sc_frag(1, m, w);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const int cc = 64 * hh + 16 * cb;
            f32x4_t tmp;
            acc_zero(tmp);
            mma16(tmp, fa, tr4<D>(qo, 16 * m, cc, lane));
            const float gpf = to_f32(sm.gp[m][w][cc + n16]);
#pragma unroll
            for (int r = 0; r < 4; ++r) DK[cb][r] += gpf * tmp[r];
          }
        }
        const PFrag4<T> fa = sc_frag(2, m, w);  // dv += A^T dy over pair (m, w)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) mma16(DV[cb], fa, tr4<D>(tdy, 16 * m, 64 * hh + 16 * cb, lane));
      }
    }

    // ---- P3: inter-chunk products (S and Lam must have landed)
    // this wave's copies are in LDS: vector-memory operations complete in issue
    // order, and at least kPfLoads loads were issued after the copies
    if (ci + G < NC) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPfLoads) : "memory");
    } else {
      vm_drain();
    }
    __syncthreads();  // B5: and every other wave's
    if constexpr (GM == kGate) {
      // the next chunk's lower bounds into the other slot (read after the next B0)
      if (wv == 0 && ci + G < NC) {
        sm.lbc[par ^ 1][c0] = plb[0];
        sm.lbc[par ^ 1][c0 + 1] = plb[1];
      }
    }
    const T *sS = sm.u.a.S, *sL = sm.u.a.L;
    float rsv = 0.f, cp[4];
    f32x4_t tq[4], tk[4], dg;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      acc_zero(tq[cb]);
      acc_zero(tk[cb]);
    }
    acc_zero(dg);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int j = 32 * ks + 8 * g;
      const PFrag<T> fdy = row8<D>(tdy, 16 * w + n16, j), fv = row8<D>(tv, 16 * w + n16, j);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int c = 64 * hh + 16 * cb + n16;
        const PFrag<T> sf = res_row8(sS, c, j), lf = res_row8(sL, c, j);
        mma(tq[cb], fdy, sf);
        mma(tk[cb], fv, lf);
        if (cb == w) mma(dg, sf, lf);
      }
    }
    {
      const int r = n16 & 3;
      rsv = (r == 0) ? dg[0] : (r == 1) ? dg[1] : (r == 2) ? dg[2] : dg[3];
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int c = 64 * hh + 16 * cb + n16;
      const float eP = sm.fac[w][0][c], eK = sm.fac[w][1][c];
      float ckp = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        DQ[cb][r] += eP * tq[cb][r];
        const float x = eK * tk[cb][r];
        DK[cb][r] += x;
        ckp += to_f32(ko[XT::at(16 * w + 4 * g + r, c)]) * x;  // ko as it entered the products
      }
      cp[cb] = group_sum(ckp);
    }
    // dv += kh Lam with kh = ko e^{Gamma - P_{w+1}} (Lam rows as k)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cc = 32 * ks + 8 * g;
      float kv[8];
      unpack8(row8<D>(ko, 16 * w + n16, cc), kv);
      const float4 e0 = ldf4(&sm.fac[w][1][cc]), e1 = ldf4(&sm.fac[w][1][cc + 4]);
      Frag f;
      f.v[0] = kv[0] * e0.x; f.v[1] = kv[1] * e0.y; f.v[2] = kv[2] * e0.z; f.v[3] = kv[3] * e0.w;
      f.v[4] = kv[4] * e1.x; f.v[5] = kv[5] * e1.y; f.v[6] = kv[6] * e1.z; f.v[7] = kv[7] * e1.w;
      const PFrag<T> khA = to_pfrag<T>(f);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) mma(DV[cb], khA, res_tr8(sL, 32 * ks, 64 * hh + 16 * cb, lane));
    }
    __syncthreads();  // B6: S, Lam, the score tiles, v and dy are dead
    if (ci + G < NC) prefetch(ci + G, kPfQL);

    // ---- P4: dv out (staged through the dead v tile, or float32 straight
    // from the accumulators), dq' and dk' staging
    if constexpr (std::is_same<TO, T>::value) {
      const GBuf bdv = win(a.dv, k);
      T *dvs = sm.v;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dvs[XT::at(16 * w + 4 * g + r, 64 * hh + 16 * cb + n16)] = from_f32<T>(DV[cb][r]);
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int idx = lane + 64 * i, t = 16 * w + (idx >> 3), col = 64 * hh + 8 * (idx & 7);
        bdv.st16<kStream>(tok(t) + (uint32_t)col * sizeof(T), *(const uint4 *)&dvs[XT::at(t, col)]);
      }
    } else {
      const GBuf bdv = wino(a.dv, k);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Pack<TO, 1> o;
          o.v[0] = DV[cb][r];
          bdv.stpack<TO, 1, kStream>(toko(16 * w + 4 * g + r) + (uint32_t)(64 * hh + 16 * cb + n16) * sizeof(TO), o);
        }
    }
    auto &ep = sm.u.e;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ep.stg[0][16 * w + 4 * g + r][64 * hh + 16 * cb + n16] = DQ[cb][r];
        ep.stg[1][16 * w + 4 * g + r][64 * hh + 16 * cb + n16] = DK[cb][r];
      }
    if (g == 0) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) ep.cpart[w][64 * hh + 16 * cb + n16] = cp[cb];
    }
    if (g == (n16 >> 2)) ep.rs[64 * hh + 16 * w + n16] = rsv;
    __syncthreads();  // B7

    // ---- P5: per token (tokens 16 w + 8 hh + t, channels c0, c0 + 1): dq = e^{ell} dq',
    // dk = e^{L - ell} dk', X = qo dq' - ko dk' with qo, ko as they entered the products
    const GBuf bdq = wino(a.dq, k), bdk = wino(a.dk, k);
    float X[8][2];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int tt = 16 * w + 8 * hh + t;
      const Pack<T, 2> qr = *(const Pack<T, 2> *)&qo[XT::at(tt, c0)];
      const Pack<T, 2> kr = *(const Pack<T, 2> *)&ko[XT::at(tt, c0)];
      const float2 d1 = *(const float2 *)&ep.stg[0][tt][c0], d2 = *(const float2 *)&ep.stg[1][tt][c0];
      const float dd1[2] = {d1.x, d1.y}, dd2[2] = {d2.x, d2.y};
      Pack<TO, 2> oq, ok;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float el = __expf(l[t][e]), ek = __expf(Lw[e] - l[t][e]);
        oq.v[e] = from_f32<TO>(el * dd1[e]);
        ok.v[e] = from_f32<TO>(ek * dd2[e]);
        X[t][e] = to_f32(qr.v[e]) * dd1[e] - to_f32(kr.v[e]) * dd2[e];
        // k tied to f: f dk (f from the prefix), subtracted from dlog f in P6;
        // it replaces the consumed dk'_t
        if (ties_k(GM) && !wide)
          ep.stg[1][tt][c0 + e] = __expf(l[t][e] - (t ? l[t - 1][e] : hoff[e])) * (ek * dd2[e]);
      }
      if (!wide) {
        bdq.stpack<TO, 2, kStream>(toko(tt) + (uint32_t)c0 * sizeof(TO), oq);
        if constexpr (reads_k(GM)) bdk.stpack<TO, 2, kStream>(toko(tt) + (uint32_t)c0 * sizeof(TO), ok);
      }
    }
    if (wide) {
      // diagonal block summed directly: dq_t adds sum_{s <= t} dA[t][s] k_s e^{ell_t - ell_s},
      // dk_t adds sum_{u >= t} dA[u][t] q_u e^{ell_u - ell_t} (every exponent <= 0)
      const GBuf bq = win(a.q, k), bv = win(a.v, k), bdy = win(a.dy, k);
      const LfRows<GM> bl = lfr(k);
      const uint32_t cb2 = (uint32_t)c0 * sizeof(T);
      float lb2[2];
      lbs(lb2);
      for (int t = 0; t < 8; ++t) {
        const int tb = 8 * hh + t, tt = 16 * w + tb;
        const Pack<T, 2> pqt = bq.ldpack<T, 2>(tok(tt) + cb2), plt = bl.template ld<T, 2>(tt, cb2);
        Pack<T, 2> pkt;
        if constexpr (reads_k(GM)) pkt = win(a.k, k).template ldpack<T, 2>(tok(tt) + cb2);
        const Pack<T, 2> pdy = bdy.ldpack<T, 2>(tok(tt) + cb2), pvt = bv.ldpack<T, 2>(tok(tt) + cb2);
        float dqd[2] = {0.f, 0.f}, dkd[2] = {0.f, 0.f}, ex[2] = {0.f, 0.f};
        for (int s_ = tb; s_ >= 0; --s_) {
          const uint32_t off = tok(16 * w + s_) + cb2;
          const Pack<T, 2> pvs = bv.ldpack<T, 2>(off), pls = bl.template ld<T, 2>(16 * w + s_, cb2);
          Pack<T, 2> pks;
          if constexpr (reads_k(GM)) pks = win(a.k, k).template ldpack<T, 2>(off);
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 2; ++e) part += to_f32(pdy.v[e]) * to_f32(pvs.v[e]);
          const float dA = wave_sum(part);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            dqd[e] += dA * k_of<GM>(pks.v[e], lfe<GM>(pls, e), lb2[e]) * __expf(ex[e]);
            ex[e] += lf_of<GM>(to_f32(lfe<GM>(pls, e)), lb2[e], 16 * w + s_ < k.len);
          }
        }
        ex[0] = ex[1] = 0.f;
        for (int u = tb; u < 16; ++u) {
          const uint32_t off = tok(16 * w + u) + cb2;
          const Pack<T, 2> pdu = bdy.ldpack<T, 2>(off), pqu = bq.ldpack<T, 2>(off);
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 2; ++e) part += to_f32(pdu.v[e]) * to_f32(pvt.v[e]);
          const float dA = wave_sum(part);
          if (u > tb) {
            const Pack<T, 2> plu = bl.template ld<T, 2>(16 * w + u, cb2);
#pragma unroll
            for (int e = 0; e < 2; ++e) ex[e] += lf_of<GM>(to_f32(lfe<GM>(plu, e)), lb2[e], 16 * w + u < k.len);
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) dkd[e] += dA * to_f32(pqu.v[e]) * __expf(ex[e]);
        }
        const float2 d1 = *(const float2 *)&ep.stg[0][tt][c0], d2 = *(const float2 *)&ep.stg[1][tt][c0];
        const float dd1[2] = {d1.x, d1.y}, dd2[2] = {d2.x, d2.y};
        Pack<TO, 2> oq, ok;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float el = __expf(l[t][e]), ek = __expf(Lw[e] - l[t][e]);
          oq.v[e] = from_f32<TO>(el * dd1[e] + dqd[e]);
          ok.v[e] = from_f32<TO>(ek * dd2[e] + dkd[e]);
          X[t][e] += to_f32(pqt.v[e]) * dqd[e] - k_of<GM>(pkt.v[e], lfe<GM>(plt, e), lb2[e]) * dkd[e];
          if (ties_k(GM))
            ep.stg[1][tt][c0 + e] = __expf(lf_of<GM>(to_f32(lfe<GM>(plt, e)), lb2[e], tt < k.len)) * (ek * dd2[e] + dkd[e]);
        }
        bdq.stpack<TO, 2, kStream>(toko(tt) + (uint32_t)c0 * sizeof(TO), oq);
        if constexpr (reads_k(GM)) bdk.stpack<TO, 2, kStream>(toko(tt) + (uint32_t)c0 * sizeof(TO), ok);
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float s_ = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) s_ += X[t][e];
      ep.tot[wv][c0 + e] = s_;
    }
    __syncthreads();  // B8: tot, cpart, rs complete

    // ---- P6: dlog f = reverse cumulative sum of X within the chunk + carry;
    // k tied to f subtracts f dk; gate mode turns that total G into dz and sums
    // G dlog f/dlb over the chunk's tokens
    {
      const GBuf bdl = wino(a.dlog_f, k);
      // per-head decay: dlog a [B,T,H], one value per token
      const GBuf bda((char *)a.dlog_f + (((size_t)(k.bh / H) * T_ + k.n * C) * H + k.bh % H) * sizeof(TO),
                     (uint32_t)(k.len * H * sizeof(TO)));
      float carry[2], dlbs[2] = {0.f, 0.f}, lb2[2];
      lbs(lb2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = c0 + e;
        carry[e] = sm.eG[c] * ep.rs[c];
#pragma unroll
        for (int i = 0; i < NB; ++i) carry[e] += ep.cpart[i][c];
#pragma unroll
        for (int o = 0; o < NWV; ++o) carry[e] += (o > wv) ? ep.tot[o][c] : 0.f;
      }
      float gsum[8];  // kScalar: each token's G summed over this lane's two channels
      // one token: its total G, then (gate mode) dz and its dlb term
      auto emit = [&](int t, const GateGrad *gg) {
        const int tt = 16 * w + 8 * hh + t;
        Pack<TO, 2> o;
        float gs = 0.f;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          carry[e] += X[t][e];
          float G = ties_k(GM) ? carry[e] - ep.stg[1][tt][c0 + e] : carry[e];
          if constexpr (GM == kGate) {
            if (tt < k.len) dlbs[e] += G * gg[e].dlb;
            G *= gg[e].dz;
          }
          o.v[e] = from_f32<TO>(G);
          gs += G;
        }
        if constexpr (GM == kScalar) {
          gsum[t] = gs;
        } else {
          bdl.stpack<TO, 2, kStream>(toko(tt) + (uint32_t)c0 * sizeof(TO), o);
        }
      };
      if (GM != kGate || !wide) {
        // f of each token from the block-local prefix of log f
#pragma unroll
        for (int t = 7; t >= 0; --t) {
          GateGrad gg[2];
          if constexpr (GM == kGate) {
#pragma unroll
            for (int e = 0; e < 2; ++e) gg[e] = gate_grad_lf(l[t][e] - (t ? l[t - 1][e] : hoff[e]), lb2[e]);
          }
          emit(t, gg);
        }
      } else {
        // a directly summed block: f from z itself
        for (int t = 7; t >= 0; --t) {
          const Pack<T, 2> pz =
              win(a.log_f, k).template ldpack<T, 2>(tok(16 * w + 8 * hh + t) + (uint32_t)c0 * sizeof(T));
          GateGrad gg[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) gg[e] = gate_grad(to_f32(pz.v[e]), lb2[e]);
          emit(t, gg);
        }
      }
      if constexpr (GM == kScalar) {
        // dlog a of the wave's eight tokens: the sums over the head's 128
        // channels, all eight reduced across the wave together.  Each exchange
        // over lane bit 5, 4, 3 hands half of the tokens still held to the
        // partner lane and adds the partner's half, so that lane bits 5..3
        // name the token left; the last three exchanges sum the rest.
        const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
        float v4[4], v2[2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v4[i] = (b5 ? gsum[i + 4] : gsum[i]) + __shfl_xor(b5 ? gsum[i] : gsum[i + 4], 32, 64);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          v2[i] = (b4 ? v4[i + 2] : v4[i]) + __shfl_xor(b4 ? v4[i] : v4[i + 2], 16, 64);
        float tot = (b3 ? v2[1] : v2[0]) + __shfl_xor(b3 ? v2[0] : v2[1], 8, 64);
        tot += __shfl_xor(tot, 4, 64);
        tot += __shfl_xor(tot, 2, 64);
        tot += __shfl_xor(tot, 1, 64);
        if ((lane & 7) == 0) {
          Pack<TO, 1> oa;
          oa.v[0] = from_f32<TO>(tot);
          bda.stpack<TO, 1, kStream>((uint32_t)(16 * w + 8 * hh + (lane >> 3)) * H * sizeof(TO), oa);
        }
      }
      if constexpr (GM == kGate) {
        // per-wave sums into the consumed dq' staging (dlb_out sums them)
        ep.stg[0][wv][c0] = dlbs[0];
        ep.stg[0][wv][c0 + 1] = dlbs[1];
      }
    }
  }
  if constexpr (GM == kGate) {
    // the last chunk's lower-bound sums
    if ((int)blockIdx.x < NC) {
      __syncthreads();
      dlb_out(ci - G);
    }
  }
}

// One persistent workgroup per compute unit: gfx950 parts have 256.  The walk
// over chunks strides by the grid and does not depend on how many workgroups
// are resident at once, so no device query is needed at launch.
constexpr int kResGrid = 256;
inline int res_grid(int nchunks) { return nchunks < kResGrid ? nchunks : kResGrid; }

template <int GM, typename TO = bf16_t>
hipError_t launch_chunk_bwd_res(const ChunkBwdArgs &a, hipStream_t stream) {
  const int nc = a.B * a.H * a.N;
  hipLaunchKernelGGL((hgrn2_chunk_bwd_res_kernel<GM, TO>), dim3(res_grid(nc)), dim3(CbwdResCfg::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hgrn2
