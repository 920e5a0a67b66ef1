// Forward without stored chunk-boundary states (gfx950): the sequence of every
// (batch, head) is cut into P segments of G chunks; each workgroup walks one
// segment's chunks in order, carrying the d x d state in float32 matrix-core
// accumulators, and writes y.  Nothing per chunk goes to memory.
//
// HGRN2 summary (paperlayer.ai) §3.2: S_t = Diag(f_t) S_{t-1} + k_t^T v_t,
// y_t = q_t S_t; §3.2 p.5: evaluated chunk by chunk in the linear-attention
// form.  Within chunk n, with the in-chunk inclusive prefix b of log f and
// its total Gamma,
//   y_t  = sum_{s <= t in chunk} (sum_c q_t[c] k_s[c] e^{b_t[c] - b_s[c]}) v_s + (q_t e^{b_t}) S
//   S   <- Diag(e^Gamma) S + sum_t Diag(e^{Gamma - b_t}) k_t^T v_t.
// The state entering segment p is the carry of the segment summaries (the
// end state of every earlier segment from a zero state, written by the state
// scan in segment mode, and the segments' total log decays), from h0:
//   S_in(0) = h0,  S_in(p + 1) = Diag(e^{a_p}) S_in(p) + S_loc(p)
// (hgrn2_seg_carry_kernel).  P = 1 needs no summaries: one pass reads every
// input once, writes y once, and the final state.
//
// Layout: one workgroup of 2 C / 16 waves per (b, h, segment), two per SIMD
// at chunk 64.  Wave (w, hh) forms the prefix of 16-token sub-block w (both
// waves of a block do), writes qo = q e^{ell}, ko = k e^{L_w - ell} and
// kh = k e^{Gamma - b_t} of the block's half hh of tokens (block-local
// prefixes ell, totals L_j, starts P_j, as the per-chunk forward), forms one
// or two of the 10 score tiles (with the gap factors between blocks, and the
// diagonal summed directly when a block decays more than kDiagLimit nats),
// which are shared through LDS, then y of block w for column half hh, and the
// state tiles S^T[16 jb.., 16 cb..] with index wv + 8 i:
//   S^T <- S^T Diag(e^Gamma) + v^T kh.
// The state's copy in the input dtype in LDS feeds the next chunk's
// inter-chunk product.
//
// bfloat16 at d = 128, chunk 64, when two workgroups per compute unit walk
// at once (PAIR, giving ACC): the state stays in the accumulators
// as S itself, wave wv holding columns 16 wv .. 16 wv + 15 for every row.  An
// accumulator tile is then already a 16-deep operand along the rows of S, so
// the inter-chunk product reads it from registers (rows scaled by e^{P_w})
// and no copy of S goes through LDS.  Each wave then writes y's column tile wv
// for all four token blocks, staged in the (dead) ko tile for full-row stores.
// The v tile arrives by asynchronous copies straight into LDS when its chunk
// starts (held in registers from the chunk before, it was spilled at this
// register budget).  Without the copy and the e^{-L} table the tiles fit in 80 KB, so two
// workgroups share a compute unit and hide each other's barriers and latency
// (at 128 registers per lane: lane-dependent values are derived anew in the
// walk so that the compiler does not keep their addresses live).
#pragma once

#include <algorithm>

#include "cfwd.h"

namespace hgrn2 {

struct SegFwdArgs {
  int B, T, H, N;                 // N chunks per sequence
  int P, G;                       // segments per (b, h), chunks per segment
  const void *q, *k, *v, *log_f;  // [B,T,H,D]; log_f holds the gate pre-activation in gate mode
  const float *lb;                // gate mode: lower bound of f, [H,D]
  const float *h0;                // P = 1: [B,H,D,D] float32 or null (zero), the initial state
  const float *sin;               // P > 1: [B,H,P,D,D] float32, entry p = the state entering segment p
  void *y;                        // [B,T,H,D], the input dtype or (out_f32) float32
  float *ht;                      // [B,H,D,D] float32 final state, or null
  int out_f32 = 0;                // bfloat16 inputs: write y as float32
  int pair = 0;                   // two workgroups per compute unit walk at once (the ACC layout, where it exists)
};

template <typename T, int D, int C, bool PAIR = false> struct SfwdCfg {
  static constexpr int NB = C / 16;             // 16-token sub-blocks
  static constexpr int NWV = 2 * NB, NT = 64 * NWV;
  static constexpr int CPL = D > 64 ? D / 64 : 1;
  static constexpr int LANES = D / CPL;
  static constexpr int JB = D / 16, CB = D / 16;
  static constexpr int KSD = D / 32;
  static constexpr int HC = D / 2 / 16;         // column tiles of one wave's half of y
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int NPAIR = NB * (NB + 1) / 2;
  static constexpr int VV = C * D / EPV, NVV = (VV + NT - 1) / NT;
  static constexpr int NTILE = JB * CB, TPW = (NTILE + NWV - 1) / NWV;  // state tiles per wave
  static constexpr int LD = RowTile<T, D>::LD;
  static_assert(D >= 32 && HC >= 1, "two column halves of at least one tile");
  // the state in the accumulators as S, for two workgroups per compute unit
  static constexpr bool ACC = PAIR && std::is_same<T, bf16_t>::value && D == 128 && C == 64;
  // kh (and, without ACC, v) is read only by transposing reads (8 rows of 32
  // bytes per instruction), which a 32-byte row padding keeps free of bank
  // conflicts; ACC has the LDS for it.  With ACC the v tile is unpadded and
  // permuted instead (sfwd_vsw), as its asynchronous copy into LDS needs.
  static constexpr int PV = ACC ? 32 : 16;
  static constexpr int LDV = RowTile<T, D, PV>::LD;
  using Sc = PFrag4<T>;  // one lane's piece of a score tile as a 16-deep operand
  struct Smem {
    T qo[C * LD];  // RowTile<T, D>; after the products, each wave's y staging
    T ko[C * LD];  // ACC: after the scores, y's staging
    T kh[C * LDV];  // k e^{Gamma - b_t}: the state update's operand
    T v[C * LDV];   // ACC: the first C * D elements, in the sfwd_vsw layout
    alignas(16) T S[ACC ? 8 : D * LD];  // copy of the state entering the chunk, row c, column j (not with ACC)
    alignas(16) Sc sc[NPAIR][64];
    alignas(16) float eL[NB][D];        // e^{L_w}, each block's decay
    alignas(16) float eLd[ACC ? 1 : NB][ACC ? 4 : D];  // e^{-L_w}, at most e^{80} (ACC: 1 / e^{L_w})
    alignas(16) float eP[NB][D];        // e^{P_w}
    alignas(16) float eG[D];            // e^{Gamma}
    int wide[NB];                       // block w's diagonal is summed directly
  };
};

// pair index p -> (i, j), i >= j, p = i (i + 1) / 2 + j
__device__ __forceinline__ int sfwd_pair_i(int p) { return p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0; }

// The v tile of the ACC layout (64 rows of 128 bfloat16): unpadded, each
// row's 16-byte chunks permuted by XOR with 2 (row & 7), a layout that an
// asynchronous copy straight into LDS can write (a wave's copy fills 1 KB
// contiguously, four whole rows).  The transposing reads take 32 bytes (two
// chunks that the permutation keeps together) from each of 4 or 8
// consecutive rows, which then fall on distinct banks.
__device__ __forceinline__ int sfwd_vsw(int r, int col) { return r * 128 + ((((col >> 3) ^ (2 * (r & 7)))) << 3) + (col & 7); }
__device__ __forceinline__ v4s_t sfwd_vtr(const bf16_t *t, int r, int n0, int lane) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s_t *)(t + sfwd_vsw(r, n0 + 4 * (lane & 3))));
}
// as tr4 and tr8 (rows r0 + 4 g + j, and r0 + 8 g + i; column n0 + n) on that layout
__device__ __forceinline__ PFrag4<bf16_t> sfwd_vtr4(const bf16_t *t, int r0, int n0, int lane) {
  PFrag4<bf16_t> f;
  f.x = sfwd_vtr(t, r0 + 4 * (lane >> 4) + ((lane & 15) >> 2), n0, lane);
  return f;
}
__device__ __forceinline__ PFrag<bf16_t> sfwd_vtr8(const bf16_t *t, int r0, int n0, int lane) {
  const int rr = r0 + 8 * (lane >> 4) + ((lane & 15) >> 2);
  union {
    v4s_t h[2];
    bf16x8_t v;
  } u;
  u.h[0] = sfwd_vtr(t, rr, n0, lane);
  u.h[1] = sfwd_vtr(t, rr + 4, n0, lane);
  PFrag<bf16_t> f;
  f.x = u.v;
  return f;
}

// TO: the element type of y (T, or float32 for bfloat16 inputs)
// PAIR: the ACC layout (bfloat16, d = 128, chunk 64), two workgroups per
// compute unit; otherwise one workgroup per compute unit, state copy in LDS
template <typename T, int D, int C, int GM, typename TO = T, bool PAIR = false>
__global__ __launch_bounds__((SfwdCfg<T, D, C, PAIR>::NT))
__attribute__((amdgpu_waves_per_eu(SfwdCfg<T, D, C, PAIR>::ACC ? 4 : 1))) void hgrn2_seg_fwd_kernel(SegFwdArgs a) {
  using Cfg = SfwdCfg<T, D, C, PAIR>;
  constexpr int NB = Cfg::NB, NWV = Cfg::NWV, NT = Cfg::NT, CPL = Cfg::CPL, JB = Cfg::JB, KSD = Cfg::KSD,
                HC = Cfg::HC, EPV = Cfg::EPV, TPW = Cfg::TPW, NPAIR = Cfg::NPAIR;
  constexpr bool ACC = Cfg::ACC;
  static_assert(!ACC || (TPW == 8 && NWV == 8 && NB == 4), "ACC: eight 16-row tiles of one column tile per wave");
  static_assert(NB == 4, "the pair decoding assumes four sub-blocks");
  using XT = RowTile<T, D>;
  constexpr int PV = Cfg::PV;
  using VT = RowTile<T, D, PV>;  // v and kh
  __shared__ typename Cfg::Smem sm;

  const int N = a.N, T_ = a.T, H = a.H, P = a.P;
  const int unit = blockIdx.x;
  const int bh = unit / P, p = unit % P;
  if (bh >= a.B * H) return;
  const int b = bh / H, h = bh % H;
  const int n0 = p * a.G, n1 = min(N, n0 + a.G);
  const int tid = threadIdx.x, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = wv >> 1, hh = wv & 1;  // token block w; half hh of its tokens (prefix) and of y's columns
  const bool has_ch = lane < Cfg::LANES;
  const int c0 = (has_ch ? lane : 0) * CPL;
  float lbv[CPL];  // gate mode: lower bounds of this lane's channels
#pragma unroll
  for (int e = 0; e < CPL; ++e) lbv[e] = GM == kGate ? a.lb[h * D + c0 + e] : 0.f;
  const uint32_t HDB = (uint32_t)H * D * sizeof(T);  // bytes from one token to the next
  const uint32_t c0b = (uint32_t)c0 * sizeof(T);
  auto tok = [&](int t) { return (uint32_t)t * HDB; };

  // ---- the state entering the segment: S^T tiles q = wv + NWV i in float32 accumulators
  const size_t SS = (size_t)D * D;
  const float *s0 = P == 1 ? (a.h0 ? a.h0 + (size_t)bh * SS : nullptr) : a.sin + ((size_t)bh * P + p) * SS;
  // (ACC: S tiles i = rows 16 i + 4 g + r, column 16 wv + n)
  f32x4_t S[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int q = wv + NWV * i, jb = q % JB, cb = q / JB;
    const int c = 16 * cb + n16, j = 16 * jb + 4 * g;
    if constexpr (ACC) {
      acc_zero(S[i]);
      if (s0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) S[i][r] = s0[(size_t)(16 * i + 4 * g + r) * D + 16 * wv + n16];
      }
    } else if (q < Cfg::NTILE && s0) {
      const float4 x = *(const float4 *)(s0 + (size_t)c * D + j);
      S[i] = f32x4_t{x.x, x.y, x.z, x.w};
    } else {
      acc_zero(S[i]);
    }
  }
  // its copy as a matrix-core operand, row c, columns j..j+3
  auto stage_state = [&]() {
    if constexpr (!ACC) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int q = wv + NWV * i, jb = q % JB, cb = q / JB;
        if (q < Cfg::NTILE) {
          Pack<T, 4> pk;
#pragma unroll
          for (int r = 0; r < 4; ++r) pk.v[r] = from_f32<T>(S[i][r]);
          *(Pack<T, 4> *)&sm.S[XT::at(16 * cb + n16, 16 * jb + 4 * g)] = pk;
        }
      }
    }
  };
  stage_state();

  // ---- a chunk's rows in registers: the v tile (16-byte vectors), q and k of
  // this wave's 8 tokens 16 w + 8 hh + t, and log f of all 16 tokens of block w
  // (both waves of a block form its prefix).  Buffer windows end at the last
  // row of the sequence: rows past it read as zero (no decay, no contribution).
  struct Regs {
    uint4 v[Cfg::NVV];
    Pack<T, CPL> q[8], k[8], l[16];
    T la;  // kScalar: log a of token 16 w + (lane & 15)
  };
  // parts of a chunk's rows: the v tile, and q, k and log f
  constexpr int kLdV = 1, kLdQKL = 2, kLdAll = 3;
  // vector-memory loads of a kLdQKL load: q and k of 8 tokens (k unless
  // formed from the gate), log f of 16 tokens (one log a with one decay per head)
  constexpr int kQKL = 8 + (reads_k(GM) ? 8 : 0) + (GM == kScalar ? 1 : 16);
  auto load = [&](Regs &r, int n, int parts) {
    // ACC (128 registers per lane): lane-dependent values derived anew, so
    // that the addresses built from them are not hoisted out of the walk and
    // kept live in registers
    const int tid = ACC ? opaque((int)threadIdx.x) : (int)threadIdx.x, lane = tid & 63;
    const int c0 = (has_ch ? lane : 0) * CPL;
    const uint32_t c0b = (uint32_t)c0 * sizeof(T);
    const int t0 = n * C, len = min(C, T_ - t0);
    const size_t cbase = (((size_t)b * T_ + t0) * H + h) * D * sizeof(T);
    const uint32_t rows = (uint32_t)len * HDB;
    const GBuf bq((const char *)a.q + cbase, rows), bv((const char *)a.v + cbase, rows);
    const GBuf bk((const char *)(reads_k(GM) ? a.k : a.q) + cbase, rows);
    const LfRows<GM> bl = lf_rows<GM, T>(a.log_f, b, T_, H, h, D, t0, len);
    if (parts & kLdV) {
#pragma unroll
      for (int i = 0; i < Cfg::NVV; ++i) {
        const int idx = min(tid + i * NT, Cfg::VV - 1);
        const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
        r.v[i] = bv.ld16(tok(row) + (uint32_t)col * sizeof(T));
      }
    }
    if (!(parts & kLdQKL)) return;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      r.q[t] = bq.template ldpack<T, CPL>(tok(16 * w + 8 * hh + t) + c0b);
      if constexpr (reads_k(GM)) r.k[t] = bk.template ldpack<T, CPL>(tok(16 * w + 8 * hh + t) + c0b);
    }
    if constexpr (GM == kScalar) {
      r.la = bl.template ld<T, 1>(16 * w + (lane & 15), 0).v[0];
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) r.l[t] = bl.template ld<T, CPL>(16 * w + t, c0b);
    }
  };

  // ACC: every prefetched register passes through an empty asm statement, so
  // that the compiler's wait for those loads (issued a chunk earlier, long
  // landed) falls here, ahead of the v tile's copies: the compiler does not
  // count the copies, and a wait of its own after them would wait for them too
  auto settle = [&](const Regs &r) {
    if constexpr (ACC) {
      static_assert(sizeof(Pack<T, CPL>) == 4, "two bfloat16 channels per lane");
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        asm volatile("" ::"v"(__builtin_bit_cast(uint32_t, r.q[t])));
        if constexpr (reads_k(GM)) asm volatile("" ::"v"(__builtin_bit_cast(uint32_t, r.k[t])));
      }
      if constexpr (GM == kScalar) {
        asm volatile("" ::"v"((uint32_t)__builtin_bit_cast(uint16_t, r.la)));
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) asm volatile("" ::"v"(__builtin_bit_cast(uint32_t, r.l[t])));
      }
    }
  };

  Regs rg;
  load(rg, n0, ACC ? kLdQKL : kLdAll);
  for (int n = n0; n < n1; ++n) {
    const int t0 = n * C, len = min(C, T_ - t0);
    // (as in load: lane-dependent values derived anew each chunk)
    const int tid = ACC ? opaque((int)threadIdx.x) : (int)threadIdx.x, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
    const int c0 = (has_ch ? lane : 0) * CPL;
    const uint32_t c0b = (uint32_t)c0 * sizeof(T);
    // ---- P0: v tile; block w's prefix (in both of its waves); qo, ko of this wave's tokens
    if constexpr (ACC) {
      settle(rg);
      // the v tile by asynchronous copies straight into LDS (the tiles are
      // free since B4), waited for before B2: wave wv copies rows 8 wv .. + 7,
      // four rows of 256 bytes per instruction; lane i lands in chunk i % 16
      // of row 4 j + i / 16 and fetches the logical chunk the swizzle puts
      // there.
      const size_t cbase = (((size_t)b * T_ + t0) * H + h) * D * sizeof(T);
      const GBuf bvc((const char *)a.v + cbase, (uint32_t)len * HDB);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 8 * wv + 4 * j + (lane >> 4);
        const int q = (lane & 15) ^ (2 * (r & 7));
        lds_dma16(bvc, tok(r) + (uint32_t)q * 16, sm.v + (8 * wv + 4 * j) * D);
      }
    } else {
#pragma unroll
      for (int i = 0; i < Cfg::NVV; ++i) {
        const int idx = tid + i * NT;
        const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
        if (idx < Cfg::VV) *(uint4 *)&sm.v[VT::at(row, col)] = rg.v[i];
      }
    }
    float kof[8][CPL];  // this wave's tokens: ko in float32, k e^{L_w - ell}
    {
      float run[CPL], ell[8][CPL], kf[8][CPL];
#pragma unroll
      for (int e = 0; e < CPL; ++e) run[e] = 0.f;
      if constexpr (ACC) {
        // (k formed only for this wave's own tokens: fewer live registers)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bool own = half == hh;  // wave-uniform
#pragma unroll
          for (int t8 = 0; t8 < 8; ++t8) {
            const int t = 8 * half + t8, tt = 16 * w + t;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
              const T lx = GM == kScalar ? readlane(rg.la, t) : rg.l[t].v[e];
              float lf;
              if (own) {
                // k of this wave's own tokens (loaded, or formed with log f)
                const T kx = reads_k(GM) ? rg.k[t8].v[e] : lx;
                lf_k<GM>(kx, lx, lbv[e], tt < len, lf, kf[t8][e]);
              } else {
                // the other half's tokens only add their log f to the prefix
                lf = lf_of<GM>(to_f32(lx), lbv[e], tt < len);
              }
              run[e] += lf;
              if (own) ell[t8][e] = run[e];
            }
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int tt = 16 * w + t;
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            const T lx = GM == kScalar ? readlane(rg.la, t) : rg.l[t].v[e];
            float lf, kv;
            // k of this wave's own tokens (loaded, or formed with log f); the
            // other half's tokens only add their log f to the prefix
            const T kx = reads_k(GM) ? rg.k[t & 7].v[e] : lx;
            lf_k<GM>(kx, lx, lbv[e], tt < len, lf, kv);
            run[e] += lf;
            if ((t >> 3) == hh) {
              ell[t & 7][e] = run[e];
              kf[t & 7][e] = kv;
            }
          }
        }
      }
      bool wd = false;
#pragma unroll
      for (int e = 0; e < CPL; ++e) wd |= has_ch && -run[e] > kDiagLimit;
      const bool wide = __ballot(wd) != 0;
      if (has_ch) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int tt = 16 * w + 8 * hh + t;
          Pack<T, CPL> oq, ok;
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            oq.v[e] = from_f32<T>(to_f32(rg.q[t].v[e]) * __expf(ell[t][e]));
            kof[t][e] = kf[t][e] * __expf(run[e] - ell[t][e]);
            ok.v[e] = from_f32<T>(kof[t][e]);
          }
          stpack<T, CPL>(&sm.qo[XT::at(tt, c0)], oq);
          stpack<T, CPL>(&sm.ko[XT::at(tt, c0)], ok);
        }
        // the block's decay e^{L_w} and its diagonal gap factor e^{-L_w} (at
        // most e^{80}): every other factor of the chunk is a product of these
        if (hh == 0) {
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            sm.eL[w][c0 + e] = __expf(run[e]);
            if constexpr (!ACC) sm.eLd[w][c0 + e] = __expf(fminf(-run[e], 80.f));
          }
        }
      }
      if (hh == 0 && lane == 0) sm.wide[w] = wide;
    }
    // the registers are consumed: the next chunk's rows
    // (ACC: q, k and log f; its v tile is copied into LDS when that chunk
    // starts.  Held in registers from here, the v vectors were spilled, and
    // the spill's store waited for the load it spilled.)
    if (n + 1 < n1) load(rg, n + 1, ACC ? kLdQKL : kLdAll);
    __syncthreads();  // B1: qo, ko, v, block decays and flags of every block

    // ---- P1: kh of this wave's tokens, e^{P_w}, e^{Gamma}; the score tiles
    if (has_ch) {
      float ea[CPL];  // e^{Gamma - P_{w+1}}
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const int c = c0 + e;
        float eb = 1.f, eg = 1.f;  // e^{P_w}, e^{Gamma}
        ea[e] = 1.f;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const float x = sm.eL[i][c];
          eb *= (i < w) ? x : 1.f;
          ea[e] *= (i > w) ? x : 1.f;
          eg *= x;
        }
        if (hh == 0) sm.eP[w][c] = eb;
        if (wv == 0) sm.eG[c] = eg;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        Pack<T, CPL> o;
#pragma unroll
        for (int e = 0; e < CPL; ++e) o.v[e] = from_f32<T>(kof[t][e] * ea[e]);
        stpack<T, CPL>(&sm.kh[VT::at(16 * w + 8 * hh + t, c0)], o);
      }
    }
    // score tile tau = wv + NWV s of pair (i, j), i >= j: X[s][t] = sum_c ko_s gap_c qo_t
    // (the transposed scores, kept as the 16-deep operand of the product with v)
#pragma unroll
    for (int s2 = 0; s2 < (NPAIR + NWV - 1) / NWV; ++s2) {
      const int tau = wv + NWV * s2;
      if (tau >= NPAIR) break;
      const int i = sfwd_pair_i(tau), j = tau - i * (i + 1) / 2;
      f32x4_t X;
      acc_zero(X);
      if (i == j && sm.wide[i]) {
        // wide in-block decay: summed directly, every exponent <= 0 (rare;
        // reloads the block's rows from global memory).  Lane (g, n) holds
        // X[s = 4g + r][t = n].
        const size_t cbase = (((size_t)b * T_ + t0) * H + h) * D * sizeof(T);
        const uint32_t rows = (uint32_t)len * HDB;
        const GBuf bq((const char *)a.q + cbase, rows);
        const GBuf bk((const char *)(reads_k(GM) ? a.k : a.q) + cbase, rows);
        const LfRows<GM> bl = lf_rows<GM, T>(a.log_f, b, T_, H, h, D, t0, len);
        for (int t = 0; t < 16; ++t) {
          float qt[CPL], ex[CPL];
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            qt[e] = 0.f;
            ex[e] = 0.f;
          }
          const Pack<T, CPL> pq = bq.template ldpack<T, CPL>(tok(16 * i + t) + c0b);
#pragma unroll
          for (int e = 0; e < CPL; ++e) qt[e] = has_ch ? to_f32(pq.v[e]) : 0.f;
          for (int sd = t; sd >= 0; --sd) {
            float part = 0.f;
            Pack<T, CPL> pk;
            if constexpr (reads_k(GM)) pk = bk.template ldpack<T, CPL>(tok(16 * i + sd) + c0b);
            const Pack<T, CPL> pls = bl.template ld<T, CPL>(16 * i + sd, c0b);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
              float lf, kv;
              lf_k<GM>(pk.v[e], lfe<GM>(pls, e), lbv[e], true, lf, kv);
              part += qt[e] * kv * __expf(ex[e]);
              ex[e] += lf;  // the factor of sd - 1 includes f_sd
            }
            const float tot = wave_sum(part);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n16 == t && 4 * g + r == sd) X[r] = tot;
          }
        }
      } else if (i == j + 1) {
        // adjacent blocks: the gap factor is e^{P_i - P_i} = 1 exactly
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int c = 32 * ks + 8 * g;
          mma(X, row8<D>(sm.ko, 16 * j + n16, c), row8<D>(sm.qo, 16 * i + n16, c));
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int c = 32 * ks + 8 * g;
          float kv[8];
          unpack8(row8<D>(sm.ko, 16 * j + n16, c), kv);
          // gap factor: e^{P_i - P_{j+1}} (the decays of the blocks between) apart,
          // e^{-L_i} (at most e^{80}) on the diagonal
          Frag fa;
#pragma unroll
          for (int e = 0; e < 8; e += 4) {
            float4 x;
            if (i == j) {
              if constexpr (ACC) {
                // e^{-L_i}: not wide, so e^{L_i} >= e^{-64}
                x = ldf4(&sm.eL[i][c + e]);
                x = make_float4(__builtin_amdgcn_rcpf(x.x), __builtin_amdgcn_rcpf(x.y), __builtin_amdgcn_rcpf(x.z),
                                __builtin_amdgcn_rcpf(x.w));
              } else {
                x = ldf4(&sm.eLd[i][c + e]);
              }
            } else {
              x = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
              for (int m = 1; m < NB - 1; ++m)
                if (m > j && m < i) {
                  const float4 L = ldf4(&sm.eL[m][c + e]);
                  x.x *= L.x; x.y *= L.y; x.z *= L.z; x.w *= L.w;
                }
            }
            fa.v[e] = kv[e] * x.x;
            fa.v[e + 1] = kv[e + 1] * x.y;
            fa.v[e + 2] = kv[e + 2] * x.z;
            fa.v[e + 3] = kv[e + 3] * x.w;
          }
          mma(X, to_pfrag<T>(fa), row8<D>(sm.qo, 16 * i + n16, c));
        }
        if (i == j) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g + r > n16) X[r] = 0.f;  // s > t
        }
      }
      sm.sc[tau][lane] = acc_to_frag4<T>(X);
    }
    if constexpr (ACC) {
      // this wave's copies of the v tile have landed: vector-memory operations
      // complete in issue order, and kQKL loads were issued after the copies
      // when a next chunk was prefetched
      if (n + 1 < n1) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kQKL) : "memory");
      } else {
        vm_drain();
      }
      // a ragged last chunk: this wave's rows past the sequence's end are
      // zero whatever the copy left there
      if (len < C) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int idx = lane + 64 * i, r = 8 * wv + (idx >> 4);
          if (r >= len) *(uint4 *)&sm.v[r * D + 8 * (idx & 15)] = uint4{0u, 0u, 0u, 0u};
        }
      }
    }
    __syncthreads();  // B2: score tiles, kh, e^{P}, e^{Gamma}, v

    if constexpr (ACC) {
      // ---- P2: y of all four token blocks for column tile wv: the scores'
      // product with v, plus (qo e^{P_w}) S from the accumulators
      f32x4_t Y[NB];
#pragma unroll
      for (int w2 = 0; w2 < NB; ++w2) acc_zero(Y[w2]);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const PFrag4<T> fv = sfwd_vtr4(sm.v, 16 * j, 16 * wv, lane);
#pragma unroll
        for (int w2 = j; w2 < NB; ++w2) mma16(Y[w2], sm.sc[w2 * (w2 + 1) / 2 + j][lane], fv);
      }
      // k slots of pair p: 0-3 <-> rows 32 p + 4 g + r (tile 2 p), 4-7 <-> rows
      // 32 p + 16 + 4 g + r (tile 2 p + 1), the same in both operands
#pragma unroll
      for (int w2 = 0; w2 < NB; ++w2) {
#pragma unroll
        for (int pp = 0; pp < TPW / 2; ++pp) {
          Frag f;
          if (w2 == 0) {  // e^{P_0} = 1
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              f.v[r] = S[2 * pp][r];
              f.v[4 + r] = S[2 * pp + 1][r];
            }
          } else {
            const float4 e0 = ldf4(&sm.eP[w2][32 * pp + 4 * g]), e1 = ldf4(&sm.eP[w2][32 * pp + 16 + 4 * g]);
            f.v[0] = S[2 * pp][0] * e0.x; f.v[1] = S[2 * pp][1] * e0.y;
            f.v[2] = S[2 * pp][2] * e0.z; f.v[3] = S[2 * pp][3] * e0.w;
            f.v[4] = S[2 * pp + 1][0] * e1.x; f.v[5] = S[2 * pp + 1][1] * e1.y;
            f.v[6] = S[2 * pp + 1][2] * e1.z; f.v[7] = S[2 * pp + 1][3] * e1.w;
          }
          const PFrag<T> qa = ld4x2(&sm.qo[XT::at(16 * w2 + n16, 32 * pp + 4 * g)],
                                    &sm.qo[XT::at(16 * w2 + n16, 32 * pp + 16 + 4 * g)]);
          mma(Y[w2], qa, to_pfrag<T>(f));
        }
      }
      // y out: float32 straight from the accumulators, else staged in the
      // dead ko tile (rows 16 w2 + 4 g + r, column 16 wv + n)
      if constexpr (!std::is_same<TO, T>::value) {
        TO *gyo = (TO *)a.y + (((size_t)b * T_ + t0) * H + h) * D;
#pragma unroll
        for (int w2 = 0; w2 < NB; ++w2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * w2 + 4 * g + r;
            if (t < len) __builtin_nontemporal_store(Y[w2][r], gyo + ((size_t)t * H * D + 16 * wv + n16));
          }
      } else {
#pragma unroll
        for (int w2 = 0; w2 < NB; ++w2)
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.ko[XT::at(16 * w2 + 4 * g + r, 16 * wv + n16)] = from_f32<T>(Y[w2][r]);
      }
      __syncthreads();  // B3: y staged

      // ---- P3: y's full rows out; the state update S <- Diag(e^Gamma) S + kh^T v
      if constexpr (std::is_same<TO, T>::value) {
        T *gy = (T *)a.y + (((size_t)b * T_ + t0) * H + h) * D;
#pragma unroll
        for (int i = 0; i < Cfg::NVV; ++i) {
          const int idx = tid + i * NT;
          const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
          if (idx < Cfg::VV && row < len) {
            const uint4 u = *(const uint4 *)&sm.ko[XT::at(row, col)];
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, u), (u32x4_t *)(gy + ((size_t)row * H * D + col)));
          }
        }
      }
      const PFrag<T> fv0 = sfwd_vtr8(sm.v, 0, 16 * wv, lane), fv1 = sfwd_vtr8(sm.v, 32, 16 * wv, lane);
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const float4 eg = ldf4(&sm.eG[16 * i + 4 * g]);
        S[i][0] *= eg.x;
        S[i][1] *= eg.y;
        S[i][2] *= eg.z;
        S[i][3] *= eg.w;
        mma(S[i], tr8<D, PV>(sm.kh, 0, 16 * i), fv0);
        mma(S[i], tr8<D, PV>(sm.kh, 32, 16 * i), fv1);
      }
    } else {
      // ---- P2: y of block w, column half hh: the scores' product with v, plus (qo e^{P_w}) S
      f32x4_t Y[HC];
#pragma unroll
      for (int cb = 0; cb < HC; ++cb) acc_zero(Y[cb]);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (j > w) continue;  // wave-uniform
        const PFrag4<T> fa = sm.sc[w * (w + 1) / 2 + j][lane];
#pragma unroll
        for (int cb = 0; cb < HC; ++cb) mma16(Y[cb], fa, tr4<D, PV>(sm.v, 16 * j, (D / 2) * hh + 16 * cb));
      }
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const int c = 32 * ks + 8 * g;
        float qv[8];
        unpack8(row8<D>(sm.qo, 16 * w + n16, c), qv);
        const float4 e0 = ldf4(&sm.eP[w][c]), e1 = ldf4(&sm.eP[w][c + 4]);
        Frag f;
        f.v[0] = qv[0] * e0.x; f.v[1] = qv[1] * e0.y; f.v[2] = qv[2] * e0.z; f.v[3] = qv[3] * e0.w;
        f.v[4] = qv[4] * e1.x; f.v[5] = qv[5] * e1.y; f.v[6] = qv[6] * e1.z; f.v[7] = qv[7] * e1.w;
        const PFrag<T> qb = to_pfrag<T>(f);
#pragma unroll
        for (int cb = 0; cb < HC; ++cb) mma(Y[cb], qb, tr8<D>(sm.S, 32 * ks, (D / 2) * hh + 16 * cb));
      }
      __syncthreads();  // B3: every wave is done with qo, the scores and the state's copy

      // ---- P3: y out (staged in this wave's half of block w's qo rows, or
      // float32 straight from the accumulators); the state update
      if constexpr (!std::is_same<TO, T>::value) {
        TO *gyo = (TO *)a.y + (((size_t)b * T_ + t0) * H + h) * D;
#pragma unroll
        for (int cb = 0; cb < HC; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * w + 4 * g + r;
            if (t < len)
              __builtin_nontemporal_store(Y[cb][r], gyo + ((size_t)t * H * D + (D / 2) * hh + 16 * cb + n16));
          }
      } else {
#pragma unroll
      for (int cb = 0; cb < HC; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.qo[XT::at(16 * w + 4 * g + r, (D / 2) * hh + 16 * cb + n16)] = from_f32<T>(Y[cb][r]);
      wave_lds_sync();
      {
        T *gy = (T *)a.y + (((size_t)b * T_ + t0) * H + h) * D;
        constexpr int RV = 16 * (D / 2) / EPV;  // 16-byte vectors in this wave's 16 half rows
#pragma unroll
        for (int i = 0; i < (RV + 63) / 64; ++i) {
          const int idx = lane + 64 * i;
          const int row = idx / (D / 2 / EPV), col = (D / 2) * hh + (idx % (D / 2 / EPV)) * EPV;
          const int t = 16 * w + row;
          if (idx < RV && t < len) {
            const uint4 u = *(const uint4 *)&sm.qo[XT::at(t, col)];
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, u), (u32x4_t *)(gy + ((size_t)t * H * D + col)));
          }
        }
      }
      }
      // S^T <- S^T Diag(e^Gamma) + v^T kh
      // (NWV = 8 divides JB for D = 128: every tile of this wave has jb = wv, and
      // the compiler keeps the two v operands across the tiles)
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int q = wv + NWV * i, jb = q % JB, cb = q / JB;
        if (q < Cfg::NTILE) {
          const float eg = sm.eG[16 * cb + n16];
#pragma unroll
          for (int r = 0; r < 4; ++r) S[i][r] *= eg;
#pragma unroll
          for (int ks = 0; ks < C / 32; ++ks) mma(S[i], tr8<D, PV>(sm.v, 32 * ks, 16 * jb), tr8<D, PV>(sm.kh, 32 * ks, 16 * cb));
        }
      }
      stage_state();
    }
    __syncthreads();  // B4: the tiles may be rewritten (and the state's copy is in place)
  }

  if (p == P - 1 && a.ht) {
    if constexpr (ACC) {
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) a.ht[(size_t)bh * SS + (size_t)(16 * i + 4 * g + r) * D + 16 * wv + n16] = S[i][r];
    } else {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int q = wv + NWV * i, jb = q % JB, cb = q / JB;
        if (q < Cfg::NTILE) {
          const int c = 16 * cb + n16, j = 16 * jb + 4 * g;
          *(float4 *)(a.ht + (size_t)bh * SS + (size_t)c * D + j) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
        }
      }
    }
  }
}

// The state entering each segment from the segments' summaries, in place in
// sin [BH, NSEG + 1, D, D] float32, whose entry p + 1 holds the end state of
// segment p from a zero state (the state scan in segment mode):
//   entry 0 <- h0 (or zero);  entry p + 1 <- Diag(e^{a_p}) entry p + entry p + 1,
// with a_p = asum [BH, NSEG, D], the segment's total log decay per channel.
// The last value is also the final state (ht, if wanted).  One thread per
// element of the d x d state, the segments in order; each thread reads its
// element of h0 before it writes the same element of ht, so ht may alias h0.
template <int D>
__global__ __launch_bounds__(256) void hgrn2_seg_carry_kernel(int BH, int NSEG, const float *h0, float *sin,
                                                              const float *asum, float *ht) {
  constexpr int PER = D * D / 256 > 0 ? D * D / 256 : 1;  // workgroups' worth of elements per (b, h)
  const size_t SS = (size_t)D * D;
  // a grid-stride walk over (b, h, element block): the grid stays small for any B * H
  for (long long blk = blockIdx.x; blk < (long long)BH * PER; blk += gridDim.x) {
    const long long bh = blk / PER;
    const int e = (int)(blk % PER) * 256 + (int)threadIdx.x;
    if (e >= D * D) continue;
    const int c = e / D;
    float cur = h0 ? h0[(size_t)bh * SS + e] : 0.f;
    float *base = sin + (size_t)bh * (NSEG + 1) * SS;
    base[e] = cur;
    // eight segments at a time: their loads are issued together, so that the
    // walk waits for one memory round trip per eight segments, not per segment
    for (int p0 = 0; p0 < NSEG; p0 += 8) {
      float loc[8], dec[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (p0 + i < NSEG) {
          loc[i] = base[(size_t)(p0 + i + 1) * SS + e];
          dec[i] = asum[((size_t)bh * NSEG + p0 + i) * D + c];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (p0 + i < NSEG) {
          cur = __expf(dec[i]) * cur + loc[i];
          base[(size_t)(p0 + i + 1) * SS + e] = cur;
        }
      }
    }
    if (ht) ht[(size_t)bh * SS + e] = cur;
  }
}

template <typename T, int D, int C, int GM, typename TO = T>
hipError_t launch_seg_fwd(const SegFwdArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)a.B * a.H * a.P));
  if constexpr (SfwdCfg<T, D, C, true>::ACC) {
    if (a.pair) {
      hipLaunchKernelGGL((hgrn2_seg_fwd_kernel<T, D, C, GM, TO, true>), grid, dim3(SfwdCfg<T, D, C, true>::NT), 0,
                         stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((hgrn2_seg_fwd_kernel<T, D, C, GM, TO>), grid, dim3(SfwdCfg<T, D, C>::NT), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_seg_carry(int BH, int NSEG, const float *h0, float *sin, const float *asum, float *ht,
                            hipStream_t stream) {
  constexpr int PER = D * D / 256 > 0 ? D * D / 256 : 1;
  const long long blocks = std::min<long long>((long long)BH * PER, 1 << 16);
  hipLaunchKernelGGL(hgrn2_seg_carry_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream, BH, NSEG, h0, sin, asum,
                     ht);
  return hipGetLastError();
}

}  // namespace hgrn2
