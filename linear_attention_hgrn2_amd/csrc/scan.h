// Chunk-boundary state scan of the HGRN2 recurrence (gfx950).
//
// HGRN2 summary (paperlayer.ai) §3.2: per head a d x d state whose rows (the
// d_k channels) are scaled by the forget gate and which receives an outer
// product write each step.  Over one chunk of C tokens with in-chunk
// inclusive prefix b_t of log f and total Gamma = b_C, the state advances as
//   S <- Diag(e^Gamma) S + sum_t Diag(e^{Gamma - b_t}) x_t^T z_t
// with (x, z) = (k, v); with tied gates k = 1 - f is formed from log f
// instead of read, and from the gate pre-activation both log f and k are
// formed (rows past the end of the sequence then decay nothing).  Walked backwards with (x, z) = (q, dy) and weights
// e^{b_t}, the same pass carries the state adjoint Lambda (the gradient of the
// loss with respect to the state at a chunk end):
//   Lambda <- Diag(e^Gamma) Lambda + sum_t Diag(e^{b_t}) q_t^T dy_t.
// Every chunk's state is written out (forward: the state after n chunks, n =
// 0..N; backward: the adjoint at the end of chunk n, n = 0..N-1) so that the
// chunk kernels can run all chunks in parallel.
//
// In segment mode (SEG, forward only) a workgroup walks only the G chunks of
// one segment of its sequence, from a zero state, and writes just the
// segment's end state (float32) and the per-channel total of its log decays:
// the summaries from which the state entering every segment is carried
// (hgrn2_seg_carry_kernel), so that the segments' outputs can then be
// computed in parallel without any per-chunk state in memory.
//
// Rows of the state evolve independently (each row is one decay channel), so
// one workgroup owns one (batch, head, CS-row slice) and holds those rows of
// the state, transposed (S^T[j][c], every column j), in float32 matrix-core
// accumulators.  Per chunk a workgroup only decays its own CS channels: thread
// tid takes channel tid % CS and the run tid / CS of TPR consecutive tokens;
// the z rows (v or dy) are shared through L2 by the slices of one head, which
// run on one XCD.
#pragma once

#include "tile.h"

namespace hgrn2 {

struct ScanArgs {
  int B, T, H, N;
  const void *x, *z, *log_f;  // [B,T,H,D]; log_f holds the gate pre-activation in gate mode
  const float *lb;            // gate mode: lower bound of f, [H,D]
  const float *s_in;          // initial state (h0 or dht), [B,H,D,D] float32, or null
  void *states;               // forward: [B,H,N+1,D,D]; backward: [B,H,N,D,D]; input dtype
  float *s_out;               // final state (ht or dh0), or null; segment mode: [B,H,NSEG+1,D,D], entry p + 1
                              // the end state of segment p (entry 0 is the carry's)
  int NSEG = 0, G = 0;        // segment mode: segments summarised per (b, h), chunks per segment
  float *asum = nullptr;      // segment mode: [B,H,NSEG,D] total log decay of each segment
};

template <typename T, int D, int C, bool REV> struct ScanCfg {
  // state rows (channels) per workgroup.  At d = 128, bf16, chunk 64, 64 rows
  // make each 128-byte line of x and log f belong to one workgroup and halve
  // the re-reads of the z rows; eight waves then keep two per SIMD.
  static constexpr bool WIDE = D >= 128 && C == 64 && sizeof(T) == 2;
  static constexpr int CS = WIDE ? 64 : (D < 32 ? D : 32);
  static constexpr int NW = WIDE ? 8 : C / 16, NT = 64 * NW;
  static constexpr int NS = D / CS;               // slices per (b, h)
  static constexpr int NR = NT / CS;              // runs of consecutive tokens per chunk
  static constexpr int TPR = C / NR;              // tokens per run (per lane)
  static_assert(NR * TPR == C, "runs tile the chunk");
  static constexpr int JB = D / 16, CBS = CS / 16;
  static constexpr int NTILE = JB * CBS;
  static constexpr int TPW = (NTILE + NW - 1) / NW;  // state tiles per wave
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int VZ = C * D / EPV;             // 16-byte vectors of one z tile
  static constexpr int NVZ = (VZ + NT - 1) / NT;
  struct Smem {
    T x[C * RowTile<T, CS, 32>::LD];    // decayed x of this slice's channels
    T z[2][C * RowTile<T, D, 32>::LD];  // z rows, double-buffered
    float Lr[NR][CS];                // run totals of log f
    float eG[CS];                    // e^Gamma
    T st[CS * RowTile<T, D>::LD];    // a state awaiting its store, rows c of the slice
  };
};

template <typename T, int D, int C, bool REV, int GM, bool SEG>
__global__ __launch_bounds__((ScanCfg<T, D, C, REV>::NT)) void hgrn2_scan_kernel(ScanArgs a) {
  static_assert(!(SEG && REV), "segment summaries are a forward pass");
  using Cfg = ScanCfg<T, D, C, REV>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, CS = Cfg::CS, NS = Cfg::NS, NR = Cfg::NR, TPR = Cfg::TPR,
                JB = Cfg::JB, EPV = Cfg::EPV;
  // rows padded by 32 bytes: the transposing operand reads are conflict-free
  using XT = RowTile<T, CS, 32>;
  using ZT = RowTile<T, D, 32>;
  __shared__ typename Cfg::Smem sm;

  // slices of one (b, h) (segment mode: of one segment) get ids equal mod 8:
  // they run on one XCD and share its L2
  const int bid = blockIdx.x;
  const int grp = bid / (8 * NS), rem = bid % (8 * NS);
  const int slice = rem / 8;
  const int unit = grp * 8 + (rem % 8);
  if (unit >= a.B * a.H * (SEG ? a.NSEG : 1)) return;
  const int bh = SEG ? unit / a.NSEG : unit;
  const int b = bh / a.H, h = bh % a.H;
  const int cs0 = slice * CS;  // first state row of this workgroup
  const int T_ = a.T, H = a.H;
  // the chunks this workgroup walks: all of them, or one segment's
  const int n0 = SEG ? (unit % a.NSEG) * a.G : 0;
  const int N = SEG ? min(a.G, a.N - n0) : a.N;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n16 = lane & 15, g = lane >> 4;
  const int cl = tid % CS, ri = tid / CS;  // prep layout: channel, run of TPR tokens
  const float lbv = GM == kGate ? a.lb[h * D + cs0 + cl] : 0.f;

  const size_t SS = (size_t)D * D;
  const uint32_t HDB = (uint32_t)H * D * sizeof(T);  // bytes from one token to the next
  // buffer window over the rows of chunk n: rows past the end of the sequence read as zero
  auto win = [&](const void *base, int n) {
    const int t0 = n * C;
    return GBuf((const char *)base + (((size_t)b * T_ + t0) * H + h) * D * sizeof(T),
                (uint32_t)min(C, T_ - t0) * HDB);
  };
  // per-lane byte offsets within a chunk window (the same for every chunk)
  const uint32_t xoff = (uint32_t)(ri * TPR) * HDB + (uint32_t)(cs0 + cl) * sizeof(T);
  uint32_t zoff[Cfg::NVZ];
#pragma unroll
  for (int i = 0; i < Cfg::NVZ; ++i) {
    const int idc = min(tid + i * NT, Cfg::VZ - 1);
    zoff[i] = (uint32_t)(idc / (D / EPV)) * HDB + (uint32_t)((idc % (D / EPV)) * EPV) * sizeof(T);
  }

  // ---- state tiles: tile q = w + NW * i (q < NTILE) covers S^T rows (j) 16 jb.. and columns (c) cs0 + 16 cb..
  f32x4_t S[Cfg::TPW];
#pragma unroll
  for (int i = 0; i < Cfg::TPW; ++i) {
    const int q = w + NW * i;
    const int jb = q % JB, cb = q / JB;
    const int c = cs0 + cb * 16 + n16, j = jb * 16 + 4 * g;
    if (q < Cfg::NTILE && a.s_in && !SEG) {
      const float4 v = *(const float4 *)(a.s_in + (size_t)bh * SS + (size_t)c * D + j);
      S[i] = f32x4_t{v.x, v.y, v.z, v.w};
    } else {
      acc_zero(S[i]);
    }
  }
  // this (b, h)'s entries of the state buffer; entry `slot` at a scalar offset
  const int nst = SEG ? 0 : REV ? N : N + 1;
  const GBuf bst((const char *)a.states + (size_t)bh * nst * SS * sizeof(T), (uint32_t)(nst * SS * sizeof(T)));
  // States leave through LDS: the tiles are written there (stage), and after
  // the next barrier every thread stores two 16-byte pieces of whole rows
  // (flush), so each store instruction writes complete 256-byte rows instead
  // of 8-byte pieces of sixteen rows.
  using STT = RowTile<T, D>;
  constexpr int VST = CS * D / EPV;  // 16-byte vectors of the slice's state rows
  int pend = -1;                     // entry staged and not yet stored
  auto stage = [&](int slot) {
    if constexpr (SEG) return;
#pragma unroll
    for (int i = 0; i < Cfg::TPW; ++i) {
      const int q = w + NW * i;
      if (q < Cfg::NTILE) {
        const int jb = q % JB, cb = q / JB;
        Pack<T, 4> p;
#pragma unroll
        for (int r = 0; r < 4; ++r) p.v[r] = from_f32<T>(S[i][r]);
        *(Pack<T, 4> *)&sm.st[STT::at(cb * 16 + n16, jb * 16 + 4 * g)] = p;
      }
    }
    pend = slot;
  };
  auto flush = [&]() {
    if (SEG || pend < 0) return;
#pragma unroll
    for (int i = 0; i < (VST + NT - 1) / NT; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
      if (idx < VST)
        bst.st16((uint32_t)((cs0 + row) * D + col) * sizeof(T), *(const uint4 *)&sm.st[STT::at(row, col)],
                 (uint32_t)(pend * SS * sizeof(T)));
    }
    pend = -1;
  };
  if (!REV) stage(0);

  // ---- register prefetch, two chunks ahead in two register sets: x, log f of
  // this lane's channel and token run; the z tile
  using XP = T[TPR];
  using ZP = uint4[Cfg::NVZ];
  // Loads go through buffer windows: rows past the end of the sequence read
  // as zero (log f = 0, x = 0, z = 0 contribute nothing), so nothing is masked
  // where they are consumed and every step issues the same loads.
  auto prefetch = [&](XP &px, XP &pl, ZP &pz, int n) {
    const LfRows<GM> bl = lf_rows<GM, T>(a.log_f, b, T_, H, h, D, n * C, min(C, T_ - n * C));
    const GBuf bz = win(a.z, n);
#pragma unroll
    for (int i = 0; i < TPR; ++i) {
      if constexpr (REV || reads_k(GM)) px[i] = win(a.x, n).template ldpack<T, 1>(xoff + (uint32_t)i * HDB).v[0];
      pl[i] = bl.template ld<T, 1>(ri * TPR + i, (uint32_t)(cs0 + cl) * sizeof(T)).v[0];
    }
#pragma unroll
    for (int i = 0; i < Cfg::NVZ; ++i) pz[i] = bz.ld16(zoff[i]);
  };

  // one chunk: consumes (px, pl, pz), then refills them with the chunk two steps on
  float gacc = 0.f;  // segment mode: this thread's channel's total log decay over the segment
  auto step = [&](XP &px, XP &pl, ZP &pz, int it) {
    const int n = REV ? N - 1 - it : n0 + it;
    T *zs = sm.z[it & 1];
    // ---- chunk-local prefix of the floored log f: within the lane's run, then across runs
    float l[TPR], kx[TPR];  // kx: k of the run's tokens (forward; formed with log f)
    float run = 0.f;
    if constexpr (GM == kGate) {
      // f from z with no logarithm: l holds products of f within the run
      // (forward: of the later tokens, e^{run - prefix}; backward: of the
      // tokens so far, e^{prefix}) and only the run total is taken to the log
      // domain, floored as the per-token floors would floor it
      float f[TPR];
#pragma unroll
      for (int i = 0; i < TPR; ++i) {
        float kk;
        gate_f_k(to_f32(pl[i]), lbv, f[i], kk);
        if (n * C + ri * TPR + i >= T_) f[i] = 1.f, kk = 0.f;  // past the end: no decay, no input
        if constexpr (!REV) kx[i] = kk;
      }
      float pp = 1.f;
      if constexpr (REV) {
#pragma unroll
        for (int i = 0; i < TPR; ++i) l[i] = pp *= f[i];
      } else {
#pragma unroll
        for (int i = TPR - 1; i >= 0; --i) {
          l[i] = pp;
          pp *= f[i];
        }
      }
      run = fmaxf(__logf(pp), TPR * kLogFloor);
    } else {
#pragma unroll
      for (int i = 0; i < TPR; ++i) {
        float lf;
        if constexpr (REV) lf = lf_of<GM>(to_f32(pl[i]), lbv, n * C + ri * TPR + i < T_);
        else lf_k<GM>(px[i], pl[i], lbv, n * C + ri * TPR + i < T_, lf, kx[i]);
        run += lf;
        l[i] = run;
      }
    }
    sm.Lr[ri][cl] = run;
#pragma unroll
    for (int i = 0; i < Cfg::NVZ; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / (D / EPV), col = (idx % (D / EPV)) * EPV;
      if (idx < Cfg::VZ) *(uint4 *)&zs[ZT::at(row, col)] = pz[i];
    }
    __syncthreads();
    // ---- decayed x: forward x e^{Gamma - b_t}, backward x e^{b_t}
    {
      float P = 0.f, G = 0.f, Q = 0.f;  // earlier runs' total, chunk total, later runs' total
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float L = sm.Lr[r][cl];
        P += (r < ri) ? L : 0.f;
        Q += (r > ri) ? L : 0.f;
        G += L;
      }
      if (ri == 0) sm.eG[cl] = __expf(G);
      gacc += G;
      if constexpr (GM == kGate) {
        // e^{b_t} (backward) or e^{Gamma - b_t} (forward) as the other runs'
        // factor times the run's own product of f
        const float e = __expf(REV ? P : Q);
#pragma unroll
        for (int i = 0; i < TPR; ++i) {
          const float xv = REV ? to_f32(px[i]) : kx[i];
          sm.x[XT::at(ri * TPR + i, cl)] = from_f32<T>(xv * (e * l[i]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < TPR; ++i) {
          const float b_t = P + l[i];
          const float ex = REV ? b_t : fminf(G - b_t, 0.f);
          const float xv = REV ? to_f32(px[i]) : kx[i];
          sm.x[XT::at(ri * TPR + i, cl)] = from_f32<T>(xv * __expf(ex));
        }
      }
    }
    flush();  // the state staged in the previous step (read here, rewritten after the next barrier)
    // this register set is consumed: fetch the chunk two steps on into it (the
    // last chunk again near the end, so every step issues the same loads)
    prefetch(px, pl, pz, REV ? max(n - 2, 0) : min(n + 2, n0 + N - 1));
    __syncthreads();
    // ---- the adjoint at the end of chunk n is the value before its update
    if (REV) stage(n);
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
            mma(S[i], tr8<D, 32>(zs, 32 * ks, 16 * jb), tr8<CS, 32>(sm.x, 32 * ks, 16 * cb));
        } else {
          mma16(S[i], tr4<D, 32>(zs, 0, 16 * jb), tr4<CS, 32>(sm.x, 0, 16 * cb));
        }
      }
    }
    if (!REV) stage(n + 1);
  };

  T px0[TPR], pl0[TPR], px1[TPR], pl1[TPR];
  uint4 pz0[Cfg::NVZ], pz1[Cfg::NVZ];
  prefetch(px0, pl0, pz0, REV ? N - 1 : n0);
  prefetch(px1, pl1, pz1, REV ? max(N - 2, 0) : n0 + min(1, N - 1));
  int it = 0;
  for (; it + 1 < N; it += 2) {
    step(px0, pl0, pz0, it);
    step(px1, pl1, pz1, it + 1);
  }
  if (it < N) step(px0, pl0, pz0, it);
  __syncthreads();
  flush();
  if (a.s_out) {
    // the final state (segment mode: the segment's end state from zero)
    const size_t so = (SEG ? (size_t)bh * (a.NSEG + 1) + unit % a.NSEG + 1 : (size_t)bh) * SS;
#pragma unroll
    for (int i = 0; i < Cfg::TPW; ++i) {
      const int q = w + NW * i;
      if (q < Cfg::NTILE) {
        const int jb = q % JB, cb = q / JB;
        const int c = cs0 + cb * 16 + n16, j = jb * 16 + 4 * g;
        *(float4 *)(a.s_out + so + (size_t)c * D + j) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
      }
    }
  }
  if (SEG && ri == 0) a.asum[(size_t)unit * D + cs0 + cl] = gacc;
}

template <typename T, int D, int C, bool REV, int GM = kUntied, bool SEG = false>
hipError_t launch_scan(const ScanArgs &a, hipStream_t stream) {
  static_assert(!(REV && GM == kTied), "the adjoint scan reads q, not k: run it untied");
  using Cfg = ScanCfg<T, D, C, REV>;
  const long long groups = ((long long)a.B * a.H * (SEG ? a.NSEG : 1) + 7) / 8;
  hipLaunchKernelGGL((hgrn2_scan_kernel<T, D, C, REV, GM, SEG>), dim3((unsigned)(groups * 8 * Cfg::NS)), dim3(Cfg::NT),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace hgrn2
