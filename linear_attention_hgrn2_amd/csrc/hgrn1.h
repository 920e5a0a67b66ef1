// HGRN1 elementwise gated recurrence (gfx950): HGRN2 summary, paperlayer.ai,
// §2.1 (the gated linear RNN that HGRN2 expands):
//   h_t[c] = f_t[c] h_{t-1}[c] + k_t[c] v_t[c],     y_t[c] = q_t[c] h_t[c],
// per channel c of [B, T, C] tensors, f = exp(log f), and in HGRN1 itself the
// input gate tied to the forget gate, k = 1 - f (GM = kTied).  The
// backward runs the adjoint g_t = q_t dy_t + f_{t+1} g_{t+1} (g_T adds dht):
//   dq_t = dy_t h_t,  dk_t = g_t v_t,  dv_t = g_t k_t,  dlog f_t = g_t f_t h_{t-1},
//   dh0 = f_1 g_1   (tied: dlog f_t - f_t dk_t, no dk).
//
// Every channel is an independent first-order scan, so the work is pure HBM
// streaming with a serial dependence along time only.  The sequence is cut
// into segments of kH1Seg tokens, eight consecutive segments form a group,
// and three passes with no waits between workgroups do the scan:
//   1. summaries: a workgroup takes one group of one batch element for 128
//      channels (a wave per segment).  Each segment's total log decay A and its
//      end state from zero (forward), or the gradient it passes to the segment
//      before from a zero gradient after it (reverse), go to LDS; then every
//      segment's exclusive combination with the group's earlier (forward) or
//      later (reverse) segments, and the group's total, go to HBM;
//   2. carries: per (b, channel) a serial pass over the groups: the state
//      entering each group (forward; the last one is hT) or the gradient
//      entering it from the right (reverse; the last one is dh0);
//   3. final: every segment again, starting from its group's carry combined
//      with its in-group prefix, writing y and the state entering the segment
//      (forward) or, with h recomputed in registers, the gradients.
// Summaries combine as (a1, b1) then (a2, b2) -> (a1 + a2, e^{a2} b1 + b2).
// A thread owns two adjacent channels (one 4-byte bf16 pair, or 8 bytes fp32)
// of one segment; a wave covers 128 consecutive channels of one token row.
#pragma once

#include "tile.h"

namespace hgrn2 {

constexpr int kH1Seg = 32;    // tokens per segment
constexpr int kH1Grp = 8;     // segments per group (waves of a summary workgroup)
constexpr int kH1Pairs = 256; // channel pairs per final-pass workgroup (four waves)

// The summaries of one direction (workspace).
struct H1Sum {
  float *PA, *PB;  // [B,S,C]: each segment's exclusive in-group combination
  float *GA, *GB;  // [B,NG,C]: each group's total
  float *gc;       // [B,NG,C]: forward state entering / reverse gradient entering each group
};

struct H1Args {
  int B, T, C, S, NG;                  // S segments, NG groups
  const void *q, *k, *v, *log_f, *dy;  // [B,T,C]
  const float *s_in;                   // forward: h0 [B,C]; reverse: dht [B,C]; or null
  float *s_out;                        // forward: hT; reverse: dh0; [B,C] or null
  H1Sum sum;                           // this pass's summaries
  H1Sum fsum;                          // final backward without saved states: the forward summaries
  float *states;                       // [B,S,C] state entering each segment: written by the final
                                       // forward (if not null), read by the final backward (if not null)
  void *y, *dq, *dk, *dv, *dlog_f;     // [B,T,C], the input dtype or (out_f32) float32
  int out_f32 = 0;                     // bfloat16 inputs: write y and the gradients as float32
};

// the workgroup's (b, segment, channel-pair block) and this thread's pair
struct H1Place {
  int b, s, p, len;
  bool valid;
  size_t rowbase;  // element index of the segment's first row, channel 0
};
__device__ __forceinline__ H1Place h1_place(const H1Args &a) {
  const int nb = (a.C / 2 + kH1Pairs - 1) / kH1Pairs;
  H1Place pl;
  pl.b = blockIdx.x / (a.S * nb);
  pl.s = (blockIdx.x / nb) % a.S;
  pl.p = (blockIdx.x % nb) * kH1Pairs + (int)threadIdx.x;
  pl.valid = pl.p < a.C / 2;
  pl.len = max(0, min(kH1Seg, a.T - pl.s * kH1Seg));
  pl.rowbase = ((size_t)pl.b * a.T + (size_t)pl.s * kH1Seg) * a.C;
  return pl;
}

// window over the segment's token rows (rows past the end of the sequence
// read as zero: log f = 0, k v = 0 leave the state unchanged)
template <typename T> __device__ __forceinline__ GBuf h1_win(const void *base, const H1Args &a, const H1Place &pl) {
  return GBuf((const char *)base + pl.rowbase * sizeof(T), (uint32_t)(pl.len * a.C * sizeof(T)));
}

// pass 1: summaries of one group (grid: B x NG x pair blocks of 64; wave j =
// segment 8 g + j).  Forward: A = sum of log f, Bs = end state from zero.
// Reverse: A as forward, Bs = the gradient passed to the segment before, from
// a zero gradient after the segment.
template <typename T, int GM, bool REV>
__global__ __launch_bounds__(64 * kH1Grp) void hgrn1_summary_kernel(H1Args a) {
  __shared__ float2 sA[kH1Grp][64], sB[kH1Grp][64];
  const int nb = (a.C / 2 + 63) / 64;
  const int b = blockIdx.x / (a.NG * nb), g = (blockIdx.x / nb) % a.NG;
  const int j = (int)threadIdx.x / 64, lane = (int)threadIdx.x % 64;
  const int s = g * kH1Grp + j, p = (blockIdx.x % nb) * 64 + lane;
  const bool valid = p < a.C / 2 && s < a.S;
  const int len = s < a.S ? min(kH1Seg, a.T - s * kH1Seg) : 0;
  const size_t rowbase = ((size_t)b * a.T + (size_t)s * kH1Seg) * a.C;
  const uint32_t RB = (uint32_t)a.C * sizeof(T), cb = (uint32_t)(2 * p) * sizeof(T),
                 rows = (uint32_t)(len * a.C * sizeof(T));
  const GBuf bl((const char *)a.log_f + rowbase * sizeof(T), rows);
  const GBuf bx((const char *)(REV ? a.q : a.k) + rowbase * sizeof(T), rows),
      bz((const char *)(REV ? a.dy : a.v) + rowbase * sizeof(T), rows);
  Pack<T, 2> pl_[kH1Seg], px[kH1Seg], pz[kH1Seg];
#pragma unroll
  for (int i = 0; i < kH1Seg; ++i) {
    pl_[i] = bl.template ldpack<T, 2>(i * RB + cb);
    if constexpr (REV || GM == kUntied) px[i] = bx.template ldpack<T, 2>(i * RB + cb);
    pz[i] = bz.template ldpack<T, 2>(i * RB + cb);
  }
  float A[2] = {0.f, 0.f}, h[2] = {0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < kH1Seg; ++jj) {
    const int i = REV ? kH1Seg - 1 - jj : jj;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float lf = floor_logf(to_f32(pl_[i].v[e])), f = __expf(lf);
      A[e] += lf;
      if constexpr (REV) {
        h[e] = f * (to_f32(px[i].v[e]) * to_f32(pz[i].v[e]) + h[e]);  // e_t = f_t (q_t dy_t + e_{t+1})
      } else {
        const float kv = GM == kTied ? tied_k_ex(lf, f) : to_f32(px[i].v[e]);
        h[e] = fmaf(f, h[e], kv * to_f32(pz[i].v[e]));
      }
    }
  }
  sA[j][lane] = make_float2(A[0], A[1]);
  sB[j][lane] = make_float2(h[0], h[1]);
  __syncthreads();
  // exclusive combination with the group's earlier (forward) or later
  // (reverse) segments, folded in the order they act on the carry (forward:
  // left to right; reverse: right to left); the last (first) wave also forms
  // the group total.  Folding segment (A, B) onto (pa, pb): x -> e^A x + B
  // after x -> e^pa x + pb.
  float pa[2] = {0.f, 0.f}, pb[2] = {0.f, 0.f};
  auto fold = [&](int i) {
    const float2 x = sA[i][lane], y = sB[i][lane];
    pb[0] = fmaf(__expf(x.x), pb[0], y.x);
    pb[1] = fmaf(__expf(x.y), pb[1], y.y);
    pa[0] += x.x;
    pa[1] += x.y;
  };
  if constexpr (REV) {
    for (int i = kH1Grp - 1; i > j; --i) fold(i);
  } else {
    for (int i = 0; i < j; ++i) fold(i);
  }
  if (valid) {
    const size_t o = ((size_t)b * a.S + s) * a.C + 2 * p;
    *(float2 *)&a.sum.PA[o] = make_float2(pa[0], pa[1]);
    *(float2 *)&a.sum.PB[o] = make_float2(pb[0], pb[1]);
  }
  if (j == (REV ? 0 : kH1Grp - 1) && p < a.C / 2) {
    fold(j);
    const size_t o = ((size_t)b * a.NG + g) * a.C + 2 * p;
    *(float2 *)&a.sum.GA[o] = make_float2(pa[0], pa[1]);
    *(float2 *)&a.sum.GB[o] = make_float2(pb[0], pb[1]);
  }
}

// pass 2: carries, one thread per (b, channel), serial over the groups.
// Forward: gc[g] = state entering group g (h0 or 0 first); s_out = hT.
// Reverse: gc[g] = gradient entering group g from the right (dht or 0 last);
// s_out = dh0.
template <bool REV>
__global__ __launch_bounds__(256) void hgrn1_carry_kernel(H1Args a) {
  const int nb = (a.C + 255) / 256;
  const int b = blockIdx.x / nb, c = (blockIdx.x % nb) * 256 + (int)threadIdx.x;
  if (c >= a.C) return;
  float x = a.s_in ? a.s_in[(size_t)b * a.C + c] : 0.f;
  const size_t base = (size_t)b * a.NG * a.C + c;
  constexpr int U = 8;  // summaries loaded ahead of their use
  for (int g0 = 0; g0 < a.NG; g0 += U) {
    float Av[U], Bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = g0 + u, g = REV ? a.NG - 1 - jj : jj;
      Av[u] = jj < a.NG ? a.sum.GA[base + (size_t)g * a.C] : 0.f;
      Bv[u] = jj < a.NG ? a.sum.GB[base + (size_t)g * a.C] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = g0 + u, g = REV ? a.NG - 1 - jj : jj;
      if (jj < a.NG) {
        a.sum.gc[base + (size_t)g * a.C] = x;
        x = fmaf(__expf(Av[u]), x, Bv[u]);
      }
    }
  }
  if (a.s_out) a.s_out[(size_t)b * a.C + c] = x;
}

// the carry entering segment s of a thread's pair: the group's carry combined
// with the segment's exclusive in-group prefix (forward) or suffix (reverse)
__device__ __forceinline__ float2 h1_seg_carry(const H1Sum &u, const H1Args &a, int b, int s, int p) {
  const size_t o = ((size_t)b * a.S + s) * a.C + 2 * p;
  const size_t og = ((size_t)b * a.NG + s / kH1Grp) * a.C + 2 * p;
  const float2 pa = *(const float2 *)&u.PA[o], pb = *(const float2 *)&u.PB[o], gc = *(const float2 *)&u.gc[og];
  return make_float2(fmaf(__expf(pa.x), gc.x, pb.x), fmaf(__expf(pa.y), gc.y, pb.y));
}

// pass 3, forward: y from the state entering the segment (TO: the element
// type of y, T or float32 for bfloat16 inputs)
template <typename T, int GM, typename TO = T>
__global__ __launch_bounds__(kH1Pairs) void hgrn1_final_fwd_kernel(H1Args a) {
  const H1Place pl = h1_place(a);
  const uint32_t RB = (uint32_t)a.C * sizeof(T), cb = (uint32_t)(2 * pl.p) * sizeof(T);
  const uint32_t RBO = (uint32_t)a.C * sizeof(TO), cbo = (uint32_t)(2 * pl.p) * sizeof(TO);
  const GBuf bq = h1_win<T>(a.q, a, pl), bk = h1_win<T>(a.k, a, pl), bv = h1_win<T>(a.v, a, pl),
             bl = h1_win<T>(a.log_f, a, pl);
  const GBuf by((char *)a.y + pl.rowbase * sizeof(TO), (uint32_t)(pl.len * a.C * sizeof(TO)));
  Pack<T, 2> pq[kH1Seg], pk[kH1Seg], pv[kH1Seg], pl_[kH1Seg];
#pragma unroll
  for (int i = 0; i < kH1Seg; ++i) {
    pq[i] = bq.template ldpack<T, 2>(i * RB + cb);
    if constexpr (GM == kUntied) pk[i] = bk.template ldpack<T, 2>(i * RB + cb);
    pv[i] = bv.template ldpack<T, 2>(i * RB + cb);
    pl_[i] = bl.template ldpack<T, 2>(i * RB + cb);
  }
  float h[2] = {0.f, 0.f};
  if (pl.valid) {
    const float2 c0 = h1_seg_carry(a.sum, a, pl.b, pl.s, pl.p);
    h[0] = c0.x;
    h[1] = c0.y;
    if (a.states) *(float2 *)&a.states[((size_t)pl.b * a.S + pl.s) * a.C + 2 * pl.p] = c0;
  }
#pragma unroll
  for (int i = 0; i < kH1Seg; ++i) {
    Pack<TO, 2> o;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float lf = floor_logf(to_f32(pl_[i].v[e])), f = __expf(lf);
      const float kv = GM == kTied ? tied_k_ex(lf, f) : to_f32(pk[i].v[e]);
      h[e] = fmaf(f, h[e], kv * to_f32(pv[i].v[e]));
      o.v[e] = from_f32<TO>(to_f32(pq[i].v[e]) * h[e]);
    }
    if (pl.valid) by.template stpack<TO, 2, kStream>(i * RBO + cbo, o);
  }
}

// pass 3, backward: h recomputed in registers from the state entering the
// segment, then the adjoint from the gradient entering it from the right, and
// the gradients.  The segment is walked in two halves of 16 tokens from the
// right (h at the midpoint first), which halves the registers the recomputed
// h and the token rows need; the first half's rows, read for the midpoint,
// wait in LDS until its own gradients, so no row is read twice.
template <typename T, int GM, typename TO = T>
__global__ __launch_bounds__(kH1Pairs) void hgrn1_final_bwd_kernel(H1Args a) {
  constexpr int HS = kH1Seg / 2;
  const H1Place pl = h1_place(a);
  const uint32_t RB = (uint32_t)a.C * sizeof(T), cb = (uint32_t)(2 * pl.p) * sizeof(T);
  // the gradients' rows (TO elements)
  const uint32_t RBO = (uint32_t)a.C * sizeof(TO), cbo = (uint32_t)(2 * pl.p) * sizeof(TO);
  const uint32_t rows = (uint32_t)(pl.len * a.C * sizeof(TO));
  const GBuf bq = h1_win<T>(a.q, a, pl), bk = h1_win<T>(a.k, a, pl), bv = h1_win<T>(a.v, a, pl),
             bl = h1_win<T>(a.log_f, a, pl), bdy = h1_win<T>(a.dy, a, pl);
  const GBuf bdq((char *)a.dq + pl.rowbase * sizeof(TO), rows), bdk((char *)a.dk + pl.rowbase * sizeof(TO), rows),
      bdv((char *)a.dv + pl.rowbase * sizeof(TO), rows), bdl((char *)a.dlog_f + pl.rowbase * sizeof(TO), rows);
  const size_t co = ((size_t)pl.b * a.S + pl.s) * a.C + 2 * pl.p;
  float2 hst = make_float2(0.f, 0.f), gin = make_float2(0.f, 0.f);  // state entering, gradient from the right
  if (pl.valid) {
    hst = a.states ? *(const float2 *)&a.states[co] : h1_seg_carry(a.fsum, a, pl.b, pl.s, pl.p);
    gin = h1_seg_carry(a.sum, a, pl.b, pl.s, pl.p);
  }
  // one token of the forward recurrence
  auto step = [&](const Pack<T, 2> &pk, const Pack<T, 2> &pv, const Pack<T, 2> &plf, float *h) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float lf = floor_logf(to_f32(plf.v[e])), f = __expf(lf);
      const float kv = GM == kTied ? tied_k_ex(lf, f) : to_f32(pk.v[e]);
      h[e] = fmaf(f, h[e], kv * to_f32(pv.v[e]));
    }
  };
  // the first half's k, v and log f: read once for the midpoint and kept in
  // this thread's own LDS slots until its gradients
  __shared__ Pack<T, 2> sk[GM == kUntied ? HS : 1][kH1Pairs], sv[HS][kH1Pairs], sl[HS][kH1Pairs];
  const int me = (int)threadIdx.x;
  float hmid[2] = {hst.x, hst.y};  // h after the first half
  {
    Pack<T, 2> k0[HS], v0[HS], l0[HS];
#pragma unroll
    for (int i = 0; i < HS; ++i) {
      if constexpr (GM == kUntied) k0[i] = bk.template ldpack<T, 2>(i * RB + cb);
      v0[i] = bv.template ldpack<T, 2>(i * RB + cb);
      l0[i] = bl.template ldpack<T, 2>(i * RB + cb);
    }
#pragma unroll
    for (int i = 0; i < HS; ++i) {
      step(k0[i], v0[i], l0[i], hmid);
      if constexpr (GM == kUntied) sk[i][me] = k0[i];
      sv[i][me] = v0[i];
      sl[i][me] = l0[i];
    }
  }
  float e_[2] = {gin.x, gin.y};  // gradient reaching h_t from later tokens, f_{t+1} g_{t+1}
  // the gradients of one half (tokens t0 .. t0 + HS - 1, h0s the state before
  // it), walked from its last token; pk, pv, pl_ hold the half's rows
  auto grads = [&](uint32_t t0, const float *h0s, const Pack<T, 2> *pk, const Pack<T, 2> *pv,
                   const Pack<T, 2> *pl_) {
    Pack<T, 2> pq[HS], pdy[HS];
#pragma unroll
    for (int i = 0; i < HS; ++i) {
      const uint32_t off = (t0 + i) * RB + cb;
      pq[i] = bq.template ldpack<T, 2>(off);
      pdy[i] = bdy.template ldpack<T, 2>(off);
    }
    float hs[HS][2];  // h after each token of the half
    {
      float h[2] = {h0s[0], h0s[1]};
#pragma unroll
      for (int i = 0; i < HS; ++i) {
        step(pk[i], pv[i], pl_[i], h);
        hs[i][0] = h[0];
        hs[i][1] = h[1];
      }
    }
#pragma unroll
    for (int i = HS - 1; i >= 0; --i) {
      Pack<TO, 2> oq, ok, ov, ol;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float lf = floor_logf(to_f32(pl_[i].v[e])), f = __expf(lf);
        const float kv = GM == kTied ? tied_k_ex(lf, f) : to_f32(pk[i].v[e]);
        const float dy = to_f32(pdy[i].v[e]), vv = to_f32(pv[i].v[e]);
        const float g = fmaf(to_f32(pq[i].v[e]), dy, e_[e]);
        const float hp = i ? hs[i - 1][e] : h0s[e];
        const float dk = g * vv;
        oq.v[e] = from_f32<TO>(dy * hs[i][e]);
        ok.v[e] = from_f32<TO>(dk);
        ov.v[e] = from_f32<TO>(g * kv);
        // tied: the total derivative, dlog f - f dk
        ol.v[e] = from_f32<TO>(GM == kTied ? f * (g * hp - dk) : g * f * hp);
        e_[e] = f * g;
      }
      if (pl.valid) {
        const uint32_t off = (t0 + i) * RBO + cbo;
        bdq.template stpack<TO, 2, kStream>(off, oq);
        if constexpr (GM == kUntied) bdk.template stpack<TO, 2, kStream>(off, ok);
        bdv.template stpack<TO, 2, kStream>(off, ov);
        bdl.template stpack<TO, 2, kStream>(off, ol);
      }
    }
  };
  {
    Pack<T, 2> k1[HS], v1[HS], l1[HS];
#pragma unroll
    for (int i = 0; i < HS; ++i) {
      const uint32_t off = (HS + i) * RB + cb;
      if constexpr (GM == kUntied) k1[i] = bk.template ldpack<T, 2>(off);
      v1[i] = bv.template ldpack<T, 2>(off);
      l1[i] = bl.template ldpack<T, 2>(off);
    }
    grads(HS, hmid, k1, v1, l1);
  }
  {
    Pack<T, 2> k0[HS], v0[HS], l0[HS];
#pragma unroll
    for (int i = 0; i < HS; ++i) {
      if constexpr (GM == kUntied) k0[i] = sk[i][me];
      v0[i] = sv[i][me];
      l0[i] = sl[i][me];
    }
    const float hfirst[2] = {hst.x, hst.y};
    grads(0, hfirst, k0, v0, l0);
  }
}

inline int h1_segments(int T) { return (T + kH1Seg - 1) / kH1Seg; }
inline int h1_groups(int S) { return (S + kH1Grp - 1) / kH1Grp; }
// grids in 64-bit arithmetic (the C ABI rejects sizes whose work-items pass 32 bits)
inline dim3 h1_sum_grid(const H1Args &a) { return dim3((unsigned)((long long)a.B * a.NG * ((a.C / 2 + 63) / 64))); }
inline dim3 h1_seg_grid(const H1Args &a) {
  return dim3((unsigned)((long long)a.B * a.S * ((a.C / 2 + kH1Pairs - 1) / kH1Pairs)));
}
inline dim3 h1_chan_grid(const H1Args &a) { return dim3((unsigned)((long long)a.B * ((a.C + 255) / 256))); }

}  // namespace hgrn2
