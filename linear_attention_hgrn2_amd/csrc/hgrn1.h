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
// into segments of kSeg tokens and scanned in three passes with no waits
// between workgroups:
//   1. summaries: per (b, segment, channel) the segment's total log decay A and
//      its end state from zero (forward), or the gradient it passes to the
//      segment before from a zero gradient after it (reverse);
//   2. carries: per (b, channel) a serial pass over the segments' summaries:
//      the state entering each segment (forward; the last one is hT) or the
//      gradient entering it from the right (reverse; the last one is dh0);
//   3. final: every segment again from its carry, writing y (forward) or, with
//      h recomputed in registers from the forward carry, the gradients.
// A thread owns two adjacent channels (one 4-byte bf16 pair, or 8 bytes fp32)
// of one segment; a wave covers 128 consecutive channels of one token row.
#pragma once

#include "tile.h"

namespace hgrn2 {

constexpr int kH1Seg = 32;    // tokens per segment
constexpr int kH1Pairs = 256; // channel pairs per workgroup (four waves)

struct H1Args {
  int B, T, C, S;                      // S = number of segments
  const void *q, *k, *v, *log_f, *dy;  // [B,T,C]
  const float *s_in;                   // forward: h0 [B,C]; reverse: dht [B,C]; or null
  float *A, *Bs;                       // [B,S,C] segment summaries (workspace)
  float *carry;                        // [B,S,C]: forward state before / reverse gradient after each segment
  const float *fcarry;                 // final backward: the forward carries [B,S,C]
  float *s_out;                        // forward: hT; reverse: dh0; [B,C] or null
  void *y, *dq, *dk, *dv, *dlog_f;     // [B,T,C]
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
  pl.len = min(kH1Seg, a.T - pl.s * kH1Seg);
  pl.rowbase = ((size_t)pl.b * a.T + (size_t)pl.s * kH1Seg) * a.C;
  return pl;
}

// window over the segment's token rows (rows past the end of the sequence
// read as zero: log f = 0, k v = 0 leave the state unchanged)
template <typename T> __device__ __forceinline__ GBuf h1_win(const void *base, const H1Args &a, const H1Place &pl) {
  return GBuf((const char *)base + pl.rowbase * sizeof(T), (uint32_t)(pl.len * a.C * sizeof(T)));
}

// pass 1: summaries.  Forward: A = sum of log f, Bs = end state from zero.
// Reverse: A as forward, Bs = the gradient passed to the segment before,
// from a zero gradient after the segment.
template <typename T, int GM, bool REV>
__global__ __launch_bounds__(kH1Pairs) void hgrn1_summary_kernel(H1Args a) {
  const H1Place pl = h1_place(a);
  const uint32_t RB = (uint32_t)a.C * sizeof(T), cb = (uint32_t)(2 * pl.p) * sizeof(T);
  const GBuf bl = h1_win<T>(a.log_f, a, pl);
  const GBuf bx = h1_win<T>(REV ? a.q : a.k, a, pl), bz = h1_win<T>(REV ? a.dy : a.v, a, pl);
  Pack<T, 2> pl_[kH1Seg], px[kH1Seg], pz[kH1Seg];
#pragma unroll
  for (int i = 0; i < kH1Seg; ++i) {
    pl_[i] = bl.template ldpack<T, 2>(i * RB + cb);
    if constexpr (REV || GM == kUntied) px[i] = bx.template ldpack<T, 2>(i * RB + cb);
    pz[i] = bz.template ldpack<T, 2>(i * RB + cb);
  }
  float A[2] = {0.f, 0.f}, h[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kH1Seg; ++j) {
    const int i = REV ? kH1Seg - 1 - j : j;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float lf = floor_logf(to_f32(pl_[i].v[e])), f = __expf(lf);
      A[e] += lf;
      if constexpr (REV) {
        h[e] = f * (to_f32(px[i].v[e]) * to_f32(pz[i].v[e]) + h[e]);  // e_t = f_t (q_t dy_t + e_{t+1})
      } else {
        const float kv = GM == kTied ? -expm1f(lf) : to_f32(px[i].v[e]);
        h[e] = fmaf(f, h[e], kv * to_f32(pz[i].v[e]));
      }
    }
  }
  if (pl.valid) {
    const size_t o = ((size_t)pl.b * a.S + pl.s) * a.C + 2 * pl.p;
    *(float2 *)&a.A[o] = make_float2(A[0], A[1]);
    *(float2 *)&a.Bs[o] = make_float2(h[0], h[1]);
  }
}

// pass 2: carries, one thread per (b, channel), serial over the segments.
// Forward: carry[s] = state before segment s (h0 or 0 first); s_out = hT.
// Reverse: carry[s] = gradient entering segment s from the right (dht or 0
// last); s_out = dh0.
template <bool REV>
__global__ __launch_bounds__(256) void hgrn1_carry_kernel(H1Args a) {
  const int nb = (a.C + 255) / 256;
  const int b = blockIdx.x / nb, c = (blockIdx.x % nb) * 256 + (int)threadIdx.x;
  if (c >= a.C) return;
  float x = a.s_in ? a.s_in[(size_t)b * a.C + c] : 0.f;
  const size_t base = (size_t)b * a.S * a.C + c;
  constexpr int U = 8;  // summaries loaded ahead of their use
  for (int s0 = 0; s0 < a.S; s0 += U) {
    float Av[U], Bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = s0 + u, s = REV ? a.S - 1 - j : j;
      Av[u] = j < a.S ? a.A[base + (size_t)s * a.C] : 0.f;
      Bv[u] = j < a.S ? a.Bs[base + (size_t)s * a.C] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = s0 + u, s = REV ? a.S - 1 - j : j;
      if (j < a.S) {
        a.carry[base + (size_t)s * a.C] = x;
        x = fmaf(__expf(Av[u]), x, Bv[u]);
      }
    }
  }
  if (a.s_out) a.s_out[(size_t)b * a.C + c] = x;
}

// pass 3, forward: y from the state entering the segment
template <typename T, int GM>
__global__ __launch_bounds__(kH1Pairs) void hgrn1_final_fwd_kernel(H1Args a) {
  const H1Place pl = h1_place(a);
  const uint32_t RB = (uint32_t)a.C * sizeof(T), cb = (uint32_t)(2 * pl.p) * sizeof(T);
  const GBuf bq = h1_win<T>(a.q, a, pl), bk = h1_win<T>(a.k, a, pl), bv = h1_win<T>(a.v, a, pl),
             bl = h1_win<T>(a.log_f, a, pl);
  const GBuf by((char *)a.y + pl.rowbase * sizeof(T), (uint32_t)(pl.len * a.C * sizeof(T)));
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
    const float2 c0 = *(const float2 *)&a.carry[((size_t)pl.b * a.S + pl.s) * a.C + 2 * pl.p];
    h[0] = c0.x;
    h[1] = c0.y;
  }
#pragma unroll
  for (int i = 0; i < kH1Seg; ++i) {
    Pack<T, 2> o;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float lf = floor_logf(to_f32(pl_[i].v[e]));
      const float kv = GM == kTied ? -expm1f(lf) : to_f32(pk[i].v[e]);
      h[e] = fmaf(__expf(lf), h[e], kv * to_f32(pv[i].v[e]));
      o.v[e] = from_f32<T>(to_f32(pq[i].v[e]) * h[e]);
    }
    if (pl.valid) by.template stpack<T, 2, kStream>(i * RB + cb, o);
  }
}

// pass 3, backward: h recomputed in registers from the forward carry, then the
// adjoint from the reverse carry, and the gradients
template <typename T, int GM>
__global__ __launch_bounds__(kH1Pairs) void hgrn1_final_bwd_kernel(H1Args a) {
  const H1Place pl = h1_place(a);
  const uint32_t RB = (uint32_t)a.C * sizeof(T), cb = (uint32_t)(2 * pl.p) * sizeof(T);
  const uint32_t rows = (uint32_t)(pl.len * a.C * sizeof(T));
  const GBuf bq = h1_win<T>(a.q, a, pl), bk = h1_win<T>(a.k, a, pl), bv = h1_win<T>(a.v, a, pl),
             bl = h1_win<T>(a.log_f, a, pl), bdy = h1_win<T>(a.dy, a, pl);
  const GBuf bdq((char *)a.dq + pl.rowbase * sizeof(T), rows), bdk((char *)a.dk + pl.rowbase * sizeof(T), rows),
      bdv((char *)a.dv + pl.rowbase * sizeof(T), rows), bdl((char *)a.dlog_f + pl.rowbase * sizeof(T), rows);
  const size_t co = ((size_t)pl.b * a.S + pl.s) * a.C + 2 * pl.p;
  float hs[kH1Seg][2];  // h after each token of the segment
  {
    Pack<T, 2> pk[kH1Seg], pv[kH1Seg], pl_[kH1Seg];
#pragma unroll
    for (int i = 0; i < kH1Seg; ++i) {
      if constexpr (GM == kUntied) pk[i] = bk.template ldpack<T, 2>(i * RB + cb);
      pv[i] = bv.template ldpack<T, 2>(i * RB + cb);
      pl_[i] = bl.template ldpack<T, 2>(i * RB + cb);
    }
    float h[2] = {0.f, 0.f};
    if (pl.valid) {
      const float2 c0 = *(const float2 *)&a.fcarry[co];
      h[0] = c0.x;
      h[1] = c0.y;
    }
#pragma unroll
    for (int i = 0; i < kH1Seg; ++i)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float lf = floor_logf(to_f32(pl_[i].v[e]));
        const float kv = GM == kTied ? -expm1f(lf) : to_f32(pk[i].v[e]);
        h[e] = fmaf(__expf(lf), h[e], kv * to_f32(pv[i].v[e]));
        hs[i][e] = h[e];
      }
  }
  float h0s[2] = {0.f, 0.f}, g_in[2] = {0.f, 0.f};
  if (pl.valid) {
    const float2 c0 = *(const float2 *)&a.fcarry[co], c1 = *(const float2 *)&a.carry[co];
    h0s[0] = c0.x;
    h0s[1] = c0.y;
    g_in[0] = c1.x;
    g_in[1] = c1.y;
  }
  Pack<T, 2> pq[kH1Seg], pk[kH1Seg], pv[kH1Seg], pl_[kH1Seg], pdy[kH1Seg];
#pragma unroll
  for (int i = 0; i < kH1Seg; ++i) {
    pq[i] = bq.template ldpack<T, 2>(i * RB + cb);
    if constexpr (GM == kUntied) pk[i] = bk.template ldpack<T, 2>(i * RB + cb);
    pv[i] = bv.template ldpack<T, 2>(i * RB + cb);
    pl_[i] = bl.template ldpack<T, 2>(i * RB + cb);
    pdy[i] = bdy.template ldpack<T, 2>(i * RB + cb);
  }
  float e_[2] = {g_in[0], g_in[1]};  // gradient reaching h_t from later tokens, f_{t+1} g_{t+1}
#pragma unroll
  for (int i = kH1Seg - 1; i >= 0; --i) {
    Pack<T, 2> oq, ok, ov, ol;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float lf = floor_logf(to_f32(pl_[i].v[e])), f = __expf(lf);
      const float kv = GM == kTied ? -expm1f(lf) : to_f32(pk[i].v[e]);
      const float dy = to_f32(pdy[i].v[e]), vv = to_f32(pv[i].v[e]);
      const float g = fmaf(to_f32(pq[i].v[e]), dy, e_[e]);
      const float hp = i ? hs[i - 1][e] : h0s[e];
      const float dk = g * vv;
      oq.v[e] = from_f32<T>(dy * hs[i][e]);
      ok.v[e] = from_f32<T>(dk);
      ov.v[e] = from_f32<T>(g * kv);
      // tied: the total derivative, dlog f - f dk
      ol.v[e] = from_f32<T>(GM == kTied ? f * (g * hp - dk) : g * f * hp);
      e_[e] = f * g;
    }
    if (pl.valid) {
      bdq.template stpack<T, 2, kStream>(i * RB + cb, oq);
      if constexpr (GM == kUntied) bdk.template stpack<T, 2, kStream>(i * RB + cb, ok);
      bdv.template stpack<T, 2, kStream>(i * RB + cb, ov);
      bdl.template stpack<T, 2, kStream>(i * RB + cb, ol);
    }
  }
}

inline int h1_segments(int T) { return (T + kH1Seg - 1) / kH1Seg; }
inline dim3 h1_seg_grid(const H1Args &a) {
  return dim3((unsigned)(a.B * a.S * ((a.C / 2 + kH1Pairs - 1) / kH1Pairs)));
}
inline dim3 h1_chan_grid(const H1Args &a) { return dim3((unsigned)(a.B * ((a.C + 255) / 256))); }

}  // namespace hgrn2
