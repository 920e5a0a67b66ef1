// Device-side building blocks shared by the HGRN2 chunk kernels (gfx950).
//
// Matrix-core convention used throughout (wave64, one 16x16 output tile per
// MFMA group):
//   lane l = 16*g + n   (n = l & 15, g = l >> 4)
//   operand fragment  : 8 values per lane ("slots" 0..7).  For D = A*B the
//                       A fragment of lane l holds A[m = n][k(g, slot)] and the
//                       B fragment holds B[k(g, slot)][col = n].  Any mapping
//                       k(g, slot) works as long as A and B use the same one,
//                       which lets us feed accumulators back in as operands.
//   accumulator       : 4 floats per lane, reg r holds D[row = 4g + r][col = n].
// An MFMA must be issued by the whole wave: lanes without data feed zeros,
// never skip the instruction under a lane-dependent branch.
// bf16 operands go through one v_mfma_f32_16x16x32_bf16; float32 operands go
// through eight v_mfma_f32_16x16x4_f32, slot i in instruction i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace hgrn2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct bf16_t {  // storage type of a bfloat16 value in memory
  uint16_t bits;
};

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x.bits) << 16);
}
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
  bf16_t r;
  r.bits = __builtin_bit_cast(uint16_t, h);
  return r;
}

// Unpack a 16-byte vector of storage values into floats.
template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;  // elements per 16 bytes
  __device__ static __forceinline__ void unpack(const uint4 &u, float *o) {
    o[0] = __uint_as_float(u.x);
    o[1] = __uint_as_float(u.y);
    o[2] = __uint_as_float(u.z);
    o[3] = __uint_as_float(u.w);
  }
};
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void unpack(const uint4 &u, float *o) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// ------------------------------------------------------------ fragments
struct Frag {
  float v[8];
};

__device__ __forceinline__ void frag_zero(Frag &f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = 0.f;
}

__device__ __forceinline__ void acc_zero(f32x4_t &a) { a = f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// D += A * B over one 32-wide k step.  Op = bf16_t: one bf16 MFMA;
// Op = float: eight float32 MFMAs.
template <typename Op> struct Mma;
template <> struct Mma<bf16_t> {
  __device__ static __forceinline__ void run(f32x4_t &acc, const Frag &a, const Frag &b) {
    bf16x8_t x, y;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = (__bf16)a.v[i];
      y[i] = (__bf16)b.v[i];
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  __device__ static __forceinline__ void run(f32x4_t &acc, const Frag &a, const Frag &b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
  }
};

// D += A * B with B carried as an unevaluated bf16 pair (hi + lo), i.e. to
// about 16 significant bits, at the cost of a second MFMA.  Used where two
// products must stay consistent enough for a later difference of them to
// cancel (the intra-chunk parts of dq and dk feed q*dq - k*dk).
template <typename Op> struct MmaSplitB;
template <> struct MmaSplitB<bf16_t> {
  __device__ static __forceinline__ void run(f32x4_t &acc, const Frag &a, const Frag &b) {
    bf16x8_t x, yh, yl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = (__bf16)a.v[i];
      yh[i] = (__bf16)b.v[i];
      yl[i] = (__bf16)(b.v[i] - (float)yh[i]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, yh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, yl, acc, 0, 0, 0);
  }
};
template <> struct MmaSplitB<float> : Mma<float> {};

// Operand pre-converted to the MFMA input type, for fragments reused many times.
template <typename Op> struct PFrag;
template <> struct PFrag<bf16_t> {
  bf16x8_t x;
  __device__ __forceinline__ void set(const Frag &f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (__bf16)f.v[i];
  }
};
template <> struct PFrag<float> {
  float x[8];
  __device__ __forceinline__ void set(const Frag &f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = f.v[i];
  }
};
__device__ __forceinline__ void mma(f32x4_t &acc, const PFrag<bf16_t> &a, const PFrag<bf16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.x, b.x, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t &acc, const PFrag<float> &a, const PFrag<float> &b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x[i], b.x[i], acc, 0, 0, 0);
}

// Operand loads straight from LDS into MFMA-ready registers.
// ld8: 8 consecutive elements (16-byte aligned for bf16, 32 for float).
// ld4x2: slots 0-3 from p0 and 4-7 from p1 (each 4 consecutive elements).
__device__ __forceinline__ PFrag<bf16_t> ld8(const bf16_t *p) {
  PFrag<bf16_t> f;
  f.x = *(const bf16x8_t *)__builtin_assume_aligned(p, 16);
  return f;
}
__device__ __forceinline__ PFrag<float> ld8(const float *p) {
  PFrag<float> f;
  const float4 *q = (const float4 *)__builtin_assume_aligned(p, 16);
  const float4 a = q[0], b = q[1];
  f.x[0] = a.x; f.x[1] = a.y; f.x[2] = a.z; f.x[3] = a.w;
  f.x[4] = b.x; f.x[5] = b.y; f.x[6] = b.z; f.x[7] = b.w;
  return f;
}
__device__ __forceinline__ PFrag<bf16_t> ld4x2(const bf16_t *p0, const bf16_t *p1) {
  union {
    uint2 u[2];
    bf16x8_t v;
  } t;
  t.u[0] = *(const uint2 *)__builtin_assume_aligned(p0, 8);
  t.u[1] = *(const uint2 *)__builtin_assume_aligned(p1, 8);
  PFrag<bf16_t> f;
  f.x = t.v;
  return f;
}
__device__ __forceinline__ PFrag<float> ld4x2(const float *p0, const float *p1) {
  PFrag<float> f;
  const float4 a = *(const float4 *)__builtin_assume_aligned(p0, 16);
  const float4 b = *(const float4 *)__builtin_assume_aligned(p1, 16);
  f.x[0] = a.x; f.x[1] = a.y; f.x[2] = a.z; f.x[3] = a.w;
  f.x[4] = b.x; f.x[5] = b.y; f.x[6] = b.z; f.x[7] = b.w;
  return f;
}
// Zero a fragment on lanes where `valid` is false, without branching (the
// bits are masked, so even inf/NaN inputs become exact zeros).
__device__ __forceinline__ PFrag<bf16_t> masked(const PFrag<bf16_t> &f, bool valid) {
  union {
    bf16x8_t v;
    uint32_t u[4];
  } t;
  t.v = f.x;
  const uint32_t m = valid ? 0xffffffffu : 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) t.u[i] &= m;
  PFrag<bf16_t> r;
  r.x = t.v;
  return r;
}
__device__ __forceinline__ PFrag<float> masked(const PFrag<float> &f, bool valid) {
  const uint32_t m = valid ? 0xffffffffu : 0u;
  PFrag<float> r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.x[i] = __uint_as_float(__float_as_uint(f.x[i]) & m);
  return r;
}
__device__ __forceinline__ void masked(Frag &f, bool valid) {
  const uint32_t m = valid ? 0xffffffffu : 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = __uint_as_float(__float_as_uint(f.v[i]) & m);
}

// Gather 8 elements p[0], p[stride], ..., p[7 * stride] (a column of a
// row-major LDS tile) straight into MFMA form.  The caller passes an
// in-bounds p for every lane; lanes with `valid` false get zeros.  bf16
// elements are loaded as 16-bit halves without a float round trip.
__device__ __forceinline__ PFrag<bf16_t> ldcol8(const bf16_t *p, int stride, bool valid) {
  PFrag<bf16_t> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.x[i] = __builtin_bit_cast(__bf16, p[i * stride].bits);
  return masked(f, valid);
}
__device__ __forceinline__ PFrag<float> ldcol8(const float *p, int stride, bool valid) {
  PFrag<float> f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.x[i] = p[i * stride];
  return masked(f, valid);
}

// 16-byte aligned float4 load from LDS (the tiles guarantee the alignment).
__device__ __forceinline__ float4 ldf4(const float *p) {
  return *(const float4 *)__builtin_assume_aligned(p, 16);
}

template <typename Op> __device__ __forceinline__ PFrag<Op> pfrag_zero() {
  Frag z;
  frag_zero(z);
  PFrag<Op> f;
  f.set(z);
  return f;
}
template <typename Op> __device__ __forceinline__ PFrag<Op> to_pfrag(const Frag &a) {
  PFrag<Op> f;
  f.set(a);
  return f;
}

// D += A * B with B given in float32 and carried as a bf16 hi + lo pair (see
// MmaSplitB); A already in MFMA form.
__device__ __forceinline__ void mma_split(f32x4_t &acc, const PFrag<bf16_t> &a, const Frag &b) {
  bf16x8_t yh, yl;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    yh[i] = (__bf16)b.v[i];
    yl[i] = (__bf16)(b.v[i] - (float)yh[i]);
  }
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.x, yh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.x, yl, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_split(f32x4_t &acc, const PFrag<float> &a, const Frag &b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x[i], b.v[i], acc, 0, 0, 0);
}

// ------------------------------------------------------------ channel-major tiles
// A [rows][C tokens] tile whose 16-byte chunks are rotated along the row by
// (row >> 3) + (row & 7).  Both the scalar column writes of the preparation
// pass (sixteen lanes writing rows 8m + e of one token) and the row-fragment
// reads of the products (sixteen lanes reading rows r..r+15 at one token)
// then touch distinct banks.  TT32: 4-byte elements (rows padded by 16 bytes
// at C = 64); TT16: 2-byte elements.
template <int C> struct TT32 {
  static constexpr int LD = (C == 64) ? C + 4 : C;
  static constexpr int NCH = C / 4;
  __device__ static __forceinline__ int at(int r, int t) {
    return r * LD + ((((t >> 2) + (r >> 3) + (r & 7)) & (NCH - 1)) << 2) + (t & 3);
  }
};
template <int C> struct TT16 {
  static constexpr int LD = C;
  static constexpr int NCH = C / 8;
  __device__ static __forceinline__ int at(int r, int t) {
    return r * LD + ((((t >> 3) + (r >> 3) + (r & 7)) & (NCH - 1)) << 3) + (t & 7);
  }
};
template <typename T, int C> struct TTile;
template <int C> struct TTile<float, C> : TT32<C> {};
template <int C> struct TTile<bf16_t, C> : TT16<C> {};

// 8 consecutive tokens t0..t0+7 (t0 a multiple of 8) of row r of a TTile.
template <int C> __device__ __forceinline__ PFrag<bf16_t> ldT8(const bf16_t *tile, int r, int t0) {
  return ld8(tile + TT16<C>::at(r, t0));
}
template <int C> __device__ __forceinline__ PFrag<float> ldT8(const float *tile, int r, int t0) {
  return ld4x2(tile + TT32<C>::at(r, t0), tile + TT32<C>::at(r, t0 + 4));
}

// ------------------------------------------------------------ misc
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Returns x, but hides its value from the optimiser.  Lane-derived indices
// are passed through this at the start of each phase of a chunk loop so that
// their LDS addresses are recomputed next to their uses instead of being
// hoisted out of the loop and kept live (which spills registers).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Floor for log f: exp(-200) is 0 in float32 and finite differences of
// prefix sums stay finite even for log f = -inf.
constexpr float kLogFloor = -200.f;
// Widest decay range (in nats) inside one 16-token sub-block for which the
// diagonal block is evaluated through the factorised matrix-core form.
// Factors then stay within exp(+-64), far from float32/bf16 overflow and
// underflow; wider blocks are evaluated directly.
constexpr float kDiagLimit = 64.f;

__device__ __forceinline__ float floor_logf(float x) { return fmaxf(x, kLogFloor); }

// How the gate arrives at a kernel (a template argument of every kernel):
//   kUntied  k and log f are separate inputs;
//   kTied    log f is the input and k = 1 - f (HGRN2 summary, paperlayer.ai,
//            §2.1 and §3.2: the input gate tied to the forget gate);
//   kGate    the gate pre-activation z and a per-channel lower bound lb are
//            the inputs: f = lb + (1 - lb) sigmoid(z), k = 1 - f (§2.2: a
//            forget gate that learns a residual above a lower bound);
//   kScalar  one log decay per head and token, log a [B,T,H], shared by every
//            channel of the head (§5: the per-head decay of other models,
//            against HGRN2's per-channel one); k is an input.
enum GateMode : int { kUntied = 0, kTied = 1, kGate = 2, kScalar = 3 };
// k is an input (and the backward writes dk)
constexpr bool reads_k(int gm) { return gm == kUntied || gm == kScalar; }
// k is tied to f (the backward writes the total derivative through log f)
constexpr bool ties_k(int gm) { return gm == kTied || gm == kGate; }

// 1 - e^x for x <= 0 without cancellation: a Taylor polynomial of e^x - 1 to
// the x^7 term for x >= -1/4 (truncation below 4e-10 relative), 1 - e^x below
// (e^x < 0.78 there, so the subtraction loses under two bits)
__device__ __forceinline__ float one_minus_exp(float x, float ex) {
  float p = fmaf(x, 1.f / 5040.f, 1.f / 720.f);
  p = fmaf(x, p, 1.f / 120.f);
  p = fmaf(x, p, 1.f / 24.f);
  p = fmaf(x, p, 1.f / 6.f);
  p = fmaf(x, p, 0.5f);
  p = fmaf(x, p, 1.f);
  return x >= -0.25f ? -x * p : 1.f - ex;
}

// HGRN2's tied input gate k = 1 - f from log f (floored), without
// cancellation for f near 1; ex = e^{log f}.  A zero log f (a row past the
// end of the sequence) gives k = 0.
__device__ __forceinline__ float tied_k_ex(float lf, float ex) { return one_minus_exp(lf, ex); }
__device__ __forceinline__ float tied_k(float log_f) {
  const float lf = floor_logf(log_f);
  return one_minus_exp(lf, __expf(lf));
}

// The gate from its pre-activation, f = lb + (1 - lb) sigmoid(z), evaluated
// with one exponential, one hardware reciprocal and one logarithm: with
// u = e^{-|z|} in (0, 1] and r = 1 / (1 + u),
//   sigmoid(z) = r (z >= 0) or u r (z < 0),  sigmoid(-z) = u r or r,
//   f = (1 + lb u) r (z >= 0)  or  (lb + u) r (z < 0),
// and for lb = 0, z < 0, log f = z + log r (no underflow of u r).  Every
// quantity is a product or sum of positive terms (no cancellation); log f
// carries an absolute error of a few 1e-8, which is what the decays see.
struct GateParts {
  float u, r;
};
__device__ __forceinline__ GateParts gate_parts(float z) {
  GateParts p;
  p.u = __expf(-fabsf(z));
  p.r = __builtin_amdgcn_rcpf(1.f + p.u);
  return p;
}

__device__ __forceinline__ float gate_log_f(float z, float lb) {
  const GateParts p = gate_parts(z);
  const bool neg0 = z < 0.f && lb == 0.f;
  const float arg = neg0 ? p.r : (z >= 0.f ? fmaf(lb, p.u, 1.f) : lb + p.u) * p.r;
  return __logf(arg) + (neg0 ? z : 0.f);
}

// f itself (and k = 1 - f) from the same pieces, with no logarithm: for the
// passes that need only products of f (e^{sums of log f}).  f may underflow
// to 0 where log f is below about -87, where e^{log f} is 0 as well.
__device__ __forceinline__ void gate_f_k(float z, float lb, float &f, float &k) {
  const GateParts p = gate_parts(z);
  const bool neg0 = z < 0.f && lb == 0.f;
  f = neg0 ? p.u * p.r : (z >= 0.f ? fmaf(lb, p.u, 1.f) : lb + p.u) * p.r;
  k = (1.f - lb) * (z >= 0.f ? p.u * p.r : p.r);
}

// k = 1 - f = (1 - lb) sigmoid(-z), without cancellation
__device__ __forceinline__ float gate_k(float z, float lb) {
  const GateParts p = gate_parts(z);
  return (1.f - lb) * (z >= 0.f ? p.u * p.r : p.r);
}

// Factors that turn the total derivative with respect to log f (with k = 1 - f
// tied to it), G = dlog f - f dk, into the gradients of the gate inputs:
//   dz = G (1 - lb) s s' / f,   dlb (one token) = G s' / f,
// with s = sigmoid(z), s' = sigmoid(-z), f = lb + (1 - lb) s.
struct GateGrad {
  float dz, dlb;
};
// from the pre-activation itself
__device__ __forceinline__ GateGrad gate_grad(float z, float lb) {
  const GateParts p = gate_parts(z);
  const float s = z >= 0.f ? p.r : p.u * p.r, sp = z >= 0.f ? p.u * p.r : p.r;
  const float inv = __builtin_amdgcn_rcpf(fmaxf(lb + (1.f - lb) * s, 1e-30f));
  GateGrad g;
  g.dz = lb > 0.f ? (1.f - lb) * s * sp * inv : sp;  // (1 - lb) s / f = 1 when lb = 0
  g.dlb = sp * inv;
  return g;
}
// from log f (floored) when z is no longer at hand: s' = (1 - f) / (1 - lb)
// and (1 - lb) s = f - lb
__device__ __forceinline__ GateGrad gate_grad_lf(float lf, float lb) {
  const float ex = __expf(lf);
  const float f = fmaxf(ex, 1e-30f), omf = one_minus_exp(lf, ex);
  const float inv = __builtin_amdgcn_rcpf((1.f - lb) * f);
  GateGrad g;
  g.dz = lb > 0.f ? (f - lb) * omf * inv : omf;
  g.dlb = omf * inv;
  return g;
}

// log f of a gate input x (floored).  kGate: x is the pre-activation and rows
// past the end of the sequence (valid = false) must decay nothing, log f = 0;
// the other modes read log f itself, which is 0 there already.
template <int GM> __device__ __forceinline__ float lf_of(float x, float lb, bool valid = true) {
  if constexpr (GM == kGate) return valid ? floor_logf(gate_log_f(x, lb)) : 0.f;
  else return floor_logf(x);
}

// log f and k of one token together (the gate pieces computed once):
// kUntied loads k, kTied forms k = 1 - e^{log f}, kGate forms both from z.
template <int GM, typename T>
__device__ __forceinline__ void lf_k(T k, T x, float lb, bool valid, float &lf, float &kv) {
  if constexpr (GM == kGate) {
    const float z = to_f32(x);
    const GateParts p = gate_parts(z);
    const bool neg0 = z < 0.f && lb == 0.f;
    const float arg = neg0 ? p.r : (z >= 0.f ? fmaf(lb, p.u, 1.f) : lb + p.u) * p.r;
    lf = valid ? floor_logf(__logf(arg) + (neg0 ? z : 0.f)) : 0.f;
    kv = (1.f - lb) * (z >= 0.f ? p.u * p.r : p.r);
  } else {
    lf = floor_logf(to_f32(x));
    kv = GM == kTied ? one_minus_exp(lf, __expf(lf)) : to_f32(k);
  }
}

// k of a token: loaded (kUntied) or formed from the gate input x
template <int GM, typename T> __device__ __forceinline__ float k_of(T k, T x, float lb = 0.f) {
  if constexpr (GM == kTied) return tied_k(to_f32(x));
  else if constexpr (GM == kGate) return gate_k(to_f32(x), lb);
  else return to_f32(k);
}

}  // namespace hgrn2
