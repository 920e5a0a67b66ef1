// LDS tiles and operand loaders for the sequence-parallel chunk kernels (gfx950).
//
// Row tiles hold [rows][W] elements with every row padded by 16 bytes: the
// row stride then moves each row four banks on, so sixteen lanes reading one
// 16-byte chunk of sixteen consecutive rows hit distinct banks, and every
// address of a tile is one per-lane base plus a compile-time offset.
//
// Operand fragments follow the convention in common.h (lane l = 16g + n; an
// operand fragment carries k-slots, an accumulator holds rows 4g + r of
// column n).  Three ways to fill a fragment from a row tile:
//   row8  : A[m][k] with k along the row (8 consecutive elements),
//   tr8   : B[k][n] with k along the rows, one column per lane (the gfx950
//           transposing LDS read, two per fragment for 16-bit data),
//   tr4   : the accumulator arrangement (rows r0 + 4g + j, column n0 + n),
//           which is also the k-slot order of a 16-deep product.
#pragma once

#include "common.h"

namespace hgrn2 {

typedef short v4s_t __attribute__((ext_vector_type(4)));

// Row-major tile of W columns padded by PADB bytes per row.  16 bytes shifts
// consecutive rows by 4 banks (16-row reads of 16 bytes per lane are
// conflict-free); 32 bytes by 8 banks (8-row transposing reads of 32 bytes per
// row are).
template <typename T, int W, int PADB = 16> struct RowTile {
  static constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int LD = W + PADB / (int)sizeof(T);  // row stride in elements
  __device__ static __forceinline__ int at(int r, int c) { return r * LD + c; }
};

// ------------------------------------------------------------ 4-slot fragments (16-deep products)
template <typename Op> struct PFrag4;
template <> struct PFrag4<bf16_t> {
  v4s_t x;
};
template <> struct PFrag4<float> {
  float x[4];
};
__device__ __forceinline__ void mma16(f32x4_t &acc, const PFrag4<bf16_t> &a, const PFrag4<bf16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.x, b.x, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4_t &acc, const PFrag4<float> &a, const PFrag4<float> &b) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x[i], b.x[i], acc, 0, 0, 0);
}
template <typename Op> __device__ __forceinline__ PFrag4<Op> acc_to_frag4(const f32x4_t &a);
template <> __device__ __forceinline__ PFrag4<bf16_t> acc_to_frag4<bf16_t>(const f32x4_t &a) {
  PFrag4<bf16_t> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.x[i] = __builtin_bit_cast(short, (__bf16)a[i]);
  return f;
}
template <> __device__ __forceinline__ PFrag4<float> acc_to_frag4<float>(const f32x4_t &a) {
  PFrag4<float> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.x[i] = a[i];
  return f;
}
// an 8-slot fragment whose slots 0-3 and 4-7 come from two accumulators
template <typename Op> __device__ __forceinline__ PFrag<Op> accs_to_frag(const f32x4_t &a, const f32x4_t &b) {
  Frag f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.v[i] = a[i];
    f.v[4 + i] = b[i];
  }
  return to_pfrag<Op>(f);
}

// ------------------------------------------------------------ loaders
// row8: elements c0..c0+7 of row r (c0 a multiple of 8)
template <int W, int PADB = 16> __device__ __forceinline__ PFrag<bf16_t> row8(const bf16_t *t, int r, int c0) {
  return ld8(t + RowTile<bf16_t, W, PADB>::at(r, c0));
}
template <int W, int PADB = 16> __device__ __forceinline__ PFrag<float> row8(const float *t, int r, int c0) {
  return ld4x2(t + RowTile<float, W, PADB>::at(r, c0), t + RowTile<float, W, PADB>::at(r, c0 + 4));
}

// one transposing read: lane (g, n) receives t[rows(g, j)][n0 + n] for j = 0..3,
// where lane (g, i) of the group supplies row rows(g, i >> 2) at column
// n0 + 4 (i & 3) (gfx950 ds_read_b64_tr_b16 semantics)
template <int W, int PADB = 16>
__device__ __forceinline__ v4s_t tr_read(const bf16_t *t, int row_of_lane, int n0, int lane) {
  const int c = n0 + 4 * (lane & 3);
  const bf16_t *p = t + RowTile<bf16_t, W, PADB>::at(row_of_lane, c);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t *)(p));
}

// tr4: accumulator arrangement, rows r0 + 4g + j, column n0 + n
template <int W, int PADB = 16> __device__ __forceinline__ PFrag4<bf16_t> tr4(const bf16_t *t, int r0, int n0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  PFrag4<bf16_t> f;
  f.x = tr_read<W, PADB>(t, r0 + 4 * g + (i >> 2), n0, i);
  return f;
}
template <int W, int PADB = 16> __device__ __forceinline__ PFrag4<bf16_t> tr4(const bf16_t *t, int r0, int n0) {
  return tr4<W, PADB>(t, r0, n0, lane_id());
}
template <int W, int PADB = 16> __device__ __forceinline__ PFrag4<float> tr4(const float *t, int r0, int n0) {
  const int lane = lane_id(), g = lane >> 4, n = lane & 15;
  PFrag4<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.x[j] = t[RowTile<float, W, PADB>::at(r0 + 4 * g + j, n0 + n)];
  return f;
}

// tr8, standard k order: slots i <-> rows r0 + 8g + i, column n0 + n
template <int W, int PADB = 16> __device__ __forceinline__ PFrag<bf16_t> tr8(const bf16_t *t, int r0, int n0) {
  const int lane = lane_id(), g = lane >> 4, i = lane & 15;
  union {
    v4s_t h[2];
    bf16x8_t v;
  } u;
  u.h[0] = tr_read<W, PADB>(t, r0 + 8 * g + (i >> 2), n0, i);
  u.h[1] = tr_read<W, PADB>(t, r0 + 8 * g + 4 + (i >> 2), n0, i);
  PFrag<bf16_t> f;
  f.x = u.v;
  return f;
}
template <int W, int PADB = 16> __device__ __forceinline__ PFrag<float> tr8(const float *t, int r0, int n0) {
  const int lane = lane_id(), g = lane >> 4, n = lane & 15;
  PFrag<float> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.x[j] = t[RowTile<float, W, PADB>::at(r0 + 8 * g + j, n0 + n)];
  return f;
}

// tr8, accumulator k order: slots 0-3 <-> rows ra + 4g + j, slots 4-7 <-> rows rb + 4g + j
// (pairs with an operand built by accs_to_frag)
template <int W, int PADB = 16> __device__ __forceinline__ PFrag<bf16_t> tr8acc(const bf16_t *t, int ra, int rb, int n0) {
  const int lane = lane_id(), g = lane >> 4, i = lane & 15;
  union {
    v4s_t h[2];
    bf16x8_t v;
  } u;
  u.h[0] = tr_read<W, PADB>(t, ra + 4 * g + (i >> 2), n0, i);
  u.h[1] = tr_read<W, PADB>(t, rb + 4 * g + (i >> 2), n0, i);
  PFrag<bf16_t> f;
  f.x = u.v;
  return f;
}
template <int W, int PADB = 16> __device__ __forceinline__ PFrag<float> tr8acc(const float *t, int ra, int rb, int n0) {
  const int lane = lane_id(), g = lane >> 4, n = lane & 15;
  PFrag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.x[j] = t[RowTile<float, W, PADB>::at(ra + 4 * g + j, n0 + n)];
    f.x[4 + j] = t[RowTile<float, W, PADB>::at(rb + 4 * g + j, n0 + n)];
  }
  return f;
}

// 8 consecutive elements of a row-major global matrix as an operand fragment
__device__ __forceinline__ PFrag<bf16_t> gload8(const bf16_t *p) {
  PFrag<bf16_t> f;
  f.x = *(const bf16x8_t *)__builtin_assume_aligned(p, 16);
  return f;
}
__device__ __forceinline__ PFrag<float> gload8(const float *p) {
  PFrag<float> f;
  const float4 *q = (const float4 *)__builtin_assume_aligned(p, 16);
  const float4 a = q[0], b = q[1];
  f.x[0] = a.x; f.x[1] = a.y; f.x[2] = a.z; f.x[3] = a.w;
  f.x[4] = b.x; f.x[5] = b.y; f.x[6] = b.z; f.x[7] = b.w;
  return f;
}
__device__ __forceinline__ void unpack8(const PFrag<bf16_t> &f, float *o) {
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)f.x[i];
}
__device__ __forceinline__ void unpack8(const PFrag<float> &f, float *o) {
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f.x[i];
}

// ------------------------------------------------------------ small groups of elements
// N consecutive elements moved as one 2-, 4-, 8- or 16-byte access
template <typename T, int N> struct Pack {
  T v[N];
};
template <typename T, int N> __device__ __forceinline__ Pack<T, N> ldpack(const T *p) {
  Pack<T, N> r;
  constexpr int BYTES = (int)sizeof(T) * N;
  if constexpr (BYTES == 2) {
    const uint16_t u = *(const uint16_t *)__builtin_assume_aligned(p, 2);
    __builtin_memcpy(&r, &u, 2);
  } else if constexpr (BYTES == 4) {
    const uint32_t u = *(const uint32_t *)__builtin_assume_aligned(p, 4);
    __builtin_memcpy(&r, &u, 4);
  } else if constexpr (BYTES == 8) {
    const uint2 u = *(const uint2 *)__builtin_assume_aligned(p, 8);
    __builtin_memcpy(&r, &u, 8);
  } else {
    static_assert(BYTES == 16, "pack size");
    const uint4 u = *(const uint4 *)__builtin_assume_aligned(p, 16);
    __builtin_memcpy(&r, &u, 16);
  }
  return r;
}
template <typename T, int N> __device__ __forceinline__ void stpack(T *p, const Pack<T, N> &r) {
  constexpr int BYTES = (int)sizeof(T) * N;
  if constexpr (BYTES == 2) {
    uint16_t u;
    __builtin_memcpy(&u, &r, 2);
    *(uint16_t *)__builtin_assume_aligned(p, 2) = u;
  } else if constexpr (BYTES == 4) {
    uint32_t u;
    __builtin_memcpy(&u, &r, 4);
    *(uint32_t *)__builtin_assume_aligned(p, 4) = u;
  } else if constexpr (BYTES == 8) {
    uint2 u;
    __builtin_memcpy(&u, &r, 8);
    *(uint2 *)__builtin_assume_aligned(p, 8) = u;
  } else {
    static_assert(BYTES == 16, "pack size");
    uint4 u;
    __builtin_memcpy(&u, &r, 16);
    *(uint4 *)__builtin_assume_aligned(p, 16) = u;
  }
}

// four values of T kept packed in registers (bf16: two per 32-bit register)
template <typename T> struct Quad;
template <> struct Quad<bf16_t> {
  uint32_t u[2] = {0u, 0u};
  __device__ __forceinline__ void set(int i, bf16_t x) {
    const uint32_t b = x.bits;
    u[i >> 1] = (i & 1) ? ((u[i >> 1] & 0xffffu) | (b << 16)) : ((u[i >> 1] & 0xffff0000u) | b);
  }
  __device__ __forceinline__ float get(int i) const {
    return __uint_as_float((i & 1) ? (u[i >> 1] & 0xffff0000u) : (u[i >> 1] << 16));
  }
};
template <> struct Quad<float> {
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void set(int i, float x) { v[i] = x; }
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};

// ------------------------------------------------------------ wave-level helpers
// Orders this wave's earlier LDS accesses before its later ones, for data
// one lane writes and another lane of the same wave reads.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// What lane i holds, on every lane (i the same on every lane).
__device__ __forceinline__ float readlane(float x, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i));
}
__device__ __forceinline__ bf16_t readlane(bf16_t x, int i) {
  bf16_t r;
  r.bits = (uint16_t)__builtin_amdgcn_readlane((int)x.bits, i);
  return r;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave (lane 0 first): a
// Kogge-Stone scan within each row of 16 lanes by DPP row shifts, then the
// row totals carried forward by the row broadcasts of lanes 15 and 31.
// Lanes a shift or broadcast does not reach add 0.
template <int CTRL, int ROW_MASK> __device__ __forceinline__ float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false);
  return x + __int_as_float(y);
}
__device__ __forceinline__ float wave_incl_scan(float x) {
  x = dpp_add<0x111, 0xf>(x);  // row_shr:1
  x = dpp_add<0x112, 0xf>(x);  // row_shr:2
  x = dpp_add<0x114, 0xf>(x);  // row_shr:4
  x = dpp_add<0x118, 0xf>(x);  // row_shr:8
  x = dpp_add<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// sum over the four lane groups g (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// A window of a global tensor addressed by 32-bit byte offsets through a
// buffer descriptor (base and size in scalar registers).  Loads at offsets at
// or past `bytes` return zero and stores there are dropped, which masks the
// rows of a partial chunk without branches or per-lane address arithmetic.
constexpr int kStream = 2;  // buffer-store cache policy: non-temporal

struct GBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ GBuf(const void *base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000)) {}
  // soff is a scalar byte offset added to every lane's; unlike off it is not
  // part of the range check, so it only carries offsets known to be in range
  __device__ __forceinline__ uint4 ld16(uint32_t off, uint32_t soff = 0) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
  }
  // stores take a cache policy: kStream (non-temporal) for outputs that are
  // written once and not read again by this kernel
  template <int POL = 0> __device__ __forceinline__ void st16(uint32_t off, const uint4 &v, uint32_t soff = 0) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, off, soff, POL);
  }
  // 8 consecutive elements as a matrix-core operand fragment
  __device__ __forceinline__ PFrag<bf16_t> frag8(const bf16_t *, uint32_t off) const {
    PFrag<bf16_t> f;
    f.x = __builtin_bit_cast(bf16x8_t, ld16(off));
    return f;
  }
  __device__ __forceinline__ PFrag<float> frag8(const float *, uint32_t off) const {
    const float4 a = __builtin_bit_cast(float4, ld16(off)), b = __builtin_bit_cast(float4, ld16(off + 16));
    PFrag<float> f;
    f.x[0] = a.x; f.x[1] = a.y; f.x[2] = a.z; f.x[3] = a.w;
    f.x[4] = b.x; f.x[5] = b.y; f.x[6] = b.z; f.x[7] = b.w;
    return f;
  }
  template <typename T, int N> __device__ __forceinline__ Pack<T, N> ldpack(uint32_t off, uint32_t soff = 0) const {
    Pack<T, N> p;
    constexpr int BYTES = (int)sizeof(T) * N;
    if constexpr (BYTES == 2) {
      const unsigned short u = __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
      __builtin_memcpy(&p, &u, 2);
    } else if constexpr (BYTES == 4) {
      const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
      __builtin_memcpy(&p, &u, 4);
    } else if constexpr (BYTES == 8) {
      const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
      __builtin_memcpy(&p, &u, 8);
    } else if constexpr (BYTES == 16) {
      const uint4 u = ld16(off, soff);
      __builtin_memcpy(&p, &u, 16);
    } else {
      static_assert(BYTES == 32, "pack size");
      const uint4 u0 = ld16(off, soff), u1 = ld16(off + 16, soff);
      __builtin_memcpy(&p, &u0, 16);
      __builtin_memcpy((char *)&p + 16, &u1, 16);
    }
    return p;
  }
  template <typename T, int N, int POL = 0>
  __device__ __forceinline__ void stpack(uint32_t off, const Pack<T, N> &p, uint32_t soff = 0) const {
    constexpr int BYTES = (int)sizeof(T) * N;
    if constexpr (BYTES == 2) {
      unsigned short u;
      __builtin_memcpy(&u, &p, 2);
      __builtin_amdgcn_raw_buffer_store_b16(u, r, off, soff, POL);
    } else if constexpr (BYTES == 4) {
      uint32_t u;
      __builtin_memcpy(&u, &p, 4);
      __builtin_amdgcn_raw_buffer_store_b32(u, r, off, soff, POL);
    } else if constexpr (BYTES == 8) {
      decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)) u;
      __builtin_memcpy(&u, &p, 8);
      __builtin_amdgcn_raw_buffer_store_b64(u, r, off, soff, POL);
    } else {
      static_assert(BYTES == 16, "pack size");
      uint4 u;
      __builtin_memcpy(&u, &p, 16);
      st16<POL>(off, u, soff);
    }
  }
};

// An asynchronous copy of 16 bytes per lane from a buffer window straight into
// LDS: lane i's bytes land at lds_base + 16 i (lds_base is the same for the
// whole wave).  Issued as a plain instruction so that the compiler does not
// make the next LDS access wait for it: the caller waits for the vector-memory
// counter to drain (and synchronises the workgroup) before anything reads the
// destination, and touches nothing there before.  No register receives data.
__device__ __forceinline__ void lds_dma16(const GBuf &b, uint32_t off, const void *lds_base) {
  const uint32_t m =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)lds_base);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds" ::"v"(off), "s"(m), "s"(b.r)
               : "memory", "m0");
#pragma clang diagnostic pop
}
// The log-decay rows of one chunk: one value per channel ([B,T,H,D], element
// c of token t) or, with one decay per head (kScalar), [B,T,H], the head's
// value broadcast over its channels.  Rows past the end read as zero.
template <int GM> struct LfRows {
  GBuf g;
  uint32_t ts;  // bytes from one token to the next
  // elements c .. c + N - 1 of token t (cb = byte offset of element c in a row)
  // (kScalar: the head's value in element 0 only; read the pack through lfe)
  template <typename T, int N> __device__ __forceinline__ Pack<T, N> ld(int t, uint32_t cb) const {
    if constexpr (GM == kScalar) {
      Pack<T, N> p;
      p.v[0] = g.template ldpack<T, 1>((uint32_t)t * ts).v[0];
      return p;
    } else {
      return g.template ldpack<T, N>((uint32_t)t * ts + cb);
    }
  }
};
// Element e of a log-decay pack.  A kScalar pack carries its one value in
// element 0 and nothing is copied into the others, so that no instruction
// right after the load waits for it.
template <int GM, typename T, int N> __device__ __forceinline__ T lfe(const Pack<T, N> &p, int e) {
  return GM == kScalar ? p.v[0] : p.v[e];
}
template <int GM, typename T>
__device__ __forceinline__ LfRows<GM> lf_rows(const void *log_f, int b, int T_, int H, int h, int D, int t0,
                                              int len) {
  const size_t w = GM == kScalar ? 1 : (size_t)D;
  return LfRows<GM>{GBuf((const char *)log_f + (((size_t)b * T_ + t0) * H + h) * w * sizeof(T),
                         (uint32_t)(len * H * w * sizeof(T))),
                    (uint32_t)(H * w * sizeof(T))};
}

// Waits until every vector-memory load of this wave, copies into LDS included, has landed.
__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace hgrn2
