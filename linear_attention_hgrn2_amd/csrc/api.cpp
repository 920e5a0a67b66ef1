// C ABI of the HGRN2 recurrence library: argument checks, dispatch, errors.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing.  The declarations and their contracts are in include/hgrn2.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <mutex>
#include <string>

#include "hgrn2.h"
#include "dispatch.h"

namespace {

thread_local std::string g_last_error;

hgrn2_status fail(hgrn2_status s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

bool valid_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool valid_chunk(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }
// dtype arguments: the input dtype, optionally with HGRN2_OUT_F32 (float32 token outputs)
int in_dtype(int t) { return t & ~HGRN2_OUT_F32; }
bool out_f32(int t) { return (t & HGRN2_OUT_F32) != 0; }
bool valid_dtype(int t) { return in_dtype(t) == HGRN2_F32 || in_dtype(t) == HGRN2_BF16; }
size_t dsize(int t) { return in_dtype(t) == HGRN2_BF16 ? 2 : 4; }  // input element
size_t osize(int t) { return out_f32(t) ? 4 : dsize(t); }          // output element
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// A launch's work-items (workgroups times their size) are counted in 32 bits
// by the dispatch packet, so every kernel's total must stay within this.
constexpr long long kMaxItems = 0xffffffffLL;

struct Range {
  const char *name;
  const void *p;
  size_t bytes;
};

bool overlap(const Range &a, const Range &b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

// Fails when any output range overlaps any input range or another output.
bool check_aliasing(const Range *ins, int nin, const Range *outs, int nout, std::string &msg) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(outs[o], ins[i])) {
        msg = std::string(outs[o].name) + " overlaps input " + ins[i].name;
        return false;
      }
    for (int p = o + 1; p < nout; ++p)
      if (overlap(outs[o], outs[p])) {
        msg = std::string(outs[o].name) + " overlaps output " + outs[p].name;
        return false;
      }
  }
  return true;
}

hgrn2_status check_common(int B, int T, int H, int DK, int DV, int chunk, int dtype) {
  if (B <= 0 || T <= 0 || H <= 0)
    return fail(HGRN2_ERR_INVALID_ARG, "B, T and H must be >= 1");
  if (DK <= 0 || DV <= 0 || chunk <= 0) return fail(HGRN2_ERR_INVALID_ARG, "DK, DV and chunk must be >= 1");
  if ((long long)B * H > (1LL << 30) || (long long)B * T * H > (1LL << 40))
    return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  if (!valid_dtype(dtype))
    return fail(HGRN2_ERR_INVALID_ARG, "dtype must be HGRN2_F32 or HGRN2_BF16 (optionally | HGRN2_OUT_F32)");
  {
    // one workgroup per chunk; 32-bit byte offsets within a chunk's token rows
    // (inputs and outputs) and within one sequence's chunk-boundary states
    const long long N = (T + (long long)chunk - 1) / chunk, E = (long long)dsize(dtype),
                    EO = (long long)osize(dtype);
    if ((long long)B * H * N >= (1LL << 31) || (long long)chunk * H * DK * EO >= (1LL << 32) ||
        (N + 1) * DK * DV * E >= (1LL << 32))
      return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  }
  if (DK != DV || !valid_d(DK))
    return fail(HGRN2_ERR_UNSUPPORTED, "need DK == DV in {16, 32, 64, 128}");
  if (!valid_chunk(chunk)) return fail(HGRN2_ERR_UNSUPPORTED, "chunk must be 16, 32, 64 or 128");
  {
    // work-items of the state scans (workgroups of eight (b, h) at a time) and
    // of the chunk kernels (one workgroup per chunk)
    const long long BH = (long long)B * H, N = (T + (long long)chunk - 1) / chunk;
    const long long scan = (BH + 7) / 8 * 8 * hgrn2::scan_items_per_bh(in_dtype(dtype), DK, chunk);
    const long long chunks = BH * N * hgrn2::chunk_items_per_chunk(chunk);
    if (scan > kMaxItems || chunks > kMaxItems) return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  }
  return HGRN2_OK;
}

hgrn2_status check_ptrs(std::initializer_list<std::pair<const char *, const void *>> req,
                        std::initializer_list<std::pair<const char *, const void *>> opt) {
  for (auto &p : req) {
    if (!p.second) return fail(HGRN2_ERR_INVALID_ARG, std::string(p.first) + " is NULL");
    if (!aligned16(p.second)) return fail(HGRN2_ERR_INVALID_ARG, std::string(p.first) + " is not 16-byte aligned");
  }
  for (auto &p : opt)
    if (p.second && !aligned16(p.second))
      return fail(HGRN2_ERR_INVALID_ARG, std::string(p.first) + " is not 16-byte aligned");
  return HGRN2_OK;
}

hgrn2_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) {
    g_last_error.clear();
    return HGRN2_OK;
  }
  if (e == hipErrorNotSupported) return fail(HGRN2_ERR_UNSUPPORTED, std::string(what) + ": no kernel for these sizes");
  return fail(HGRN2_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

using hgrn2::kGate;
using hgrn2::kScalar;
using hgrn2::kTied;
using hgrn2::kUntied;
using hgrn2::reads_k;

// the adjoint scan reads log f (formed from z in gate mode, one per head with
// a scalar decay) and never k
int adjoint_gm(int gm) { return gm == kGate || gm == kScalar ? gm : kUntied; }

bool fwd_exists(int dtype, int D, int C, int gm = kUntied) {
  return hgrn2::dispatch_scan(dtype, D, C, false, gm, nullptr, nullptr) == hipSuccess &&
         hgrn2::dispatch_scan(dtype, D, C, true, adjoint_gm(gm), nullptr, nullptr) == hipSuccess &&
         hgrn2::dispatch_chunk_fwd(dtype, D, C, gm, nullptr, nullptr) == hipSuccess;
}

bool bwd_exists(int dtype, int D, int C, int gm = kUntied) {
  return hgrn2::dispatch_chunk_bwd(dtype, D, C, gm, nullptr, nullptr) == hipSuccess;
}

// bytes of the per-chunk lower-bound gradient sums (gate mode), [B, H, N, DK] float32
size_t dlb_part_bytes(int B, int T, int H, int DK, int chunk) {
  return (size_t)B * H * (size_t)((T + chunk - 1) / chunk) * DK * sizeof(float);
}

// bytes of the state adjoints at every chunk end, [B, H, N, DK, DV] in the input dtype
size_t adjoint_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype) {
  return (size_t)B * H * (size_t)((T + chunk - 1) / chunk) * DK * DV * dsize(dtype);
}


// ---- the forward without stored chunk-boundary states (sfwd.h): each
// sequence is cut into P segments of G chunks so that about seg_units()
// workgroups walk segments at once; P - 1 segment summaries (P when only the
// final state is wanted) are carried into the state entering every segment.
// The walk fits two workgroups per compute unit where it keeps its state in
// the accumulators (bfloat16, d = 128, chunk 64), one elsewhere; gfx950 parts
// have 256 compute units.  The second workgroup per unit pays for the extra
// summaries only when each segment walks at least kSegMinG chunks.
int seg_units(int dtype, int D, int chunk) { return (dtype == 1 && D == 128 && chunk == 64) ? 512 : 256; }
constexpr long long kSegMinG = 8;

struct SegPlan {
  int P, G, NSEG;
  bool pair;  // planned for two walking workgroups per compute unit
};

SegPlan seg_plan(int dtype, int D, int B, int T, int H, int chunk, bool want_y) {
  const long long BH = (long long)B * H, N = (T + (long long)chunk - 1) / chunk;
  auto plan = [&](long long units) {
    const long long Pt = std::min<long long>(N, std::max<long long>(1, (units + BH - 1) / BH));
    SegPlan sp;
    sp.G = (int)((N + Pt - 1) / Pt);
    sp.P = (int)((N + sp.G - 1) / sp.G);  // no empty segment
    sp.NSEG = want_y ? sp.P - 1 : sp.P;
    sp.pair = units > 256 && BH * sp.P > 256;
    return sp;
  };
  const long long units = seg_units(dtype, D, chunk);
  SegPlan sp = plan(units);
  if (units > 256 && sp.P > 1 && sp.G < kSegMinG) sp = plan(256);
  return sp;
}

bool seg_exists(int dtype, int D, int chunk, int gm) {
  return hgrn2::dispatch_seg_fwd(dtype, D, chunk, gm, nullptr, nullptr) == hipSuccess &&
         hgrn2::dispatch_seg_scan(dtype, D, chunk, gm, nullptr, nullptr) == hipSuccess;
}

// workspace of the forward without stored states: the states entering the
// segments [B,H,NSEG+1,D,D] and the segments' log decay totals [B,H,NSEG,D],
// float32, sized for NSEG = P (the larger case)
size_t seg_ws_bytes(int dtype, int B, int T, int H, int D, int chunk, bool want_y) {
  const SegPlan sp = seg_plan(dtype, D, B, T, H, chunk, want_y);
  const size_t BH = (size_t)B * H;
  return (BH * (sp.NSEG + 1) * D * D + BH * sp.NSEG * D) * sizeof(float);
}

hgrn2_status launch_scan(int dtype, int D, int chunk, bool reverse, int gm, int B, int T, int H, const void *x,
                         const void *z, const void *log_f, const float *lb, const float *s_in, void *states,
                         float *s_out, void *stream, const char *what) {
  hgrn2::ScanArgs sa;
  sa.B = B;
  sa.T = T;
  sa.H = H;
  sa.N = (T + chunk - 1) / chunk;
  sa.x = x;
  sa.z = z;
  sa.log_f = log_f;
  sa.lb = lb;
  sa.s_in = s_in;
  sa.states = states;
  sa.s_out = s_out;
  return hip_status(hgrn2::dispatch_scan(dtype, D, chunk, reverse, gm, &sa, (hipStream_t)stream), what);
}

hgrn2_status launch_chunk_fwd(int dtype, bool of32, int D, int chunk, int gm, int B, int T, int H, const void *q,
                              const void *k, const void *v, const void *log_f, const float *lb, const void *states,
                              void *y, void *stream, const char *what) {
  hgrn2::ChunkFwdArgs ca;
  ca.out_f32 = of32;
  ca.B = B;
  ca.T = T;
  ca.H = H;
  ca.N = (T + chunk - 1) / chunk;
  ca.q = q;
  ca.k = k;
  ca.v = v;
  ca.log_f = log_f;
  ca.lb = lb;
  ca.states = states;
  ca.y = y;
  return hip_status(hgrn2::dispatch_chunk_fwd(dtype, D, chunk, gm, &ca, (hipStream_t)stream), what);
}

hgrn2_status launch_chunk_bwd(int dtype, bool of32, int D, int chunk, int gm, int B, int T, int H, const void *q,
                              const void *k, const void *v, const void *log_f, const float *lb, const void *dy,
                              const void *states, const void *lam, void *dq, void *dk, void *dv, void *dlog_f,
                              float *dlb_part, void *stream, const char *what) {
  hgrn2::ChunkBwdArgs a;
  a.out_f32 = of32;
  a.B = B;
  a.T = T;
  a.H = H;
  a.N = (T + chunk - 1) / chunk;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_f = log_f;
  a.dy = dy;
  a.states = states;
  a.lam = lam;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_f = dlog_f;
  a.lb = lb;
  a.dlb = dlb_part;
  return hip_status(hgrn2::dispatch_chunk_bwd(dtype, D, chunk, gm, &a, (hipStream_t)stream), what);
}

// ---- scratch of the allocation-free backward (hgrn2_bwd_noalloc)
// Device memory of a fixed size in the library's own code object: every GPU
// the library runs on holds one copy until the process ends.  In host code
// the array's name is only a host-side handle; the device address of each
// GPU's copy comes from hipGetSymbolAddress with that GPU current, once, and
// only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[HGRN2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // each device's address of `scratch`, set once

// The current device's address of `scratch` (looked up on the first call on
// that device), or null with the error message set.
void *scratch_ptr(hgrn2_status &st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    st = fail(HGRN2_ERR_HIP, std::string("hgrn2_bwd_noalloc: no current device (") +
                                 (e != hipSuccess ? hipGetErrorString(e) : "device index out of range") + ")");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      st = fail(HGRN2_ERR_HIP, std::string("hgrn2_bwd_noalloc: scratch address: ") + hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  st = HGRN2_OK;
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int hgrn2_abi_version(void) { return HGRN2_ABI_VERSION; }

const char *hgrn2_status_string(int s) {
  switch (s) {
    case HGRN2_OK: return "HGRN2_OK";
    case HGRN2_ERR_INVALID_ARG: return "HGRN2_ERR_INVALID_ARG";
    case HGRN2_ERR_UNSUPPORTED: return "HGRN2_ERR_UNSUPPORTED";
    case HGRN2_ERR_WORKSPACE: return "HGRN2_ERR_WORKSPACE";
    case HGRN2_ERR_HIP: return "HGRN2_ERR_HIP";
  }
  return "HGRN2_UNKNOWN_STATUS";
}

const char *hgrn2_last_error(void) { return g_last_error.c_str(); }

int hgrn2_supported(int D, int chunk, int dtype) {
  if (!valid_d(D) || !valid_chunk(chunk) || !valid_dtype(dtype)) return 0;
  // every bfloat16 kernel also exists with float32 outputs
  dtype = in_dtype(dtype);
  return fwd_exists(dtype, D, chunk) && bwd_exists(dtype, D, chunk) ? 1 : 0;
}

int hgrn2_num_chunks(int T, int chunk) {
  if (T <= 0 || chunk <= 0) return 0;
  return (T + chunk - 1) / chunk;
}

size_t hgrn2_states_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || DK <= 0 || DV <= 0 || chunk <= 0 || !valid_dtype(dtype)) return 0;
  const size_t N = (size_t)hgrn2_num_chunks(T, chunk);
  return (size_t)B * H * (N + 1) * DK * DV * dsize(dtype);
}

size_t hgrn2_fwd_workspace_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                                 int have_states) {
  if (have_states) return 0;
  if (B <= 0 || T <= 0 || H <= 0 || DK <= 0 || DV <= 0 || chunk <= 0 || !valid_dtype(dtype)) return 0;
  if (DK == DV && seg_exists(in_dtype(dtype), DK, chunk, kUntied))
    return seg_ws_bytes(in_dtype(dtype), B, T, H, DK, chunk, false);
  return hgrn2_states_bytes(B, T, H, DK, DV, chunk, dtype);
}

size_t hgrn2_bwd_workspace_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                                 int have_states) {
  if (B <= 0 || T <= 0 || H <= 0 || DK <= 0 || DV <= 0 || chunk <= 0 || !valid_dtype(dtype)) return 0;
  return adjoint_bytes(B, T, H, DK, DV, chunk, dtype) +
         (have_states ? 0 : hgrn2_states_bytes(B, T, H, DK, DV, chunk, dtype));
}

// ---- implementations shared by the entry points of the three gate modes.
// kTied: k = 1 - exp(log f) is formed in the kernels (k is NULL), and the
// backward writes the total dlog f and no dk (dk is NULL).  kGate: the log_f
// pointer carries the pre-activation z, lb [H, DK] the lower bound; log f and
// k are formed in the kernels, and the backward writes dz (through the dlog_f
// pointer) and dlb [H, DK].

static hgrn2_status need_k(int gm, const void *k, const char *name) {
  if (!reads_k(gm)) return HGRN2_OK;
  return check_ptrs({{name, k}}, {});
}

static hgrn2_status need_lb(int gm, const void *lb, const char *name) {
  if (gm != kGate) return HGRN2_OK;
  if (!lb) return fail(HGRN2_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (((uintptr_t)lb & 3u) != 0) return fail(HGRN2_ERR_INVALID_ARG, std::string(name) + " is not 4-byte aligned");
  return HGRN2_OK;
}

static const char *gate_name(int gm) { return gm == kGate ? "z" : gm == kScalar ? "log_a" : "log_f"; }
static const char *dgate_name(int gm) { return gm == kGate ? "dz" : gm == kScalar ? "dlog_a" : "dlog_f"; }
// bytes of the log-decay input (and of its gradient): one per head with a scalar decay
static size_t gate_bytes(int gm, size_t tok, int DK) { return gm == kScalar ? tok / DK : tok; }

static hgrn2_status fwd_impl(int gm, const char *fn, int B, int T, int H, int DK, int DV, int chunk, int dtype,
                             const void *q, const void *k, const void *v, const void *log_f, const float *lb,
                             const float *h0, void *y, float *ht, void *states_out, void *ws, size_t ws_bytes,
                             void *stream) {
  hgrn2_status st = check_common(B, T, H, DK, DV, chunk, dtype);
  if (st != HGRN2_OK) return st;
  const bool of32 = out_f32(dtype);
  const size_t toko = (size_t)B * T * H * DK * osize(dtype);  // bytes of y
  dtype = in_dtype(dtype);
  st = check_ptrs({{"q", q}, {"v", v}, {gate_name(gm), log_f}},
                  {{"h0", h0}, {"y", y}, {"ht", ht}, {"states_out", states_out}, {"ws", ws}});
  if (st == HGRN2_OK) st = need_k(gm, k, "k");
  if (st == HGRN2_OK) st = need_lb(gm, lb, "lower_bound");
  if (st != HGRN2_OK) return st;
  if (!fwd_exists(dtype, DK, chunk, gm))
    return fail(HGRN2_ERR_UNSUPPORTED, "no forward kernel for this D, chunk and dtype");
  const size_t tok = (size_t)B * T * H * DK * dsize(dtype);
  const size_t sb = (size_t)B * H * DK * DV * sizeof(float);
  const size_t lbb = (size_t)H * DK * sizeof(float);
  if (!states_out && seg_exists(dtype, DK, chunk, gm)) {
    // no state is kept for a backward: walk segments, carrying the state on chip
    const SegPlan sp = seg_plan(dtype, DK, B, T, H, chunk, y != nullptr);
    const size_t need = seg_ws_bytes(dtype, B, T, H, DK, chunk, false);
    if (sp.NSEG > 0 && (!ws || ws_bytes < need))
      return fail(HGRN2_ERR_WORKSPACE, "workspace smaller than hgrn2_fwd_workspace_bytes()");
    const Range ins[] = {{"q", q, tok},
                         {"k", reads_k(gm) ? k : nullptr, tok},
                         {"v", v, tok},
                         {gate_name(gm), log_f, gate_bytes(gm, tok, DK)},
                         {"h0", (ht == h0) ? nullptr : h0, sb},
                         {"lower_bound", gm == kGate ? lb : nullptr, lbb}};
    const Range outs[] = {{"y", y, toko}, {"ht", ht, sb}, {"ws", sp.NSEG > 0 ? ws : nullptr, need}};
    std::string msg;
    if (!check_aliasing(ins, 6, outs, 3, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);
    if (ht == h0 && ht && (overlap(Range{"y", y, toko}, Range{"h0", h0, sb}) ||
                           (sp.NSEG > 0 && overlap(Range{"ws", ws, need}, Range{"h0", h0, sb}))))
      return fail(HGRN2_ERR_INVALID_ARG, "an output overlaps h0");
    if (!reads_k(gm)) k = nullptr;
    if (gm != kGate) lb = nullptr;
    const long long BH = (long long)B * H;
    float *sin = (float *)ws;
    float *asum = sp.NSEG > 0 ? sin + (size_t)BH * (sp.NSEG + 1) * DK * DV : nullptr;
    if (sp.NSEG > 0) {
      // the end state of every summarised segment from zero, and its total log decay
      hgrn2::ScanArgs sa;
      sa.B = B;
      sa.T = T;
      sa.H = H;
      sa.N = (T + chunk - 1) / chunk;
      sa.x = k;
      sa.z = v;
      sa.log_f = log_f;
      sa.lb = lb;
      sa.s_in = nullptr;
      sa.states = nullptr;
      sa.s_out = sin;
      sa.NSEG = sp.NSEG;
      sa.G = sp.G;
      sa.asum = asum;
      st = hip_status(hgrn2::dispatch_seg_scan(dtype, DK, chunk, gm, &sa, (hipStream_t)stream), fn);
      if (st != HGRN2_OK) return st;
      // the state entering every segment (and, with no y, the final state)
      st = hip_status(hgrn2::dispatch_seg_carry(DK, (int)BH, sp.NSEG, h0, sin, asum, y ? nullptr : ht,
                                                (hipStream_t)stream),
                      fn);
      if (st != HGRN2_OK || !y) return st;
    }
    hgrn2::SegFwdArgs fa;
    fa.B = B;
    fa.T = T;
    fa.H = H;
    fa.N = (T + chunk - 1) / chunk;
    fa.P = sp.P;
    fa.G = sp.G;
    fa.q = q;
    fa.k = k;
    fa.v = v;
    fa.log_f = log_f;
    fa.lb = lb;
    fa.h0 = sp.P == 1 ? h0 : nullptr;
    fa.sin = sp.P == 1 ? nullptr : sin;
    fa.y = y;
    fa.ht = ht;
    fa.out_f32 = of32;
    fa.pair = sp.pair ? 1 : 0;
    return hip_status(hgrn2::dispatch_seg_fwd(dtype, DK, chunk, gm, &fa, (hipStream_t)stream), fn);
  }
  const size_t stb = hgrn2_states_bytes(B, T, H, DK, DV, chunk, dtype);
  void *states = states_out;
  if (!states) {
    if (!ws || ws_bytes < stb)
      return fail(HGRN2_ERR_WORKSPACE, "states_out is NULL: need a workspace of hgrn2_states_bytes()");
    states = ws;
  }
  // ht may be exactly h0 (each workgroup reads its slice of h0 before it
  // writes the same slice of ht); any other overlap is an error.
  const Range ins[] = {{"q", q, tok},
                       {"k", reads_k(gm) ? k : nullptr, tok},
                       {"v", v, tok},
                       {gate_name(gm), log_f, gate_bytes(gm, tok, DK)},
                       {"h0", (ht == h0) ? nullptr : h0, sb},
                       {"lower_bound", gm == kGate ? lb : nullptr, lbb}};
  const Range outs[] = {{"y", y, toko}, {"ht", ht, sb}, {states_out ? "states_out" : "ws", states, stb}};
  std::string msg;
  if (!check_aliasing(ins, 6, outs, 3, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);
  if (ht == h0 && ht && (overlap(Range{"y", y, toko}, Range{"h0", h0, sb}) ||
                         overlap(Range{"states", states, stb}, Range{"h0", h0, sb})))
    return fail(HGRN2_ERR_INVALID_ARG, "an output overlaps h0");

  if (!reads_k(gm)) k = nullptr;
  if (gm != kGate) lb = nullptr;
  st = launch_scan(dtype, DK, chunk, false, gm, B, T, H, k, v, log_f, lb, h0, states, ht, stream, fn);
  if (st != HGRN2_OK || !y) return st;
  return launch_chunk_fwd(dtype, of32, DK, chunk, gm, B, T, H, q, k, v, log_f, lb, states, y, stream, fn);
}

static hgrn2_status bwd_impl(int gm, const char *fn, int B, int T, int H, int DK, int DV, int chunk, int dtype,
                             const void *q, const void *k, const void *v, const void *log_f, const float *lb,
                             const float *h0, const void *states_in, const void *dy, const float *dht, void *dq,
                             void *dk, void *dv, void *dlog_f, float *dlb, float *dh0, void *ws, size_t ws_bytes,
                             void *stream) {
  hgrn2_status st = check_common(B, T, H, DK, DV, chunk, dtype);
  if (st != HGRN2_OK) return st;
  const bool of32 = out_f32(dtype);
  const size_t toko = (size_t)B * T * H * DK * osize(dtype);  // bytes of each token gradient
  dtype = in_dtype(dtype);
  st = check_ptrs({{"q", q}, {"v", v}, {gate_name(gm), log_f}, {"dy", dy}, {"dq", dq}, {"dv", dv},
                   {dgate_name(gm), dlog_f}},
                  {{"h0", h0}, {"states_in", states_in}, {"dht", dht}, {"dh0", dh0}, {"ws", ws}});
  if (st == HGRN2_OK) st = need_k(gm, k, "k");
  if (st == HGRN2_OK) st = need_k(gm, dk, "dk");
  if (st == HGRN2_OK) st = need_lb(gm, lb, "lower_bound");
  if (st == HGRN2_OK) st = need_lb(gm, dlb, "dlower_bound");
  if (st != HGRN2_OK) return st;
  if (!bwd_exists(dtype, DK, chunk, gm) || !fwd_exists(dtype, DK, chunk, gm))
    return fail(HGRN2_ERR_UNSUPPORTED, "no backward kernel for this D, chunk and dtype");
  const size_t tok = (size_t)B * T * H * DK * dsize(dtype);
  const size_t sb = (size_t)B * H * DK * DV * sizeof(float);
  const size_t stb = hgrn2_states_bytes(B, T, H, DK, DV, chunk, dtype);
  const size_t lamb = adjoint_bytes(B, T, H, DK, DV, chunk, dtype);
  const size_t partb = gm == kGate ? dlb_part_bytes(B, T, H, DK, chunk) : 0;
  const size_t need = lamb + partb + (states_in ? 0 : stb);
  // the lower-bound sum runs H * (DK / min(DK, 64)) workgroups of 1024 work-items
  if (gm == kGate && (long long)H * (DK / (DK < 64 ? DK : 64)) * 1024 > kMaxItems)
    return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  if (!ws || ws_bytes < need)
    return fail(HGRN2_ERR_WORKSPACE, "workspace smaller than hgrn2_bwd_workspace_bytes()");
  if (!reads_k(gm)) k = dk = nullptr;
  if (gm != kGate) lb = dlb = nullptr;
  const size_t lbb = (size_t)H * DK * sizeof(float), gb = gate_bytes(gm, tok, DK), gbo = gate_bytes(gm, toko, DK);
  const void *states = states_in;
  const Range ins[] = {{"q", q, tok},           {"k", k, tok},          {"v", v, tok},
                       {gate_name(gm), log_f, gb}, {"h0", h0, sb},     {"dy", dy, tok},
                       {"dht", dht, sb},        {"states_in", states_in, stb}, {"lower_bound", lb, lbb}};
  const Range outs[] = {{"dq", dq, toko}, {"dk", dk, toko},         {"dv", dv, toko}, {dgate_name(gm), dlog_f, gbo},
                        {"dh0", dh0, sb}, {"dlower_bound", dlb, lbb}, {"ws", ws, need}};
  std::string msg;
  if (!check_aliasing(ins, 9, outs, 7, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);

  // workspace: adjoints, then (gate mode) the per-chunk dlb sums, then (if
  // not given) the recomputed states
  float *part = gm == kGate ? (float *)((char *)ws + lamb) : nullptr;
  if (!states) {
    // recompute the chunk-boundary states with the forward state scan
    void *sws = (char *)ws + lamb + partb;
    st = launch_scan(dtype, DK, chunk, false, gm, B, T, H, k, v, log_f, lb, h0, sws, nullptr, stream, fn);
    if (st != HGRN2_OK) return st;
    states = sws;
  }
  // the state adjoint at every chunk end (reverse scan), then all chunks' gradients
  st = launch_scan(dtype, DK, chunk, true, adjoint_gm(gm), B, T, H, q, dy, log_f, lb, dht, ws, dh0, stream, fn);
  if (st != HGRN2_OK) return st;
  st = launch_chunk_bwd(dtype, of32, DK, chunk, gm, B, T, H, q, k, v, log_f, lb, dy, states, ws, dq, dk, dv, dlog_f,
                        part, stream, fn);
  if (st != HGRN2_OK || gm != kGate) return st;
  return hip_status(hgrn2::dispatch_dlb_reduce(B, H, hgrn2_num_chunks(T, chunk), DK, part, dlb, (hipStream_t)stream),
                    fn);
}

static hgrn2_status fwd_chunk_impl(int gm, const char *fn, int B, int T, int H, int DK, int DV, int chunk,
                                   int dtype, const void *q, const void *k, const void *v, const void *log_f,
                                   const void *states, void *y, void *stream) {
  hgrn2_status st = check_common(B, T, H, DK, DV, chunk, dtype);
  if (st != HGRN2_OK) return st;
  const bool of32 = out_f32(dtype);
  const size_t toko = (size_t)B * T * H * DK * osize(dtype);
  dtype = in_dtype(dtype);
  st = check_ptrs({{"q", q}, {"v", v}, {"log_f", log_f}, {"states", states}, {"y", y}}, {});
  if (st == HGRN2_OK) st = need_k(gm, k, "k");
  if (st != HGRN2_OK) return st;
  if (hgrn2::dispatch_chunk_fwd(dtype, DK, chunk, gm, nullptr, nullptr) != hipSuccess)
    return fail(HGRN2_ERR_UNSUPPORTED, "no forward kernel for this D, chunk and dtype");
  if (!reads_k(gm)) k = nullptr;
  const size_t tok = (size_t)B * T * H * DK * dsize(dtype);
  const size_t stb = hgrn2_states_bytes(B, T, H, DK, DV, chunk, dtype);
  const Range ins[] = {{"q", q, tok}, {"k", k, tok}, {"v", v, tok}, {"log_f", log_f, tok}, {"states", states, stb}};
  const Range outs[] = {{"y", y, toko}};
  std::string msg;
  if (!check_aliasing(ins, 5, outs, 1, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);
  return launch_chunk_fwd(dtype, of32, DK, chunk, gm, B, T, H, q, k, v, log_f, nullptr, states, y, stream, fn);
}

static hgrn2_status bwd_chunk_impl(int gm, const char *fn, int B, int T, int H, int DK, int DV, int chunk,
                                   int dtype, const void *q, const void *k, const void *v, const void *log_f,
                                   const void *states, const void *adjoints, const void *dy, void *dq, void *dk,
                                   void *dv, void *dlog_f, void *stream) {
  hgrn2_status st = check_common(B, T, H, DK, DV, chunk, dtype);
  if (st != HGRN2_OK) return st;
  const bool of32 = out_f32(dtype);
  const size_t toko = (size_t)B * T * H * DK * osize(dtype);
  dtype = in_dtype(dtype);
  st = check_ptrs({{"q", q}, {"v", v}, {"log_f", log_f}, {"states", states}, {"adjoints", adjoints}, {"dy", dy},
                   {"dq", dq}, {"dv", dv}, {"dlog_f", dlog_f}},
                  {});
  if (st == HGRN2_OK) st = need_k(gm, k, "k");
  if (st == HGRN2_OK) st = need_k(gm, dk, "dk");
  if (st != HGRN2_OK) return st;
  if (!bwd_exists(dtype, DK, chunk, gm))
    return fail(HGRN2_ERR_UNSUPPORTED, "no backward kernel for this D, chunk and dtype");
  if (!reads_k(gm)) k = dk = nullptr;
  const size_t tok = (size_t)B * T * H * DK * dsize(dtype);
  const size_t stb = hgrn2_states_bytes(B, T, H, DK, DV, chunk, dtype);
  const size_t lamb = adjoint_bytes(B, T, H, DK, DV, chunk, dtype);
  const Range ins[] = {{"q", q, tok},           {"k", k, tok},   {"v", v, tok},
                       {"log_f", log_f, tok},   {"dy", dy, tok}, {"states", states, stb},
                       {"adjoints", adjoints, lamb}};
  const Range outs[] = {{"dq", dq, toko}, {"dk", dk, toko}, {"dv", dv, toko}, {"dlog_f", dlog_f, toko}};
  std::string msg;
  if (!check_aliasing(ins, 7, outs, 4, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);
  return launch_chunk_bwd(dtype, of32, DK, chunk, gm, B, T, H, q, k, v, log_f, nullptr, dy, states, adjoints, dq, dk,
                          dv, dlog_f, nullptr, stream, fn);
}

static hgrn2_status decode_impl(int gm, const char *fn, int B, int H, int DK, int DV, int dtype, const void *q,
                                const void *k, const void *v, const void *log_f, const float *lb, float *state,
                                void *y, void *stream) {
  if (B <= 0 || H <= 0) return fail(HGRN2_ERR_INVALID_ARG, "B and H must be >= 1");
  if ((long long)B * H > (1LL << 30)) return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  if (!valid_dtype(dtype))
    return fail(HGRN2_ERR_INVALID_ARG, "dtype must be HGRN2_F32 or HGRN2_BF16 (optionally | HGRN2_OUT_F32)");
  if (DK != DV || !valid_d(DK)) return fail(HGRN2_ERR_UNSUPPORTED, "need DK == DV in {16, 32, 64, 128}");
  const bool of32 = out_f32(dtype);
  const size_t veco = (size_t)B * H * DK * osize(dtype);  // bytes of y
  dtype = in_dtype(dtype);
  // one workgroup per (b, h)
  if ((long long)B * H * hgrn2::decode_items_per_bh(DK) > kMaxItems) return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  hgrn2_status st = check_ptrs({{"q", q}, {"v", v}, {gate_name(gm), log_f}, {"state", state}, {"y", y}}, {});
  if (st == HGRN2_OK) st = need_k(gm, k, "k");
  if (st == HGRN2_OK) st = need_lb(gm, lb, "lower_bound");
  if (st != HGRN2_OK) return st;
  if (!reads_k(gm)) k = nullptr;
  if (gm != kGate) lb = nullptr;
  const size_t vec = (size_t)B * H * DK * dsize(dtype);
  const size_t sb = (size_t)B * H * DK * DV * sizeof(float);
  const size_t lbb = (size_t)H * DK * sizeof(float);
  const Range ins[] = {{"q", q, vec}, {"k", k, vec}, {"v", v, vec}, {gate_name(gm), log_f, gate_bytes(gm, vec, DK)},
                       {"lower_bound", lb, lbb}};
  const Range outs[] = {{"y", y, veco}, {"state", state, sb}};
  std::string msg;
  if (!check_aliasing(ins, 5, outs, 2, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);
  hgrn2::DecodeArgs a;
  a.B = B;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_f = log_f;
  a.lb = lb;
  a.state = state;
  a.y = y;
  a.out_f32 = of32;
  return hip_status(hgrn2::dispatch_decode(dtype, DK, gm, a, (hipStream_t)stream), fn);
}

// ---- independent gates

hgrn2_status hgrn2_fwd(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                       const void *k, const void *v, const void *log_f, const float *h0, void *y,
                       float *ht, void *states_out, void *ws, size_t ws_bytes, void *stream) {
  return fwd_impl(kUntied, "hgrn2_fwd", B, T, H, DK, DV, chunk, dtype, q, k, v, log_f, nullptr, h0, y, ht,
                  states_out, ws, ws_bytes, stream);
}

hgrn2_status hgrn2_bwd(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                       const void *k, const void *v, const void *log_f, const float *h0,
                       const void *states_in, const void *dy, const float *dht, void *dq,
                       void *dk, void *dv, void *dlog_f, float *dh0, void *ws, size_t ws_bytes,
                       void *stream) {
  return bwd_impl(kUntied, "hgrn2_bwd", B, T, H, DK, DV, chunk, dtype, q, k, v, log_f, nullptr, h0, states_in, dy,
                  dht, dq, dk, dv, dlog_f, nullptr, dh0, ws, ws_bytes, stream);
}

hgrn2_status hgrn2_bwd_noalloc(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                               const void *k, const void *v, const void *log_f, const float *h0,
                               const void *states_in, const void *dy, const float *dht, void *dq, void *dk,
                               void *dv, void *dlog_f, float *dh0, void *stream) {
  // the sizes are checked before the scratch is looked up: a rejected call
  // makes no HIP call at all
  const size_t need = hgrn2_bwd_workspace_bytes(B, T, H, DK, DV, chunk, dtype, states_in != nullptr);
  if (need > (size_t)HGRN2_NOALLOC_SCRATCH_BYTES) {
    hgrn2_status st = check_common(B, T, H, DK, DV, chunk, dtype);
    if (st != HGRN2_OK) return st;
    return fail(HGRN2_ERR_WORKSPACE, "hgrn2_bwd_noalloc: the backward needs " + std::to_string(need) +
                                         " bytes of scratch, more than its " +
                                         std::to_string((size_t)HGRN2_NOALLOC_SCRATCH_BYTES) +
                                         " (use hgrn2_bwd with a workspace)");
  }
  hgrn2_status st = check_common(B, T, H, DK, DV, chunk, dtype);
  if (st != HGRN2_OK) return st;
  st = check_ptrs({{"q", q}, {"v", v}, {"log_f", log_f}, {"dy", dy}, {"dq", dq}, {"dv", dv}, {"dlog_f", dlog_f},
                   {"k", k}, {"dk", dk}},
                  {{"h0", h0}, {"states_in", states_in}, {"dht", dht}, {"dh0", dh0}});
  if (st != HGRN2_OK) return st;
  void *ws = scratch_ptr(st);
  if (!ws) return st;
  return bwd_impl(kUntied, "hgrn2_bwd_noalloc", B, T, H, DK, DV, chunk, dtype, q, k, v, log_f, nullptr, h0,
                  states_in, dy, dht, dq, dk, dv, dlog_f, nullptr, dh0, ws, (size_t)HGRN2_NOALLOC_SCRATCH_BYTES,
                  stream);
}

hgrn2_status hgrn2_fwd_chunk(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                             const void *k, const void *v, const void *log_f, const void *states, void *y,
                             void *stream) {
  return fwd_chunk_impl(kUntied, "hgrn2_fwd_chunk", B, T, H, DK, DV, chunk, dtype, q, k, v, log_f, states, y,
                        stream);
}

hgrn2_status hgrn2_bwd_adjoint(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                               const void *log_f, const void *dy, const float *dht, void *adjoints, float *dh0,
                               void *stream) {
  hgrn2_status st = check_common(B, T, H, DK, DV, chunk, dtype);
  if (st != HGRN2_OK) return st;
  dtype = in_dtype(dtype);  // no token output
  st = check_ptrs({{"q", q}, {"log_f", log_f}, {"dy", dy}, {"adjoints", adjoints}}, {{"dht", dht}, {"dh0", dh0}});
  if (st != HGRN2_OK) return st;
  if (hgrn2::dispatch_scan(dtype, DK, chunk, true, kUntied, nullptr, nullptr) != hipSuccess)
    return fail(HGRN2_ERR_UNSUPPORTED, "no adjoint scan kernel for this D, chunk and dtype");
  const size_t tok = (size_t)B * T * H * DK * dsize(dtype);
  const size_t sb = (size_t)B * H * DK * DV * sizeof(float);
  const size_t lamb = adjoint_bytes(B, T, H, DK, DV, chunk, dtype);
  const Range ins[] = {{"q", q, tok}, {"log_f", log_f, tok}, {"dy", dy, tok}, {"dht", dht, sb}};
  const Range outs[] = {{"adjoints", adjoints, lamb}, {"dh0", dh0, sb}};
  std::string msg;
  if (!check_aliasing(ins, 4, outs, 2, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);
  return launch_scan(dtype, DK, chunk, true, kUntied, B, T, H, q, dy, log_f, nullptr, dht, adjoints, dh0, stream,
                     "hgrn2_bwd_adjoint");
}

hgrn2_status hgrn2_bwd_chunk(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                             const void *k, const void *v, const void *log_f, const void *states,
                             const void *adjoints, const void *dy, void *dq, void *dk, void *dv, void *dlog_f,
                             void *stream) {
  return bwd_chunk_impl(kUntied, "hgrn2_bwd_chunk", B, T, H, DK, DV, chunk, dtype, q, k, v, log_f, states, adjoints,
                        dy, dq, dk, dv, dlog_f, stream);
}

hgrn2_status hgrn2_decode_step(int B, int H, int DK, int DV, int dtype, const void *q, const void *k,
                               const void *v, const void *log_f, float *state, void *y, void *stream) {
  return decode_impl(kUntied, "hgrn2_decode_step", B, H, DK, DV, dtype, q, k, v, log_f, nullptr, state, y, stream);
}

// ---- tied gates (k = 1 - exp(log f))

hgrn2_status hgrn2_fwd_tied(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                            const void *v, const void *log_f, const float *h0, void *y, float *ht,
                            void *states_out, void *ws, size_t ws_bytes, void *stream) {
  return fwd_impl(kTied, "hgrn2_fwd_tied", B, T, H, DK, DV, chunk, dtype, q, nullptr, v, log_f, nullptr, h0, y, ht,
                  states_out, ws, ws_bytes, stream);
}

hgrn2_status hgrn2_bwd_tied(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                            const void *v, const void *log_f, const float *h0, const void *states_in,
                            const void *dy, const float *dht, void *dq, void *dv, void *dlog_f, float *dh0,
                            void *ws, size_t ws_bytes, void *stream) {
  return bwd_impl(kTied, "hgrn2_bwd_tied", B, T, H, DK, DV, chunk, dtype, q, nullptr, v, log_f, nullptr, h0,
                  states_in, dy, dht, dq, nullptr, dv, dlog_f, nullptr, dh0, ws, ws_bytes, stream);
}

hgrn2_status hgrn2_fwd_chunk_tied(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                                  const void *v, const void *log_f, const void *states, void *y, void *stream) {
  return fwd_chunk_impl(kTied, "hgrn2_fwd_chunk_tied", B, T, H, DK, DV, chunk, dtype, q, nullptr, v, log_f, states,
                        y, stream);
}

hgrn2_status hgrn2_bwd_chunk_tied(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                                  const void *v, const void *log_f, const void *states, const void *adjoints,
                                  const void *dy, void *dq, void *dv, void *dlog_f, void *stream) {
  return bwd_chunk_impl(kTied, "hgrn2_bwd_chunk_tied", B, T, H, DK, DV, chunk, dtype, q, nullptr, v, log_f, states,
                        adjoints, dy, dq, nullptr, dv, dlog_f, stream);
}

hgrn2_status hgrn2_decode_step_tied(int B, int H, int DK, int DV, int dtype, const void *q, const void *v,
                                    const void *log_f, float *state, void *y, void *stream) {
  return decode_impl(kTied, "hgrn2_decode_step_tied", B, H, DK, DV, dtype, q, nullptr, v, log_f, nullptr, state, y,
                     stream);
}

// ---- gate from its pre-activation (f = lb + (1 - lb) sigmoid(z), k = 1 - f)

size_t hgrn2_bwd_gate_workspace_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype, int have_states) {
  const size_t base = hgrn2_bwd_workspace_bytes(B, T, H, DK, DV, chunk, dtype, have_states);
  return base ? base + dlb_part_bytes(B, T, H, DK, chunk) : 0;
}

hgrn2_status hgrn2_fwd_gate(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                            const void *v, const void *z, const float *lower_bound, const float *h0, void *y,
                            float *ht, void *states_out, void *ws, size_t ws_bytes, void *stream) {
  return fwd_impl(kGate, "hgrn2_fwd_gate", B, T, H, DK, DV, chunk, dtype, q, nullptr, v, z, lower_bound, h0, y, ht,
                  states_out, ws, ws_bytes, stream);
}

hgrn2_status hgrn2_bwd_gate(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                            const void *v, const void *z, const float *lower_bound, const float *h0,
                            const void *states_in, const void *dy, const float *dht, void *dq, void *dv, void *dz,
                            float *dlower_bound, float *dh0, void *ws, size_t ws_bytes, void *stream) {
  return bwd_impl(kGate, "hgrn2_bwd_gate", B, T, H, DK, DV, chunk, dtype, q, nullptr, v, z, lower_bound, h0,
                  states_in, dy, dht, dq, nullptr, dv, dz, dlower_bound, dh0, ws, ws_bytes, stream);
}

hgrn2_status hgrn2_decode_step_gate(int B, int H, int DK, int DV, int dtype, const void *q, const void *v,
                                    const void *z, const float *lower_bound, float *state, void *y, void *stream) {
  return decode_impl(kGate, "hgrn2_decode_step_gate", B, H, DK, DV, dtype, q, nullptr, v, z, lower_bound, state, y,
                     stream);
}

// ---- one decay per head (log a [B,T,H])

hgrn2_status hgrn2_fwd_scalar(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                              const void *k, const void *v, const void *log_a, const float *h0, void *y, float *ht,
                              void *states_out, void *ws, size_t ws_bytes, void *stream) {
  return fwd_impl(kScalar, "hgrn2_fwd_scalar", B, T, H, DK, DV, chunk, dtype, q, k, v, log_a, nullptr, h0, y, ht,
                  states_out, ws, ws_bytes, stream);
}

hgrn2_status hgrn2_bwd_scalar(int B, int T, int H, int DK, int DV, int chunk, int dtype, const void *q,
                              const void *k, const void *v, const void *log_a, const float *h0,
                              const void *states_in, const void *dy, const float *dht, void *dq, void *dk, void *dv,
                              void *dlog_a, float *dh0, void *ws, size_t ws_bytes, void *stream) {
  return bwd_impl(kScalar, "hgrn2_bwd_scalar", B, T, H, DK, DV, chunk, dtype, q, k, v, log_a, nullptr, h0,
                  states_in, dy, dht, dq, dk, dv, dlog_a, nullptr, dh0, ws, ws_bytes, stream);
}

hgrn2_status hgrn2_decode_step_scalar(int B, int H, int DK, int DV, int dtype, const void *q, const void *k,
                                      const void *v, const void *log_a, float *state, void *y, void *stream) {
  return decode_impl(kScalar, "hgrn2_decode_step_scalar", B, H, DK, DV, dtype, q, k, v, log_a, nullptr, state, y,
                     stream);
}

// ---- HGRN1 elementwise scan

static hgrn2_status h1_check(int B, int T, int C, int dtype, int tied) {
  if (B <= 0 || T <= 0 || C <= 0) return fail(HGRN2_ERR_INVALID_ARG, "B, T and C must be >= 1");
  if ((long long)B * T * C > (1LL << 40) || (long long)B * C > (1LL << 30))
    return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  if (!valid_dtype(dtype))
    return fail(HGRN2_ERR_INVALID_ARG, "dtype must be HGRN2_F32 or HGRN2_BF16 (optionally | HGRN2_OUT_F32)");
  // a segment's 32 token rows (inputs and outputs) are addressed with 32-bit byte offsets
  if (32LL * C * (long long)osize(dtype) >= (1LL << 32)) return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  if (tied != 0 && tied != 1) return fail(HGRN2_ERR_INVALID_ARG, "tied must be 0 or 1");
  if (C % 2 != 0) return fail(HGRN2_ERR_UNSUPPORTED, "C must be even");
  {
    // work-items of the three passes: summaries (B * groups * ceil(C/128)
    // workgroups of 64 * kH1Grp), carries (B * ceil(C/256) of 256) and the
    // segment pass (B * segments * ceil(C/512) of kH1Pairs)
    const long long S = hgrn2::h1_segments(T), NG = hgrn2::h1_groups((int)S), P = C / 2;
    const long long sum = (long long)B * NG * ((P + 63) / 64) * 64 * hgrn2::kH1Grp;
    const long long carry = (long long)B * ((C + 255) / 256) * 256;
    const long long seg = (long long)B * S * ((P + hgrn2::kH1Pairs - 1) / hgrn2::kH1Pairs) * hgrn2::kH1Pairs;
    if (sum > kMaxItems || carry > kMaxItems || seg > kMaxItems) return fail(HGRN2_ERR_INVALID_ARG, "problem too large");
  }
  return HGRN2_OK;
}

size_t hgrn1_states_bytes(int B, int T, int C) {
  if (B <= 0 || T <= 0 || C <= 0) return 0;
  return (size_t)B * hgrn2::h1_segments(T) * C * sizeof(float);
}

// one direction's summaries: segment prefixes (2 [B,S,C]) and group totals
// and carries (3 [B,NG,C]), float32
static size_t h1_sum_bytes(int B, int T, int C) {
  const int S = hgrn2::h1_segments(T), NG = hgrn2::h1_groups(S);
  return ((size_t)2 * S + (size_t)3 * NG) * B * C * sizeof(float);
}

size_t hgrn1_fwd_workspace_bytes(int B, int T, int C, int have_states) {
  (void)have_states;
  if (B <= 0 || T <= 0 || C <= 0) return 0;
  return h1_sum_bytes(B, T, C);
}

size_t hgrn1_bwd_workspace_bytes(int B, int T, int C, int have_states) {
  if (B <= 0 || T <= 0 || C <= 0) return 0;
  return h1_sum_bytes(B, T, C) * (have_states ? 1 : 2);
}

static hgrn2::H1Sum h1_sum_at(void *base, int B, int T, int C) {
  const int S = hgrn2::h1_segments(T), NG = hgrn2::h1_groups(S);
  const size_t sb = (size_t)B * S * C, gb = (size_t)B * NG * C;
  float *f = (float *)base;
  hgrn2::H1Sum u;
  u.PA = f;
  u.PB = f + sb;
  u.GA = f + 2 * sb;
  u.GB = f + 2 * sb + gb;
  u.gc = f + 2 * sb + 2 * gb;
  return u;
}

static hgrn2::H1Args h1_args(int B, int T, int C) {
  hgrn2::H1Args a{};
  a.B = B;
  a.T = T;
  a.C = C;
  a.S = hgrn2::h1_segments(T);
  a.NG = hgrn2::h1_groups(a.S);
  return a;
}

static hgrn2_status h1_launch(int op, int dtype, int gm, const hgrn2::H1Args &a, void *stream, const char *fn) {
  return hip_status(hgrn2::dispatch_hgrn1(op, dtype, gm, a, (hipStream_t)stream), fn);
}

hgrn2_status hgrn1_fwd(int B, int T, int C, int dtype, int tied, const void *q, const void *k, const void *v,
                       const void *log_f, const float *h0, void *y, float *hT, float *states_out, void *ws,
                       size_t ws_bytes, void *stream) {
  const char *fn = "hgrn1_fwd";
  hgrn2_status st = h1_check(B, T, C, dtype, tied);
  if (st != HGRN2_OK) return st;
  const bool of32 = out_f32(dtype);
  const size_t toko = (size_t)B * T * C * osize(dtype);  // bytes of y
  dtype = in_dtype(dtype);
  st = check_ptrs({{"q", q}, {"v", v}, {"log_f", log_f}, {"y", y}},
                  {{"h0", h0}, {"hT", hT}, {"states_out", states_out}, {"ws", ws}});
  if (st == HGRN2_OK) st = need_k(tied ? kTied : kUntied, k, "k");
  if (st != HGRN2_OK) return st;
  const size_t tok = (size_t)B * T * C * dsize(dtype), sb = hgrn1_states_bytes(B, T, C),
               hb = (size_t)B * C * sizeof(float);
  const size_t need = hgrn1_fwd_workspace_bytes(B, T, C, states_out != nullptr);
  if (!ws || ws_bytes < need) return fail(HGRN2_ERR_WORKSPACE, "workspace smaller than hgrn1_fwd_workspace_bytes()");
  if (tied) k = nullptr;
  const Range ins[] = {{"q", q, tok}, {"k", k, tok}, {"v", v, tok}, {"log_f", log_f, tok}, {"h0", h0, hb}};
  const Range outs[] = {{"y", y, toko}, {"hT", hT, hb}, {"states_out", states_out, sb}, {"ws", ws, need}};
  std::string msg;
  if (!check_aliasing(ins, 5, outs, 4, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);
  hgrn2::H1Args a = h1_args(B, T, C);
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_f = log_f;
  a.s_in = h0;
  a.s_out = hT;
  a.sum = h1_sum_at(ws, B, T, C);
  a.states = states_out;
  a.y = y;
  a.out_f32 = of32;
  const int gm = tied ? kTied : kUntied;
  if ((st = h1_launch(hgrn2::kH1SummaryFwd, dtype, gm, a, stream, fn)) != HGRN2_OK) return st;
  if ((st = h1_launch(hgrn2::kH1CarryFwd, dtype, gm, a, stream, fn)) != HGRN2_OK) return st;
  return h1_launch(hgrn2::kH1FinalFwd, dtype, gm, a, stream, fn);
}

hgrn2_status hgrn1_bwd(int B, int T, int C, int dtype, int tied, const void *q, const void *k, const void *v,
                       const void *log_f, const float *h0, const float *states_in, const void *dy, const float *dht,
                       void *dq, void *dk, void *dv, void *dlog_f, float *dh0, void *ws, size_t ws_bytes,
                       void *stream) {
  const char *fn = "hgrn1_bwd";
  hgrn2_status st = h1_check(B, T, C, dtype, tied);
  if (st != HGRN2_OK) return st;
  const bool of32 = out_f32(dtype);
  const size_t toko = (size_t)B * T * C * osize(dtype);  // bytes of each gradient
  dtype = in_dtype(dtype);
  st = check_ptrs({{"q", q}, {"v", v}, {"log_f", log_f}, {"dy", dy}, {"dq", dq}, {"dv", dv}, {"dlog_f", dlog_f}},
                  {{"h0", h0}, {"states_in", states_in}, {"dht", dht}, {"dh0", dh0}, {"ws", ws}});
  const int gm = tied ? kTied : kUntied;
  if (st == HGRN2_OK) st = need_k(gm, k, "k");
  if (st == HGRN2_OK) st = need_k(gm, dk, "dk");
  if (st != HGRN2_OK) return st;
  const size_t tok = (size_t)B * T * C * dsize(dtype), sb = hgrn1_states_bytes(B, T, C),
               hb = (size_t)B * C * sizeof(float);
  const size_t need = hgrn1_bwd_workspace_bytes(B, T, C, states_in != nullptr);
  if (!ws || ws_bytes < need) return fail(HGRN2_ERR_WORKSPACE, "workspace smaller than hgrn1_bwd_workspace_bytes()");
  if (tied) k = dk = nullptr;
  const Range ins[] = {{"q", q, tok},   {"k", k, tok},   {"v", v, tok},   {"log_f", log_f, tok},
                       {"h0", h0, hb},  {"dy", dy, tok}, {"dht", dht, hb}, {"states_in", states_in, sb}};
  const Range outs[] = {{"dq", dq, toko}, {"dk", dk, toko}, {"dv", dv, toko}, {"dlog_f", dlog_f, toko},
                        {"dh0", dh0, hb}, {"ws", ws, need}};
  std::string msg;
  if (!check_aliasing(ins, 8, outs, 6, msg)) return fail(HGRN2_ERR_INVALID_ARG, msg);
  hgrn2::H1Args a = h1_args(B, T, C);
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_f = log_f;
  a.dy = dy;
  a.out_f32 = of32;
  a.states = const_cast<float *>(states_in);  // read only by the final backward
  if (!states_in) {
    // the forward summaries and group carries; the final backward combines them
    // into the state entering each segment
    a.sum = h1_sum_at((char *)ws + h1_sum_bytes(B, T, C), B, T, C);
    a.s_in = h0;
    a.s_out = nullptr;
    if ((st = h1_launch(hgrn2::kH1SummaryFwd, dtype, gm, a, stream, fn)) != HGRN2_OK) return st;
    if ((st = h1_launch(hgrn2::kH1CarryFwd, dtype, gm, a, stream, fn)) != HGRN2_OK) return st;
    a.fsum = a.sum;
  }
  // reverse: the gradient entering every segment from the right, then the gradients
  a.sum = h1_sum_at(ws, B, T, C);
  a.s_in = dht;
  a.s_out = dh0;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_f = dlog_f;
  if ((st = h1_launch(hgrn2::kH1SummaryRev, dtype, gm, a, stream, fn)) != HGRN2_OK) return st;
  if ((st = h1_launch(hgrn2::kH1CarryRev, dtype, gm, a, stream, fn)) != HGRN2_OK) return st;
  return h1_launch(hgrn2::kH1FinalBwd, dtype, gm, a, stream, fn);
}

}  // extern "C"
