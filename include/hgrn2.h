/*
 * hgrn2.h -- C ABI of the MI355X (gfx950) HGRN2 recurrence library.
 *
 * The operation (HGRN2: Gated Linear RNNs with State Expansion, paperlayer.ai
 * summary, §3.2 "HGRN2"): for every batch element b and head h, a d_k x d_v
 * matrix state S whose rows (decay channels) are scaled by the forget gate
 * f_t = exp(log_f_t) and which receives the outer product of the input-gate
 * vector k_t with the input v_t; the output is the matrix-vector product of
 * the output gate q_t with the state, taken after the update:
 *
 *     S_t = Diag(f_t) S_{t-1} + k_t^T v_t,        y_t = q_t S_t,
 *
 * (HGRN2 ties k = 1 - f, §2.1 and §3.2 p.5; here k is an input of its own so
 * the caller can tie it or not).  Training uses the chunkwise linear-attention
 * form of this recurrence (§3.2 p.5: identical to GLA's, so chunkwise
 * algorithms apply); inference uses the recurrent form one token at a time
 * (§1: linear inference complexity).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates or frees memory, keeps no global state and never synchronises:
 *     every call only enqueues kernels on `stream` (a hipStream_t, or NULL for
 *     the default stream) and returns.
 *   - Token tensors q, k, log_f, v, y and their gradients are contiguous
 *     row-major [B, T, H, D] (D fastest), 16-byte aligned.  States
 *     (h0, ht, dht, dh0, the decode state) are float32 [B, H, DK, DV], DV
 *     fastest, 16-byte aligned.
 *   - dtype: HGRN2_F32 (float) or HGRN2_BF16 (bfloat16 bits), the dtype of
 *     the token inputs (q, k, v, log_f, dy) and of the stored chunk-boundary
 *     states and adjoints.  y and all token gradients have the input dtype,
 *     unless HGRN2_OUT_F32 is or'ed into dtype: then they are float32,
 *     written straight from the float32 accumulators (no bfloat16 rounding
 *     of the results).  "output dtype" below means that choice.
 *     Accumulation is float32.
 *   - Supported sizes: DK == DV == D in {16, 32, 64, 128}; chunk in
 *     {16, 32, 64, 128} (float32 at D = 128 only up to chunk 64: its chunk-128
 *     tiles exceed the 160 KB of LDS); any B, H >= 1 and T >= 1 (a partial
 *     last chunk is masked).
 *     hgrn2_supported() tells which (D, chunk, dtype) combinations have a
 *     kernel; others return HGRN2_ERR_UNSUPPORTED.  Kernels address a
 *     chunk's token rows and one sequence's chunk-boundary states with 32-bit
 *     byte offsets and launch one workgroup per chunk, so with N =
 *     ceil(T / chunk) and E the element size a call returns
 *     HGRN2_ERR_INVALID_ARG ("problem too large") unless B*H*N < 2^31,
 *     chunk*H*D*E < 2^32 and (N + 1)*D*D*E < 2^32 (bf16, D = 128: T up to
 *     about 8.4 million tokens per sequence at chunk 64), B*H <= 2^30,
 *     B*T*H <= 2^40, and every kernel the call launches has fewer than 2^32
 *     work-items (the dispatch counts them in 32 bits): B*H*N*4*chunk for the
 *     chunk kernels, ceil(B*H/8)*8 times at most 2048 (D = 128, chunk 128)
 *     for the state scans, B*H times min(D*D/4, 256) for the decode step.
 *   - Gate precondition: log_f <= 0 and not NaN.  -inf (f = 0) is allowed;
 *     kernels floor log_f at -200, where exp() is already 0 in float32.
 *   - Errors: arguments are checked before anything is launched; on an
 *     argument error nothing is enqueued.  A launch failure returns
 *     HGRN2_ERR_HIP.  hgrn2_last_error() gives a message for the last failing
 *     call on the calling thread.  No C++ exception crosses this boundary.
 *   - Outputs must not alias inputs, except where stated.
 */
#ifndef HGRN2_H
#define HGRN2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HGRN2_ABI_VERSION 9

typedef enum {
  HGRN2_OK = 0,
  HGRN2_ERR_INVALID_ARG = 1, /* null required pointer, size <= 0, misalignment, aliasing */
  HGRN2_ERR_UNSUPPORTED = 2, /* valid arguments with no kernel (D, chunk, dtype)          */
  HGRN2_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required               */
  HGRN2_ERR_HIP = 4          /* the HIP runtime reported an error at launch              */
} hgrn2_status;

typedef enum { HGRN2_F32 = 0, HGRN2_BF16 = 1 } hgrn2_dtype;

/* Or'ed into the dtype argument of any call (HGRN2_BF16 | HGRN2_OUT_F32):
 * the call's token outputs (y of the forwards and decode steps; dq, dk, dv
 * and dlog_f / dz / dlog_a of the backwards) are float32 [.., D] tensors,
 * 4 bytes per element, while its token inputs, dy included, keep the input
 * dtype.  A no-op with HGRN2_F32.  Sizes of states, adjoints and workspaces
 * do not change.  Any other bit set is HGRN2_ERR_INVALID_ARG. */
#define HGRN2_OUT_F32 0x100

/* HGRN2_ABI_VERSION of the built library. */
int hgrn2_abi_version(void);

/* Static English name of a status code. */
const char *hgrn2_status_string(int status);

/* Message describing the last non-OK return on the calling thread ("" if none). */
const char *hgrn2_last_error(void);

/* 1 if a kernel exists for DK = DV = D, this chunk size and this dtype, else 0. */
int hgrn2_supported(int D, int chunk, int dtype);

/* Number of chunks, ceil(T / chunk). */
int hgrn2_num_chunks(int T, int chunk);

/* Bytes of the chunk-boundary state buffer: B*H*(N+1)*DK*DV*sizeof(dtype),
 * N = ceil(T/chunk).  Entry n (n = 0..N) is the state after the first n
 * chunks, rounded to `dtype` (the input dtype of the call), entry 0 being h0
 * (or zero) and entry N the final state.  Layout [B, H, N+1, DK, DV].  The
 * recurrence itself always carries its state in float32; these rounded copies
 * only feed the backward, whose matrix-core products consume the state in the
 * input dtype anyway.  Returns 0 for invalid arguments. */
size_t hgrn2_states_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype);

/* Workspace bytes hgrn2_fwd needs: 0 when the caller passes states_out.  With
 * states_out = NULL, where the forward without stored states exists (chunk
 * 64; bf16 with D in {32, 64, 128}, float32 with D in {32, 64}): the segment
 * summaries, 4 * B*H*((P+1)*DK*DV + P*DK) bytes for the P segments of each
 * sequence (see hgrn2_fwd; a few MB); elsewhere hgrn2_states_bytes(...) (the
 * chunk-boundary states are then written to the workspace, which the
 * per-chunk outputs read). */
size_t hgrn2_fwd_workspace_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                                 int have_states);

/* Workspace bytes hgrn2_bwd needs: the state adjoint at every chunk end,
 * B*H*N*DK*DV*sizeof(dtype), plus hgrn2_states_bytes(...) when the caller
 * passes states_in = NULL (the states are then recomputed into the workspace). */
size_t hgrn2_bwd_workspace_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                                 int have_states);

/*
 * Chunked forward (HGRN2 summary §3.2 p.5, chunkwise form of the recurrence).
 * With states_out (the training forward): two launches on `stream`, a scan
 * over the chunks of every (b, h) that writes each chunk-boundary state, then
 * the outputs of all chunks in parallel from those states (the second is
 * hgrn2_fwd_chunk); with y = NULL only the scan runs.
 * With states_out = NULL (inference, where that path exists: see
 * hgrn2_fwd_workspace_bytes): no chunk-boundary state is stored.  Each
 * sequence is cut into P segments of G chunks, P = about U / (B*H) (at
 * least 1, at most the chunks; U = 512 for bf16 at D 128, whose segment walk
 * runs two workgroups per compute unit, else 256), and up to three launches
 * run: the end state
 * and total decay of each of the first P - 1 segments from a zero state (a
 * scan over the segment), their carry into the state entering every segment,
 * and the segments' outputs, each segment walked chunk by chunk with its state
 * on chip.  With P = 1 only the last launch runs and every input is read once.
 * With y = NULL the first two run over all P segments and give ht.  Otherwise
 * the chunk-boundary states go to ws as with states_out.
 *   q, k, log_f : [B,T,H,DK] dtype      v : [B,T,H,DV] dtype
 *   h0          : [B,H,DK,DV] float32, or NULL for a zero initial state
 *   y           : [B,T,H,DV] output dtype (written), or NULL (states and ht only)
 *   ht          : [B,H,DK,DV] float32 final state, or NULL (not wanted).
 *                 ht may alias h0.
 *   states_out  : hgrn2_states_bytes() bytes of chunk-boundary states (input
 *                 dtype) for the backward, or NULL (then they go to ws).
 *   ws, ws_bytes: workspace (see hgrn2_fwd_workspace_bytes); may be NULL/0
 *                 when states_out is given.
 */
hgrn2_status hgrn2_fwd(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                       const void *q, const void *k, const void *v, const void *log_f,
                       const float *h0, void *y, float *ht, void *states_out, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * Chunked backward by reverse chunk scan of the state adjoint, for the loss
 * L = sum(y * dy) + sum(ht * dht).  Launches on `stream`: the forward state
 * scan when states_in is NULL, then hgrn2_bwd_adjoint (adjoints into the
 * front of ws), then hgrn2_bwd_chunk.  Gradients are partial derivatives with k
 * and log_f independent; a caller that ties k = 1 - exp(log_f) adds
 * -exp(log_f) * dk to dlog_f itself.
 *   q, k, v, log_f, h0 : as passed to hgrn2_fwd (same chunk size)
 *   states_in   : the states_out of that hgrn2_fwd call, or NULL (recompute;
 *                 needs a workspace of hgrn2_states_bytes())
 *   dy          : [B,T,H,DV] dtype
 *   dht         : [B,H,DK,DV] float32, or NULL (zero)
 *   dq, dk, dlog_f : [B,T,H,DK] output dtype (written)
 *   dv          : [B,T,H,DV] output dtype (written)
 *   dh0         : [B,H,DK,DV] float32 (written), or NULL (not wanted)
 *   ws, ws_bytes: workspace of at least hgrn2_bwd_workspace_bytes() bytes
 *                 (always needed: it holds the adjoints).
 */
hgrn2_status hgrn2_bwd(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                       const void *q, const void *k, const void *v, const void *log_f,
                       const float *h0, const void *states_in, const void *dy,
                       const float *dht, void *dq, void *dk, void *dv, void *dlog_f,
                       float *dh0, void *ws, size_t ws_bytes, void *stream);

/*
 * hgrn2_bwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight training or serving loops,
 * harnesses that forbid allocation).  Same arguments, checks, kernels and
 * results as hgrn2_bwd (bit for bit), except ws and ws_bytes: the adjoints (and
 * the recomputed chunk-boundary states when states_in is NULL) go to a
 * scratch array of HGRN2_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * every GPU it runs on until the process ends (256 MiB: the adjoints of
 * B8 H16 T4096 at D = 128, chunk 64, bf16, with the states passed in).  A call
 * that needs more returns HGRN2_ERR_WORKSPACE before anything is enqueued.
 * The call itself allocates nothing.  Every call on one GPU uses that GPU's
 * one scratch array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller; consecutive calls
 * on one stream are safe.  Nothing in the scratch needs to start at zero.
 */
#define HGRN2_NOALLOC_SCRATCH_BYTES (256u << 20)
hgrn2_status hgrn2_bwd_noalloc(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                               const void *q, const void *k, const void *v, const void *log_f,
                               const float *h0, const void *states_in, const void *dy,
                               const float *dht, void *dq, void *dk, void *dv, void *dlog_f,
                               float *dh0, void *stream);

/*
 * The single launches that hgrn2_fwd and hgrn2_bwd are made of, for callers
 * that schedule or time them one by one.  Same conventions and checks as the
 * composite calls; each enqueues exactly one kernel.
 *
 * hgrn2_fwd_chunk: y of every chunk from the chunk-boundary states that
 * hgrn2_fwd(..., y = NULL, states_out = states, ...) wrote (chunkwise form,
 * HGRN2 summary §3.2 p.5): y = (in-chunk decayed scores) v + (q scaled by the
 * in-chunk cumulative decay) S_{start of chunk}.
 *   states : [B,H,N+1,DK,DV] dtype, read      y : [B,T,H,DV] output dtype, written
 */
hgrn2_status hgrn2_fwd_chunk(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                             const void *q, const void *k, const void *v, const void *log_f,
                             const void *states, void *y, void *stream);

/*
 * hgrn2_bwd_adjoint: the gradient of the loss with respect to the state at
 * every chunk end, by a reverse scan over the chunks (the adjoint of the
 * recurrence: Lambda_{t-1} = Diag(f_t) Lambda_t + q_t^T dy_t, from
 * Lambda_T = dht).
 *   adjoints : [B,H,N,DK,DV] dtype (written): entry n is the adjoint of the
 *              state after chunk n+1 (n = 0..N-1), B*H*N*DK*DV*sizeof(dtype)
 *              bytes (= hgrn2_bwd_workspace_bytes(..., have_states = 1)).
 *   dht      : [B,H,DK,DV] float32, or NULL (zero)
 *   dh0      : [B,H,DK,DV] float32 (written), or NULL (not wanted)
 */
hgrn2_status hgrn2_bwd_adjoint(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                               const void *q, const void *log_f, const void *dy,
                               const float *dht, void *adjoints, float *dh0, void *stream);

/*
 * hgrn2_bwd_chunk: dq, dk, dv and dlog_f of every chunk, all chunks in
 * parallel, from the chunk-boundary states (states, as for hgrn2_fwd_chunk)
 * and the adjoints that hgrn2_bwd_adjoint wrote.  Outputs as for hgrn2_bwd.
 */
hgrn2_status hgrn2_bwd_chunk(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                             const void *q, const void *k, const void *v, const void *log_f,
                             const void *states, const void *adjoints, const void *dy, void *dq,
                             void *dk, void *dv, void *dlog_f, void *stream);

/*
 * One recurrent decode step (HGRN2 summary §1, recurrent inference): for every
 * (b, h), S <- Diag(exp(log_f)) S + k^T v in place, then y = q S.
 *   q, k, log_f : [B,H,DK] dtype      v : [B,H,DV] dtype
 *   state       : [B,H,DK,DV] float32, read and overwritten
 *   y           : [B,H,DV] output dtype (written)
 * Any D in {16, 32, 64, 128} with DK == DV; dtype F32 or BF16 (| HGRN2_OUT_F32).
 */
hgrn2_status hgrn2_decode_step(int B, int H, int DK, int DV, int dtype, const void *q,
                               const void *k, const void *v, const void *log_f,
                               float *state, void *y, void *stream);

/*
 * Tied gates.  HGRN2 ties the input gate to the forget gate, k = 1 - f
 * (HGRN2 summary §2.1 and §3.2 p.5).  These entry points take no k: the
 * kernels form k = -expm1(log_f) from log_f itself (exact near f = 1), which
 * saves one token tensor of reads per launch that used k.  The backward
 * returns the total derivative with respect to log_f,
 *     dlog_f = (partial through the decay) - exp(log_f) * (partial wrt k),
 * and no dk.  Everything else (layouts, states, workspaces, errors) is as for
 * the untied calls with the same names.
 */
hgrn2_status hgrn2_fwd_tied(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                            const void *q, const void *v, const void *log_f, const float *h0,
                            void *y, float *ht, void *states_out, void *ws, size_t ws_bytes,
                            void *stream);
hgrn2_status hgrn2_bwd_tied(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                            const void *q, const void *v, const void *log_f, const float *h0,
                            const void *states_in, const void *dy, const float *dht, void *dq,
                            void *dv, void *dlog_f, float *dh0, void *ws, size_t ws_bytes,
                            void *stream);
hgrn2_status hgrn2_fwd_chunk_tied(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                                  const void *q, const void *v, const void *log_f,
                                  const void *states, void *y, void *stream);
hgrn2_status hgrn2_bwd_chunk_tied(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                                  const void *q, const void *v, const void *log_f,
                                  const void *states, const void *adjoints, const void *dy,
                                  void *dq, void *dv, void *dlog_f, void *stream);
hgrn2_status hgrn2_decode_step_tied(int B, int H, int DK, int DV, int dtype, const void *q,
                                    const void *v, const void *log_f, float *state, void *y,
                                    void *stream);

/*
 * Gate from its pre-activation.  HGRN's forget gate has an additive lower
 * bound per layer and learns a residual above it (HGRN2 summary §2.2: lower
 * bounds built per layer, the forget gate learning residuals above them); with
 * the input gate tied as above:
 *     f = lb + (1 - lb) * sigmoid(z),        k = 1 - f = (1 - lb) * sigmoid(-z).
 * These entry points take the pre-activation z [B, T, H, DK] (input dtype, in
 * place of log_f) and the lower bound lower_bound [H, DK] (float32, one value
 * per head channel, 0 <= lb < 1; a scalar bound is the same value everywhere;
 * 4-byte aligned) and form log f and k in the kernels, so no log_f or k
 * tensor is ever written or read.  Rows past the end of the sequence decay
 * nothing.  Precondition: z finite.
 *
 * hgrn2_bwd_gate returns, with G = dlog_f - f dk the total derivative through
 * log f (the tied-gate backward's dlog_f) and s = sigmoid(z), s' = sigmoid(-z):
 *     dz            = G (1 - lb) s s' / f                    [B, T, H, DK], output dtype
 *     dlower_bound  = sum over b and t of G s' / f            [H, DK], float32, overwritten
 * and no dk.  dlower_bound is summed per chunk into the workspace and then over
 * chunks in a fixed order (repeat runs agree bit for bit).  Its workspace is
 * hgrn2_bwd_gate_workspace_bytes() (the untied size plus B*H*N*DK floats).
 * For lb = 0 and z below about -88, f underflows in float32 and the dlb term
 * of that token is infinite (its exact value exceeds the float32 range).
 * Everything else (layouts, states, errors) is as for the untied calls.
 */
size_t hgrn2_bwd_gate_workspace_bytes(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                                      int have_states);
hgrn2_status hgrn2_fwd_gate(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                            const void *q, const void *v, const void *z, const float *lower_bound,
                            const float *h0, void *y, float *ht, void *states_out, void *ws,
                            size_t ws_bytes, void *stream);
hgrn2_status hgrn2_bwd_gate(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                            const void *q, const void *v, const void *z, const float *lower_bound,
                            const float *h0, const void *states_in, const void *dy,
                            const float *dht, void *dq, void *dv, void *dz, float *dlower_bound,
                            float *dh0, void *ws, size_t ws_bytes, void *stream);
hgrn2_status hgrn2_decode_step_gate(int B, int H, int DK, int DV, int dtype, const void *q,
                                    const void *v, const void *z, const float *lower_bound,
                                    float *state, void *y, void *stream);

/*
 * One decay per head.  Other models share one forget-gate value across a
 * head's state (HGRN2 summary §5: Mamba2, xLSTM and Gated Retention share one
 * decay per head for tensor-core efficiency, where HGRN2 keeps one per
 * dimension).  These entry points take log_a [B, T, H] (input dtype; decode:
 * [B, H]) in place of log_f, the same for every row of head h's state:
 *     S_t = a_t S_{t-1} + k_t^T v_t,        y_t = q_t S_t,
 * with k an input.  The backward returns dlog_a [B, T, H] (output dtype), the
 * sum over the head's channels of the per-channel derivative, and dk.  The
 * log-decay bytes shrink by D.  Everything else (layouts, states, workspaces,
 * errors, gate preconditions on log_a) is as for the untied calls.
 */
hgrn2_status hgrn2_fwd_scalar(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                              const void *q, const void *k, const void *v, const void *log_a,
                              const float *h0, void *y, float *ht, void *states_out, void *ws,
                              size_t ws_bytes, void *stream);
hgrn2_status hgrn2_bwd_scalar(int B, int T, int H, int DK, int DV, int chunk, int dtype,
                              const void *q, const void *k, const void *v, const void *log_a,
                              const float *h0, const void *states_in, const void *dy,
                              const float *dht, void *dq, void *dk, void *dv, void *dlog_a,
                              float *dh0, void *ws, size_t ws_bytes, void *stream);
hgrn2_status hgrn2_decode_step_scalar(int B, int H, int DK, int DV, int dtype, const void *q,
                                      const void *k, const void *v, const void *log_a, float *state,
                                      void *y, void *stream);

/*
 * HGRN1: the elementwise gated linear recurrence that HGRN2 expands (HGRN2
 * summary §2.1), per channel c of [B, T, C] tensors:
 *     h_t[c] = f_t[c] h_{t-1}[c] + k_t[c] v_t[c],     y_t[c] = q_t[c] h_t[c],
 * f = exp(log_f), q the output gate, v the input; tied = 1 ties the input gate
 * to the forget gate, k = 1 - f (HGRN1's own form; k and dk are then NULL and
 * dlog_f is the total derivative dlog_f - f dk).  It is HGRN2's recurrence
 * with d_k = d_v = 1.  C = the channels of a token row (heads times head
 * width), any even C >= 2 with 32*C*E < 2^32 (E the element size: a
 * segment's rows are addressed with 32-bit byte offsets); any B, T >= 1 with
 * B*C <= 2^30 and B*T*C <= 2^40.  Token tensors [B, T, C] in dtype (y and
 * the gradients in the output dtype, as for the HGRN2 calls), 16-byte
 * aligned; h0, hT, dht, dh0 float32 [B, C] (optional, NULL = zero / not
 * written).
 *
 * The sequence is scanned in segments of 32 tokens, eight segments to a
 * group.  states_out (optional) receives the state entering every segment,
 * float32 [B, S, C] with S = ceil(T / 32) (hgrn1_states_bytes()); hgrn1_bwd
 * takes it as states_in or, with NULL, recomputes what it needs in the
 * workspace.  Workspaces: hgrn1_fwd_workspace_bytes(), hgrn1_bwd_workspace_bytes()
 * (have_states = whether states_in is passed to the backward; the forward's
 * size does not depend on it).  Each call enqueues three kernels (summaries of
 * every group of segments, a serial pass over the groups per channel, the
 * segments again), five for a backward that recomputes the states.  Errors as
 * for the other calls; C odd is HGRN2_ERR_UNSUPPORTED.
 */
size_t hgrn1_states_bytes(int B, int T, int C);
size_t hgrn1_fwd_workspace_bytes(int B, int T, int C, int have_states);
size_t hgrn1_bwd_workspace_bytes(int B, int T, int C, int have_states);
hgrn2_status hgrn1_fwd(int B, int T, int C, int dtype, int tied, const void *q, const void *k,
                       const void *v, const void *log_f, const float *h0, void *y, float *hT,
                       float *states_out, void *ws, size_t ws_bytes, void *stream);
hgrn2_status hgrn1_bwd(int B, int T, int C, int dtype, int tied, const void *q, const void *k,
                       const void *v, const void *log_f, const float *h0, const float *states_in,
                       const void *dy, const float *dht, void *dq, void *dk, void *dv,
                       void *dlog_f, float *dh0, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HGRN2_H */
