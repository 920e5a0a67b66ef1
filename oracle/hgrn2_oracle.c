/*
 * HGRN2 recurrence oracle: plain, slow, float64, CPU only.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this file's library.  It shares no code with the GPU
 * path and is never used to produce a product result.
 *
 * What it computes (HGRN2: Gated Linear RNNs with State Expansion, paperlayer.ai
 * summary, §3.2 "HGRN2"): per batch element and head, a d_k x d_v matrix state
 * whose rows (the decay channels) are scaled by the forget gate and which
 * receives the outer product of the input-gate vector with the input; the
 * output is the matrix-vector product of the output gate with the state.  In
 * linear-attention notation (same page, §3.2 p.5: identical to GLA's
 * recurrence with q = output gate, k = 1 - f, v = input):
 *
 *     f_t      = exp(log_f_t)                     (log_f = -inf gives f = 0)
 *     S_t[c,j] = f_t[c] * S_{t-1}[c,j] + k_t[c] * v_t[j]
 *     y_t[j]   = sum_c q_t[c] * S_t[c,j]          (read out after the update)
 *     S_0      = h0, or zero
 *
 * The backward is hand-written backpropagation through time of exactly that
 * loop, with the scalar loss sum(y * dy) + sum(S_T * dht); every input is an
 * independent variable (k is not tied to log_f here).
 *
 * Layouts: q, k, log_f [B,T,H,DK]; v, y, dy [B,T,H,DV]; states [B,H,DK,DV],
 * all row-major, float64.  (b,h) pairs are independent and are spread over
 * OpenMP threads; nothing else is reordered.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_CKPT 64 /* backward keeps every 64th state and recomputes the rest */

static size_t tok_off(int T, int H, int D, int b, int t, int h) {
  return (((size_t)b * T + t) * H + h) * (size_t)D;
}

/* One step of the recurrence for one (b,h): S <- diag(f) S + k v^T. */
static void step_state(int DK, int DV, double *S, const double *k, const double *v,
                       const double *log_f) {
  for (int c = 0; c < DK; ++c) {
    const double f = exp(log_f[c]);
    double *row = S + (size_t)c * DV;
    for (int j = 0; j < DV; ++j) row[j] = f * row[j] + k[c] * v[j];
  }
}

/* y[j] = sum_c q[c] S[c,j] */
static void readout(int DK, int DV, const double *S, const double *q, double *y) {
  for (int j = 0; j < DV; ++j) y[j] = 0.0;
  for (int c = 0; c < DK; ++c) {
    const double *row = S + (size_t)c * DV;
    for (int j = 0; j < DV; ++j) y[j] += q[c] * row[j];
  }
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Forward: y [B,T,H,DV]; ht [B,H,DK,DV] (may be NULL); h0 may be NULL (zero). */
void oracle_fwd(int B, int T, int H, int DK, int DV, const double *q, const double *k,
                const double *v, const double *log_f, const double *h0, double *y,
                double *ht) {
  const size_t SS = (size_t)DK * DV;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh) {
    const int b = bh / H, h = bh % H;
    double *S = (double *)malloc(SS * sizeof(double));
    if (h0) memcpy(S, h0 + (size_t)bh * SS, SS * sizeof(double));
    else memset(S, 0, SS * sizeof(double));
    for (int t = 0; t < T; ++t) {
      step_state(DK, DV, S, k + tok_off(T, H, DK, b, t, h), v + tok_off(T, H, DV, b, t, h),
                 log_f + tok_off(T, H, DK, b, t, h));
      readout(DK, DV, S, q + tok_off(T, H, DK, b, t, h), y + tok_off(T, H, DV, b, t, h));
    }
    if (ht) memcpy(ht + (size_t)bh * SS, S, SS * sizeof(double));
    free(S);
  }
}

/*
 * Backward by backpropagation through time.  G holds dL/dS_t for the step
 * being undone:
 *   G   += q_t dy_t^T
 *   dq_t = S_t dy_t,  dk_t = G v_t,  dv_t = G^T k_t
 *   dlog_f_t[c] = f_t[c] * sum_j G[c,j] S_{t-1}[c,j]
 *   G    = diag(f_t) G                    (gradient flowing into S_{t-1})
 * and dh0 = G after the first step.  dht and h0 may be NULL (zero); dh0 may
 * be NULL (not wanted).
 */
void oracle_bwd(int B, int T, int H, int DK, int DV, const double *q, const double *k,
                const double *v, const double *log_f, const double *h0, const double *dy,
                const double *dht, double *dq, double *dk, double *dv, double *dlog_f,
                double *dh0) {
  const size_t SS = (size_t)DK * DV;
  const int nck = (T + ORACLE_CKPT - 1) / ORACLE_CKPT;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh) {
    const int b = bh / H, h = bh % H;
    /* checkpoints: ck[m] = S_{m*CKPT} (state before step m*CKPT+1) */
    double *ck = (double *)malloc((size_t)(nck + 1) * SS * sizeof(double));
    double *seg = (double *)malloc((size_t)(ORACLE_CKPT + 1) * SS * sizeof(double));
    double *G = (double *)malloc(SS * sizeof(double));
    double *S = (double *)malloc(SS * sizeof(double));
    if (h0) memcpy(S, h0 + (size_t)bh * SS, SS * sizeof(double));
    else memset(S, 0, SS * sizeof(double));
    for (int t = 0; t < T; ++t) {
      if (t % ORACLE_CKPT == 0) memcpy(ck + (size_t)(t / ORACLE_CKPT) * SS, S, SS * sizeof(double));
      step_state(DK, DV, S, k + tok_off(T, H, DK, b, t, h), v + tok_off(T, H, DV, b, t, h),
                 log_f + tok_off(T, H, DK, b, t, h));
    }
    if (dht) memcpy(G, dht + (size_t)bh * SS, SS * sizeof(double));
    else memset(G, 0, SS * sizeof(double));
    for (int m = nck - 1; m >= 0; --m) {
      const int t0 = m * ORACLE_CKPT;
      const int t1 = (t0 + ORACLE_CKPT < T) ? t0 + ORACLE_CKPT : T;
      /* seg[i] = S_{t0+i}, i = 0..t1-t0 (S_u is the state after u steps) */
      memcpy(seg, ck + (size_t)m * SS, SS * sizeof(double));
      for (int t = t0; t < t1; ++t) {
        double *dst = seg + (size_t)(t - t0 + 1) * SS;
        memcpy(dst, seg + (size_t)(t - t0) * SS, SS * sizeof(double));
        step_state(DK, DV, dst, k + tok_off(T, H, DK, b, t, h), v + tok_off(T, H, DV, b, t, h),
                   log_f + tok_off(T, H, DK, b, t, h));
      }
      for (int t = t1 - 1; t >= t0; --t) {
        const double *St = seg + (size_t)(t - t0 + 1) * SS;  /* state after this step */
        const double *Sp = seg + (size_t)(t - t0) * SS;      /* state before it */
        const double *qt = q + tok_off(T, H, DK, b, t, h);
        const double *kt = k + tok_off(T, H, DK, b, t, h);
        const double *vt = v + tok_off(T, H, DV, b, t, h);
        const double *lt = log_f + tok_off(T, H, DK, b, t, h);
        const double *gy = dy + tok_off(T, H, DV, b, t, h);
        double *gq = dq + tok_off(T, H, DK, b, t, h);
        double *gk = dk + tok_off(T, H, DK, b, t, h);
        double *gv = dv + tok_off(T, H, DV, b, t, h);
        double *gl = dlog_f + tok_off(T, H, DK, b, t, h);
        for (int c = 0; c < DK; ++c)
          for (int j = 0; j < DV; ++j) G[(size_t)c * DV + j] += qt[c] * gy[j];
        for (int c = 0; c < DK; ++c) {
          double aq = 0.0, ak = 0.0, al = 0.0;
          for (int j = 0; j < DV; ++j) {
            aq += St[(size_t)c * DV + j] * gy[j];
            ak += G[(size_t)c * DV + j] * vt[j];
            al += G[(size_t)c * DV + j] * Sp[(size_t)c * DV + j];
          }
          gq[c] = aq;
          gk[c] = ak;
          gl[c] = exp(lt[c]) * al;
        }
        for (int j = 0; j < DV; ++j) {
          double a = 0.0;
          for (int c = 0; c < DK; ++c) a += G[(size_t)c * DV + j] * kt[c];
          gv[j] = a;
        }
        for (int c = 0; c < DK; ++c) {
          const double f = exp(lt[c]);
          for (int j = 0; j < DV; ++j) G[(size_t)c * DV + j] *= f;
        }
      }
    }
    if (dh0) memcpy(dh0 + (size_t)bh * SS, G, SS * sizeof(double));
    free(ck);
    free(seg);
    free(G);
    free(S);
  }
}

/* One recurrent decode step (HGRN2 summary §1: recurrent inference with
 * linear cost): state [B,H,DK,DV] updated in place, then y [B,H,DV] read out
 * from the updated state.  q, k, log_f [B,H,DK]; v [B,H,DV]. */
void oracle_decode(int B, int H, int DK, int DV, const double *q, const double *k,
                   const double *v, const double *log_f, double *state, double *y) {
  const size_t SS = (size_t)DK * DV;
#pragma omp parallel for schedule(static)
  for (int bh = 0; bh < B * H; ++bh) {
    double *S = state + (size_t)bh * SS;
    step_state(DK, DV, S, k + (size_t)bh * DK, v + (size_t)bh * DV, log_f + (size_t)bh * DK);
    readout(DK, DV, S, q + (size_t)bh * DK, y + (size_t)bh * DV);
  }
}
