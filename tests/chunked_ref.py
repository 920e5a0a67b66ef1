"""Float64 numpy model of the chunked algorithm the GPU kernels implement.

Not the oracle and not product code: a design check.  It evaluates the
recurrence chunk by chunk with exactly the factorisation the kernels use
(block-local prefixes of log f inside 16-token sub-blocks, every exponent
anchored so that it is <= 0 except on diagonal sub-blocks, which fall back to
direct evaluation when their decay range is too wide), so that the algebra can
be checked against the step-by-step oracle on the CPU.

Chunked form (HGRN2 summary, paperlayer.ai, §3.2 p.5: the recurrence is GLA's,
so chunkwise algorithms apply).  For one chunk with prefix b_t = sum_{r<=t} log f_r:
    Y       = tril(A) V + (q * e^b) S_prev,   A[t,s] = sum_c q_t k_s e^{b_t - b_s}
    S_next  = e^Gamma * S_prev + (k * e^{Gamma - b})^T V
and the backward runs the adjoint Lam of the chunk-end state in reverse:
    dq  = dA (k e^{b_t-b_s}) + e^b * (dY S_prev^T),      dA = tril(dY V^T)
    dk  = dA^T (q e^{b_t-b_s}) + e^{Gamma-b} * (V Lam^T)
    dv  = A^T dY + (k e^{Gamma-b}) Lam
    dlog_f_t = sum_{t'>=t in chunk} (q dq - k dk)_{t'} + rowsum(S_next * Lam)
    Lam_prev = e^Gamma * Lam + (q e^b)^T dY
"""

from __future__ import annotations

import numpy as np

FLOOR = -200.0     # log f floor: exp(-200) is 0 in float32, and it keeps differences finite
DIAG_LIMIT = 64.0  # widest in-block decay for which the diagonal block is factorised


def _chunk_prefix(lf, SB):
    """Block-local inclusive prefixes ell [C, D], block totals L [NB, D],
    block starts P [NB, D] (chunk-relative), chunk total Gamma [D]."""
    C, D = lf.shape
    NB = C // SB
    ell = np.zeros_like(lf)
    L = np.zeros((NB, D))
    for i in range(NB):
        blk = np.cumsum(lf[i * SB:(i + 1) * SB], axis=0)
        ell[i * SB:(i + 1) * SB] = blk
        L[i] = blk[-1]
    P = np.concatenate([np.zeros((1, D)), np.cumsum(L, axis=0)[:-1]], axis=0)
    return ell, L, P, L.sum(axis=0)


def _scores(q, k, ell, L, SB):
    """A[t,s] (causal) through the anchored factorisation."""
    C = q.shape[0]
    NB = C // SB
    A = np.zeros((C, C))
    for i in range(NB):
        ti = slice(i * SB, (i + 1) * SB)
        Qt = q[ti] * np.exp(ell[ti])                                   # <= |q|
        for j in range(i):
            sj = slice(j * SB, (j + 1) * SB)
            gap = L[j + 1:i].sum(axis=0)                                # <= 0
            Kt = k[sj] * np.exp((L[j] - ell[sj]) + gap)                 # <= |k|
            A[ti, sj] = Qt @ Kt.T
        if (-L[i]).max() <= DIAG_LIMIT:
            Kd = k[ti] * np.exp(-ell[ti])                               # >= |k|, bounded
            A[ti, ti] = np.tril(Qt @ Kd.T)
        else:
            d = ell[ti][:, None, :] - ell[ti][None, :, :]               # [t, s, c]
            A[ti, ti] = np.tril((q[ti][:, None, :] * k[ti][None, :, :] *
                                 np.exp(np.minimum(d, 0.0))).sum(-1))
    return A


def forward(q, k, v, log_f, h0=None, C=64, SB=16):
    """y, ht for [B,T,H,D] float64 inputs by the chunked algorithm."""
    B, T, H, D = q.shape
    DV = v.shape[-1]
    N = (T + C - 1) // C
    y = np.zeros((B, T, H, DV))
    ht = np.zeros((B, H, D, DV))
    for b in range(B):
        for h in range(H):
            S = np.zeros((D, DV)) if h0 is None else h0[b, h].copy()
            for n in range(N):
                t0, t1 = n * C, min(T, (n + 1) * C)
                Lt = t1 - t0
                qc, kc, vc, lc = (np.zeros((C, x.shape[-1])) for x in (q, k, v, q))
                qc[:Lt], kc[:Lt], vc[:Lt] = q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h]
                lc[:Lt] = np.maximum(log_f[b, t0:t1, h], FLOOR)
                ell, L, P, G = _chunk_prefix(lc, SB)
                blk = np.repeat(np.arange(C // SB), SB)
                A = _scores(qc, kc, ell, L, SB)
                Qh = qc * np.exp(P[blk] + ell)
                Kh = kc * np.exp((G - P[blk] - L[blk]) + (L[blk] - ell))
                Y = A @ vc + Qh @ S
                S = np.exp(G)[:, None] * S + Kh.T @ vc
                y[b, t0:t1, h] = Y[:Lt]
            ht[b, h] = S
    return y, ht


def backward(q, k, v, log_f, dy, h0=None, dht=None, C=64, SB=16):
    """dq, dk, dv, dlog_f, dh0 by the chunked algorithm (states recomputed)."""
    B, T, H, D = q.shape
    DV = v.shape[-1]
    N = (T + C - 1) // C
    NB = C // SB
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(q)]
    dh0 = np.zeros((B, H, D, DV))
    blk = np.repeat(np.arange(NB), SB)
    for b in range(B):
        for h in range(H):
            chunks = []
            S = np.zeros((D, DV)) if h0 is None else h0[b, h].copy()
            states = [S.copy()]
            for n in range(N):
                t0, t1 = n * C, min(T, (n + 1) * C)
                Lt = t1 - t0
                qc, kc, vc, lc, gc = (np.zeros((C, x.shape[-1])) for x in (q, k, v, q, v))
                qc[:Lt], kc[:Lt], vc[:Lt] = q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h]
                lc[:Lt] = np.maximum(log_f[b, t0:t1, h], FLOOR)
                gc[:Lt] = dy[b, t0:t1, h]
                ell, L, P, G = _chunk_prefix(lc, SB)
                Kh = kc * np.exp((G - P[blk] - L[blk]) + (L[blk] - ell))
                S = np.exp(G)[:, None] * S + Kh.T @ vc
                states.append(S.copy())
                chunks.append((t0, t1, qc, kc, vc, lc, gc, ell, L, P, G, Kh))
            Lam = np.zeros((D, DV)) if dht is None else dht[b, h].copy()
            for n in range(N - 1, -1, -1):
                t0, t1, qc, kc, vc, lc, gc, ell, L, P, G, Kh = chunks[n]
                Lt = t1 - t0
                Sp, Sn = states[n], states[n + 1]
                A = _scores(qc, kc, ell, L, SB)
                dA = np.tril(gc @ vc.T)
                # dq: row block i anchored at its own start P_i
                dq = np.zeros((C, D))
                dk = np.zeros((C, D))
                for i in range(NB):
                    ti = slice(i * SB, (i + 1) * SB)
                    acc = np.zeros((SB, D))
                    for j in range(i):
                        sj = slice(j * SB, (j + 1) * SB)
                        Kt = kc[sj] * np.exp((L[j] - ell[sj]) + L[j + 1:i].sum(axis=0))
                        acc += dA[ti, sj] @ Kt
                    if (-L[i]).max() <= DIAG_LIMIT:
                        acc += dA[ti, ti] @ (kc[ti] * np.exp(-ell[ti]))
                        dq[ti] = np.exp(ell[ti]) * acc
                    else:
                        d = ell[ti][:, None, :] - ell[ti][None, :, :]
                        diag = (dA[ti, ti][:, :, None] * kc[ti][None] *
                                np.exp(np.minimum(d, 0.0))).sum(1)
                        dq[ti] = np.exp(ell[ti]) * acc + diag
                # dk: column block j anchored at its own end E_j
                for j in range(NB):
                    sj = slice(j * SB, (j + 1) * SB)
                    acc = np.zeros((SB, D))
                    for i in range(j + 1, NB):
                        ti = slice(i * SB, (i + 1) * SB)
                        Qt = qc[ti] * np.exp(ell[ti] + L[j + 1:i].sum(axis=0))
                        acc += dA[ti, sj].T @ Qt
                    if (-L[j]).max() <= DIAG_LIMIT:
                        acc += dA[sj, sj].T @ (qc[sj] * np.exp(ell[sj] - L[j]))
                        dk[sj] = np.exp(L[j] - ell[sj]) * acc
                    else:
                        d = ell[sj][:, None, :] - ell[sj][None, :, :]           # [t, s, c]
                        diag = (dA[sj, sj][:, :, None] * qc[sj][:, None, :] *
                                np.exp(np.minimum(d, 0.0))).sum(0)
                        dk[sj] = np.exp(L[j] - ell[sj]) * acc + diag
                dq += np.exp(P[blk] + ell) * (gc @ Sp.T)
                dk += np.exp((G - P[blk] - L[blk]) + (L[blk] - ell)) * (vc @ Lam.T)
                dv = A.T @ gc + Kh @ Lam
                u = qc * dq - kc * dk
                dl = np.flip(np.cumsum(np.flip(u, 0), 0), 0) + (Sn * Lam).sum(1)[None, :]
                Qh = qc * np.exp(P[blk] + ell)
                Lam = np.exp(G)[:, None] * Lam + Qh.T @ gc
                for o, val in zip(out, (dq, dk, dv, dl)):
                    o[b, t0:t1, h] = val[:Lt]
            dh0[b, h] = Lam
    return (*out, dh0)


def _bf16(x):
    """Round to the nearest bfloat16 (ties to even), as float64."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + ((u >> 16) & 1) + 0x7FFF) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def forward_bf16_points(q, k, v, log_f, C=64, SB=16, round_operands=True):
    """y of one sequence ([T, D] float64 inputs, zero initial state) by the
    chunk forward's arithmetic with bfloat16 rounding where the bf16 kernels
    round: the decayed score operands q e^{ell}, k e^{L - ell} (and k e^{ell}
    times its gap factor off the adjacent blocks), the score tile, the state
    and the inter-chunk operand, the scan's decayed k, and y.
    round_operands=False keeps the decayed q and k operands (and the scan's
    decayed k) in float64 and rounds the rest.  Diagonal blocks wider than
    DIAG_LIMIT are not modelled (the workloads here have none)."""
    T, D = q.shape
    N = (T + C - 1) // C
    R = _bf16 if round_operands else (lambda x: x)
    y = np.zeros((T, D))
    S = np.zeros((D, D))
    NB = C // SB
    for n in range(N):
        t0, t1 = n * C, min(T, (n + 1) * C)
        Lt = t1 - t0
        qc, kc, vc, lc = (np.zeros((C, D)) for _ in range(4))
        qc[:Lt], kc[:Lt], vc[:Lt] = q[t0:t1], k[t0:t1], v[t0:t1]
        lc[:Lt] = np.maximum(log_f[t0:t1], FLOOR)
        ell, L, P, G = _chunk_prefix(lc, SB)
        assert (-L).max() <= DIAG_LIMIT
        qo = R(qc * np.exp(ell))
        ko = R(kc * np.exp(np.repeat(L, SB, 0) - ell))
        A = np.zeros((C, C))
        for i in range(NB):
            ti = slice(i * SB, (i + 1) * SB)
            for j in range(i + 1):
                sj = slice(j * SB, (j + 1) * SB)
                if j == i - 1:
                    kt = ko[sj]                                  # gap factor exactly 1
                else:
                    gap = np.exp(np.minimum(-L[i], 80.0)) if j == i else np.exp(P[i] - P[j + 1])
                    kt = R(ko[sj] * gap)
                blk = qo[ti] @ kt.T
                A[ti, sj] = np.tril(blk) if j == i else blk
        qb = R(qo * np.exp(np.repeat(P, SB, 0)))
        Y = _bf16(A) @ vc + qb @ _bf16(S)
        xd = R(kc * np.exp(np.minimum(G - np.cumsum(lc, 0), 0.0)))
        S = np.exp(G)[:, None] * S + xd.T @ vc
        y[t0:t1] = _bf16(Y)[:Lt]
    return y
