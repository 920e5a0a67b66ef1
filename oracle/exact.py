"""Exact rational-arithmetic HGRN2 recurrence for tiny inputs.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).  Pure-Python loops over
``fractions.Fraction``; meant for T <= 8 and d <= 4.

Same recurrence as the C oracle (HGRN2 summary, paperlayer.ai, §3.2): the
state's rows are scaled by the forget gate, the outer product k_t v_t^T is
added, and the output is q_t read through the updated state.  Here the forget
gate is given directly as a rational f in [0, 1] (no logarithm), so every
result is exact.
"""

from __future__ import annotations

from fractions import Fraction


def _zeros(r, c):
    return [[Fraction(0)] * c for _ in range(r)]


def forward(q, k, v, f, h0=None):
    """q, k, f: [T][DK]; v: [T][DV]; h0: [DK][DV] or None.  Returns (y [T][DV], S_T)."""
    T, DK, DV = len(q), len(q[0]), len(v[0])
    S = [row[:] for row in h0] if h0 is not None else _zeros(DK, DV)
    ys = []
    for t in range(T):
        for c in range(DK):
            for j in range(DV):
                S[c][j] = f[t][c] * S[c][j] + k[t][c] * v[t][j]
        ys.append([sum((q[t][c] * S[c][j] for c in range(DK)), Fraction(0)) for j in range(DV)])
    return ys, S


def backward(q, k, v, f, dy, h0=None, dht=None):
    """Exact BPTT of L = sum(y*dy) + sum(S_T*dht).

    Returns (dq, dk, dv, df, dh0), where df is dL/df (not d/dlog f; the
    log-gradient is f * df)."""
    T, DK, DV = len(q), len(q[0]), len(v[0])
    states = [[row[:] for row in h0] if h0 is not None else _zeros(DK, DV)]
    for t in range(T):
        P = states[-1]
        states.append([[f[t][c] * P[c][j] + k[t][c] * v[t][j] for j in range(DV)]
                       for c in range(DK)])
    G = [row[:] for row in dht] if dht is not None else _zeros(DK, DV)
    dq = [None] * T
    dk = [None] * T
    dv = [None] * T
    df = [None] * T
    for t in range(T - 1, -1, -1):
        for c in range(DK):
            for j in range(DV):
                G[c][j] += q[t][c] * dy[t][j]
        St, Sp = states[t + 1], states[t]
        dq[t] = [sum((St[c][j] * dy[t][j] for j in range(DV)), Fraction(0)) for c in range(DK)]
        dk[t] = [sum((G[c][j] * v[t][j] for j in range(DV)), Fraction(0)) for c in range(DK)]
        dv[t] = [sum((G[c][j] * k[t][c] for c in range(DK)), Fraction(0)) for j in range(DV)]
        df[t] = [sum((G[c][j] * Sp[c][j] for j in range(DV)), Fraction(0)) for c in range(DK)]
        G = [[f[t][c] * G[c][j] for j in range(DV)] for c in range(DK)]
    return dq, dk, dv, df, G
