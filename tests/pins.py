"""Pins for the CPU oracle: checks against facts fixed by the mathematics,
not by the oracle itself.

Every pin takes an oracle handle (``oracle.Oracle``) so that the mutation
test can run the same pins against deliberately broken copies of the oracle
and show that each plausible mistake fails at least one pin.

Sources (HGRN2: Gated Linear RNNs with State Expansion, paperlayer.ai summary):
  §3.2 "HGRN2": outer-product state expansion, diagonal forget gate,
        matrix-vector readout; multi-head state d_h x d_h;
  §3.2 p.5: identical to GLA's recurrence (linear-attention form);
  §2.1: gated linear RNN with the input gate tied as one minus the forget gate
        (the elementwise case, recovered here as d_k = d_v = 1);
  §1: recurrent inference with linear cost (the decode step).
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_exact.json")


def _rng(seed):
    return np.random.default_rng(seed)


def rand_inputs(seed, B=2, T=37, H=3, DK=5, DV=4, h0=True, lo=-1.5):
    r = _rng(seed)
    q = r.standard_normal((B, T, H, DK))
    k = r.standard_normal((B, T, H, DK))
    v = r.standard_normal((B, T, H, DV))
    log_f = r.uniform(lo, 0.0, (B, T, H, DK))
    hh = r.standard_normal((B, H, DK, DV)) if h0 else None
    return q, k, v, log_f, hh


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- forward pins

def closed_form(q, k, v, log_f, h0):
    """Quadratic closed form of the recurrence, written independently of the
    step loop:  y_t = sum_c q_t[c] (P_{0,t}[c] h0[c,:] + sum_{s<=t} P_{s,t}[c] k_s[c] v_s),
    P_{s,t}[c] = prod_{r=s+1..t} f_r[c] (and P_{0,t} includes f_0..f_t).
    Uses cumulative sums of log f inside one (b,h) slice."""
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    y = np.zeros((B, T, H, DV))
    for b in range(B):
        for h in range(H):
            cum = np.cumsum(log_f[b, :, h, :], axis=0)          # sum_{r<=t} log f_r
            for t in range(T):
                dec = np.exp(cum[t][None, :] - cum[: t + 1])    # [s, c] = prod_{r=s+1..t} f_r
                w = (q[b, t, h][None, :] * k[b, : t + 1, h] * dec).sum(axis=1)  # [s]
                y[b, t, h] = w @ v[b, : t + 1, h]
                if h0 is not None:
                    y[b, t, h] += (q[b, t, h] * np.exp(cum[t])) @ h0[b, h]
    return y


def pin_closed_form(orc):
    q, k, v, lf, h0 = rand_inputs(1)
    y, _ = orc.forward(q, k, v, lf, h0)
    assert rel(y, closed_form(q, k, v, lf, h0)) < 1e-12


def pin_limit_f_one(orc):
    """f == 1 (log f = 0): causal linear attention tril(Q K^T) V + Q h0."""
    q, k, v, lf, h0 = rand_inputs(2)
    lf = np.zeros_like(lf)
    y, ht = orc.forward(q, k, v, lf, h0)
    B, T, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            ref = np.tril(Q @ K.T) @ V + Q @ h0[b, h]
            assert rel(y[b, :, h], ref) < 1e-12
            assert rel(ht[b, h], h0[b, h] + K.T @ V) < 1e-12


def pin_limit_f_zero(orc):
    """f == 0 (log f = -inf): the state is replaced every step, y_t = (q_t . k_t) v_t."""
    q, k, v, lf, h0 = rand_inputs(3)
    lf = np.full_like(lf, -np.inf)
    y, ht = orc.forward(q, k, v, lf, h0)
    ref = (q * k).sum(-1, keepdims=True) * v
    assert rel(y, ref) < 1e-13
    ref_ht = k[:, -1][..., :, None] * v[:, -1][..., None, :]
    assert rel(ht, ref_ht) < 1e-13


def pin_scalar_scan(orc):
    """d_k = d_v = 1 is the elementwise gated linear recurrence
    h_t = f_t h_{t-1} + k_t v_t, y_t = q_t h_t (a first-order linear scan)."""
    r = _rng(4)
    T = 50
    q, k, v = r.standard_normal((3, 1, T, 1, 1))
    f = r.uniform(0.0, 1.0, (1, T, 1, 1))
    y, ht = orc.forward(q, k, v, np.log(f), None)
    hs = 0.0
    out = []
    for t in range(T):
        hs = f[0, t, 0, 0] * hs + k[0, t, 0, 0] * v[0, t, 0, 0]
        out.append(q[0, t, 0, 0] * hs)
    assert rel(y[0, :, 0, 0], out) < 1e-13
    assert abs(ht[0, 0, 0, 0] - hs) < 1e-12 * max(1.0, abs(hs))


def _frac_mat(m):
    return [[Fraction(x) for x in row] for row in m]


def pin_golden_exact(orc):
    """The C oracle reproduces the exact rational fixture (one channel reset by
    f = 0, one channel with f = 1) to float64 rounding."""
    g = json.load(open(GOLDEN))
    f = _frac_mat(g["f"])
    to = lambda m: np.array([[float(x) for x in row] for row in _frac_mat(m)])
    q, k, v, h0, dy, dht = (to(g[n]) for n in ("q", "k", "v", "h0", "dy", "dht"))
    fl = np.array([[float(x) for x in row] for row in f])
    with np.errstate(divide="ignore"):
        lf = np.log(fl)
    y, ht = orc.forward(q[None, :, None], k[None, :, None], v[None, :, None],
                        lf[None, :, None], h0[None, None])
    assert rel(y[0, :, 0], to(g["y"])) < 1e-14
    assert rel(ht[0, 0], to(g["ht"])) < 1e-14
    dq, dk, dv, dl, dh0 = orc.backward(q[None, :, None], k[None, :, None], v[None, :, None],
                                       lf[None, :, None], dy[None, :, None], h0[None, None],
                                       dht[None, None])
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (dl, "dlog_f")):
        assert rel(got[0, :, 0], to(g[name])) < 1e-14, name
    assert rel(dh0[0, 0], to(g["dh0"])) < 1e-14


def golden_closed_form_exact():
    """The fixture itself against the closed form in exact arithmetic."""
    g = json.load(open(GOLDEN))
    q, k, v, f, h0 = (_frac_mat(g[n]) for n in ("q", "k", "v", "f", "h0"))
    T, DK, DV = len(q), len(q[0]), len(v[0])
    y = _frac_mat(g["y"])
    for t in range(T):
        for j in range(DV):
            acc = Fraction(0)
            for c in range(DK):
                p0 = Fraction(1)
                for r in range(0, t + 1):
                    p0 *= f[r][c]
                inner = p0 * h0[c][j]
                for s in range(t + 1):
                    p = Fraction(1)
                    for r in range(s + 1, t + 1):
                        p *= f[r][c]
                    inner += p * k[s][c] * v[s][j]
                acc += q[t][c] * inner
            assert acc == y[t][j], (t, j)


def pin_linearity(orc):
    """y is linear in (v, h0) jointly; heads and batch entries are independent."""
    q, k, v, lf, h0 = rand_inputs(5)
    _, _, v2, _, h02 = rand_inputs(6)
    y1, t1 = orc.forward(q, k, v, lf, h0)
    y2, t2 = orc.forward(q, k, v2, lf, h02)
    y3, t3 = orc.forward(q, k, 2.0 * v - 3.0 * v2, lf, 2.0 * h0 - 3.0 * h02)
    assert rel(y3, 2.0 * y1 - 3.0 * y2) < 1e-12
    assert rel(t3, 2.0 * t1 - 3.0 * t2) < 1e-12
    # permuting heads / batch permutes the outputs
    ph = [2, 0, 1]
    yp, tp = orc.forward(q[:, :, ph], k[:, :, ph], v[:, :, ph], lf[:, :, ph], h0[:, ph])
    assert np.array_equal(yp, y1[:, :, ph]) and np.array_equal(tp, t1[:, ph])
    yb, tb = orc.forward(q[::-1], k[::-1], v[::-1], lf[::-1], h0[::-1])
    assert np.array_equal(yb, y1[::-1]) and np.array_equal(tb, t1[::-1])


def pin_state_carry(orc):
    """Running [0, T1) then [T1, T) from the carried state equals one run."""
    q, k, v, lf, h0 = rand_inputs(7, T=41)
    y, ht = orc.forward(q, k, v, lf, h0)
    T1 = 17
    ya, ha = orc.forward(q[:, :T1], k[:, :T1], v[:, :T1], lf[:, :T1], h0)
    yb, hb = orc.forward(q[:, T1:], k[:, T1:], v[:, T1:], lf[:, T1:], ha)
    assert rel(np.concatenate([ya, yb], axis=1), y) < 1e-13
    assert rel(hb, ht) < 1e-13


def pin_decode(orc):
    """A decode step is one forward step from the given state, read out after
    the update."""
    q, k, v, lf, h0 = rand_inputs(8, T=1)
    y, ht = orc.forward(q, k, v, lf, h0)
    yd, Sd = orc.decode_step(q[:, 0], k[:, 0], v[:, 0], lf[:, 0], h0)
    assert rel(yd, y[:, 0]) < 1e-14 and rel(Sd, ht) < 1e-14
    # and against the definition written out in numpy
    f = np.exp(lf[:, 0])
    Sref = f[..., :, None] * h0 + k[:, 0][..., :, None] * v[:, 0][..., None, :]
    yref = np.einsum("bhc,bhcj->bhj", q[:, 0], Sref)
    assert rel(Sd, Sref) < 1e-14 and rel(yd, yref) < 1e-13


# --------------------------------------------------------------- backward pins

def _loss(orc, q, k, v, lf, h0, dy, dht):
    y, ht = orc.forward(q, k, v, lf, h0)
    return float((y * dy).sum() + (ht * dht).sum())


def pin_finite_differences(orc):
    """Central differences of L = sum(y dy) + sum(ht dht) for every input element."""
    q, k, v, lf, h0 = rand_inputs(9, B=1, T=9, H=2, DK=3, DV=2)
    r = _rng(10)
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    grads = orc.backward(q, k, v, lf, dy, h0, dht)
    args = [q, k, v, lf, h0]
    eps = 1e-6
    for ai, g in enumerate(grads):
        x = args[ai]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(orc, *args, dy, dht)
            x[idx] = old - eps
            lm = _loss(orc, *args, dy, dht)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        assert rel(g, num) < 1e-7, ("input", ai, rel(g, num))


def pin_autograd(orc):
    """Gradients against torch float64 autograd through a plain loop of the
    recurrence (no hand-derived backward involved)."""
    import torch
    q, k, v, lf, h0 = rand_inputs(11, B=2, T=13, H=2, DK=4, DV=3)
    r = _rng(12)
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v, lf, h0)]
    tq, tk, tv, tl, th = ts
    S = th
    ys = []
    for t in range(q.shape[1]):
        S = torch.exp(tl[:, t])[..., :, None] * S + tk[:, t][..., :, None] * tv[:, t][..., None, :]
        ys.append(torch.einsum("bhc,bhcj->bhj", tq[:, t], S))
    Y = torch.stack(ys, dim=1)
    L = (Y * torch.tensor(dy)).sum() + (S * torch.tensor(dht)).sum()
    L.backward()
    got = orc.backward(q, k, v, lf, dy, h0, dht)
    for g, t in zip(got, ts):
        assert rel(g, t.grad.numpy()) < 1e-12


def pin_dlogf_identity(orc):
    """dlog_f_r = sum_{t>=r} (q*dq - k*dk)_t + rowsum(S_T * dht): the gradient
    of the log-gate equals a reverse cumulative sum of q.dq - k.dk plus the
    final-state term (follows from d/dlog f_r scaling every path through r)."""
    q, k, v, lf, h0 = rand_inputs(13, T=23)
    r = _rng(14)
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    dq, dk, dv, dl, dh0 = orc.backward(q, k, v, lf, dy, h0, dht)
    _, ht = orc.forward(q, k, v, lf, h0)
    u = q * dq - k * dk
    rc = np.flip(np.cumsum(np.flip(u, axis=1), axis=1), axis=1)
    ref = rc + (ht * dht).sum(-1)[:, None]
    assert rel(dl, ref) < 1e-12


def pin_bwd_limits(orc):
    """f == 1: gradients of causal linear attention in closed matrix form."""
    q, k, v, lf, h0 = rand_inputs(15, B=1, H=1, T=11, h0=False)
    lf = np.zeros_like(lf)
    r = _rng(16)
    dy = r.standard_normal(v.shape)
    dq, dk, dv, dl, dh0 = orc.backward(q, k, v, lf, dy, None, None)
    Q, K, V, dY = q[0, :, 0], k[0, :, 0], v[0, :, 0], dy[0, :, 0]
    M = np.tril(np.ones((Q.shape[0],) * 2))
    dA = (dY @ V.T) * M
    assert rel(dq[0, :, 0], dA @ K) < 1e-12
    assert rel(dk[0, :, 0], dA.T @ Q) < 1e-12
    assert rel(dv[0, :, 0], ((Q @ K.T) * M).T @ dY) < 1e-12
    assert rel(dh0[0, 0], Q.T @ dY) < 1e-12


# ---------------------------------------------------------------- tied gates

def _loss_tied(orc, q, v, lf, h0, dy, dht):
    import oracle as o
    y, ht = orc.forward(q, o.tied_k(lf), v, lf, h0)
    return float((y * dy).sum() + (ht * dht).sum())


def pin_tied_finite_differences(orc):
    """k = 1 - exp(log_f): central differences of the loss in (q, v, log_f, h0),
    with k recomputed from every perturbed log_f, against backward_tied."""
    import oracle as o
    q, _, v, lf, h0 = rand_inputs(17, B=1, T=8, H=2, DK=3, DV=2)
    r = _rng(18)
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    grads = o.backward_tied(q, v, lf, dy, h0, dht)
    args = [q, v, lf, h0]
    eps = 1e-6
    for ai, g in enumerate(grads):
        x = args[ai]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss_tied(orc, *args, dy, dht)
            x[idx] = old - eps
            lm = _loss_tied(orc, *args, dy, dht)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        assert rel(g, num) < 1e-7, ("input", ai, rel(g, num))


def pin_tied_autograd(orc):
    """Tied gradients against torch float64 autograd through a plain loop that
    forms k = 1 - exp(log_f) itself."""
    import torch
    import oracle as o
    q, _, v, lf, h0 = rand_inputs(19, B=2, T=11, H=2, DK=4, DV=3)
    r = _rng(20)
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, v, lf, h0)]
    tq, tv, tl, th = ts
    tk = 1.0 - torch.exp(tl)
    S = th
    ys = []
    for t in range(q.shape[1]):
        S = torch.exp(tl[:, t])[..., :, None] * S + tk[:, t][..., :, None] * tv[:, t][..., None, :]
        ys.append(torch.einsum("bhc,bhcj->bhj", tq[:, t], S))
    Y = torch.stack(ys, dim=1)
    L = (Y * torch.tensor(dy)).sum() + (S * torch.tensor(dht)).sum()
    L.backward()
    got = o.backward_tied(q, v, lf, dy, h0, dht)
    for g, t in zip(got, ts):
        assert rel(g, t.grad.numpy()) < 1e-12
    y, ht = o.forward_tied(q, v, lf, h0)
    assert rel(y, Y.detach().numpy()) < 1e-13 and rel(ht, S.detach().numpy()) < 1e-13


# ---------------------------------------------------------------- gate from its pre-activation

def _gate_inputs(seed, B=1, T=7, H=2, DK=3, DV=2):
    r = _rng(seed)
    q = r.standard_normal((B, T, H, DK))
    v = r.standard_normal((B, T, H, DV))
    z = r.standard_normal((B, T, H, DK)) * 1.5
    lam = r.uniform(0.0, 0.9, (H, DK))
    h0 = r.standard_normal((B, H, DK, DV))
    return q, v, z, lam, h0


def pin_gate_log_sigmoid(orc):
    """With lam = 0 the gate is a plain sigmoid: log f is torch's logsigmoid and
    k is sigmoid(-z), over a range that overflows a naive exp; with lam > 0, log f
    and k against the direct formula at moderate z, and f + k = 1."""
    import torch
    import oracle as o
    z = np.concatenate([np.linspace(-700.0, 700.0, 2801), [-1e-9, 0.0, 1e-9]])
    tz = torch.tensor(z, dtype=torch.float64)
    assert np.max(np.abs(o.gate_log_f(z, 0.0) - torch.nn.functional.logsigmoid(tz).numpy())) < 1e-13
    assert np.max(np.abs(o.gate_k(z, 0.0) - torch.sigmoid(-tz).numpy())) < 1e-15
    zm = np.linspace(-30.0, 30.0, 601)
    for lam in (0.1, 0.5, 0.97):
        direct = np.log(lam + (1.0 - lam) * torch.sigmoid(torch.tensor(zm, dtype=torch.float64)).numpy())
        assert np.max(np.abs(o.gate_log_f(zm, lam) - direct)) < 1e-14, lam
        assert np.max(np.abs(np.exp(o.gate_log_f(zm, lam)) + o.gate_k(zm, lam) - 1.0)) < 1e-14, lam
        assert np.all(o.gate_log_f(zm, lam) >= np.log(lam) - 1e-15)   # f never falls below lam


def _loss_gate(orc, q, v, z, lam, h0, dy, dht):
    import oracle as o
    y, ht = orc.forward(q, o.gate_k(z, lam), v, o.gate_log_f(z, lam), h0)
    return float((y * dy).sum() + (ht * dht).sum())


def pin_gate_finite_differences(orc):
    """Central differences of the loss in (q, v, z, lam, h0) against backward_gate."""
    import oracle as o
    q, v, z, lam, h0 = _gate_inputs(23)
    r = _rng(24)
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    dq, dv, dz, dlam, dh0 = o.backward_gate(q, v, z, lam, dy, h0, dht)
    args = [q, v, z, lam, h0]
    eps = 1e-6
    for ai, g in enumerate((dq, dv, dz, dlam, dh0)):
        x = args[ai]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss_gate(orc, *args, dy, dht)
            x[idx] = old - eps
            lm = _loss_gate(orc, *args, dy, dht)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        assert rel(g, num) < 1e-7, ("input", ai, rel(g, num))


def pin_gate_autograd(orc):
    """Gate-mode gradients against torch float64 autograd through a plain loop
    that forms f = lam + (1 - lam) sigmoid(z) and k = 1 - f itself."""
    import torch
    import oracle as o
    q, v, z, lam, h0 = _gate_inputs(25, B=2, T=9, H=2, DK=4, DV=3)
    r = _rng(26)
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, v, z, lam, h0)]
    tq, tv, tz, tlam, th = ts
    f = tlam + (1.0 - tlam) * torch.sigmoid(tz)
    tk = 1.0 - f
    S = th
    ys = []
    for t in range(q.shape[1]):
        S = f[:, t][..., :, None] * S + tk[:, t][..., :, None] * tv[:, t][..., None, :]
        ys.append(torch.einsum("bhc,bhcj->bhj", tq[:, t], S))
    Y = torch.stack(ys, dim=1)
    L = (Y * torch.tensor(dy)).sum() + (S * torch.tensor(dht)).sum()
    L.backward()
    got = o.backward_gate(q, v, z, lam, dy, h0, dht)
    for g, t in zip(got, ts):
        assert rel(g, t.grad.numpy()) < 1e-12
    y, ht = o.forward_gate(q, v, z, lam, h0)
    assert rel(y, Y.detach().numpy()) < 1e-13 and rel(ht, S.detach().numpy()) < 1e-13


# ---------------------------------------------------------------- HGRN1 elementwise recurrence

def pin_hgrn1_geometric(orc):
    """HGRN1 with a constant gate f and a constant input i, tied (k = 1 - f),
    output gate 1: h_t = f^t h0 + (1 - f^t) i, the closed form of a first-order
    linear recurrence with constant coefficients."""
    import oracle as o
    B, T, C = 2, 23, 5
    r = _rng(31)
    f = r.uniform(0.2, 0.99, (1, 1, C))
    i = r.standard_normal((B, 1, C))
    h0 = r.standard_normal((B, C))
    lf = np.broadcast_to(np.log(f), (B, T, C)).copy()
    v = np.broadcast_to(i, (B, T, C)).copy()
    q = np.ones((B, T, C))
    y, hT = o.hgrn1_forward(q, None, v, lf, h0, tied=True)
    tt = np.arange(1, T + 1)[None, :, None]
    ref = f ** tt * h0[:, None, :] + (1.0 - f ** tt) * i
    assert rel(y, ref) < 1e-13 and rel(hT, ref[:, -1]) < 1e-13


def pin_hgrn1_finite_differences(orc):
    """HGRN1 gradients (untied and tied) against central differences of the loss
    sum(y dy) + sum(hT dht) in every input."""
    import oracle as o
    B, T, C = 1, 9, 3
    r = _rng(32)
    q, k, v = (r.standard_normal((B, T, C)) for _ in range(3))
    lf = r.uniform(-1.5, 0.0, (B, T, C))
    h0 = r.standard_normal((B, C))
    dy = r.standard_normal((B, T, C))
    dht = r.standard_normal((B, C))
    for tied in (False, True):
        def loss(q, k, v, lf, h0):
            y, hT = o.hgrn1_forward(q, k, v, lf, h0, tied=tied)
            return float((y * dy).sum() + (hT * dht).sum())
        dq, dk, dv, dl, dh0 = o.hgrn1_backward(q, k, v, lf, dy, h0, dht, tied=tied)
        args = [q, k, v, lf, h0]
        for ai, g in ((0, dq), (1, dk), (2, dv), (3, dl), (4, dh0)):
            if g is None:
                continue
            x = args[ai]
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                old = x[idx]
                x[idx] = old + 1e-6
                lp = loss(*args)
                x[idx] = old - 1e-6
                lm = loss(*args)
                x[idx] = old
                num[idx] = (lp - lm) / 2e-6
            assert rel(g, num) < 1e-7, (tied, ai, rel(g, num))


# ---------------------------------------------------------------- scalar decay per head

def pin_scalar_decay_autograd(orc):
    """Scalar-decay gradients against torch float64 autograd through a plain
    loop that scales the whole state by one a_t per head."""
    import torch
    import oracle as o
    q, k, v, _, h0 = rand_inputs(41, B=2, T=10, H=2, DK=4, DV=3)
    r = _rng(42)
    la = r.uniform(-1.5, 0.0, q.shape[:3])
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, la, h0)]
    tq, tk, tv, tla, th = ts
    S = th
    ys = []
    for t in range(q.shape[1]):
        S = torch.exp(tla[:, t])[..., None, None] * S + tk[:, t][..., :, None] * tv[:, t][..., None, :]
        ys.append(torch.einsum("bhc,bhcj->bhj", tq[:, t], S))
    Y = torch.stack(ys, dim=1)
    L = (Y * torch.tensor(dy)).sum() + (S * torch.tensor(dht)).sum()
    L.backward()
    got = o.backward_scalar(q, k, v, la, dy, h0, dht)
    for g, t in zip(got, ts):
        assert rel(g, t.grad.numpy()) < 1e-12
    y, ht = o.forward_scalar(q, k, v, la, h0)
    assert rel(y, Y.detach().numpy()) < 1e-13 and rel(ht, S.detach().numpy()) < 1e-13


def pin_scalar_decay_finite_differences(orc):
    """Central differences of the loss in log_a against backward_scalar's dlog_a."""
    import oracle as o
    q, k, v, _, h0 = rand_inputs(43, B=1, T=7, H=2, DK=3, DV=2)
    r = _rng(44)
    la = r.uniform(-1.5, 0.0, q.shape[:3])
    dy = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    g = o.backward_scalar(q, k, v, la, dy, h0, dht)[3]
    num = np.zeros_like(la)
    for idx in np.ndindex(la.shape):
        old = la[idx]
        la[idx] = old + 1e-6
        yp, hp = orc.forward(q, k, v, np.repeat(la[..., None], 3, axis=-1), h0)
        la[idx] = old - 1e-6
        ym, hm = orc.forward(q, k, v, np.repeat(la[..., None], 3, axis=-1), h0)
        la[idx] = old
        num[idx] = (((yp - ym) * dy).sum() + ((hp - hm) * dht).sum()) / 2e-6
    assert rel(g, num) < 1e-7



def pin_decode_variants(orc):
    """The tied, gate and per-head decode steps: each is one step of its
    forward from the given state, and equals the one-step definition written
    out in numpy (S' = f S + k^T v, y = q S'), with f and k formed directly:
    f = exp(log f), k = 1 - f (tied); f = lam + (1 - lam) / (1 + e^-z),
    k = 1 - f (gate); one f per head (scalar)."""
    import oracle as o
    q, k, v, lf, h0 = rand_inputs(51, T=1)
    r = _rng(52)
    B, _, H, DK = q.shape

    def one_step(f, kk):
        S = f[..., :, None] * h0 + kk[..., :, None] * v[:, 0][..., None, :]
        return np.einsum("bhc,bhcj->bhj", q[:, 0], S), S

    # tied
    yd, Sd = o.decode_step_tied(q[:, 0], v[:, 0], lf[:, 0], h0)
    y1, h1 = o.forward_tied(q, v, lf, h0)
    f = np.exp(lf[:, 0])
    yr, Sr = one_step(f, 1.0 - f)
    assert rel(yd, y1[:, 0]) < 1e-14 and rel(Sd, h1) < 1e-14
    assert rel(yd, yr) < 1e-12 and rel(Sd, Sr) < 1e-12
    # gate from the pre-activation with a per-channel lower bound
    z = r.normal(0.0, 2.0, (B, 1, H, DK))
    lam = r.uniform(0.0, 0.9, (H, DK))
    yd, Sd = o.decode_step_gate(q[:, 0], v[:, 0], z[:, 0], lam, h0)
    y1, h1 = o.forward_gate(q, v, z, lam, h0)
    f = lam + (1.0 - lam) / (1.0 + np.exp(-z[:, 0]))
    yr, Sr = one_step(f, 1.0 - f)
    assert rel(yd, y1[:, 0]) < 1e-14 and rel(Sd, h1) < 1e-14
    assert rel(yd, yr) < 1e-12 and rel(Sd, Sr) < 1e-12
    # one decay per head
    la = r.uniform(-1.5, 0.0, (B, 1, H))
    yd, Sd = o.decode_step_scalar(q[:, 0], k[:, 0], v[:, 0], la[:, 0], h0)
    y1, h1 = o.forward_scalar(q, k, v, la, h0)
    yr, Sr = one_step(np.repeat(np.exp(la[:, 0])[..., None], DK, axis=-1), k[:, 0])
    assert rel(yd, y1[:, 0]) < 1e-14 and rel(Sd, h1) < 1e-14
    assert rel(yd, yr) < 1e-12 and rel(Sd, Sr) < 1e-12

ALL_PINS = [pin_closed_form, pin_limit_f_one, pin_limit_f_zero, pin_scalar_scan,
            pin_golden_exact, pin_linearity, pin_state_carry, pin_decode,
            pin_finite_differences, pin_autograd, pin_dlogf_identity, pin_bwd_limits,
            pin_tied_finite_differences, pin_tied_autograd,
            pin_gate_log_sigmoid, pin_gate_finite_differences, pin_gate_autograd,
            pin_hgrn1_geometric, pin_hgrn1_finite_differences,
            pin_scalar_decay_autograd, pin_scalar_decay_finite_differences, pin_decode_variants]
GATE_PINS = [pin_gate_log_sigmoid, pin_gate_finite_differences, pin_gate_autograd]
