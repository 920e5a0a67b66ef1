"""CPU float64 oracle for the HGRN2 recurrence.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg import this package.  The product path
(``linear_attention_hgrn2_amd``) never imports it.

The arithmetic lives in ``hgrn2_oracle.c`` (step-by-step recurrence, hand
backpropagation through time, one decode step), compiled with gcc into
``liboracle_hgrn2.so`` next to it.  This module only converts arrays to
contiguous float64 and calls it.  ``exact`` holds an exact rational-arithmetic
version of the same loops for tiny inputs.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hgrn2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_hgrn2.so")
_lib = None

__all__ = ["build", "forward", "backward", "decode_step", "forward_tied", "backward_tied",
           "decode_step_tied", "tied_k", "gate_log_f", "gate_k", "gate_partials", "forward_gate",
           "backward_gate", "decode_step_gate", "hgrn1_forward", "hgrn1_backward", "forward_scalar",
           "backward_scalar", "decode_step_scalar", "threads", "Oracle", "default"]


def build(force: bool = True) -> str:
    """Compile the C oracle (gcc, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes handle on one build of the C oracle (the default build, or a
    differently compiled copy that a test supplies)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_fwd.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_bwd.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_decode.argtypes = [I, I, I, I, P, P, P, P, P, P]
        lib.oracle_threads.restype = I
        self.lib = lib
        self.path = path

    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    def forward(self, q, k, v, log_f, h0=None):
        q, k, v, log_f, h0 = map(_f64, (q, k, v, log_f, h0))
        B, T, H, DK = q.shape
        DV = v.shape[-1]
        assert k.shape == q.shape and log_f.shape == q.shape and v.shape == (B, T, H, DV)
        if h0 is not None:
            assert h0.shape == (B, H, DK, DV)
        y = np.zeros((B, T, H, DV))
        ht = np.zeros((B, H, DK, DV))
        self.lib.oracle_fwd(B, T, H, DK, DV, _p(q), _p(k), _p(v), _p(log_f), _p(h0),
                            _p(y), _p(ht))
        return y, ht

    def backward(self, q, k, v, log_f, dy, h0=None, dht=None):
        q, k, v, log_f, dy, h0, dht = map(_f64, (q, k, v, log_f, dy, h0, dht))
        B, T, H, DK = q.shape
        DV = v.shape[-1]
        assert dy.shape == v.shape
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        dl = np.zeros_like(log_f)
        dh0 = np.zeros((B, H, DK, DV))
        self.lib.oracle_bwd(B, T, H, DK, DV, _p(q), _p(k), _p(v), _p(log_f), _p(h0), _p(dy),
                            _p(dht), _p(dq), _p(dk), _p(dv), _p(dl), _p(dh0))
        return dq, dk, dv, dl, dh0

    def decode_step(self, q, k, v, log_f, state):
        q, k, v, log_f = map(_f64, (q, k, v, log_f))
        S = np.array(state, dtype=np.float64, copy=True, order="C")
        B, H, DK = q.shape
        DV = v.shape[-1]
        y = np.zeros((B, H, DV))
        self.lib.oracle_decode(B, H, DK, DV, _p(q), _p(k), _p(v), _p(log_f), _p(S), _p(y))
        return y, S


def _load() -> Oracle:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = Oracle(_LIB)
    return _lib


def default() -> Oracle:
    """The oracle built from ``hgrn2_oracle.c``."""
    return _load()


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return _load().threads()


def forward(q, k, v, log_f, h0=None):
    """y [B,T,H,DV], ht [B,H,DK,DV] of the step recurrence, float64.

    q, k, log_f: [B,T,H,DK]; v: [B,T,H,DV]; h0: [B,H,DK,DV] or None (zero)."""
    return _load().forward(q, k, v, log_f, h0)


def backward(q, k, v, log_f, dy, h0=None, dht=None):
    """(dq, dk, dv, dlog_f, dh0) of L = sum(y*dy) + sum(ht*dht), float64.

    k and log_f are independent inputs (no tying)."""
    return _load().backward(q, k, v, log_f, dy, h0, dht)


def decode_step(q, k, v, log_f, state):
    """One recurrent step: returns (y [B,H,DV], new state [B,H,DK,DV]); the
    input state array is not modified."""
    return _load().decode_step(q, k, v, log_f, state)


# ------------------------------------------------------------------ tied gates
# HGRN2 ties the input gate to the forget gate, k = 1 - f (HGRN2 summary,
# paperlayer.ai, §2.1 and §3.2).  With log_f the only gate input, k is a
# function of it, and the loss reaches log_f both through the decay and
# through k: d/dlog_f = (partial through the decay) + (dk/dlog_f) * dk with
# dk/dlog_f = -exp(log_f).


def tied_k(log_f):
    """k = 1 - f = -expm1(log_f), float64, without cancellation for f near 1."""
    return -np.expm1(np.asarray(log_f, dtype=np.float64))


def forward_tied(q, v, log_f, h0=None):
    """forward() with k = 1 - exp(log_f)."""
    return forward(q, tied_k(log_f), v, log_f, h0)


def backward_tied(q, v, log_f, dy, h0=None, dht=None):
    """(dq, dv, dlog_f, dh0) with k = 1 - exp(log_f): dlog_f is the total
    derivative, the partial through the decay minus exp(log_f) * dk."""
    lf = np.asarray(log_f, dtype=np.float64)
    dq, dk, dv, dl, dh0 = backward(q, tied_k(lf), v, lf, dy, h0, dht)
    return dq, dv, dl - np.exp(lf) * dk, dh0


def decode_step_tied(q, v, log_f, state):
    """decode_step() with k = 1 - exp(log_f)."""
    return decode_step(q, tied_k(log_f), v, log_f, state)


# ------------------------------------------------------------------ gate from its pre-activation
# HGRN's forget gate has an additive lower bound: the gate learns a residual
# above a lower bound lam that the layer supplies (HGRN2 summary,
# paperlayer.ai, §2.2: lower bounds per layer, forget gate learning residuals
# above them).  Read here as
#     f = lam + (1 - lam) * sigmoid(z),      k = 1 - f = (1 - lam) * sigmoid(-z),
# with z [B,T,H,DK] the pre-activation and lam [H,DK] the lower bound of each
# head channel.  The loss reaches z and lam through log f (the decay) and
# through k (the tied input gate); the chain rule over the partial gradients
# of the recurrence gives dz and dlam (summed over batch and time).


def _sig_pair(z):
    """(sigmoid(z), sigmoid(-z)) in float64 without overflow."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    hi, lo = 1.0 / (1.0 + e), e / (1.0 + e)
    return np.where(z >= 0, hi, lo), np.where(z >= 0, lo, hi)


def gate_log_f(z, lam):
    """log f = log(lam + (1 - lam) sigmoid(z)), float64, stable for any z:
    for z >= 0 (u = e^-z <= 1) it is log1p(lam u) - log1p(u); for z < 0
    (u = e^z < 1) it is log(lam + u) - log1p(u).  lam broadcasts over [..., H, DK]."""
    z = np.asarray(z, dtype=np.float64)
    lam = np.broadcast_to(np.asarray(lam, dtype=np.float64), z.shape)
    u = np.exp(-np.abs(z))
    with np.errstate(divide="ignore"):
        neg = np.log(lam + u) - np.log1p(u)
    pos = np.log1p(lam * u) - np.log1p(u)
    return np.where(z >= 0, pos, neg)


def gate_k(z, lam):
    """k = 1 - f = (1 - lam) sigmoid(-z), float64."""
    lam = np.asarray(lam, dtype=np.float64)
    return (1.0 - lam) * _sig_pair(z)[1]


def gate_partials(z, lam):
    """(dlog_f/dz, dk/dz, dlog_f/dlam, dk/dlam) at every element, float64:
    with s = sigmoid(z), s' = sigmoid(-z), f = lam + (1 - lam) s:
    dlog_f/dz = (1 - lam) s s' / f,  dk/dz = -(1 - lam) s s',
    dlog_f/dlam = s' / f,            dk/dlam = -s'."""
    z = np.asarray(z, dtype=np.float64)
    lam = np.broadcast_to(np.asarray(lam, dtype=np.float64), z.shape)
    s, sp = _sig_pair(z)
    f = lam + (1.0 - lam) * s
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(lam == 0.0, 1.0, (1.0 - lam) * s / f)   # (1 - lam) s / f, -> 1 as lam -> 0
        dl_dlam = sp / f
    return ratio * sp, -(1.0 - lam) * s * sp, dl_dlam, -sp


def forward_gate(q, v, z, lam, h0=None):
    """forward() with log f and k formed from the pre-activation z and the lower bound lam [H,DK]."""
    return forward(q, gate_k(z, lam), v, gate_log_f(z, lam), h0)


def backward_gate(q, v, z, lam, dy, h0=None, dht=None):
    """(dq, dv, dz, dlam, dh0): dz [B,T,H,DK] and dlam [H,DK] by the chain rule
    through log f and k; dlam sums over batch and time."""
    dq, dk, dv, dl, dh0 = backward(q, gate_k(z, lam), v, gate_log_f(z, lam), dy, h0, dht)
    a, b, c, d = gate_partials(z, lam)
    dz = dl * a + dk * b
    dlam = (dl * c + dk * d).sum(axis=(0, 1))
    return dq, dv, dz, dlam, dh0


def decode_step_gate(q, v, z, lam, state):
    """decode_step() with log f and k formed from z [B,H,DK] and lam [H,DK]."""
    return decode_step(q, gate_k(z, lam), v, gate_log_f(z, lam), state)


# ------------------------------------------------------------------ HGRN1 elementwise recurrence
# HGRN's gated linear RNN (HGRN2 summary, paperlayer.ai, §2.1): per channel c,
#     h_t[c] = f_t[c] h_{t-1}[c] + k_t[c] v_t[c],     y_t[c] = q_t[c] h_t[c],
# with the input gate k = 1 - f in HGRN1 itself (tied) and q the output gate.
# It is the HGRN2 recurrence with d_k = d_v = 1 and every channel its own
# head, so it runs through the same step loop: [B, T, C] becomes
# [B, T, C, 1] with C heads.


def _h1(x):
    return None if x is None else np.asarray(x, dtype=np.float64)[..., None]


def hgrn1_forward(q, k, v, log_f, h0=None, tied=False):
    """(y [B,T,C], hT [B,C]).  tied: k = 1 - exp(log_f) (k is ignored)."""
    lf = np.asarray(log_f, dtype=np.float64)
    kk = tied_k(lf) if tied else k
    h0_ = None if h0 is None else np.asarray(h0, dtype=np.float64)[..., None, None]
    y, ht = forward(_h1(q), _h1(kk), _h1(v), _h1(lf), h0_)
    return y[..., 0], ht[..., 0, 0]


def hgrn1_backward(q, k, v, log_f, dy, h0=None, dht=None, tied=False):
    """(dq, dk or None, dv, dlog_f, dh0) of the loss sum(y dy) + sum(hT dht);
    tied: dlog_f is the total derivative (dlog_f - f dk) and dk is None."""
    lf = np.asarray(log_f, dtype=np.float64)
    kk = tied_k(lf) if tied else k
    h0_ = None if h0 is None else np.asarray(h0, dtype=np.float64)[..., None, None]
    dht_ = None if dht is None else np.asarray(dht, dtype=np.float64)[..., None, None]
    dq, dk, dv, dl, dh0 = backward(_h1(q), _h1(kk), _h1(v), _h1(lf), _h1(dy), h0_, dht_)
    dq, dk, dv, dl, dh0 = dq[..., 0], dk[..., 0], dv[..., 0], dl[..., 0], dh0[..., 0, 0]
    if tied:
        return dq, None, dv, dl - np.exp(lf) * dk, dh0
    return dq, dk, dv, dl, dh0


# ------------------------------------------------------------------ scalar decay per head
# The per-head scalar decay that other models use in place of HGRN2's
# per-channel gate (HGRN2 summary, paperlayer.ai, §5: Mamba2, xLSTM and Gated
# Retention share one decay per head; HGRN2 keeps one per dimension): one
# log a_t per (b, t, h), the same for every row of that head's state.  The
# recurrence is HGRN2's with log_f[..., c] = log a for every channel c, and the
# gradient of log a sums the per-channel one over the channels.


def _bcast(log_a, D):
    la = np.asarray(log_a, dtype=np.float64)
    return np.repeat(la[..., None], D, axis=-1)


def forward_scalar(q, k, v, log_a, h0=None):
    """forward() with one log decay per (b, t, h), log_a [B,T,H]."""
    return forward(q, k, v, _bcast(log_a, np.shape(q)[-1]), h0)


def backward_scalar(q, k, v, log_a, dy, h0=None, dht=None):
    """(dq, dk, dv, dlog_a [B,T,H], dh0)."""
    dq, dk, dv, dl, dh0 = backward(q, k, v, _bcast(log_a, np.shape(q)[-1]), dy, h0, dht)
    return dq, dk, dv, dl.sum(axis=-1), dh0


def decode_step_scalar(q, k, v, log_a, state):
    """decode_step() with log_a [B,H]."""
    return decode_step(q, k, v, _bcast(log_a, np.shape(q)[-1]), state)
