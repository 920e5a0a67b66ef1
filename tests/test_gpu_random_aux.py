"""Randomised GPU parity of the decode step and of the HGRN1 scan, cases
drawn from fixed master seeds (the same on every run), each compared with the
float64 oracle by the metrics of tests/gpu_util.py against the dtype's
tolerance.

Decode (HGRN2 summary, paperlayer.ai, §1: inference keeps only the state and
advances it one token at a time): a random gate mode (untied, tied, gate from
z, one decay per head), dtype, head size, batch and head counts, gate regime,
and (bfloat16) bfloat16 or float32 y; y and the state updated in place.  The
one-token y is a dot product over the head's channels, so its comparison also
gets the magnitude of its terms (the oracle on absolute values).

HGRN1 (§2.2, the elementwise recurrence HGRN2 expands): tied or untied gates,
dtype, batch, a length from one token to several 256-token groups, an even
channel count, gate regime, with or without h0 and dht, with saved or
recomputed segment states.

HGRN2_RANDOM_DECODE and HGRN2_RANDOM_HGRN1 set the counts (default 12 each)."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu

MASTER_SEED = 40961
N_DECODE = int(os.environ.get("HGRN2_RANDOM_DECODE", "12"))
N_HGRN1 = int(os.environ.get("HGRN2_RANDOM_HGRN1", "12"))


def _draw_decode(i):
    r = np.random.default_rng(MASTER_SEED + 7919 * i)
    return dict(gm=str(r.choice(["untied", "tied", "gate", "scalar"])), dtype=str(r.choice(["bf16", "f32"])),
                D=int(r.choice([16, 32, 64, 128])), B=int(r.integers(1, 9)), H=int(r.integers(1, 9)),
                lam=float(r.choice([0.0, 0.3, 0.6, 0.9, 0.97])), out32=bool(r.integers(0, 2)),
                seed=int(r.integers(1, 1 << 30)))


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode_case(i):
    import torch
    import linear_attention_hgrn2_amd as m
    c = _draw_decode(i)
    dt, D, gm, B, H = c["dtype"], c["D"], c["gm"], c["B"], c["H"]
    print("decode case %d: %s" % (i, c), flush=True)
    w = synth.Workload("decode", B=B, H=H, T=1, D=D, chunk=0, dtype="f32", lam=c["lam"], qscale=1.0, h0std=0.5,
                       train=False, seed=c["seed"])
    d = synth.generate_decode(w)
    conv = (lambda a: a) if dt == "f32" else synth.f32_to_bf16_bits
    d["la"] = np.ascontiguousarray(d["log_f"][..., 0])
    x = {n: to_dev(conv(d[n]), dt) for n in ("q", "k", "v", "log_f", "z", "la")}
    f = {n: synth.to_f64(conv(d[n]), dt) for n in ("q", "k", "v", "log_f", "z", "la")}
    lb = synth.lower_bounds(H, D, c["lam"], 0.2, seed=c["seed"] + 1)
    S = to_dev(d["state"], "f32")
    S0 = d["state"].astype(np.float64)
    od = torch.float32 if (c["out32"] and dt == "bf16") else None
    if gm == "untied":
        y = m.decode_step(x["q"], x["k"], x["v"], x["log_f"], S, out_dtype=od)
        yr, Sr = oracle.decode_step(f["q"], f["k"], f["v"], f["log_f"], S0)
        k, lf = np.abs(f["k"]), f["log_f"]
    elif gm == "tied":
        y = m.decode_step_tied(x["q"], x["v"], x["log_f"], S, out_dtype=od)
        yr, Sr = oracle.decode_step_tied(f["q"], f["v"], f["log_f"], S0)
        k, lf = oracle.tied_k(f["log_f"]), f["log_f"]
    elif gm == "gate":
        y = m.decode_step_gate(x["q"], x["v"], x["z"], to_dev(lb, "f32"), S, out_dtype=od)
        lb64 = lb.astype(np.float64)
        yr, Sr = oracle.decode_step_gate(f["q"], f["v"], f["z"], lb64, S0)
        k, lf = oracle.gate_k(f["z"], lb64), oracle.gate_log_f(f["z"], lb64)
    else:
        y = m.decode_step_scalar(x["q"], x["k"], x["v"], x["la"], S, out_dtype=od)
        yr, Sr = oracle.decode_step_scalar(f["q"], f["k"], f["v"], f["la"], S0)
        k, lf = np.abs(f["k"]), np.repeat(f["la"][..., None], D, axis=-1)
    torch.cuda.synchronize()
    assert y.dtype == (torch.float32 if od is not None or dt == "f32" else torch.bfloat16)
    ya, _ = oracle.decode_step(np.abs(f["q"]), k, np.abs(f["v"]), lf, np.abs(S0))
    ey = errors(to_host64(y)[:, None], yr[:, None], "token", ya[:, None], dt)
    es = errors(to_host64(S), Sr, "state")
    print("  y %s | state %s" % (fmt(ey), fmt(es)), flush=True)
    assert worst(ey) <= TOL[dt] and worst(es) <= TOL[dt], (i, c, fmt(ey), fmt(es))


def _draw_h1(i):
    r = np.random.default_rng(MASTER_SEED + 1 + 6101 * i)
    return dict(tied=bool(r.integers(0, 2)), dtype=str(r.choice(["bf16", "f32"])), B=int(r.integers(1, 5)),
                T=int(r.integers(1, 3001)), C=2 * int(r.integers(1, 401)),
                lam=float(r.choice([0.0, 0.3, 0.6, 0.9, 0.97])), h0=bool(r.integers(0, 2)),
                dht=bool(r.integers(0, 2)), saved=bool(r.integers(0, 2)), seed=int(r.integers(1, 1 << 30)))


def _err3(a, b):
    """errors() of a [B, T, C] token tensor or of a [B, C] state (one slice per
    batch element, one row per channel)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.ndim == 2:
        return errors(a[:, None, :, None], b[:, None, :, None], "state")
    return errors(a, b, "btc")


@pytest.mark.parametrize("i", range(N_HGRN1))
def test_random_hgrn1_case(i):
    import torch
    import linear_attention_hgrn2_amd as m
    c = _draw_h1(i)
    dt, B, T, C, tied = c["dtype"], c["B"], c["T"], c["C"], c["tied"]
    print("hgrn1 case %d: %s" % (i, c), flush=True)
    w = synth.Workload("h1", B=B, H=C // 2, T=T, D=2, chunk=0, dtype=dt, lam=c["lam"], qscale=1.0, h0std=0.0,
                       train=True, seed=c["seed"])
    d = synth.generate(w)
    x = {n: d[n].reshape(B, T, C) for n in ("q", "k", "v", "log_f", "dy")}
    rr = np.random.default_rng(c["seed"] + 1)
    h0 = rr.standard_normal((B, C)).astype(np.float32) if c["h0"] else None
    dht = (0.5 * rr.standard_normal((B, C))).astype(np.float32) if c["dht"] else None
    q, k, v, lf, dy = (to_dev(x[n], dt) for n in ("q", "k", "v", "log_f", "dy"))
    kk = None if tied else k
    y, ht, st = m.hgrn1_fwd(q, kk, v, lf, to_dev(h0, "f32"), tied=tied, want_states=c["saved"])
    g = m.hgrn1_bwd(q, kk, v, lf, dy, to_dev(h0, "f32"), to_dev(dht, "f32"), st if c["saved"] else None, tied=tied)
    torch.cuda.synchronize()
    f = {n: synth.to_f64(x[n], dt) for n in ("q", "k", "v", "log_f", "dy")}
    h064 = None if h0 is None else h0.astype(np.float64)
    dht64 = None if dht is None else dht.astype(np.float64)
    fk = None if tied else f["k"]
    yr, htr = oracle.hgrn1_forward(f["q"], fk, f["v"], f["log_f"], h064, tied=tied)
    gr = oracle.hgrn1_backward(f["q"], fk, f["v"], f["log_f"], f["dy"], h064, dht64, tied=tied)
    errs = {"y": _err3(to_host64(y), yr), "hT": _err3(to_host64(ht), htr)}
    for name, a, r in zip(("dq", "dk", "dv", "dlog_f", "dh0"), g, gr):
        if r is not None and a is not None:
            errs[name] = _err3(to_host64(a), r)
    print("  " + "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items()), flush=True)
    for name, e in errs.items():
        assert worst(e) <= TOL[dt], (i, c, name, fmt(e))
