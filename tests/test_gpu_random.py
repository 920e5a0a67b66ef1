"""Randomised GPU parity: cases drawn from a fixed master seed, each a random
gate mode (untied, tied, gate from z, one decay per head), dtype, head size,
chunk size, ragged length (shorter than one chunk up to several chunks),
batch and head counts, decay regime, with or without an initial state and a
final-state gradient, with saved or recomputed boundary states, through the
segmented or the stored-state forward, and (bfloat16) with bfloat16 or
float32 outputs.  Every output is compared with the float64 oracle by the
metrics of tests/gpu_util.py against the dtype's tolerance; sequences shorter
than one 16-token sub-block also pass the oracle's run on the inputs' absolute
values, the magnitude of the terms each output sums (the arithmetic's rounding
scale for outputs that cancel their terms).

HGRN2_RANDOM_CASES sets the number of cases (default 24); the cases are the
same on every run.  A second stream of medium cases (HGRN2_RANDOM_MEDIUM,
default 6) draws up to 4 x 16 sequences of up to 2048 tokens (at most 32768
token-heads), so that the persistent backward walks several chunks per
workgroup and the scans many chunks per sequence.  A third stream
(HGRN2_RANDOM_PAIRED, default 6) draws bfloat16 d = 128 chunk-64 cases of 33
to 96 sequences long enough that the forward without stored states walks two
workgroups per compute unit (segments of at least 8 chunks), with ragged
lengths, so that the paired walk's copies of the v tile into LDS, its
uneven last segments and its ragged last chunks meet random inputs in every
gate mode."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import MIN_NORM_ROWS, TOL, errors, fmt, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu

MASTER_SEED = 20241
N_CASES = int(os.environ.get("HGRN2_RANDOM_CASES", "24"))
N_MEDIUM = int(os.environ.get("HGRN2_RANDOM_MEDIUM", "6"))
N_PAIRED = int(os.environ.get("HGRN2_RANDOM_PAIRED", "6"))


def _draw(i):
    r = np.random.default_rng(MASTER_SEED + 7919 * i)
    c = dict(gm=str(r.choice(["untied", "tied", "gate", "scalar"])), dtype=str(r.choice(["bf16", "f32"])),
             D=int(r.choice([16, 32, 64, 128])), C=int(r.choice([16, 32, 64, 128])),
             B=int(r.integers(1, 4)), H=int(r.integers(1, 4)), lam=float(r.choice([0.0, 0.3, 0.6, 0.9, 0.97])),
             h0=bool(r.integers(0, 2)), dht=bool(r.integers(0, 2)), saved=bool(r.integers(0, 2)),
             out32=bool(r.integers(0, 2)), seed=int(r.integers(1, 1 << 30)))
    c["T"] = int(r.integers(1, 4 * c["C"] + 38))
    return c


def _draw_medium(i):
    r = np.random.default_rng(MASTER_SEED + 1 + 6101 * i)
    c = dict(gm=str(r.choice(["untied", "tied", "gate", "scalar"])), dtype=str(r.choice(["bf16", "f32"])),
             D=int(r.choice([64, 128])), C=int(r.choice([16, 32, 64, 128])),
             B=int(r.integers(1, 5)), H=int(r.integers(1, 17)), lam=float(r.choice([0.0, 0.3, 0.6, 0.9, 0.97])),
             h0=bool(r.integers(0, 2)), dht=bool(r.integers(0, 2)), saved=bool(r.integers(0, 2)),
             out32=bool(r.integers(0, 2)), seed=int(r.integers(1, 1 << 30)))
    c["T"] = int(r.integers(64, min(2048, 32768 // (c["B"] * c["H"])) + 1))
    return c


def _draw_paired(i):
    r = np.random.default_rng(MASTER_SEED + 2 + 4513 * i)
    B = int(r.integers(1, 4))
    H = int(r.integers(-(-33 // B), 96 // B + 1))
    c = dict(gm=str(r.choice(["untied", "tied", "gate", "scalar"])), dtype="bf16", D=128, C=64, B=B, H=H,
             lam=float(r.choice([0.0, 0.3, 0.6, 0.9, 0.97])), h0=bool(r.integers(0, 2)), dht=bool(r.integers(0, 2)),
             saved=bool(r.integers(0, 2)), out32=bool(r.integers(0, 2)), seed=int(r.integers(1, 1 << 30)))
    pt = -(-512 // (B * H))                     # segments per sequence the plan aims at
    n = int(r.integers(8 * pt, 10 * pt + 1))    # chunks: segments of at least 8
    c["T"] = (n - 1) * 64 + int(r.integers(1, 65))
    return c


def _label(c):
    return "%s %s D%d C%d B%d H%d T%d lam%.2f%s%s%s%s" % (
        c["gm"], c["dtype"], c["D"], c["C"], c["B"], c["H"], c["T"], c["lam"], " h0" if c["h0"] else "",
        " dht" if c["dht"] else "", " saved" if c["saved"] else " recomputed",
        " out-f32" if c["out32"] and c["dtype"] == "bf16" else "")


def _terms(c, f, h064, dht64, lb64):
    """The magnitude of the terms each output sums: the oracle on the absolute
    values of q, k, v, h0, dy and dht, with the same decays (and, tied or from
    z, the same k = 1 - f >= 0).  Every output of the recurrence is a sum of
    products of these inputs with positive weights, so this is the sum of its
    terms' magnitudes; the tied and gate chain rules combine two such partials
    with signed factors, whose magnitudes add."""
    gm = c["gm"]
    A = lambda x: None if x is None else np.abs(x)
    q, v, dy, h0, dht = A(f["q"]), A(f["v"]), A(f["dy"]), A(h064), A(dht64)
    if gm == "untied":
        k, lf = A(f["k"]), f["log_f"]
    elif gm == "tied":
        lf = f["log_f"]
        k = oracle.tied_k(lf)
    elif gm == "gate":
        lf, k = oracle.gate_log_f(f["z"], lb64), oracle.gate_k(f["z"], lb64)
    else:
        lf, k = np.repeat(f["la"][..., None], c["D"], axis=-1), A(f["k"])
    y, ht = oracle.forward(q, k, v, lf, h0)
    dq, dk, dv, dl, dh0 = oracle.backward(q, k, v, lf, dy, h0, dht)
    t = dict(y=y, ht=ht, dq=dq, dk=dk, dv=dv, dh0=dh0)
    if gm == "untied":
        t["dlog_f"] = dl
    elif gm == "tied":
        t["dlog_f"] = dl + np.exp(np.maximum(lf, -200.0)) * dk
    elif gm == "gate":
        a, b, cc, d = oracle.gate_partials(f["z"], lb64)
        t["dz"] = dl * np.abs(a) + dk * np.abs(b)
        t["dlb"] = (dl * np.abs(cc) + dk * np.abs(d)).sum(axis=(0, 1))
    else:
        t["dlog_a"] = dl.sum(axis=-1)
    return t


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    _run(i, _draw(i))


@pytest.mark.parametrize("i", range(N_MEDIUM))
def test_random_medium_case(i):
    _run(i, _draw_medium(i))


@pytest.mark.parametrize("i", range(N_PAIRED))
def test_random_paired_walk_case(i):
    from tests.test_gpu_segfwd import _plan
    c = _draw_paired(i)
    assert _plan(c["B"], c["H"], c["T"])[2], "the case must take the paired walk"
    _run(i, c)


def _run(i, c):
    import torch
    import linear_attention_hgrn2_amd as m
    dt, D, C, gm = c["dtype"], c["D"], c["C"], c["gm"]
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    if not m.supported(D, C, tdt):
        pytest.skip("no kernel for D %d, chunk %d, %s" % (D, C, dt))
    print("case %d: %s" % (i, _label(c)), flush=True)
    w = synth.Workload("random", B=c["B"], H=c["H"], T=c["T"], D=D, chunk=0, dtype=dt, lam=c["lam"], qscale=1.0,
                       h0std=0.5 if c["h0"] else 0.0, train=True, seed=c["seed"])
    d = synth.generate(w)
    lb = synth.lower_bounds(c["H"], D, c["lam"], 0.2, seed=c["seed"] + 1)
    la = np.ascontiguousarray(d["log_f"][..., 0])
    rr = np.random.default_rng(c["seed"] + 2)
    dht = (rr.standard_normal((c["B"], c["H"], D, D)) * 0.5).astype(np.float32) if c["dht"] else None
    x = {n: to_dev(d[n], dt) for n in ("q", "k", "v", "log_f", "z", "dy")}
    x["la"] = to_dev(la, dt)
    lbd, h0, dhtd = to_dev(lb, "f32"), to_dev(d["h0"], "f32"), to_dev(dht, "f32")
    od = torch.float32 if (c["out32"] and dt == "bf16") else None
    kw = dict(chunk=C, out_dtype=od)

    def fwd(want_states):
        if gm == "untied":
            return m.fwd(x["q"], x["k"], x["v"], x["log_f"], h0, want_states=want_states, **kw)
        if gm == "tied":
            return m.fwd_tied(x["q"], x["v"], x["log_f"], h0, want_states=want_states, **kw)
        if gm == "gate":
            return m.fwd_gate(x["q"], x["v"], x["z"], lbd, h0, want_states=want_states, **kw)
        return m.fwd_scalar(x["q"], x["k"], x["v"], x["la"], h0, want_states=want_states, **kw)

    y, ht, _ = fwd(False)             # no states kept: the segmented forward where it exists
    _, _, st = fwd(True)
    st = st if c["saved"] else None
    if gm == "untied":
        g = m.bwd(x["q"], x["k"], x["v"], x["log_f"], x["dy"], h0, dhtd, st, **kw)
        got = dict(dq=g[0], dk=g[1], dv=g[2], dlog_f=g[3], dh0=g[4])
    elif gm == "tied":
        g = m.bwd_tied(x["q"], x["v"], x["log_f"], x["dy"], h0, dhtd, st, **kw)
        got = dict(dq=g[0], dv=g[1], dlog_f=g[2], dh0=g[3])
    elif gm == "gate":
        g = m.bwd_gate(x["q"], x["v"], x["z"], lbd, x["dy"], h0, dhtd, st, **kw)
        got = dict(dq=g[0], dv=g[1], dz=g[2], dlb=g[3], dh0=g[4])
    else:
        g = m.bwd_scalar(x["q"], x["k"], x["v"], x["la"], x["dy"], h0, dhtd, st, **kw)
        got = dict(dq=g[0], dk=g[1], dv=g[2], dlog_a=g[3], dh0=g[4])
    torch.cuda.synchronize()

    f = {n: synth.to_f64(d[n], dt) for n in ("q", "k", "v", "log_f", "z", "dy")}
    f["la"] = synth.to_f64(la, dt)
    h064 = None if d["h0"] is None else d["h0"].astype(np.float64)
    dht64 = None if dht is None else dht.astype(np.float64)
    lb64 = lb.astype(np.float64)
    if gm == "untied":
        yr, htr = oracle.forward(f["q"], f["k"], f["v"], f["log_f"], h064)
        gr = oracle.backward(f["q"], f["k"], f["v"], f["log_f"], f["dy"], h064, dht64)
        ref = dict(dq=gr[0], dk=gr[1], dv=gr[2], dlog_f=gr[3], dh0=gr[4])
    elif gm == "tied":
        yr, htr = oracle.forward_tied(f["q"], f["v"], f["log_f"], h064)
        gr = oracle.backward_tied(f["q"], f["v"], f["log_f"], f["dy"], h064, dht64)
        ref = dict(dq=gr[0], dv=gr[1], dlog_f=gr[2], dh0=gr[3])
    elif gm == "gate":
        yr, htr = oracle.forward_gate(f["q"], f["v"], f["z"], lb64, h064)
        gr = oracle.backward_gate(f["q"], f["v"], f["z"], lb64, f["dy"], h064, dht64)
        ref = dict(dq=gr[0], dv=gr[1], dz=gr[2], dlb=gr[3], dh0=gr[4])
    else:
        yr, htr = oracle.forward_scalar(f["q"], f["k"], f["v"], f["la"], h064)
        gr = oracle.backward_scalar(f["q"], f["k"], f["v"], f["la"], f["dy"], h064, dht64)
        ref = dict(dq=gr[0], dk=gr[1], dv=gr[2], dlog_a=gr[3], dh0=gr[4])

    terms = _terms(c, f, h064, dht64, lb64) if c["T"] < MIN_NORM_ROWS else {}

    def err(name, a, r):
        a, r = to_host64(a), np.asarray(r, np.float64)
        tm = terms.get(name)
        if name in ("ht", "dh0"):
            return errors(a, r, "state", tm, dt)
        if name == "dlb":
            return errors(a[None, :, :, None], r[None, :, :, None], "state", None if tm is None else tm[None, :, :, None], dt)
        if name == "dlog_a":
            return errors(a[..., None], r[..., None], "token", None if tm is None else tm[..., None], dt)
        return errors(a, r, "token", tm, dt)

    errs = {"y": err("y", y, yr), "ht": err("ht", ht, htr)}
    errs.update({n: err(n, got[n], ref[n]) for n in ref})
    print("  " + "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert worst(e) <= TOL[dt], (i, _label(c), n, fmt(e))
