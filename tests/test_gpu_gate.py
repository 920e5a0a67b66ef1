"""GPU parity of the gate-from-pre-activation entry points (f = lb + (1 - lb)
sigmoid(z), k = 1 - f, both formed in the kernels; the backward returns dz and
the lower-bound gradient summed over batch and time) against the float64
oracle's gate functions, on the same seeded inputs: z rounded to the input
dtype, the lower bound [H, D] in float32.  Tolerances as for the untied path:
normwise relative error per (b, h) slice (per tensor for the [H, D] lower-bound
gradient) <= 2e-2 (bf16), <= 1e-4 (fp32)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, slice_rel, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu


def _case(dtype, B, T, H, D, lam=0.3, spread=0.25, seed=7, h0std=0.0, qscale=1.0):
    w = synth.Workload("case", B=B, H=H, T=T, D=D, chunk=0, dtype=dtype, lam=lam, qscale=qscale, h0std=h0std,
                       train=True, seed=seed)
    d = synth.generate(w)
    d["lb"] = synth.lower_bounds(H, D, lam, spread, seed=seed + 3)
    return d


def _dht(d):
    rng = np.random.default_rng(d["seed"] + 99)
    return (rng.standard_normal((d["B"], d["H"], d["D"], d["D"])) * 0.5).astype(np.float32)


def _rel(a, b):
    """errors() of a per-head [H, D] float32 gradient (one slice per head, one
    row per channel), as the worst of its three metrics."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return worst(errors(a[None, :, :, None], b[None, :, :, None], "state"))


def _run(d, chunk):
    import torch
    import linear_attention_hgrn2_amd as m
    dt = d["dtype"]
    q, v, z, dy = (to_dev(d[n], dt) for n in ("q", "v", "z", "dy"))
    lb = to_dev(d["lb"], "f32")
    h0 = to_dev(d["h0"], "f32")
    dht = to_dev(_dht(d), "f32")
    y, ht, st = m.fwd_gate(q, v, z, lb, h0, chunk=chunk, want_states=True)
    g = m.bwd_gate(q, v, z, lb, dy, h0, dht, st, chunk=chunk)
    torch.cuda.synchronize()
    return y, ht, g


def _check(d, chunk, label=""):
    dt = d["dtype"]
    y, ht, (dq, dv, dz, dlb, dh0) = _run(d, chunk)
    x = {n: synth.to_f64(d[n], dt) for n in ("q", "v", "z", "dy")}
    lb = d["lb"].astype(np.float64)
    h0 = None if d["h0"] is None else d["h0"].astype(np.float64)
    yr, htr = oracle.forward_gate(x["q"], x["v"], x["z"], lb, h0)
    gr = oracle.backward_gate(x["q"], x["v"], x["z"], lb, x["dy"], h0, _dht(d).astype(np.float64))
    errs = {"y": slice_rel(to_host64(y), yr), "ht": slice_rel(to_host64(ht), htr, token_major=False)}
    for name, a, r in zip(("dq", "dv", "dz"), (dq, dv, dz), gr[:3]):
        errs[name] = slice_rel(to_host64(a), r)
    errs["dlb"] = _rel(to_host64(dlb), gr[3])
    errs["dh0"] = slice_rel(to_host64(dh0), gr[4], token_major=False)
    print("%s gate D=%d C=%d %s: %s" % (label, d["D"], chunk, dt, " ".join("%s %.3e" % e for e in errs.items())),
          flush=True)
    for name, e in errs.items():
        assert e <= TOL[dt], (name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,C", [(16, 16), (32, 32), (64, 64), (128, 16), (128, 32), (128, 64)])
def test_gate_shapes(dtype, D, C):
    """A ragged last chunk in every case: rows past the end must decay nothing
    (ht and dh0 see it)."""
    import linear_attention_hgrn2_amd as m
    import torch
    if not m.supported(D, C, torch.float32 if dtype == "f32" else torch.bfloat16):
        pytest.skip("no kernel for this combination")
    d = _case(dtype, B=2, T=2 * C + 7, H=2, D=D, h0std=0.5)
    _check(d, C)


@pytest.mark.parametrize("lam,spread", [(0.0, 0.0), (0.97, 0.02)])
def test_gate_lower_bound_regimes_f32(lam, spread):
    """float32 (tolerance 1e-4) with no lower bound and with gates near one,
    where log f is small and its absolute accuracy matters most."""
    d = _case("f32", B=2, T=5 * 64 + 3, H=3, D=64, lam=lam, spread=spread, h0std=0.2)
    _check(d, 64, label="f32 lam=%.2f+-%.2f" % (lam, spread))


@pytest.mark.parametrize("lam,spread", [(0.0, 0.0), (0.5, 0.45), (0.97, 0.02)])
def test_gate_lower_bound_regimes_d128(lam, spread):
    """No lower bound (plain sigmoid gate), bounds spread over (0.05, 0.95), and
    bounds near one (gates near one, small k); d = 128, chunk 64, bf16, several
    chunks per workgroup."""
    d = _case("bf16", B=3, T=20 * 64 + 13, H=5, D=128, lam=lam, spread=spread, h0std=0.2)
    _check(d, 64, label="lam=%.2f+-%.2f" % (lam, spread))


def test_gate_extreme_preactivations_d128():
    """Saturated gates (|z| up to 30) and lower bounds 0 and 0.99 on some
    channels; in-block decays wide enough for the directly summed diagonal.
    (A bound of 0 is not combined with z far below 0: there the lower-bound
    gradient of a token is G / f with f tiny, exact but ill-conditioned.)"""
    d = _case("bf16", B=1, T=300, H=2, D=128, lam=0.3, spread=0.3, h0std=0.3)
    z = synth.to_f64(d["z"], "bf16")
    z[0, 3, 0, :] = -30.0
    z[0, 20:40, 1, 2] = 30.0
    z[0, 70:90, 1, :8] = -12.0
    d["z"] = synth.f32_to_bf16_bits(z.astype(np.float32))
    d["lb"][1, 8:12] = 0.0
    d["lb"][0, 4:8] = 0.99
    _check(d, 64, label="extreme")
    _check(d, 16, label="extreme")


def test_gate_repeat_runs_are_bitwise_equal():
    import torch
    d = _case("bf16", B=2, T=5 * 64 + 9, H=3, D=128, h0std=0.3)
    a = _run(d, 64)
    b = _run(d, 64)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert torch.equal(x, y)


def test_gate_train_full():
    """The training shape (B8 H16 T4096 d128, chunk 64, bf16) in gate mode with
    lower bounds around 0.3: every (b, h) against the oracle, and the
    lower-bound gradient of every head summed over the whole batch."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate("train_bf16", lam=0.3)
    d["lb"] = synth.lower_bounds(d["H"], d["D"], 0.3, 0.25, seed=11)
    q, v, z, dy = (to_dev(d[n], "bf16") for n in ("q", "v", "z", "dy"))
    lb = to_dev(d["lb"], "f32")
    y, _, st = m.fwd_gate(q, v, z, lb, None, chunk=64, want_ht=False, want_states=True)
    dq, dv, dz, dlb, _ = m.bwd_gate(q, v, z, lb, dy, None, None, st, chunk=64, want_dh0=False)
    torch.cuda.synchronize()
    x = {n: synth.to_f64(d[n], "bf16") for n in ("q", "v", "z", "dy")}
    lbh = d["lb"].astype(np.float64)
    yr, _ = oracle.forward_gate(x["q"], x["v"], x["z"], lbh, None)
    errs = {"y": errors(to_host64(y), yr)}
    del yr
    gr = oracle.backward_gate(x["q"], x["v"], x["z"], lbh, x["dy"], None, None)
    for name, a, r in zip(("dq", "dv", "dz"), (dq, dv, dz), gr[:3]):
        errs[name] = errors(to_host64(a), r)
    a, r = to_host64(dlb), gr[3]
    errs["dlb"] = errors(a[None, :, :, None], r[None, :, :, None], "state")
    print("gate train, all 128 (b,h): %s" % "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items()), flush=True)
    for name, e in errs.items():
        assert worst(e) <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 128])
def test_gate_decode(dtype, D):
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate_decode("decode_f32", B=3, H=5, D=D, seed=13)
    lbv = synth.lower_bounds(5, D, 0.5, 0.4, seed=17)
    conv = (lambda a: a) if dtype == "f32" else (lambda a: synth.f32_to_bf16_bits(a))
    q, v, z = (to_dev(conv(d[n]), dtype) for n in ("q", "v", "z"))
    S = to_dev(d["state"], "f32")
    y = m.decode_step_gate(q, v, z, to_dev(lbv, "f32"), S)
    torch.cuda.synchronize()
    x = {n: synth.to_f64(conv(d[n]), dtype) for n in ("q", "v", "z")}
    yr, Sr = oracle.decode_step_gate(x["q"], x["v"], x["z"], lbv.astype(np.float64), d["state"].astype(np.float64))
    ey = worst(errors(to_host64(y)[:, None], yr[:, None]))
    es = worst(errors(to_host64(S), Sr, "state"))
    print("gate decode D=%d %s: y %.3e state %.3e" % (D, dtype, ey, es), flush=True)
    assert ey <= TOL[dtype] and es <= 1e-5
