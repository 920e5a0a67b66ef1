"""GPU parity of the one-decay-per-head entry points (log_a [B, T, H] shared
by every channel of a head; k an input; the backward returns dlog_a summed over
the head's channels) against the float64 oracle's scalar-decay functions, on
the same seeded inputs.  The per-head decay is the first channel's log f of
the generator's gates.  Normwise relative error per (b, h) slice <= 2e-2
(bf16), <= 1e-4 (fp32)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, slice_rel, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu


def _case(dtype, B, T, H, D, lam=0.3, seed=9, h0std=0.5):
    w = synth.Workload("case", B=B, H=H, T=T, D=D, chunk=0, dtype=dtype, lam=lam, qscale=1.0, h0std=h0std,
                       train=True, seed=seed)
    d = synth.generate(w)
    d["log_a"] = np.ascontiguousarray(d["log_f"][..., 0])
    return d


def _dht(d):
    rng = np.random.default_rng(d["seed"] + 99)
    return (rng.standard_normal((d["B"], d["H"], d["D"], d["D"])) * 0.5).astype(np.float32)


def _run(d, chunk):
    import torch
    import linear_attention_hgrn2_amd as m
    dt = d["dtype"]
    q, k, v, la, dy = (to_dev(d[n], dt) for n in ("q", "k", "v", "log_a", "dy"))
    h0 = to_dev(d["h0"], "f32")
    dht = to_dev(_dht(d), "f32")
    y, ht, st = m.fwd_scalar(q, k, v, la, h0, chunk=chunk, want_states=True)
    g = m.bwd_scalar(q, k, v, la, dy, h0, dht, st, chunk=chunk)
    torch.cuda.synchronize()
    return y, ht, g


def _check(d, chunk, label=""):
    dt = d["dtype"]
    y, ht, (dq, dk, dv, dla, dh0) = _run(d, chunk)
    x = {n: synth.to_f64(d[n], dt) for n in ("q", "k", "v", "log_a", "dy")}
    h0 = None if d["h0"] is None else d["h0"].astype(np.float64)
    yr, htr = oracle.forward_scalar(x["q"], x["k"], x["v"], x["log_a"], h0)
    gr = oracle.backward_scalar(x["q"], x["k"], x["v"], x["log_a"], x["dy"], h0, _dht(d).astype(np.float64))
    errs = {"y": slice_rel(to_host64(y), yr), "ht": slice_rel(to_host64(ht), htr, token_major=False)}
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), gr[:3]):
        errs[name] = slice_rel(to_host64(a), r)
    errs["dlog_a"] = slice_rel(to_host64(dla)[..., None], gr[3][..., None])
    errs["dh0"] = slice_rel(to_host64(dh0), gr[4], token_major=False)
    print("%s scalar D=%d C=%d %s: %s" % (label, d["D"], chunk, dt, " ".join("%s %.3e" % e for e in errs.items())),
          flush=True)
    for name, e in errs.items():
        assert e <= TOL[dt], (name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,C", [(16, 16), (32, 32), (64, 64), (128, 16), (128, 32), (128, 64)])
def test_scalar_shapes(dtype, D, C):
    import linear_attention_hgrn2_amd as m
    import torch
    if not m.supported(D, C, torch.float32 if dtype == "f32" else torch.bfloat16):
        pytest.skip("no kernel for this combination")
    _check(_case(dtype, B=2, T=2 * C + 7, H=2, D=D), C)


@pytest.mark.parametrize("lam", [0.0, 0.97])
def test_scalar_decay_regimes_d128(lam):
    _check(_case("bf16", B=3, T=20 * 64 + 13, H=5, D=128, lam=lam, h0std=0.2), 64, label="lam=%.2f" % lam)


def test_scalar_extreme_decays_d128():
    """Full resets (log a = -inf), the -200 floor and in-block decays wide
    enough for the directly summed diagonal, all channels of a head at once."""
    d = _case("bf16", B=1, T=300, H=2, D=128, lam=0.0, h0std=0.3)
    la = synth.to_f64(d["log_a"], "bf16")
    la[0, 3, 0] = -np.inf
    la[0, 20, 1] = -200.0
    la[0, 70:80, 1] = -9.0
    d["log_a"] = synth.f32_to_bf16_bits(la.astype(np.float32))
    _check(d, 64, label="extreme")
    _check(d, 16, label="extreme")


def test_scalar_repeat_runs_are_bitwise_equal():
    import torch
    d = _case("bf16", B=2, T=5 * 64 + 9, H=3, D=128)
    a, b = _run(d, 64), _run(d, 64)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert torch.equal(x, y)


def test_scalar_train_full():
    """The training shape (B8 H16 T4096 d128, chunk 64, bf16) with one decay per
    head; every (b, h) against the oracle."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate("train_bf16", lam=0.3)
    la = np.ascontiguousarray(d["log_f"][..., 0])
    q, k, v, dy = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "dy"))
    lat = to_dev(la, "bf16")
    y, _, st = m.fwd_scalar(q, k, v, lat, None, chunk=64, want_ht=False, want_states=True)
    dq, dk, dv, dla, _ = m.bwd_scalar(q, k, v, lat, dy, None, None, st, chunk=64, want_dh0=False)
    torch.cuda.synchronize()
    x = {n: synth.to_f64(d[n], "bf16") for n in ("q", "k", "v", "dy")}
    la64 = synth.to_f64(la, "bf16")
    yr, _ = oracle.forward_scalar(x["q"], x["k"], x["v"], la64, None)
    errs = {"y": errors(to_host64(y), yr)}
    del yr
    gr = oracle.backward_scalar(x["q"], x["k"], x["v"], la64, x["dy"], None, None)
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), gr[:3]):
        errs[name] = errors(to_host64(a), r)
    errs["dlog_a"] = errors(to_host64(dla)[..., None], gr[3][..., None])
    print("scalar train, all 128 (b,h): %s" % "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items()), flush=True)
    for name, e in errs.items():
        assert worst(e) <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 128])
def test_scalar_decode(dtype, D):
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate_decode("decode_f32", B=3, H=5, D=D, seed=13)
    la = np.ascontiguousarray(d["log_f"][..., 0])
    conv = (lambda a: a) if dtype == "f32" else (lambda a: synth.f32_to_bf16_bits(a))
    q, k, v = (to_dev(conv(d[n]), dtype) for n in ("q", "k", "v"))
    S = to_dev(d["state"], "f32")
    y = m.decode_step_scalar(q, k, v, to_dev(conv(la), dtype), S)
    torch.cuda.synchronize()
    x = {n: synth.to_f64(conv(d[n]), dtype) for n in ("q", "k", "v")}
    yr, Sr = oracle.decode_step_scalar(x["q"], x["k"], x["v"], synth.to_f64(conv(la), dtype),
                                       d["state"].astype(np.float64))
    ey = worst(errors(to_host64(y)[:, None], yr[:, None]))
    es = worst(errors(to_host64(S), Sr, "state"))
    print("scalar decode D=%d %s: y %.3e state %.3e" % (D, dtype, ey, es), flush=True)
    assert ey <= TOL[dtype] and es <= 1e-5
