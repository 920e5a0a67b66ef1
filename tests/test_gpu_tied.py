"""GPU parity of the tied-gate entry points (k = 1 - exp(log_f), formed in the
kernels; the backward returns the total derivative with respect to log_f)
against the float64 oracle's tied functions, on the same seeded inputs (the
k the generators draw is not used).  Tolerances as for the untied path:
normwise relative error per (b, h) slice <= 2e-2 (bf16), <= 1e-4 (fp32)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, inputs64, slice_rel, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu


def _case(dtype, B, T, H, D, lam=0.0, seed=7, h0std=0.0, qscale=None):
    w = synth.Workload("case", B=B, H=H, T=T, D=D, chunk=0, dtype=dtype, lam=lam,
                       qscale=(1.0 / np.sqrt(D) if qscale is None else qscale), h0std=h0std,
                       train=True, seed=seed)
    return synth.generate(w)


def _dht(d):
    rng = np.random.default_rng(d["seed"] + 99)
    return (rng.standard_normal((d["B"], d["H"], d["D"], d["D"])) * 0.5).astype(np.float32)


def _check(d, chunk, label=""):
    import torch
    import linear_attention_hgrn2_amd as m
    dt = d["dtype"]
    q, v, lf, dy = (to_dev(d[n], dt) for n in ("q", "v", "log_f", "dy"))
    h0 = to_dev(d["h0"], "f32")
    dht_np = _dht(d)
    dht = to_dev(dht_np, "f32")
    y, ht, st = m.fwd_tied(q, v, lf, h0, chunk=chunk, want_states=True)
    dq, dv, dl, dh0 = m.bwd_tied(q, v, lf, dy, h0, dht, st, chunk=chunk)
    torch.cuda.synchronize()
    x = inputs64(d)
    yr, htr = oracle.forward_tied(x["q"], x["v"], x["log_f"], x["h0"])
    gr = oracle.backward_tied(x["q"], x["v"], x["log_f"], x["dy"], x["h0"], dht_np.astype(np.float64))
    errs = {"y": slice_rel(to_host64(y), yr), "ht": slice_rel(to_host64(ht), htr, token_major=False)}
    for name, g, r in zip(("dq", "dv", "dlog_f"), (dq, dv, dl), gr[:3]):
        errs[name] = slice_rel(to_host64(g), r)
    errs["dh0"] = slice_rel(to_host64(dh0), gr[3], token_major=False)
    print("%s tied D=%d C=%d %s: %s" % (label, d["D"], chunk, dt, " ".join("%s %.3e" % e for e in errs.items())),
          flush=True)
    for name, e in errs.items():
        assert e <= TOL[dt], (name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,C", [(16, 16), (32, 32), (64, 64), (128, 16), (128, 32), (128, 64)])
def test_tied_shapes(dtype, D, C):
    import linear_attention_hgrn2_amd as m
    import torch
    if not m.supported(D, C, torch.float32 if dtype == "f32" else torch.bfloat16):
        pytest.skip("no kernel for this combination")
    d = _case(dtype, B=2, T=2 * C + 7, H=2, D=D, lam=0.3, h0std=0.5, qscale=1.0)
    _check(d, C)


@pytest.mark.parametrize("lam", [0.0, 0.97])
def test_tied_gate_regimes_d128(lam):
    """Gates far from 1 (lower bound 0) and near 1 (0.97, where k = 1 - f is
    small and must be formed without cancellation), d = 128, chunk 64, bf16,
    several chunks per workgroup."""
    d = _case("bf16", B=3, T=20 * 64 + 13, H=5, D=128, lam=lam, h0std=0.2, qscale=1.0)
    _check(d, 64, label="lam=%.2f" % lam)


def test_tied_extreme_gates_d128():
    """Full resets (k = 1), the -200 floor and in-block decays that force the
    directly summed diagonal, with tied gates."""
    d = _case("bf16", B=1, T=300, H=2, D=128, lam=0.0, h0std=0.3, qscale=1.0)
    lf = synth.to_f64(d["log_f"], "bf16")
    lf[0, 3, 0, :] = -np.inf
    lf[0, 20, 1, 2] = -200.0
    lf[0, 40:44, 0, 1] = -30.0
    lf[0, 70:80, 1, :] = -9.0
    d["log_f"] = synth.f32_to_bf16_bits(lf.astype(np.float32))
    _check(d, 64, label="extreme")
    _check(d, 16, label="extreme")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tied_staged_launches_equal_composite_calls(dtype):
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case(dtype, B=2, T=3 * 64 + 11, H=3, D=128, lam=0.3, h0std=0.5, qscale=1.0)
    q, v, lf, dy = (to_dev(d[n], dtype) for n in ("q", "v", "log_f", "dy"))
    h0 = to_dev(d["h0"], "f32")
    dht = to_dev(_dht(d), "f32")
    y, ht, st = m.fwd_tied(q, v, lf, h0, chunk=64, want_states=True)
    g = m.bwd_tied(q, v, lf, dy, h0, dht, st, chunk=64)
    _, ht2, st2 = m.fwd_tied(q, v, lf, h0, chunk=64, want_states=True, want_y=False)
    y2 = m.fwd_chunk_tied(q, v, lf, st2, chunk=64)
    lam, dh02 = m.bwd_adjoint(q, lf, dy, dht, chunk=64, want_dh0=True)
    g2 = m.bwd_chunk_tied(q, v, lf, dy, st2, lam, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(st, st2) and torch.equal(ht, ht2) and torch.equal(y, y2)
    assert torch.equal(g[3], dh02)
    for a, b in zip(g[:3], g2):
        assert torch.equal(a, b)


def test_tied_train_full():
    """The training shape (B8 H16 T4096 d128, chunk 64, bf16, lower bound 0.3)
    in the configuration the benchmark's tied leg times; every (b, h)."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate("train_bf16", lam=0.3)
    q, v, lf, dy = (to_dev(d[n], "bf16") for n in ("q", "v", "log_f", "dy"))
    y, _, st = m.fwd_tied(q, v, lf, None, chunk=64, want_ht=False, want_states=True)
    dq, dv, dl, _ = m.bwd_tied(q, v, lf, dy, None, None, st, chunk=64, want_dh0=False)
    torch.cuda.synchronize()
    x = inputs64(d)
    yr, _ = oracle.forward_tied(x["q"], x["v"], x["log_f"], None)
    errs = {"y": errors(to_host64(y), yr)}
    del yr
    gr = oracle.backward_tied(x["q"], x["v"], x["log_f"], x["dy"], None, None)
    for name, g, r in zip(("dq", "dv", "dlog_f"), (dq, dv, dl), gr[:3]):
        errs[name] = errors(to_host64(g), r)
    print("tied train, all 128 (b,h): %s" % "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items()), flush=True)
    for name, e in errs.items():
        assert worst(e) <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 128])
def test_tied_decode(dtype, D):
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate_decode("decode_f32", B=3, H=5, D=D, seed=13)
    conv = (lambda a: a) if dtype == "f32" else (lambda a: synth.f32_to_bf16_bits(a))
    q, v, lf = (to_dev(conv(d[n]), dtype) for n in ("q", "v", "log_f"))
    S = to_dev(d["state"], "f32")
    y = m.decode_step_tied(q, v, lf, S)
    torch.cuda.synchronize()
    x = {n: synth.to_f64(conv(d[n]), dtype) for n in ("q", "v", "log_f")}
    yr, Sr = oracle.decode_step_tied(x["q"], x["v"], x["log_f"], d["state"].astype(np.float64))
    ey = worst(errors(to_host64(y)[:, None], yr[:, None]))
    es = worst(errors(to_host64(S), Sr, "state"))
    print("tied decode D=%d %s: y %.3e state %.3e" % (D, dtype, ey, es), flush=True)
    assert ey <= TOL[dtype] and es <= 1e-5
