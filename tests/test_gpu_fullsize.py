"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The GPU computes every (b, h) and the oracle recomputes
every (b, h) sequence in full; every slice, row and element is compared
(tests/gpu_util.py: normwise per slice, per row and per element, 2e-2 for
bf16 and 1e-4 for float32)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, inputs64, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu


def _fwd_full(name):
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate(name)
    dt = d["dtype"]
    q, k, v, lf = (to_dev(d[n], dt) for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    y, ht, _ = m.fwd(q, k, v, lf, h0, chunk=d["chunk"])
    torch.cuda.synchronize()
    x = inputs64(d)
    yr, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], x["h0"])
    ey = errors(to_host64(y), yr)
    eh = errors(to_host64(ht), htr, "state")
    print("%s full fwd, all %d (b,h): y %s | ht %s" % (name, d["B"] * d["H"], fmt(ey), fmt(eh)), flush=True)
    assert worst(ey) <= TOL[dt] and worst(eh) <= TOL[dt]


def test_fwd_bf16_full():
    """B4 H8 T2048 d128, lower bound 0.5, chunk 64."""
    _fwd_full("fwd_bf16")


def test_long_bf16_full():
    """B1 H32 T32768 d128, lower bound 0.97, random float32 initial state, final state out."""
    _fwd_full("long_bf16")


@pytest.mark.parametrize("lam", synth.TRAIN_LAMBDAS)
def test_train_bf16_full(lam):
    """B8 H16 T4096 d128: forward saving states, then backward from them; all
    128 (b, h) sequences against the oracle."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate("train_bf16", lam=lam)
    C = d["chunk"]
    q, k, v, lf, dy = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f", "dy"))
    y, _, states = m.fwd(q, k, v, lf, None, chunk=C, want_ht=False, want_states=True)
    dq, dk, dv, dl, _ = m.bwd(q, k, v, lf, dy, None, None, states, chunk=C, want_dh0=False)
    torch.cuda.synchronize()
    x = inputs64(d)
    del d
    yr, _ = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], None)
    errs = {"y": errors(to_host64(y), yr)}
    del yr
    gr = oracle.backward(x["q"], x["k"], x["v"], x["log_f"], x["dy"], None, None)
    for name, g, r in zip(("dq", "dk", "dv", "dlog_f"), (dq, dk, dv, dl), gr[:4]):
        errs[name] = errors(to_host64(g), r)
    print("train_bf16 lam=%.1f, all 128 (b,h): %s" % (lam, "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items())),
          flush=True)
    for name, e in errs.items():
        assert worst(e) <= TOL["bf16"], (name, e)


def test_decode_full():
    """B256 H16 d128, float32 state, one step in place; every (b, h)."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate_decode("decode_f32")
    q, k, v, lf = (to_dev(d[n], "f32") for n in ("q", "k", "v", "log_f"))
    S = to_dev(d["state"], "f32")
    y = m.decode_step(q, k, v, lf, S)
    torch.cuda.synchronize()
    yr, Sr = oracle.decode_step(d["q"], d["k"], d["v"], d["log_f"], d["state"])
    ey = errors(to_host64(y)[:, None], yr[:, None])   # [B, 1, H, D]: one token per sequence
    es = errors(to_host64(S), Sr, "state")
    print("decode full, all 4096 (b,h): y %s | state %s" % (fmt(ey), fmt(es)), flush=True)
    assert worst(ey) <= TOL["f32"] and worst(es) <= 1e-5
