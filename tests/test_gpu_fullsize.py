"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The GPU computes every (b, h); the oracle recomputes a few
sampled (b, h) sequences in full, which are compared slice by slice
(normwise relative error; 2e-2 for bf16, 1e-4 for float32)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, inputs64, select_bh, slice_rel, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _pairs(B, H, n, seed):
    r = np.random.default_rng(seed)
    idx = r.choice(B * H, size=min(n, B * H), replace=False)
    return [(int(i) // H, int(i) % H) for i in sorted(idx)]


def _fwd_full(name, lam=None, nsample=3):
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate(name, lam=lam)
    dt = d["dtype"]
    q, k, v, lf = (to_dev(d[n], dt) for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    y, ht, _ = m.fwd(q, k, v, lf, h0, chunk=d["chunk"])
    torch.cuda.synchronize()
    pairs = _pairs(d["B"], d["H"], nsample, d["seed"])
    x = inputs64(d)
    sub = {n: select_bh(x[n], pairs) for n in ("q", "k", "v", "log_f")}
    h0s = select_bh(x["h0"], pairs, token_major=False)
    yr, htr = oracle.forward(sub["q"], sub["k"], sub["v"], sub["log_f"], h0s)
    yg = select_bh(to_host64(y), pairs)
    hg = select_bh(to_host64(ht), pairs, token_major=False)
    ey, eh = slice_rel(yg, yr), slice_rel(hg, htr, token_major=False)
    print("%s full fwd pairs %s: y %.3e ht %.3e" % (name, pairs, ey, eh), flush=True)
    assert ey <= TOL[dt] and eh <= TOL[dt]


def test_fwd_bf16_full():
    """B4 H8 T2048 d128, lower bound 0.5, chunk 64."""
    _fwd_full("fwd_bf16")


def test_long_bf16_full():
    """B1 H32 T32768 d128, lower bound 0.97, random float32 initial state, final state out."""
    _fwd_full("long_bf16", nsample=2)


@pytest.mark.parametrize("lam", synth.TRAIN_LAMBDAS)
def test_train_bf16_full(lam):
    """B8 H16 T4096 d128: forward saving states, then backward from them."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate("train_bf16", lam=lam)
    C = d["chunk"]
    q, k, v, lf, dy = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f", "dy"))
    y, _, states = m.fwd(q, k, v, lf, None, chunk=C, want_ht=False, want_states=True)
    dq, dk, dv, dl, _ = m.bwd(q, k, v, lf, dy, None, None, states, chunk=C, want_dh0=False)
    torch.cuda.synchronize()
    pairs = _pairs(d["B"], d["H"], 2, d["seed"] + int(lam * 10))
    x = inputs64(d)
    sub = {n: select_bh(x[n], pairs) for n in ("q", "k", "v", "log_f", "dy")}
    yr, _ = oracle.forward(sub["q"], sub["k"], sub["v"], sub["log_f"], None)
    gr = oracle.backward(sub["q"], sub["k"], sub["v"], sub["log_f"], sub["dy"], None, None)
    errs = {"y": slice_rel(select_bh(to_host64(y), pairs), yr)}
    for name, g, r in zip(("dq", "dk", "dv", "dlog_f"), (dq, dk, dv, dl), gr[:4]):
        errs[name] = slice_rel(select_bh(to_host64(g), pairs), r)
    print("train_bf16 lam=%.1f pairs %s: %s" % (lam, pairs, " ".join("%s %.3e" % e for e in errs.items())),
          flush=True)
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)


def test_decode_full():
    """B256 H16 d128, float32 state, one step in place."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate_decode("decode_f32")
    q, k, v, lf = (to_dev(d[n], "f32") for n in ("q", "k", "v", "log_f"))
    S = to_dev(d["state"], "f32")
    y = m.decode_step(q, k, v, lf, S)
    torch.cuda.synchronize()
    pairs = _pairs(d["B"], d["H"], 64, 3)
    bi = [b for b, _ in pairs]
    hi = [h for _, h in pairs]
    yr, Sr = oracle.decode_step(d["q"][bi, hi][:, None], d["k"][bi, hi][:, None], d["v"][bi, hi][:, None],
                                d["log_f"][bi, hi][:, None], d["state"][bi, hi][:, None])
    yg = to_host64(y)[bi, hi][:, None]
    Sg = to_host64(S)[bi, hi][:, None]
    ey = max(np.linalg.norm(yg[i] - yr[i]) / np.linalg.norm(yr[i]) for i in range(len(pairs)))
    es = max(np.linalg.norm(Sg[i] - Sr[i]) / np.linalg.norm(Sr[i]) for i in range(len(pairs)))
    print("decode full: y %.3e state %.3e" % (ey, es), flush=True)
    assert ey <= TOL["f32"] and es <= 1e-5
