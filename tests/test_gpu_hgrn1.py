"""GPU parity of the HGRN1 elementwise recurrence (hgrn1_fwd / hgrn1_bwd over
[B, T, C]) against the float64 oracle's HGRN1 functions (the step loop with
one channel per head), on the same seeded inputs.  Every channel sequence,
token row and element is compared (tests/gpu_util.py, layout "btc"; the final
states [B, C] per batch element and per channel): <= 2e-2 (bf16), <= 1e-4
(fp32)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu


def _inputs(dtype, B, T, C, lam=0.3, seed=5):
    """HGRN1 inputs from the same generator as the HGRN2 workloads: [B, T, H, D]
    with H D = C read as [B, T, C]; h0 and dht float32 [B, C]."""
    H, D = C // 2, 2
    w = synth.Workload("h1", B=B, H=H, T=T, D=D, chunk=0, dtype=dtype, lam=lam, qscale=1.0, h0std=0.0,
                       train=True, seed=seed)
    d = synth.generate(w)
    r = np.random.default_rng(seed + 1)
    out = {n: d[n].reshape(B, T, C) for n in ("q", "k", "v", "log_f", "dy")}
    out["h0"] = r.standard_normal((B, C)).astype(np.float32)
    out["dht"] = (0.5 * r.standard_normal((B, C))).astype(np.float32)
    out["dtype"] = dtype
    return out


def _err(a, b):
    """errors() of a [B, T, C] token tensor ("btc") or a [B, C] state (one
    slice per batch element, one row per channel)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.ndim == 2:
        return errors(a[:, None, :, None], b[:, None, :, None], "state")
    return errors(a, b, "btc")


def _run(x, tied, with_states=True):
    import torch
    import linear_attention_hgrn2_amd as m
    dt = x["dtype"]
    q, k, v, lf, dy = (to_dev(x[n], dt) for n in ("q", "k", "v", "log_f", "dy"))
    h0, dht = to_dev(x["h0"], "f32"), to_dev(x["dht"], "f32")
    y, ht, st = m.hgrn1_fwd(q, k, v, lf, h0, tied=tied, want_states=with_states)
    g = m.hgrn1_bwd(q, k, v, lf, dy, h0, dht, st, tied=tied)
    torch.cuda.synchronize()
    return y, ht, st, g


def _check(x, tied, label=""):
    dt = x["dtype"]
    y, ht, _, (dq, dk, dv, dl, dh0) = _run(x, tied)
    f = {n: synth.to_f64(x[n], dt) for n in ("q", "k", "v", "log_f", "dy")}
    h0, dht = x["h0"].astype(np.float64), x["dht"].astype(np.float64)
    yr, htr = oracle.hgrn1_forward(f["q"], f["k"], f["v"], f["log_f"], h0, tied=tied)
    gr = oracle.hgrn1_backward(f["q"], f["k"], f["v"], f["log_f"], f["dy"], h0, dht, tied=tied)
    errs = {"y": _err(to_host64(y), yr), "hT": _err(to_host64(ht), htr)}
    for name, a, r in zip(("dq", "dk", "dv", "dlog_f", "dh0"), (dq, dk, dv, dl, dh0), gr):
        if r is not None:
            errs[name] = _err(to_host64(a), r)
    print("%s hgrn1 %s %s tied=%d: %s" % (label, dt, tuple(x["q"].shape), tied,
                                          "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items())), flush=True)
    for name, e in errs.items():
        assert worst(e) <= TOL[dt], (name, e)


@pytest.mark.parametrize("tied", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C", [(2, 70, 6), (3, 32, 256), (2, 1, 130), (2, 257, 512), (1, 1000, 1024)])
def test_hgrn1_shapes(dtype, tied, B, T, C):
    """Ragged last segments (70, 257, 1000 tokens), a single token, a single
    segment, and channel counts that fill a workgroup partly (6, 130)."""
    _check(_inputs(dtype, B, T, C), tied)


@pytest.mark.parametrize("lam", [0.0, 0.97])
def test_hgrn1_gate_regimes(lam):
    """Gates far from one (many tokens forget almost everything) and near one."""
    _check(_inputs("bf16", 2, 600, 256, lam=lam), True, label="lam=%.2f" % lam)


def test_hgrn1_saved_states_equal_recomputed_and_repeat_is_bitwise():
    import torch
    import linear_attention_hgrn2_amd as m
    x = _inputs("bf16", 2, 300, 512)
    a = _run(x, True, with_states=True)
    b = _run(x, True, with_states=False)
    c = _run(x, True, with_states=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for u, w in zip(a[3], b[3]):
        assert (u is None and w is None) or torch.equal(u, w)
    assert torch.equal(a[2], c[2])
    for u, w in zip(a[3], c[3]):
        assert (u is None and w is None) or torch.equal(u, w)


def test_hgrn1_full_size_all_channels():
    """B8 T4096 C2048 (the training workload's H16 x d128 channels), bf16, tied,
    as the benchmark runs it; the oracle recomputes every channel."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = synth.generate("train_bf16", lam=0.3)
    B, T, C = d["B"], d["T"], d["H"] * d["D"]
    x = {n: d[n].reshape(B, T, C) for n in ("q", "v", "log_f", "dy")}
    q, v, lf, dy = (to_dev(x[n], "bf16") for n in ("q", "v", "log_f", "dy"))
    y, ht, st = m.hgrn1_fwd(q, None, v, lf, None, tied=True, want_states=True)
    dq, _, dv, dl, _ = m.hgrn1_bwd(q, None, v, lf, dy, None, None, st, tied=True, want_dh0=False)
    torch.cuda.synchronize()
    f = {n: synth.to_f64(x[n], "bf16") for n in ("q", "v", "log_f", "dy")}
    yr, htr = oracle.hgrn1_forward(f["q"], None, f["v"], f["log_f"], None, tied=True)
    errs = {"y": _err(to_host64(y), yr), "hT": _err(to_host64(ht), htr)}
    del yr
    gr = oracle.hgrn1_backward(f["q"], None, f["v"], f["log_f"], f["dy"], None, None, tied=True)
    for name, a, r in zip(("dq", "dv", "dlog_f"), (dq, dv, dl), (gr[0], gr[2], gr[3])):
        errs[name] = _err(to_host64(a), r)
    print("hgrn1 full size, all %d channels: %s" % (B * C, "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items())),
          flush=True)
    for name, e in errs.items():
        assert worst(e) <= TOL["bf16"], (name, e)
