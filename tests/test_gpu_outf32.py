"""GPU parity of float32 outputs for bfloat16 inputs (HGRN2_OUT_F32; the
binding's out_dtype=torch.float32), for every entry point with token outputs,
in every gate mode and on every kernel path: the segmented forward (chunk 64),
the stored-state forward (other chunks, or states kept), the resident backward
(D = 128, chunk 64), the generic backward, the decode step and HGRN1.

Two checks per output:
  1. the float32 values meet the float64 oracle within the bfloat16 tolerance
     (the inputs and the matrix-core operands are still bfloat16; only the
     final rounding of the results is skipped);
  2. rounded to bfloat16 (to nearest even, as the kernels round) they equal,
     bit for bit, the outputs of the same call without the flag: both compute
     the same float32 values and differ only in the store.
float32 results that never had a bfloat16 form (ht, dh0, the lower-bound
gradient, the decode state) are bitwise equal between the two calls."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu

MODES = ("untied", "tied", "gate", "scalar")


def _case(B, T, H, D, seed=11):
    w = synth.Workload("case", B=B, H=H, T=T, D=D, chunk=0, dtype="bf16", lam=0.3, qscale=1.0, h0std=0.5,
                       train=True, seed=seed)
    d = synth.generate(w)
    d["lb"] = synth.lower_bounds(H, D, 0.3, 0.25, seed=seed + 3)
    d["log_a"] = np.ascontiguousarray(d["log_f"][..., 0])
    r = np.random.default_rng(seed + 99)
    d["dht"] = (r.standard_normal((B, H, D, D)) * 0.5).astype(np.float32)
    return d


def _dev(d):
    x = {n: to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f", "z", "dy", "log_a")}
    x["lb"] = to_dev(d["lb"], "f32")
    x["h0"] = to_dev(d["h0"], "f32")
    x["dht"] = to_dev(d["dht"], "f32")
    return x


def _fwd(m, gm, x, chunk, out_dtype, want_states):
    kw = dict(chunk=chunk, want_states=want_states, out_dtype=out_dtype)
    if gm == "untied":
        return m.fwd(x["q"], x["k"], x["v"], x["log_f"], x["h0"], **kw)
    if gm == "tied":
        return m.fwd_tied(x["q"], x["v"], x["log_f"], x["h0"], **kw)
    if gm == "gate":
        return m.fwd_gate(x["q"], x["v"], x["z"], x["lb"], x["h0"], **kw)
    return m.fwd_scalar(x["q"], x["k"], x["v"], x["log_a"], x["h0"], **kw)


def _bwd(m, gm, x, states, chunk, out_dtype):
    """Gradients as a dict name -> tensor (token gradients and float32 ones)."""
    kw = dict(chunk=chunk, out_dtype=out_dtype)
    q, v, dy, h0, dht = x["q"], x["v"], x["dy"], x["h0"], x["dht"]
    if gm == "untied":
        g = m.bwd(q, x["k"], v, x["log_f"], dy, h0, dht, states, **kw)
        return dict(dq=g[0], dk=g[1], dv=g[2], dlog_f=g[3], dh0=g[4])
    if gm == "tied":
        g = m.bwd_tied(q, v, x["log_f"], dy, h0, dht, states, **kw)
        return dict(dq=g[0], dv=g[1], dlog_f=g[2], dh0=g[3])
    if gm == "gate":
        g = m.bwd_gate(q, v, x["z"], x["lb"], dy, h0, dht, states, **kw)
        return dict(dq=g[0], dv=g[1], dz=g[2], dlb=g[3], dh0=g[4])
    g = m.bwd_scalar(q, x["k"], v, x["log_a"], dy, h0, dht, states, **kw)
    return dict(dq=g[0], dk=g[1], dv=g[2], dlog_a=g[3], dh0=g[4])


def _oracle(gm, d):
    f = {n: synth.to_f64(d[n], "bf16") for n in ("q", "k", "v", "log_f", "z", "dy", "log_a")}
    h0, dht = d["h0"].astype(np.float64), d["dht"].astype(np.float64)
    lb = d["lb"].astype(np.float64)
    if gm == "untied":
        (y, ht), g = (oracle.forward(f["q"], f["k"], f["v"], f["log_f"], h0),
                      oracle.backward(f["q"], f["k"], f["v"], f["log_f"], f["dy"], h0, dht))
        return y, ht, dict(dq=g[0], dk=g[1], dv=g[2], dlog_f=g[3], dh0=g[4])
    if gm == "tied":
        (y, ht), g = (oracle.forward_tied(f["q"], f["v"], f["log_f"], h0),
                      oracle.backward_tied(f["q"], f["v"], f["log_f"], f["dy"], h0, dht))
        return y, ht, dict(dq=g[0], dv=g[1], dlog_f=g[2], dh0=g[3])
    if gm == "gate":
        (y, ht), g = (oracle.forward_gate(f["q"], f["v"], f["z"], lb, h0),
                      oracle.backward_gate(f["q"], f["v"], f["z"], lb, f["dy"], h0, dht))
        return y, ht, dict(dq=g[0], dv=g[1], dz=g[2], dlb=g[3], dh0=g[4])
    (y, ht), g = (oracle.forward_scalar(f["q"], f["k"], f["v"], f["log_a"], h0),
                  oracle.backward_scalar(f["q"], f["k"], f["v"], f["log_a"], f["dy"], h0, dht))
    return y, ht, dict(dq=g[0], dk=g[1], dv=g[2], dlog_a=g[3], dh0=g[4])


def _err(name, got, ref):
    a, b = to_host64(got), np.asarray(ref, np.float64)
    if name in ("ht", "dh0"):
        return errors(a, b, "state")
    if name == "dlb":
        return errors(a[None, :, :, None], b[None, :, :, None], "state")
    if name == "dlog_a":
        return errors(a[..., None], b[..., None], "token")
    return errors(a, b, "token")


def _same_after_rounding(name, o32, o16):
    import torch
    if o16.dtype == torch.float32:  # never rounded: the same float32 values
        assert torch.equal(o32, o16), name
        return
    assert o32.dtype == torch.float32, (name, o32.dtype)
    r = o32.to(torch.bfloat16)
    if not torch.equal(r.view(torch.int16), o16.view(torch.int16)):
        bad = (r.view(torch.int16) != o16.view(torch.int16)).nonzero()
        raise AssertionError("%s: %d of %d values differ after rounding, first at %s"
                             % (name, bad.shape[0], o16.numel(), tuple(bad[0].tolist())))


@pytest.mark.parametrize("gm", MODES)
@pytest.mark.parametrize("D,C", [(128, 64), (64, 64), (128, 32), (32, 128), (128, 128), (16, 16)])
def test_out_f32_fwd_bwd(gm, D, C):
    """Forward (segmented walk when no state is kept, stored-state otherwise)
    and backward, every gate mode; D 128 / chunk 64 is the resident backward."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case(B=2, T=3 * C + 21, H=3, D=D)
    x = _dev(d)
    y32, ht32, _ = _fwd(m, gm, x, C, torch.float32, False)        # no states: the segmented walk (chunk 64)
    y16, ht16, _ = _fwd(m, gm, x, C, None, False)
    ys16, _, st = _fwd(m, gm, x, C, None, True)
    ys32, hts32, st32 = _fwd(m, gm, x, C, torch.float32, True)    # stored states
    g32 = _bwd(m, gm, x, st, C, torch.float32)
    g16 = _bwd(m, gm, x, st, C, None)
    torch.cuda.synchronize()
    _same_after_rounding("y (walk)", y32, y16)
    assert torch.equal(ht32, ht16)
    assert torch.equal(st32.view(torch.int16), st.view(torch.int16))  # states keep the input dtype
    _same_after_rounding("y (stored)", ys32, ys16)
    for n in g16:
        _same_after_rounding(n, g32[n], g16[n])
    yr, htr, gr = _oracle(gm, d)
    errs = {"y": _err("y", y32, yr), "y_stored": _err("y", ys32, yr), "ht": _err("ht", ht32, htr)}
    errs.update({n: _err(n, g32[n], gr[n]) for n in gr})
    print("out f32 %s D=%d C=%d: %s" % (gm, D, C, "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items())),
          flush=True)
    for n, e in errs.items():
        assert worst(e) <= TOL["bf16"], (n, fmt(e))


def test_out_f32_flag_is_a_no_op_for_float32_inputs():
    """float32 inputs write float32 anyway: with the flag the calls give the
    same bits as without it (forward walk and stored-state, backward)."""
    import torch
    import linear_attention_hgrn2_amd as m
    w = synth.Workload("case", B=2, H=2, T=150, D=64, chunk=0, dtype="f32", lam=0.3, qscale=1.0, h0std=0.5,
                       train=True, seed=4)
    d = synth.generate(w)
    q, k, v, lf, dy = (to_dev(d[n], "f32") for n in ("q", "k", "v", "log_f", "dy"))
    h0 = to_dev(d["h0"], "f32")
    outs = {}
    for od in (torch.float32, None):
        y, ht, _ = m.fwd(q, k, v, lf, h0, chunk=64, out_dtype=od)
        ys, _, st = m.fwd(q, k, v, lf, h0, chunk=64, want_states=True, out_dtype=od)
        g = m.bwd(q, k, v, lf, dy, h0, None, st, chunk=64, out_dtype=od)
        outs[od] = (y, ht, ys) + tuple(g)
    torch.cuda.synchronize()
    for a, b in zip(outs[torch.float32], outs[None]):
        assert a.dtype == b.dtype == torch.float32
        assert torch.equal(a, b)


def test_out_f32_is_closer_to_the_oracle():
    """The float32 outputs lose no accuracy to the bfloat16 ones: their
    normwise error is at most that of the rounded outputs (rounding adds
    about 2^-9 relative per element on top)."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case(B=2, T=300, H=3, D=128, seed=21)
    x = _dev(d)
    y32, _, st = _fwd(m, "untied", x, 64, torch.float32, True)
    y16, _, _ = _fwd(m, "untied", x, 64, None, True)
    g32 = _bwd(m, "untied", x, st, 64, torch.float32)
    g16 = _bwd(m, "untied", x, st, 64, None)
    torch.cuda.synchronize()
    yr, _, gr = _oracle("untied", d)
    for n, a, b, r in [("y", y32, y16, yr)] + [(k, g32[k], g16[k], gr[k]) for k in ("dq", "dk", "dv", "dlog_f")]:
        e32, e16 = _err(n, a, r)["norm"], _err(n, b, r)["norm"]
        print("%s: float32 out %.3e, bfloat16 out %.3e" % (n, e32, e16), flush=True)
        assert e32 <= e16 * 1.0001 + 1e-7, (n, e32, e16)


@pytest.mark.parametrize("gm", MODES)
@pytest.mark.parametrize("D", [16, 128])
def test_out_f32_decode(gm, D):
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case(B=3, T=1, H=4, D=D, seed=5)
    x = {n: t[:, 0].contiguous() for n, t in _dev(d).items() if n in ("q", "k", "v", "log_f", "z", "log_a")}
    s0 = to_dev(d["h0"], "f32")
    lb = to_dev(d["lb"], "f32")
    outs = {}
    for od in (torch.float32, None):
        s = s0.clone()
        if gm == "untied":
            y = m.decode_step(x["q"], x["k"], x["v"], x["log_f"], s, out_dtype=od)
        elif gm == "tied":
            y = m.decode_step_tied(x["q"], x["v"], x["log_f"], s, out_dtype=od)
        elif gm == "gate":
            y = m.decode_step_gate(x["q"], x["v"], x["z"], lb, s, out_dtype=od)
        else:
            y = m.decode_step_scalar(x["q"], x["k"], x["v"], x["log_a"], s, out_dtype=od)
        outs[od] = (y, s)
    torch.cuda.synchronize()
    # an output of the wrong dtype or shape is refused before anything runs
    with pytest.raises(ValueError):
        m.decode_step(x["q"], x["k"], x["v"], x["log_f"], s0.clone(), out_dtype=torch.float32,
                      y=torch.empty_like(x["q"]))
    with pytest.raises(ValueError):
        m.decode_step(x["q"], x["k"], x["v"], x["log_f"], s0.clone(), y=torch.empty_like(x["q"])[:, :1])
    (y32, s32), (y16, s16) = outs[torch.float32], outs[None]
    assert torch.equal(s32, s16)
    _same_after_rounding("y", y32, y16)
    yr, _, _ = _oracle(gm, d)  # T = 1: the forward's one output is the decode step's
    e = errors(to_host64(y32)[:, None], np.asarray(yr, np.float64), "token")
    assert worst(e) <= TOL["bf16"], fmt(e)


@pytest.mark.parametrize("tied", [False, True])
def test_out_f32_hgrn1(tied):
    import torch
    import linear_attention_hgrn2_amd as m
    B, T, C = 2, 300, 258
    w = synth.Workload("h1", B=B, H=C // 2, T=T, D=2, chunk=0, dtype="bf16", lam=0.3, qscale=1.0, h0std=0.0,
                       train=True, seed=17)
    d = synth.generate(w)
    x = {n: to_dev(d[n].reshape(B, T, C), "bf16") for n in ("q", "k", "v", "log_f", "dy")}
    r = np.random.default_rng(18)
    h0 = torch.from_numpy(r.standard_normal((B, C)).astype(np.float32)).cuda()
    dht = torch.from_numpy((0.5 * r.standard_normal((B, C))).astype(np.float32)).cuda()
    k = None if tied else x["k"]
    res = {}
    for od in (torch.float32, None):
        y, ht, st = m.hgrn1_fwd(x["q"], k, x["v"], x["log_f"], h0, tied=tied, want_states=True, out_dtype=od)
        g = m.hgrn1_bwd(x["q"], k, x["v"], x["log_f"], x["dy"], h0, dht, st, tied=tied, out_dtype=od)
        res[od] = (y, ht) + tuple(g)
    torch.cuda.synchronize()
    names = ("y", "ht", "dq", "dk", "dv", "dlog_f", "dh0")
    for n, a, b in zip(names, res[torch.float32], res[None]):
        if a is None:
            continue
        _same_after_rounding(n, a, b)
    f = {n: synth.to_f64(d[n].reshape(B, T, C), "bf16") for n in ("q", "k", "v", "log_f", "dy")}
    h064, dht64 = h0.double().cpu().numpy(), dht.double().cpu().numpy()
    yr, _ = oracle.hgrn1_forward(f["q"], None if tied else f["k"], f["v"], f["log_f"], h064, tied=tied)
    gr = oracle.hgrn1_backward(f["q"], None if tied else f["k"], f["v"], f["log_f"], f["dy"], h064, dht64,
                               tied=tied)
    for n, a, ref in zip(("y", "dq", "dk", "dv", "dlog_f"), (res[torch.float32][0],) + res[torch.float32][2:6],
                         (yr,) + tuple(gr[:4])):
        if a is None:
            continue
        e = errors(to_host64(a), np.asarray(ref, np.float64), "btc")
        assert worst(e) <= TOL["bf16"], (n, fmt(e))


def test_out_f32_autograd():
    """hgrn2_chunk(out_dtype=float32): y in float32; the backward takes dy in
    the input dtype and returns the same gradients as the functional call."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case(B=1, T=200, H=2, D=64, seed=3)
    x = _dev(d)
    leaves = [x[n].clone().requires_grad_(True) for n in ("q", "k", "v", "log_f")]
    h0 = x["h0"].clone().requires_grad_(True)
    y, ht = m.hgrn2_chunk(*leaves, h0, 64, out_dtype=torch.float32)
    assert y.dtype == torch.float32 and ht.dtype == torch.float32
    dy32 = x["dy"].float()
    (y * dy32).sum().backward()
    torch.cuda.synchronize()
    _, _, st = m.fwd(x["q"], x["k"], x["v"], x["log_f"], x["h0"], chunk=64, want_states=True)
    g = m.bwd(x["q"], x["k"], x["v"], x["log_f"], x["dy"], x["h0"], None, st, chunk=64)
    torch.cuda.synchronize()
    for leaf, ref in zip(leaves + [h0], g):
        assert leaf.grad.dtype == ref.dtype
        assert torch.equal(leaf.grad, ref)
