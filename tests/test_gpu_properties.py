"""Properties of the recurrence checked on the HIP path (d = 128, chunk 64, in
bfloat16 and float32: the resident backward and the general one).

HGRN2 summary (paperlayer.ai) §3.2: S_t = Diag(f_t) S_{t-1} + k_t^T v_t,
y_t = q_t S_t, per (batch, head) with no coupling between them (§3.2 p.5: the
heads are independent recurrences).  Hence:
  - f = 1 everywhere (log f = 0) is causal linear attention,
    y = tril(Q K^T) V + Q h0, and f = 0 everywhere (log f = -inf) leaves one
    term per token, y_t = (q_t . k_t) v_t: both against the oracle, whose pins
    fix these limits;
  - permuting batch elements and heads permutes the outputs, bit for bit;
  - y and the final state are linear in (v, h0): scaling both by a power of
    two scales them exactly; y(v1 + v2) = y(v1) + y(v2) within tolerance;
  - value column j of y, of the final state and of dv depends on value
    column j of v, h0 and dy only: changing the other columns leaves it
    unchanged, bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, inputs64, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu

D, C = 128, 64


def _case(dtype, B=2, T=3 * 64 + 21, H=3, lam=0.3, seed=31, h0std=0.3):
    w = synth.Workload("prop", B=B, H=H, T=T, D=D, chunk=C, dtype=dtype, lam=lam, qscale=1.0 / np.sqrt(D),
                       h0std=h0std, train=True, seed=seed)
    return synth.generate(w)


def _dht(d):
    rng = np.random.default_rng(d["seed"] + 99)
    return (rng.standard_normal((d["B"], d["H"], D, D)) * 0.5).astype(np.float32)


def _store(x64, dtype):
    return x64.astype(np.float32) if dtype == "f32" else synth.f32_to_bf16_bits(x64.astype(np.float32))


def _run(tensors, dtype):
    """Forward saving states, then backward; every output, on the host in float64."""
    import torch
    import linear_attention_hgrn2_amd as m
    q, k, v, lf, dy = (to_dev(tensors[n], dtype) for n in ("q", "k", "v", "log_f", "dy"))
    h0, dht = to_dev(tensors["h0"], "f32"), to_dev(tensors["dht"], "f32")
    y, ht, st = m.fwd(q, k, v, lf, h0, chunk=C, want_states=True)
    dq, dk, dv, dl, dh0 = m.bwd(q, k, v, lf, dy, h0, dht, st, chunk=C)
    torch.cuda.synchronize()
    return {n: to_host64(t) for n, t in zip(("y", "ht", "dq", "dk", "dv", "dlog_f", "dh0"),
                                            (y, ht, dq, dk, dv, dl, dh0))}


def _tensors(d):
    return {n: d[n] for n in ("q", "k", "v", "log_f", "dy", "h0")} | {"dht": _dht(d)}


def _against_oracle(d, t, label):
    dt = d["dtype"]
    got = _run(t, dt)
    x = {n: synth.to_f64(t[n], dt) for n in ("q", "k", "v", "log_f", "dy")}
    h0, dht = t["h0"].astype(np.float64), t["dht"].astype(np.float64)
    yr, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], h0)
    gr = oracle.backward(x["q"], x["k"], x["v"], x["log_f"], x["dy"], h0, dht)
    refs = {"y": yr, "ht": htr, "dq": gr[0], "dk": gr[1], "dv": gr[2], "dlog_f": gr[3], "dh0": gr[4]}
    errs = {n: errors(got[n], r, "state" if n in ("ht", "dh0") else "token") for n, r in refs.items()}
    print("%s %s: %s" % (label, dt, "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items())), flush=True)
    return got, refs, errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_forgetting_is_causal_linear_attention(dtype):
    """log f = 0 on every token (f = 1): the oracle is pinned to
    tril(Q K^T) V + Q h0 here; the kernels must meet it (the cumulative decay
    and every gap factor are exactly 1)."""
    d = _case(dtype)
    t = _tensors(d)
    t["log_f"] = _store(np.zeros(d["q"].shape), dtype)
    _, _, errs = _against_oracle(d, t, "f=1")
    for n, e in errs.items():
        assert worst(e) <= TOL[dtype], (n, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_forgetting_keeps_one_term_per_token(dtype):
    """log f = -inf on every token (f = 0): y_t = (q_t . k_t) v_t, the final
    state is k_T^T v_T, and nothing reaches h0 or the decay: dlog f and dh0
    are zero in exact arithmetic (their reference slices are all zero and are
    compared in absolute terms; the kernels' cancellation residue must stay
    far below the tolerance), and no NaN may appear (the kernels floor log f
    at -200)."""
    d = _case(dtype)
    t = _tensors(d)
    t["log_f"] = _store(np.full(d["q"].shape, -np.inf), dtype)
    got, refs, errs = _against_oracle(d, t, "f=0")
    assert not np.any(refs["dlog_f"]) and not np.any(refs["dh0"])
    for n, e in errs.items():
        assert worst(e) <= TOL[dtype], (n, e)
    # the one-term form itself, on the GPU's y (the oracle's pins fix it too)
    x = {n: synth.to_f64(t[n], dtype) for n in ("q", "k", "v")}
    direct = (x["q"] * x["k"]).sum(-1, keepdims=True) * x["v"]
    assert worst(errors(got["y"], direct)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batch_and_head_permutation_is_bitwise(dtype):
    """Batch elements and heads are independent recurrences computed by the
    same operations in the same order wherever they sit in the tensors."""
    d = _case(dtype, B=3, H=4)
    t = _tensors(d)
    base = _run(t, dtype)
    pb, ph = np.array([2, 0, 1]), np.array([3, 1, 0, 2])
    tp = {n: np.ascontiguousarray(t[n][pb][:, :, ph]) for n in ("q", "k", "v", "log_f", "dy")}
    tp.update({n: np.ascontiguousarray(t[n][pb][:, ph]) for n in ("h0", "dht")})
    perm = _run(tp, dtype)
    for n, a in base.items():
        want = a[pb][:, ph] if n in ("ht", "dh0") else a[pb][:, :, ph]
        assert np.array_equal(perm[n], want), n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_linearity_in_v_and_h0(dtype):
    """y and ht are linear in (v, h0) jointly, and every gradient is linear in
    (dy, dht): scaling by 2 (exact in both dtypes) scales the outputs exactly;
    the sum of two value inputs gives the sum of the outputs within tolerance.
    (Lower bound 0.5 keeps every decayed product in float32's normal range, so
    that no subnormal flush can tell x from 2 x.)"""
    d = _case(dtype, lam=0.5)
    t = _tensors(d)
    base = _run(t, dtype)
    t2 = dict(t)
    t2["v"] = _store(2.0 * synth.to_f64(t["v"], dtype), dtype)
    t2["h0"] = (2.0 * t["h0"]).astype(np.float32)
    t2["dy"] = _store(2.0 * synth.to_f64(t["dy"], dtype), dtype)
    t2["dht"] = (2.0 * t["dht"]).astype(np.float32)
    sc = _run(t2, dtype)
    assert np.array_equal(sc["y"], 2.0 * base["y"]) and np.array_equal(sc["ht"], 2.0 * base["ht"])
    # q, k and log f enter the gradients through (v, h0) once and (dy, dht) once
    for n in ("dq", "dk", "dlog_f"):
        assert np.array_equal(sc[n], 4.0 * base[n]), n
    assert np.array_equal(sc["dv"], 2.0 * base["dv"]) and np.array_equal(sc["dh0"], 2.0 * base["dh0"])
    # additivity: a second value input (and initial state)
    r = np.random.default_rng(5)
    v2 = r.standard_normal(d["q"].shape) / np.sqrt(D)
    h2 = (0.3 * r.standard_normal(t["h0"].shape)).astype(np.float32)
    tb = dict(t, v=_store(v2, dtype), h0=h2)
    vs = synth.to_f64(t["v"], dtype) + synth.to_f64(tb["v"], dtype)
    ts = dict(t, v=_store(vs, dtype), h0=(t["h0"].astype(np.float64) + h2).astype(np.float32))
    ob, osum = _run(tb, dtype), _run(ts, dtype)
    ey = errors(osum["y"], base["y"] + ob["y"])
    eh = errors(osum["ht"], base["ht"] + ob["ht"], "state")
    print("additivity %s: y %s | ht %s" % (dtype, fmt(ey), fmt(eh)), flush=True)
    assert worst(ey) <= TOL[dtype] and worst(eh) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_value_columns_are_independent_bitwise(dtype):
    """Changing value columns J of v, h0 (and of dy, dht) leaves the other
    columns of y, ht (and dv) bit for bit unchanged."""
    d = _case(dtype)
    t = _tensors(d)
    base = _run(t, dtype)
    J = np.arange(0, D, 3)
    keep = np.setdiff1d(np.arange(D), J)
    r = np.random.default_rng(9)
    tc = {n: t[n].copy() for n in t}
    v = synth.to_f64(t["v"], dtype)
    v[..., J] = r.standard_normal(v[..., J].shape) / np.sqrt(D)
    tc["v"] = _store(v, dtype)
    dy = synth.to_f64(t["dy"], dtype)
    dy[..., J] = r.standard_normal(dy[..., J].shape)
    tc["dy"] = _store(dy, dtype)
    tc["h0"][..., J] = (0.3 * r.standard_normal(tc["h0"][..., J].shape)).astype(np.float32)
    tc["dht"][..., J] = (0.5 * r.standard_normal(tc["dht"][..., J].shape)).astype(np.float32)
    ch = _run(tc, dtype)
    for n in ("y", "ht", "dv", "dh0"):
        assert np.array_equal(ch[n][..., keep], base[n][..., keep]), n
        assert not np.array_equal(ch[n][..., J], base[n][..., J]), n


@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("use_ht", [False, True])
def test_autograd_wrapper(with_h0, use_ht):
    """hgrn2_chunk under torch autograd: the gradients torch hands back for
    q, k, v, log f (and h0) are the oracle's, for a loss that uses y alone or
    y and the final state."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case("bf16", B=2, T=2 * 64 + 9, H=2, h0std=0.3 if with_h0 else 0.0)
    leaves = {n: to_dev(d[n], "bf16").requires_grad_(True) for n in ("q", "k", "v", "log_f")}
    h0 = to_dev(d["h0"], "f32").requires_grad_(True) if with_h0 else None
    dy = to_dev(d["dy"], "bf16")
    dht_np = _dht(d)
    y, ht = m.hgrn2_chunk(leaves["q"], leaves["k"], leaves["v"], leaves["log_f"], h0, chunk=C)
    loss = (y.float() * dy.float()).sum()
    if use_ht:
        loss = loss + (ht * to_dev(dht_np, "f32")).sum()
    loss.backward()
    torch.cuda.synchronize()
    x = inputs64(d)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["log_f"], x["dy"], x["h0"],
                          dht_np.astype(np.float64) if use_ht else None)
    errs = {n: errors(to_host64(leaves[n].grad), r) for n, r in zip(("q", "k", "v", "log_f"), ref[:4])}
    if with_h0:
        errs["h0"] = errors(to_host64(h0.grad), ref[4], "state")
    print("autograd h0=%d ht=%d: %s" % (with_h0, use_ht, "; ".join("%s %s" % (n, fmt(e)) for n, e in errs.items())),
          flush=True)
    for n, e in errs.items():
        assert worst(e) <= TOL["bf16"], (n, e)
