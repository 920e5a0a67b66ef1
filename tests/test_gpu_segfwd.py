"""The forward without stored chunk-boundary states (hgrn2_fwd with
states_out = NULL at chunk 64): sequences cut into P segments whose end
states are summarised, carried, and then walked with the state on chip
(HGRN2 summary, paperlayer.ai, §3.2 p.5: the chunkwise form; §1: inference
keeps only the state).  Against the oracle (every slice, row and element):
one segment per sequence (B*H >= 256), many segments with a ragged last one,
the final state alone (y = NULL), ht aliasing h0 across segments, every gate
mode, float32, decays wide enough for the directly summed diagonal, and
agreement with the forward that stores its states.  bfloat16 at d = 128 walks
two workgroups per compute unit (the state kept in the accumulators) where the
plan fills both; the paired-walk tests cover that layout in every gate mode."""
import functools

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, errors, fmt, inputs64, to_dev, to_host64, worst

pytestmark = pytest.mark.gpu


def _case(dtype, B, T, H, D, lam=0.3, seed=41, h0std=0.3):
    w = synth.Workload("seg", B=B, H=H, T=T, D=D, chunk=64, dtype=dtype, lam=lam, qscale=1.0 / np.sqrt(D),
                       h0std=h0std, train=False, seed=seed)
    return synth.generate(w)


def _plan(B, H, T, dtype="bf16", D=128):
    """The segments the library cuts and whether two workgroups per compute
    unit walk them (mirrors the ABI's rule, for the report)."""
    N, BH = -(-T // 64), B * H

    def plan(u):
        Pt = min(N, max(1, -(-u // BH)))
        G = -(-N // Pt)
        return -(-N // G), G

    units = 512 if (dtype == "bf16" and D == 128) else 256
    P, G = plan(units)
    if units > 256 and P > 1 and G < 8:
        units = 256
        P, G = plan(units)
    return P, G, units > 256 and BH * P > 256


def _check(d, label=""):
    import torch
    import linear_attention_hgrn2_amd as m
    dt = d["dtype"]
    q, k, v, lf = (to_dev(d[n], dt) for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    y, ht, _ = m.fwd(q, k, v, lf, h0, chunk=64)
    torch.cuda.synchronize()
    x = inputs64(d)
    yr, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], x["h0"])
    ey, eh = errors(to_host64(y), yr), errors(to_host64(ht), htr, "state")
    P, G, pair = _plan(d["B"], d["H"], d["T"], dt, d["D"])
    print("%s seg fwd %s B%d H%d T%d D%d (P=%d G=%d%s): y %s | ht %s" % (
        label, dt, d["B"], d["H"], d["T"], d["D"], P, G, ", paired" if pair else "", fmt(ey), fmt(eh)), flush=True)
    assert worst(ey) <= TOL[dt] and worst(eh) <= TOL[dt]
    return y, ht


@pytest.mark.parametrize("dtype,D", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("f32", 32), ("f32", 64)])
def test_many_segments_ragged(dtype, D):
    """8 segments of one chunk, the last chunk partial; 4 segments of 6 chunks."""
    _check(_case(dtype, B=1, T=7 * 64 + 5, H=3, D=D))
    _check(_case(dtype, B=8, T=23 * 64 + 9, H=8, D=D, seed=42))


def test_one_segment_per_sequence():
    """B*H = 256 sequences: P = 1, one pass with no summaries."""
    _check(_case("bf16", B=16, T=3 * 64 + 1, H=16, D=128))


def test_segments_longer_than_one_chunk_with_wide_decays():
    """Full resets, the -200 floor and in-block decays past kDiagLimit, in several segments."""
    d = _case("bf16", B=2, T=20 * 64 + 3, H=2, D=128, lam=0.0)
    lf = synth.to_f64(d["log_f"], "bf16")
    lf[0, 3, 0, :] = -np.inf
    lf[0, 20, 1, 2] = -200.0
    lf[0, 400:404, 0, 1] = -30.0
    lf[1, 700:710, 1, :] = -9.0
    d["log_f"] = synth.f32_to_bf16_bits(lf.astype(np.float32))
    _check(d, "wide")


def test_final_state_alone():
    """y = NULL: the summaries of every segment carried to the final state."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case("bf16", B=2, T=11 * 64 + 30, H=3, D=128)
    q, k, v, lf = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f"))
    _, ht, _ = m.fwd(q, k, v, lf, to_dev(d["h0"], "f32"), chunk=64, want_y=False)
    torch.cuda.synchronize()
    x = inputs64(d)
    _, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], x["h0"])
    e = errors(to_host64(ht), htr, "state")
    print("seg ht alone: %s" % fmt(e), flush=True)
    assert worst(e) <= TOL["bf16"]


def test_ht_aliases_h0_across_segments():
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case("bf16", B=1, T=9 * 64 + 7, H=2, D=128)
    q, k, v, lf = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    y_ref, ht_ref, _ = m.fwd(q, k, v, lf, h0.clone(), chunk=64)
    s = h0.clone()
    y, _, _ = m.fwd(q, k, v, lf, s, chunk=64, ht=s)
    torch.cuda.synchronize()
    assert torch.equal(s, ht_ref) and torch.equal(y, y_ref)


def test_repeat_runs_are_bitwise_equal():
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case("bf16", B=2, T=9 * 64 + 7, H=3, D=128)
    q, k, v, lf = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    a = m.fwd(q, k, v, lf, h0, chunk=64)
    b = m.fwd(q, k, v, lf, h0, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_agrees_with_the_stored_state_forward():
    """The same outputs as the forward that stores its chunk-boundary states,
    within tolerance (the operation order differs at segment boundaries), and
    a sequence split at a chunk multiple with its state carried agrees too."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case("bf16", B=2, T=10 * 64 + 21, H=3, D=128)
    q, k, v, lf = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    y, ht, _ = m.fwd(q, k, v, lf, h0, chunk=64)
    ys, hts, _ = m.fwd(q, k, v, lf, h0, chunk=64, want_states=True)
    T1 = 4 * 64
    part = lambda t, a, b: t[:, a:b].contiguous()
    y1, ht1, _ = m.fwd(*(part(t, 0, T1) for t in (q, k, v, lf)), h0, chunk=64)
    y2, ht2, _ = m.fwd(*(part(t, T1, d["T"]) for t in (q, k, v, lf)), ht1, chunk=64)
    torch.cuda.synchronize()
    e = {"y": errors(to_host64(y), to_host64(ys)), "ht": errors(to_host64(ht), to_host64(hts), "state"),
         "split y": errors(to_host64(torch.cat([y1, y2], 1)), to_host64(y)),
         "split ht": errors(to_host64(ht2), to_host64(ht), "state")}
    print("seg vs stored: %s" % "; ".join("%s %s" % (n, fmt(v_)) for n, v_ in e.items()), flush=True)
    for n, v_ in e.items():
        assert worst(v_) <= TOL["bf16"], n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_modes(dtype):
    """Tied gates, the gate from its pre-activation and one decay per head,
    forward without states, against their oracles."""
    import torch
    import linear_attention_hgrn2_amd as m
    D = 64 if dtype == "f32" else 128
    d = _case(dtype, B=2, T=9 * 64 + 13, H=3, D=D)
    q, v, lf, z, k = (to_dev(d[n], dtype) for n in ("q", "v", "log_f", "z", "k"))
    h0 = to_dev(d["h0"], "f32")
    lbn = synth.lower_bounds(d["H"], D, 0.3, 0.25, seed=3)
    la = np.ascontiguousarray(d["log_f"][..., 0])
    x = {n: synth.to_f64(d[n], dtype) for n in ("q", "v", "log_f", "z", "k")}
    h064 = d["h0"].astype(np.float64)
    out = {"tied": m.fwd_tied(q, v, lf, h0, chunk=64)[:2],
           "gate": m.fwd_gate(q, v, z, to_dev(lbn, "f32"), h0, chunk=64)[:2],
           "scalar": m.fwd_scalar(q, k, v, to_dev(la, dtype), h0, chunk=64)[:2]}
    torch.cuda.synchronize()
    ref = {"tied": oracle.forward_tied(x["q"], x["v"], x["log_f"], h064),
           "gate": oracle.forward_gate(x["q"], x["v"], x["z"], lbn.astype(np.float64), h064),
           "scalar": oracle.forward_scalar(x["q"], x["k"], x["v"], synth.to_f64(la, dtype), h064)}
    for mode in out:
        ey = errors(to_host64(out[mode][0]), ref[mode][0])
        eh = errors(to_host64(out[mode][1]), ref[mode][1], "state")
        print("seg %s %s: y %s | ht %s" % (mode, dtype, fmt(ey), fmt(eh)), flush=True)
        assert worst(ey) <= TOL[dtype] and worst(eh) <= TOL[dtype], mode


# B5 H13 T4049: 65 sequences of 64 chunks (the last one 17 tokens), cut into
# 8 segments of 8 chunks: 520 workgroups, two per compute unit
PAIRED = dict(B=5, T=63 * 64 + 17, H=13, D=128)


@functools.lru_cache(maxsize=1)
def _paired_inputs():
    return _case("bf16", lam=0.5, seed=51, **PAIRED)


def test_paired_walk_plan():
    assert _plan(PAIRED["B"], PAIRED["H"], PAIRED["T"]) == (8, 8, True)
    assert _plan(4, 8, 2048) == (8, 4, False)       # segments of 2 chunks would be too short
    assert _plan(1, 32, 32768) == (16, 32, True)


@pytest.mark.parametrize("mode", ["untied", "tied", "gate", "scalar"])
def test_paired_walk(mode):
    """The two-per-compute-unit walk in every gate mode, with an initial state
    and the final state, against the oracle."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = _paired_inputs()
    q, k, v, lf, z = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f", "z"))
    h0 = to_dev(d["h0"], "f32")
    x = {n: synth.to_f64(d[n], "bf16") for n in ("q", "k", "v", "log_f", "z")}
    h064 = d["h0"].astype(np.float64)
    if mode == "untied":
        y, ht, _ = m.fwd(q, k, v, lf, h0, chunk=64)
        yr, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], h064)
    elif mode == "tied":
        y, ht, _ = m.fwd_tied(q, v, lf, h0, chunk=64)
        yr, htr = oracle.forward_tied(x["q"], x["v"], x["log_f"], h064)
    elif mode == "gate":
        lbn = synth.lower_bounds(d["H"], 128, 0.5, 0.25, seed=5)
        y, ht, _ = m.fwd_gate(q, v, z, to_dev(lbn, "f32"), h0, chunk=64)
        yr, htr = oracle.forward_gate(x["q"], x["v"], x["z"], lbn.astype(np.float64), h064)
    else:
        la = np.ascontiguousarray(d["log_f"][..., 0])
        y, ht, _ = m.fwd_scalar(q, k, v, to_dev(la, "bf16"), h0, chunk=64)
        yr, htr = oracle.forward_scalar(x["q"], x["k"], x["v"], synth.to_f64(la, "bf16"), h064)
    torch.cuda.synchronize()
    ey, eh = errors(to_host64(y), yr), errors(to_host64(ht), htr, "state")
    print("paired walk %s: y %s | ht %s" % (mode, fmt(ey), fmt(eh)), flush=True)
    assert worst(ey) <= TOL["bf16"] and worst(eh) <= TOL["bf16"]


def test_paired_walk_f32_out_and_wide_decays():
    """float32 y from the accumulators, full resets, the -200 floor and
    in-block decays past kDiagLimit, in the paired walk."""
    import torch
    import linear_attention_hgrn2_amd as m
    d = _case("bf16", lam=0.0, seed=52, **PAIRED)
    lf = synth.to_f64(d["log_f"], "bf16")
    lf[0, 3, 0, :] = -np.inf
    lf[1, 20, 1, 2] = -200.0
    lf[2, 400:404, 5, 1] = -30.0
    lf[4, 2000:2010, 12, :] = -9.0
    d["log_f"] = synth.f32_to_bf16_bits(lf.astype(np.float32))
    q, k, v, lfd = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    y, ht, _ = m.fwd(q, k, v, lfd, h0, chunk=64, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert y.dtype == torch.float32
    x = inputs64(d)
    yr, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], x["h0"])
    ey, eh = errors(to_host64(y), yr), errors(to_host64(ht), htr, "state")
    print("paired walk, float32 y, wide decays: y %s | ht %s" % (fmt(ey), fmt(eh)), flush=True)
    assert worst(ey) <= TOL["bf16"] and worst(eh) <= TOL["bf16"]


def test_paired_walk_uneven_segments():
    """The paired walk where the segments do not divide the sequence: B2 H20
    T6369 is 40 sequences of 100 chunks (the last one 33 tokens), cut into 13
    segments of 8 chunks, the last of them 4 chunks long; no initial state."""
    assert _plan(2, 20, 99 * 64 + 33) == (13, 8, True)
    _check(_case("bf16", B=2, T=99 * 64 + 33, H=20, D=128, lam=0.6, seed=53, h0std=0.0), "uneven")
