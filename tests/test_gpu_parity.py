"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
identical seeded inputs.  Every slice, row and element is compared
(tests/gpu_util.py): <= 2e-2 for bfloat16 inputs and <= 1e-4 for float32
inputs.  The forwards here without states_out take the segmented path where
it exists (chunk 64)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, inputs64, select_bh, slice_rel, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _hip():
    import linear_attention_hgrn2_amd as m
    return m


def _case(dtype, B, T, H, D, lam=0.0, seed=7, h0std=0.0, qscale=None, train=True):
    w = synth.Workload("case", B=B, H=H, T=T, D=D, chunk=0, dtype=dtype, lam=lam,
                       qscale=(1.0 / np.sqrt(D) if qscale is None else qscale), h0std=h0std,
                       train=train, seed=seed)
    return synth.generate(w)


def _fwd_check(d, chunk, label=""):
    m = _hip()
    import torch
    dt = d["dtype"]
    q, k, v, lf = (to_dev(d[n], dt) for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    y, ht, _ = m.fwd(q, k, v, lf, h0, chunk=chunk)
    torch.cuda.synchronize()
    x = inputs64(d)
    yr, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], x["h0"])
    ey = slice_rel(to_host64(y), yr)
    eh = slice_rel(to_host64(ht), htr, token_major=False)
    print("%s fwd D=%d C=%d %s: y %.3e ht %.3e" % (label, d["D"], chunk, dt, ey, eh), flush=True)
    assert ey <= TOL[dt], ey
    assert eh <= TOL[dt], eh
    return y, ht


def _bwd_check(d, chunk, use_states=True, with_dht=True, label=""):
    m = _hip()
    import torch
    dt = d["dtype"]
    q, k, v, lf, dy = (to_dev(d[n], dt) for n in ("q", "k", "v", "log_f", "dy"))
    h0 = to_dev(d["h0"], "f32")
    rng = np.random.default_rng(d["seed"] + 99)
    dht_np = (rng.standard_normal((d["B"], d["H"], d["D"], d["D"])) * 0.5).astype(np.float32) if with_dht else None
    dht = to_dev(dht_np, "f32")
    states = None
    if use_states:
        _, _, states = m.fwd(q, k, v, lf, h0, chunk=chunk, want_ht=False, want_states=True)
    dq, dk, dv, dl, dh0 = m.bwd(q, k, v, lf, dy, h0, dht, states, chunk=chunk)
    torch.cuda.synchronize()
    x = inputs64(d)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["log_f"], x["dy"], x["h0"],
                          None if dht_np is None else dht_np.astype(np.float64))
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv", "dlog_f"), (dq, dk, dv, dl), ref[:4]):
        errs[name] = slice_rel(to_host64(g), r)
    errs["dh0"] = slice_rel(to_host64(dh0), ref[4], token_major=False)
    print("%s bwd D=%d C=%d %s: %s" % (label, d["D"], chunk, dt,
                                       " ".join("%s %.3e" % kv for kv in errs.items())), flush=True)
    for name, e in errs.items():
        assert e <= TOL[dt], (name, e)


# ------------------------------------------------------------------ forward

def test_fwd_tiny_f32_workload():
    """The tiny float32 workload: B1 H2 T256 d16, chunk 16, zero initial state."""
    d = synth.generate("tiny_f32")
    _fwd_check(d, 16, "tiny_f32")


ALL_DC = [(D, C) for D in (16, 32, 64, 128) for C in (16, 32, 64, 128)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,C", ALL_DC)
def test_fwd_shapes(dtype, D, C):
    import linear_attention_hgrn2_amd as m
    import torch
    if not m.supported(D, C, torch.float32 if dtype == "f32" else torch.bfloat16):
        pytest.skip("no kernel for this combination")
    d = _case(dtype, B=2, T=3 * C + 5, H=3, D=D, lam=0.3, h0std=0.5, qscale=1.0)
    _fwd_check(d, C)


def test_fwd_extreme_gates():
    """log f = -inf (reset), -200 (floor) and decays wide enough to force the
    direct evaluation of diagonal sub-blocks."""
    for dtype in ("f32", "bf16"):
        d = _case(dtype, B=1, T=150, H=2, D=64, lam=0.0, h0std=0.3, qscale=1.0)
        lf = synth.to_f64(d["log_f"], dtype)
        lf[0, 3, 0, :] = -np.inf
        lf[0, 20, 1, 2] = -200.0
        lf[0, 40:44, 0, 1] = -30.0   # 120 nats inside one 16-token block
        lf[0, 70:80, 1, :] = -9.0
        d["log_f"] = lf.astype(np.float32) if dtype == "f32" else synth.f32_to_bf16_bits(lf.astype(np.float32))
        _fwd_check(d, 64, "extreme")
        _fwd_check(d, 16, "extreme")


def test_fwd_ht_aliases_h0():
    m = _hip()
    import torch
    d = _case("f32", B=2, T=70, H=2, D=32, h0std=1.0, qscale=1.0)
    q, k, v, lf = (to_dev(d[n], "f32") for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    _, ht_ref, _ = m.fwd(q, k, v, lf, h0.clone(), chunk=32)
    s = h0.clone()
    m.fwd(q, k, v, lf, s, chunk=32, ht=s)
    torch.cuda.synchronize()
    assert torch.equal(s, ht_ref)


# ----------------------------------------------------------------- backward

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,C", ALL_DC)
def test_bwd_shapes(dtype, D, C):
    import linear_attention_hgrn2_amd as m
    import torch
    if not m.supported(D, C, torch.float32 if dtype == "f32" else torch.bfloat16):
        pytest.skip("no kernel for this combination")
    d = _case(dtype, B=2, T=2 * C + 7, H=2, D=D, lam=0.3, h0std=0.5, qscale=1.0)
    _bwd_check(d, C)


def test_bwd_recompute_states_and_no_dht():
    d = _case("bf16", B=1, T=200, H=2, D=128, lam=0.0, h0std=0.0, qscale=1.0)
    _bwd_check(d, 64, use_states=False, with_dht=False, label="recompute")


def test_bwd_extreme_gates():
    for dtype in ("f32", "bf16"):
        d = _case(dtype, B=1, T=150, H=2, D=64, lam=0.0, h0std=0.3, qscale=1.0)
        lf = synth.to_f64(d["log_f"], dtype)
        lf[0, 3, 0, :] = -np.inf
        lf[0, 20, 1, 2] = -200.0
        lf[0, 40:44, 0, 1] = -30.0
        lf[0, 70:80, 1, :] = -9.0
        d["log_f"] = lf.astype(np.float32) if dtype == "f32" else synth.f32_to_bf16_bits(lf.astype(np.float32))
        _bwd_check(d, 64, label="extreme")
        _bwd_check(d, 16, label="extreme")


def test_bwd_extreme_gates_d128():
    """d = 128, chunk 64 in bfloat16 (the training shape's kernel): blocks whose
    in-block decay forces the directly summed diagonal, a full reset and the
    -200 floor, in several chunks."""
    d = _case("bf16", B=1, T=300, H=2, D=128, lam=0.0, h0std=0.3, qscale=1.0)
    lf = synth.to_f64(d["log_f"], "bf16")
    lf[0, 3, 0, :] = -np.inf
    lf[0, 20, 1, 2] = -200.0
    lf[0, 40:44, 0, 1] = -30.0
    lf[0, 70:80, 1, :] = -9.0
    lf[0, 200:216, 0, 5] = -5.0
    d["log_f"] = synth.f32_to_bf16_bits(lf.astype(np.float32))
    _bwd_check(d, 64, label="extreme d128")


def test_bwd_many_chunks_per_workgroup():
    """More chunks than workgroups at d = 128, chunk 64 (bfloat16), with a
    ragged last chunk: each workgroup walks several chunks."""
    d = _case("bf16", B=3, T=20 * 64 + 13, H=5, D=128, lam=0.3, h0std=0.2, qscale=1.0)
    _bwd_check(d, 64, label="many chunks")


# ------------------------------------------------------------------- decode

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_decode(dtype, D):
    m = _hip()
    import torch
    d = synth.generate_decode("decode_f32", B=3, H=5, D=D, seed=11)
    conv = (lambda a: a) if dtype == "f32" else (lambda a: synth.f32_to_bf16_bits(a))
    q, k, v, lf = (to_dev(conv(d[n]), dtype) for n in ("q", "k", "v", "log_f"))
    S = to_dev(d["state"], "f32")
    y = m.decode_step(q, k, v, lf, S)
    torch.cuda.synchronize()
    x = {n: synth.to_f64(conv(d[n]), dtype) for n in ("q", "k", "v", "log_f")}
    yr, Sr = oracle.decode_step(x["q"], x["k"], x["v"], x["log_f"], d["state"].astype(np.float64))
    ey = np.linalg.norm(to_host64(y) - yr) / np.linalg.norm(yr)
    es = np.linalg.norm(to_host64(S) - Sr) / np.linalg.norm(Sr)
    print("decode D=%d %s: y %.3e state %.3e" % (D, dtype, ey, es), flush=True)
    assert ey <= TOL[dtype] and es <= 1e-5


# ------------------------------------------------------------ staged launches

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_staged_launches_equal_composite_calls(dtype):
    """hgrn2_fwd_chunk, hgrn2_bwd_adjoint and hgrn2_bwd_chunk run the kernels
    hgrn2_fwd / hgrn2_bwd are made of, in the same order on the same inputs,
    so their results are bit-for-bit those of the composite calls (which the
    other tests hold to the oracle)."""
    m = _hip()
    import torch
    d = _case(dtype, B=2, T=3 * 64 + 11, H=3, D=64, lam=0.3, h0std=0.5, qscale=1.0)
    C = 64
    q, k, v, lf, dy = (to_dev(d[n], dtype) for n in ("q", "k", "v", "log_f", "dy"))
    h0 = to_dev(d["h0"], "f32")
    rng = np.random.default_rng(d["seed"] + 99)
    dht = to_dev((rng.standard_normal(tuple(h0.shape)) * 0.5).astype(np.float32), "f32")
    y, ht, states = m.fwd(q, k, v, lf, h0, chunk=C, want_states=True)
    dq, dk, dv, dl, dh0 = m.bwd(q, k, v, lf, dy, h0, dht, states, chunk=C)
    _, ht2, states2 = m.fwd(q, k, v, lf, h0, chunk=C, want_states=True, y=torch.empty_like(y))
    y2 = m.fwd_chunk(q, k, v, lf, states2, chunk=C)
    lam, dh02 = m.bwd_adjoint(q, lf, dy, dht, chunk=C, want_dh0=True)
    g2 = m.bwd_chunk(q, k, v, lf, dy, states2, lam, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(states, states2) and torch.equal(ht, ht2)
    assert torch.equal(y, y2)
    assert torch.equal(dh0, dh02)
    for a, b in zip((dq, dk, dv, dl), g2):
        assert torch.equal(a, b)


# ------------------------------------------------- fixed-order bitwise checks

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeat_runs_are_bitwise_equal(dtype):
    """No kernel reorders its arithmetic between runs (no atomics, a fixed chunk
    to workgroup assignment): two identical calls give identical bits."""
    m = _hip()
    import torch
    d = _case(dtype, B=3, T=5 * 64 + 9, H=5, D=128, lam=0.3, h0std=0.5, qscale=1.0)
    q, k, v, lf, dy = (to_dev(d[n], dtype) for n in ("q", "k", "v", "log_f", "dy"))
    h0 = to_dev(d["h0"], "f32")
    outs = []
    for _ in range(2):
        y, ht, st = m.fwd(q, k, v, lf, h0, chunk=64, want_states=True)
        g = m.bwd(q, k, v, lf, dy, h0, ht * 0.5, st, chunk=64)
        outs.append((y, ht, st) + tuple(g))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_carry_split_is_bitwise(dtype):
    """Splitting a sequence at a multiple of the chunk and carrying the final
    state in as the next call's initial state repeats the same operations in
    the same order on the forward that stores its chunk-boundary states:
    outputs and final state match bit for bit.  (The forward without stored
    states cuts the sequence into segments whose boundaries depend on the
    length, so there the split agrees within tolerance: test_gpu_segfwd.)"""
    m = _hip()
    import torch
    C, T1 = 64, 3 * 64
    d = _case(dtype, B=2, T=T1 + 2 * 64 + 21, H=3, D=128, lam=0.5, h0std=0.3, qscale=1.0)
    q, k, v, lf = (to_dev(d[n], dtype) for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    y, ht, _ = m.fwd(q, k, v, lf, h0, chunk=C, want_states=True)
    part = lambda t, a, b: t[:, a:b].contiguous()
    y1, ht1, _ = m.fwd(*(part(t, 0, T1) for t in (q, k, v, lf)), h0, chunk=C, want_states=True)
    y2, ht2, _ = m.fwd(*(part(t, T1, d["T"]) for t in (q, k, v, lf)), ht1, chunk=C, want_states=True)
    torch.cuda.synchronize()
    assert torch.equal(y[:, :T1], y1)
    assert torch.equal(y[:, T1:], y2)
    assert torch.equal(ht, ht2)


def test_chunk_sizes_agree_with_each_other():
    """Chunks of 16, 32, 64 and 128 tokens (bfloat16, d = 128) each meet the
    oracle's tolerance and agree with one another within it."""
    m = _hip()
    import torch
    d = _case("bf16", B=2, T=3 * 128 + 5, H=2, D=128, lam=0.3, h0std=0.3, qscale=1.0)
    q, k, v, lf, dy = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f", "dy"))
    h0 = to_dev(d["h0"], "f32")
    res = {}
    for C in (16, 32, 64, 128):
        y, ht, st = m.fwd(q, k, v, lf, h0, chunk=C, want_states=True)
        g = m.bwd(q, k, v, lf, dy, h0, None, st, chunk=C)
        res[C] = (y, ht) + tuple(g)
    torch.cuda.synchronize()
    x = inputs64(d)
    yr, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], x["h0"])
    gr = oracle.backward(x["q"], x["k"], x["v"], x["log_f"], x["dy"], x["h0"], None)
    refs = (yr, htr) + tuple(gr)
    for C, outs in res.items():
        for i, (o, r) in enumerate(zip(outs, refs)):
            tm = i not in (1, 6)
            assert slice_rel(to_host64(o), r, token_major=tm) <= TOL["bf16"], (C, i)
    for i in range(len(refs)):
        tm = i not in (1, 6)
        for C in (16, 32, 128):
            e = slice_rel(to_host64(res[C][i]), to_host64(res[64][i]), token_major=tm)
            print("chunk %d vs 64, output %d: %.3e" % (C, i, e), flush=True)
            assert e <= TOL["bf16"], (C, i, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_equals_forward_at_one_token(dtype):
    """A decode step is the chunked forward at T = 1 from the same state."""
    m = _hip()
    import torch
    d = synth.generate_decode("decode_f32", B=4, H=3, D=128, seed=21)
    conv = (lambda a: a) if dtype == "f32" else (lambda a: synth.f32_to_bf16_bits(a))
    q, k, v, lf = (to_dev(conv(d[n]), dtype) for n in ("q", "k", "v", "log_f"))
    S = to_dev(d["state"], "f32")
    yf, htf, _ = m.fwd(q[:, None].contiguous(), k[:, None].contiguous(), v[:, None].contiguous(),
                       lf[:, None].contiguous(), S.clone(), chunk=16)
    yd = m.decode_step(q, k, v, lf, S)
    torch.cuda.synchronize()
    ey = np.linalg.norm(to_host64(yd) - to_host64(yf[:, 0])) / np.linalg.norm(to_host64(yf[:, 0]))
    es = np.linalg.norm(to_host64(S) - to_host64(htf)) / np.linalg.norm(to_host64(htf))
    print("decode vs forward at T=1 %s: y %.3e state %.3e" % (dtype, ey, es), flush=True)
    assert ey <= TOL[dtype] and es <= 1e-5
