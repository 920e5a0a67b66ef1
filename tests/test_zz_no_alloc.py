"""hgrn2_bwd_noalloc (the backward with the library's own scratch in place of
a workspace) gives exactly hgrn2_bwd's results, call after call on one GPU:
first at the size that fills the scratch (the B8 H16 T4096 d128 training
batch, states passed in), then a smaller float32 call that recomputes the
states, then a bf16 call again; each compared bit for bit with hgrn2_bwd on
the same inputs."""
import numpy as np
import pytest

import synth
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _case(dtype, B, T, H, D, lam, seed, h0std):
    w = synth.Workload("noalloc", B=B, H=H, T=T, D=D, chunk=0, dtype=dtype, lam=lam, qscale=1.0 / np.sqrt(D),
                       h0std=h0std, train=True, seed=seed)
    return synth.generate(w)


def _both(d, chunk, with_states, with_dht):
    import torch
    import linear_attention_hgrn2_amd as m
    dt = d["dtype"]
    q, k, v, lf, dy = (to_dev(d[n], dt) for n in ("q", "k", "v", "log_f", "dy"))
    h0 = to_dev(d["h0"], "f32")
    dht = None
    if with_dht:
        r = np.random.default_rng(d["seed"] + 99)
        dht = to_dev((0.5 * r.standard_normal((d["B"], d["H"], d["D"], d["D"]))).astype(np.float32), "f32")
    st = m.fwd(q, k, v, lf, h0, chunk=chunk, want_ht=False, want_y=False, want_states=True)[2] if with_states else None
    a = m.bwd_noalloc(q, k, v, lf, dy, h0, dht, st, chunk=chunk, want_dh0=h0 is not None)
    b = m.bwd(q, k, v, lf, dy, h0, dht, st, chunk=chunk, want_dh0=h0 is not None)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dlog_f", "dh0"), a, b):
        assert (x is None) == (y is None), name
        if x is not None:
            assert torch.isfinite(x.float()).all(), name
            assert torch.equal(x, y), name


def test_noalloc_equals_workspace_backward_call_after_call():
    import linear_attention_hgrn2_amd as m
    w = synth.WORKLOADS["train_bf16"]
    need = m.lib().hgrn2_bwd_workspace_bytes(w.B, w.T, w.H, w.D, w.D, w.chunk, 1, 1)
    assert need == m.NOALLOC_SCRATCH_BYTES      # the training batch fills the scratch exactly
    print("noalloc: B8 H16 T4096 d128 bf16 chunk 64, states passed in", flush=True)
    _both(synth.generate("train_bf16", lam=0.3), 64, with_states=True, with_dht=False)
    print("noalloc: B1 H2 T70 d32 f32 chunk 32, states recomputed", flush=True)
    _both(_case("f32", 1, 70, 2, 32, 0.3, 5, 0.5), 32, with_states=False, with_dht=True)
    print("noalloc: B2 H3 T329 d128 bf16 chunk 64, states recomputed", flush=True)
    _both(_case("bf16", 2, 5 * 64 + 9, 3, 128, 0.0, 6, 0.3), 64, with_states=False, with_dht=True)


def test_noalloc_rejects_more_than_its_scratch():
    import linear_attention_hgrn2_amd as m
    w = synth.WORKLOADS["train_bf16"]
    # the training batch without its states: adjoints plus recomputed states exceed the scratch
    P = 1 << 16
    r = m.lib().hgrn2_bwd_noalloc(w.B, w.T, w.H, w.D, w.D, w.chunk, 1, P, P, P, P, None, None, P, None,
                                  P, P, P, P, None, None)
    assert r == 3 and b"scratch" in m.lib().hgrn2_last_error()
