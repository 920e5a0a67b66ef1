"""The backward of every gate mode with the chunk-boundary states recomputed
(states NULL: the workspace holds them) is bit-identical to the backward
given the forward's saved states: the recomputation runs the same scan on the
same inputs.  bf16 and fp32, ragged T, nonzero h0 and dht."""
import numpy as np
import pytest

import synth
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _inputs(dtype, B=2, T=3 * 64 + 11, H=3, D=128, seed=21):
    w = synth.Workload("rc", B=B, H=H, T=T, D=D, chunk=0, dtype=dtype, lam=0.3, qscale=1.0, h0std=0.5,
                       train=True, seed=seed)
    d = synth.generate(w)
    r = np.random.default_rng(seed + 1)
    d["dht"] = (0.5 * r.standard_normal((B, H, D, D))).astype(np.float32)
    d["lb"] = synth.lower_bounds(H, D, 0.3, 0.25, seed=seed + 2)
    d["log_a"] = np.ascontiguousarray(d["log_f"][..., 0])
    return d


def _equal(a, b):
    import torch
    for x, y in zip(a, b):
        assert (x is None and y is None) or torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["tied", "gate", "scalar"])
def test_recomputed_states_bitwise(mode, dtype):
    import torch
    import linear_attention_hgrn2_amd as m
    d = _inputs(dtype)
    dev = {n: to_dev(d[n], dtype) for n in ("q", "k", "v", "log_f", "dy", "z", "log_a")}
    h0, dht = to_dev(d["h0"], "f32"), to_dev(d["dht"], "f32")
    q, k, v, dy = dev["q"], dev["k"], dev["v"], dev["dy"]
    if mode == "tied":
        _, _, st = m.fwd_tied(q, v, dev["log_f"], h0, chunk=64, want_states=True)
        run = lambda s: m.bwd_tied(q, v, dev["log_f"], dy, h0, dht, s, chunk=64)
    elif mode == "gate":
        lb = torch.from_numpy(d["lb"]).float().cuda()
        _, _, st = m.fwd_gate(q, v, dev["z"], lb, h0, chunk=64, want_states=True)
        run = lambda s: m.bwd_gate(q, v, dev["z"], lb, dy, h0, dht, s, chunk=64)
    else:
        _, _, st = m.fwd_scalar(q, k, v, dev["log_a"], h0, chunk=64, want_states=True)
        run = lambda s: m.bwd_scalar(q, k, v, dev["log_a"], dy, h0, dht, s, chunk=64)
    saved = run(st)
    recomputed = run(None)
    torch.cuda.synchronize()
    print("%s %s: %d outputs compared" % (mode, dtype, sum(x is not None for x in saved)), flush=True)
    _equal(saved, recomputed)
