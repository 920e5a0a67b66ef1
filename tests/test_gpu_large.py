"""Token tensors past 4 GiB: B2 H16 d128, T = 524388 bf16 (2.15e9 elements per
token tensor, 8.6 GB of chunk-boundary states), forward and backward with the
kernels and chunk size of the training workload.  Full resets (f = 0) every
1024 tokens split every sequence into windows that start from a zero state,
so the float64 oracle recomputes whole windows on their own: the one that
holds the 4 GiB byte offset of the token tensors, the last (ragged) one, and
the first, at the highest and lowest (b, h).  Normwise relative error per
window <= 2e-2 (every slice, row and element of the window).  The forward
without stored states (segmented) is checked on the same windows."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, slice_rel

pytestmark = pytest.mark.gpu


def test_token_tensors_beyond_4gib():
    import torch
    import linear_attention_hgrn2_amd as m
    B, H, D, C, R = 2, 16, 128, 64, 1024
    T = 524288 + 100
    print("large: B%d H%d T%d d%d, %.1f GB per token tensor" % (B, H, T, D, B * T * H * D * 2 / 1e9), flush=True)
    x = synth.large_device_inputs(B, T, H, D, seed=77, reset_every=R)
    q, k, v, lf, dy = (x[n] for n in ("q", "k", "v", "log_f", "dy"))
    y, _, st = m.fwd(q, k, v, lf, None, chunk=C, want_ht=False, want_states=True)
    dq, dk, dv, dl, _ = m.bwd(q, k, v, lf, dy, None, None, st, chunk=C, want_dh0=False)
    torch.cuda.synchronize()
    del st
    # the forward without stored states (segments walked with the state on chip)
    ys, _, _ = m.fwd(q, k, v, lf, None, chunk=C, want_ht=False)
    torch.cuda.synchronize()
    # token of b = 1 at element 2^31 (byte offset 2^32 of a bf16 tensor)
    t_cross = (1 << 31) // (H * D) - T
    windows = [(1, H - 1, (t_cross // R) * R), (1, H - 1, ((T - 1) // R) * R), (0, 0, 0), (1, 3, (t_cross // R) * R)]
    host = lambda t, b, h, t0, t1: t[b, t0:t1, h].float().cpu().numpy().astype(np.float64)[None, :, None, :]
    for b, h, t0 in windows:
        t1 = min(t0 + R, T)
        w = {n: host(x[n], b, h, t0, t1) for n in ("q", "k", "v", "log_f", "dy")}
        yr, _ = oracle.forward(w["q"], w["k"], w["v"], w["log_f"], None)
        gr = oracle.backward(w["q"], w["k"], w["v"], w["log_f"], w["dy"], None, None)
        errs = {"y": slice_rel(host(y, b, h, t0, t1), yr), "y (no states)": slice_rel(host(ys, b, h, t0, t1), yr)}
        for name, a, r in zip(("dq", "dk", "dv", "dlog_f"), (dq, dk, dv, dl), gr[:4]):
            errs[name] = slice_rel(host(a, b, h, t0, t1), r)
        print("window b=%d h=%d tokens %d..%d: %s" % (b, h, t0, t1, " ".join("%s %.3e" % e for e in errs.items())),
              flush=True)
        for name, e in errs.items():
            assert e <= TOL["bf16"], (name, e)
    del x, q, k, v, lf, dy, y, ys, dq, dk, dv, dl
    torch.cuda.empty_cache()
