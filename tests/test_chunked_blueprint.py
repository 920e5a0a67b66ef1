"""The chunked factorisation used by the GPU kernels, modelled in float64
numpy, against the step-by-step oracle.  CPU only; validates the algebra
(anchoring, diagonal fallback, tail masking, boundary carries) before any
kernel runs it."""
import numpy as np
import pytest

import oracle
from tests import chunked_ref
from tests.pins import rel


def _inputs(seed, B=1, T=75, H=2, D=8, lo=-1.0, extreme=False):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((B, T, H, D)) for _ in range(3))
    lf = r.uniform(lo, 0.0, (B, T, H, D))
    if extreme:
        lf[0, 3, 0, :] = -np.inf          # full reset
        lf[0, 20, 1, 2] = -200.0          # floor value
        lf[0, 40:44, 0, 1] = -30.0        # wide decay range inside one sub-block
    h0 = r.standard_normal((B, H, D, D))
    dy = r.standard_normal((B, T, H, D))
    dht = r.standard_normal((B, H, D, D))
    return q, k, v, lf, h0, dy, dht


@pytest.mark.parametrize("C,SB", [(16, 16), (32, 16), (64, 16), (16, 4), (32, 8)])
@pytest.mark.parametrize("extreme", [False, True])
def test_chunked_forward_matches_oracle(C, SB, extreme):
    q, k, v, lf, h0, dy, dht = _inputs(1, extreme=extreme)
    y, ht = oracle.forward(q, k, v, lf, h0)
    yc, hc = chunked_ref.forward(q, k, v, lf, h0, C=C, SB=SB)
    assert rel(yc, y) < 1e-12
    assert rel(hc, ht) < 1e-12


@pytest.mark.parametrize("C,SB", [(16, 16), (32, 16), (64, 16), (32, 8)])
@pytest.mark.parametrize("extreme", [False, True])
def test_chunked_backward_matches_oracle(C, SB, extreme):
    q, k, v, lf, h0, dy, dht = _inputs(2, extreme=extreme)
    ref = oracle.backward(q, k, v, lf, dy, h0, dht)
    got = chunked_ref.backward(q, k, v, lf, dy, h0, dht, C=C, SB=SB)
    for name, g, r in zip(("dq", "dk", "dv", "dlog_f", "dh0"), got, ref):
        assert rel(g, r) < 1e-11, (name, rel(g, r))


def test_wide_decay_triggers_fallback():
    """The extreme inputs really exercise the diagonal fallback."""
    _, _, _, lf, _, _, _ = _inputs(1, extreme=True)
    blk = np.maximum(lf[0, 32:48, 0, :], chunked_ref.FLOOR).sum(0)
    assert (-blk).max() > chunked_ref.DIAG_LIMIT
