"""The comparison metrics of the GPU parity tests (tests/gpu_util.py) on
planted errors, on the CPU: a slice norm over thousands of tokens misses one
wrong token row and one wrong element; the row and element terms do not."""
import numpy as np

from tests.gpu_util import TOL, errors, worst


def _ref(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def test_identical_is_zero():
    r = _ref((2, 64, 3, 16))
    e = errors(r.copy(), r)
    assert (e["norm"], e["row"], e["elem"]) == (0.0, 0.0, 0.0)


def test_one_wrong_token_row_is_caught_by_the_row_term():
    r = _ref((2, 4096, 2, 128))
    g = r.copy()
    g[1, 1234, 0] = 0.0                      # one token row of one (b, h) lost
    e = errors(g, r)
    assert e["norm"] <= TOL["bf16"]          # 1/64 of the slice norm: the norm alone passes it
    assert e["row"] > 0.4 and worst(e) > TOL["bf16"]


def test_one_wrong_element_is_caught_by_the_element_term():
    r = _ref((1, 512, 1, 64))
    g = r.copy()
    i = np.argmax(np.abs(r))
    g.flat[i] *= 1.05                        # 5% off on a large element
    e = errors(g, r)
    assert e["norm"] < TOL["bf16"] and e["row"] < TOL["bf16"]
    assert e["elem"] > TOL["bf16"]


def test_rounding_noise_at_bf16_scale_passes():
    """Noise of 5e-3 of the slice rms on every element (the size of the bf16
    paths' normwise errors) over 8 million elements stays under the bound."""
    r = _ref((4, 4096, 4, 128))
    g = r + 5e-3 * np.random.default_rng(1).standard_normal(r.shape)
    assert worst(errors(g, r)) <= TOL["bf16"]


def test_element_scale_follows_its_row():
    """Rows ten times larger than the rest of the slice (a decaying initial
    state) carry rounding noise ten times larger: measured against their own
    row's magnitude, not the slice's."""
    r = _ref((1, 4096, 1, 128))
    r[:, :300] *= 10.0
    noise = 4e-3 * np.random.default_rng(2).standard_normal(r.shape)
    noise[:, :300] *= 10.0
    assert worst(errors(r + noise, r)) <= TOL["bf16"]


def test_state_and_channel_layouts():
    r = _ref((2, 3, 16, 16))
    g = r.copy()
    g[1, 2, 5] += 0.5                        # one state row
    e = errors(g, r, "state")
    assert e["row"] > TOL["bf16"] and e["elem"] > TOL["bf16"]
    r = _ref((2, 300, 8))
    g = r.copy()
    g[0, 17, 3] = -g[0, 17, 3]               # one element of one channel sequence
    assert errors(g, r, "btc")["elem"] > TOL["bf16"]


def test_nonfinite_fails_and_zero_reference_is_absolute():
    r = _ref((1, 8, 1, 4))
    g = r.copy()
    g[0, 3, 0, 1] = np.nan
    assert worst(errors(g, r)) == float("inf")
    z = np.zeros((1, 8, 1, 4))
    e = errors(z + 1e-9, z)
    assert worst(e) < 1e-8


def test_one_value_rows_use_the_element_term():
    """Rows of a single value (the per-head dlog_a [B, T, H], read as rows of
    one): the row term is the element term.  A near-cancelling value off by
    2.4% of its slice's rms (what bfloat16 operand rounding leaves on a sum
    whose terms are hundreds of times the result) passes; a value off by 20%
    of the slice rms fails; so does a lost token."""
    r = _ref((3, 200, 3, 1)) * 20.0
    rms = np.sqrt(np.mean(r[2, :, 0, 0] ** 2))
    g = r.copy()
    g[2, 1, 0, 0] = -0.88
    r2 = r.copy()
    r2[2, 1, 0, 0] = -0.88 + 0.024 * rms
    e = errors(g, r2)
    assert e["row"] == e["elem"] and worst(e) <= TOL["bf16"]
    g = r.copy()
    g[1, 5, 2, 0] += 0.2 * rms
    assert worst(errors(g, r)) > TOL["bf16"]
    g = r.copy()
    g[0, 17, 1, 0] = 0.0
    assert worst(errors(g, r)) > TOL["bf16"] or abs(r[0, 17, 1, 0]) < 0.06 * rms


def test_short_slices_use_the_row_term():
    """Sequences shorter than one 16-token sub-block: the norm term is the row
    term.  A one-token row off by 2.8% in every element (what bf16 operand
    rounding leaves on a score whose terms cancel thirty-fold) passes; 10% off
    fails; at 16 tokens the slice norm applies again."""
    r = _ref((2, 1, 2, 64))
    g = r.copy()
    g[0, 0, 1] *= 1.028
    e = errors(g, r)
    assert e["norm"] == e["row"] and worst(e) <= TOL["bf16"]
    g = r.copy()
    g[1, 0, 0] *= 1.10
    assert worst(errors(g, r)) > TOL["bf16"]
    r = _ref((1, 16, 1, 64))
    g = r * 1.028
    e = errors(g, r)
    assert e["norm"] > TOL["bf16"] and e["norm"] != e["row"]


def test_short_slices_measure_against_their_terms():
    """A one-token slice whose score q.k cancels its terms 200-fold: the
    bf16 kernels' rounding (the float64 model of their rounding points) is
    several percent of y itself, so the plain metric fails it; measured
    against the magnitude of y's terms (the oracle on absolute values) it
    passes, while one channel of q with its sign flipped still fails."""
    import oracle
    from tests import chunked_ref as cr
    rng = np.random.default_rng(7)
    B, T, H, D = 1, 1, 2, 64
    q = cr._bf16(rng.standard_normal((B, T, H, D)))
    k = cr._bf16(rng.standard_normal((B, T, H, D)))
    for h in range(H):                              # q.k about 1/200 of sum |q k|
        qk = q[0, 0, h] * k[0, 0, h]
        c = int(np.argmax(np.abs(q[0, 0, h])))
        want = 0.005 * np.abs(qk).sum()
        k[0, 0, h, c] = cr._bf16(np.array([k[0, 0, h, c] + (want - qk.sum()) / q[0, 0, h, c]]))[0]
    v = cr._bf16(rng.standard_normal((B, T, H, D)))
    lf = np.full((B, T, H, D), np.log(0.9))
    ref, _ = oracle.forward(q, k, v, lf, None)
    got = np.stack([cr.forward_bf16_points(q[0, :, h], k[0, :, h], v[0, :, h], lf[0, :, h], C=16)
                    for h in range(H)], axis=1)[None]
    terms, _ = oracle.forward(np.abs(q), np.abs(k), np.abs(v), lf, None)
    assert worst(errors(got, ref)) > TOL["bf16"]
    assert worst(errors(got, ref, "token", terms)) <= TOL["bf16"]
    q2 = q.copy()
    q2[..., 5] = -q2[..., 5]
    bad, _ = oracle.forward(q2, k, v, lf, None)
    assert worst(errors(bad, ref, "token", terms)) > TOL["bf16"]
