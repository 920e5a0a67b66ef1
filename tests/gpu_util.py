"""Helpers shared by the GPU parity tests: move synthetic inputs to the GPU,
run the oracle on the same values, compare them.

Comparison metrics (all three must be <= the dtype's tolerance, TOL):
  norm  the largest normwise relative error over slices,
        ||gpu - ref||_F / ||ref||_F;
  row   the largest error of one row (one token's D values of a head, one
        token's C channels, one state row), relative to that row's reference
        norm plus the slice's root-mean-square row norm:
        ||gpu_t - ref_t|| / (||ref_t|| + rms_t ||ref_t||);
  elem  the largest error of one element, relative to its reference value
        plus three times the typical magnitude around it, the larger of its
        row's and its slice's root-mean-square value:
        |gpu - ref| / (|ref| + 3 max(rms(ref_t), rms(ref))).
A slice is one (b, h) sequence of a [B, T, H, D] tensor, one (b, h) matrix of
a [B, H, D, D] state, or one (b, c) channel sequence of a [B, T, C] tensor.
A slice of fewer than MIN_NORM_ROWS rows (sequences shorter than one 16-token
sub-block) is held to the row term in place of the norm term: its norm is
then the relative error of one or a few rows, with nothing to average over.
With one token a row of y is one score times v, and that score a dot product
of q e^{ell} (a bf16 operand) with k: where its terms cancel thirty-fold, the
operand rounding alone leaves about 3% in every element of the row (a float64
model of the kernels' rounding points reproduces the GPU's error to three
digits, and drops it tenfold without the operand rounding).  The row term
measures that row against its norm plus the slice's rms row norm, as it does
every row of every slice.  Where the comparison also has the magnitude of the
terms each output sums (`terms`: the oracle on the absolute values of the
inputs, |q|, |k|, |v|, |h0|, |dy|, |dht| with f unchanged, which for these
sums of products with positive weights is the sum of the terms' magnitudes),
a short slice's row and element denominators also get TERMS_FRAC of it: a
path rounds a term at most about five times at its unit roundoff (bf16:
decayed operands, score tile, state, output), so the fraction is five unit
roundoffs over the tolerance, 5 * 2^-9 / 2e-2 (about 1/2) for bf16 and
5 * 2^-24 / 1e-4 for float32.  An output that cancels its terms almost completely is then held
to the rounding its arithmetic allows, not to its own tiny magnitude.
The row and element terms catch localised errors that a slice norm over
hundreds of thousands of values would hide (one wrong token row of a 4096-token
slice moves its norm by only about 1/64).  Where a row holds a single value
(the per-head dlog_a [B, T, H], a per-channel [H, D] or [B, C] quantity read
as rows of one), the row term would be the element term with a factor 1, so
the element term stands for it: it already checks every row.

The element scale follows the magnitude of the element's own row because
magnitudes, and the rounding noise that comes with them, vary along a
sequence: a decaying initial state makes the first thousand outputs of the
long-context workload about ten times larger than the later ones.  The factor
3 comes from the bf16 paths' arithmetic: the decayed q and k enter the score
products as bf16 operands (relative rounding 2^-9 each), so an output that is a
near-cancellation of terms several times its row's magnitude carries an error
of a few percent of that magnitude.  Over the 67 million elements of a full
training batch the largest such error is 4.2% of its row's rms (the element
metric with factor 2 gave 2.1e-2); a float64 emulation of the kernels'
rounding points reproduces that element's error exactly, and removing the
operand roundings from the emulation removes it.  With 3, the threshold for an
element whose true value is near zero is 6% of its neighbourhood's magnitude,
1.4 times that extreme, while an element off by more than 6% of its
neighbourhood's magnitude (or 2% of its own value) fails.  A slice whose
reference is exactly zero is compared in absolute terms.  Any NaN or infinity
in the GPU result fails.
"""

from __future__ import annotations

import numpy as np
import torch

import synth

TOL = {"bf16": 2e-2, "f32": 1e-4}
MIN_NORM_ROWS = 16
TERMS_FRAC = {"bf16": 5 * 2.0 ** -9 / TOL["bf16"], "f32": 5 * 2.0 ** -24 / TOL["f32"]}


def to_dev(a: np.ndarray | None, dtype: str):
    """Storage array (float32, or uint16 bfloat16 bits) -> CUDA tensor."""
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def _nz(x):
    """Denominators: zero (an all-zero reference) becomes one (absolute error)."""
    return np.where(x > 0, x, 1.0)


def errors(got: np.ndarray, ref: np.ndarray, layout: str = "token", terms: np.ndarray | None = None,
           dtype: str = "bf16") -> dict:
    """The three metrics above for `got` against `ref`.

    layout: "token" [B, T, H, D] (slices (b, h), rows = tokens), "state"
    [B, H, D, D] (slices (b, h), rows = state rows), "btc" [B, T, C] (slices
    (b, c), rows = tokens of one batch element).  terms: the magnitude of the
    terms each reference value sums, same shape (used for short slices of the
    input dtype `dtype`)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return {"norm": float("inf"), "row": float("inf"), "elem": float("inf"), "elem_at": "non-finite"}
    if got.size == 0:
        return {"norm": 0.0, "row": 0.0, "elem": 0.0, "elem_at": ""}
    d = got - ref
    if layout == "token":       # [B, T, H, D]
        s_ax, r_ax = (1, 3), 3
        slice_b = lambda x: x[:, None, :, None]      # [B, H] -> broadcast over [B, T, H, D]
        row_b = lambda x: x[:, None, :]              # [B, H] -> broadcast over rows [B, T, H]
    elif layout == "state":     # [B, H, D, D]
        s_ax, r_ax = (2, 3), 3
        slice_b = lambda x: x[:, :, None, None]
        row_b = lambda x: x[:, :, None]
    elif layout == "btc":       # [B, T, C]: slices (b, c) along T; rows = tokens of b
        B, T, C = ref.shape
        n = np.sqrt((d * d).sum(axis=1))             # [B, C]
        rn = np.sqrt((ref * ref).sum(axis=1))
        norm = float(np.max(n / _nz(rn)))
        rms = rn / np.sqrt(T)
        re = np.sqrt((d * d).sum(axis=2))            # [B, T]
        rr = np.sqrt((ref * ref).sum(axis=2))
        rs = np.sqrt((rr * rr).mean(axis=1))         # [B]
        row = float(np.max(re / _nz(rr + rs[:, None])))
        scale = np.maximum(rms[:, None, :], (rr / np.sqrt(C))[:, :, None])
        return {"norm": row if T < MIN_NORM_ROWS else norm, "row": row, **_elem(d, ref, scale)}
    else:
        raise ValueError(layout)
    n = np.sqrt((d * d).sum(axis=s_ax))
    rn = np.sqrt((ref * ref).sum(axis=s_ax))
    norm = float(np.max(n / _nz(rn)))
    count = ref.shape[s_ax[0]] * ref.shape[s_ax[1]]
    rms = rn / np.sqrt(count)
    re = np.sqrt((d * d).sum(axis=r_ax))
    rr = np.sqrt((ref * ref).sum(axis=r_ax))
    nrows = ref.shape[s_ax[0]]
    rs = rn / np.sqrt(nrows)                         # rms row norm of the slice
    width = ref.shape[r_ax]
    scale = np.maximum(slice_b(rms), (rr / np.sqrt(width))[..., None])
    short = nrows < MIN_NORM_ROWS
    ta = np.zeros_like(ref) if (terms is None or not short) else TERMS_FRAC[dtype] * np.abs(np.asarray(terms, np.float64))
    el = _elem(d, ref, scale, ta)
    ra = np.sqrt((ta * ta).sum(axis=r_ax))
    row = el["elem"] if width == 1 else float(np.max(re / _nz(rr + row_b(rs) + ra)))
    return {"norm": row if short else norm, "row": row, **el}


def _elem(d, ref, scale, extra=0.0):
    """The element metric, and where its worst element is (index, error,
    reference, scale) for the report.  extra: a further per-element term of
    the denominator (a short slice's share of its terms' magnitude)."""
    scale = np.broadcast_to(scale, ref.shape)
    ratio = np.abs(d) / _nz(np.abs(ref) + 3.0 * scale + extra)
    i = int(np.argmax(ratio))
    at = np.unravel_index(i, ref.shape)
    return {"elem": float(ratio.flat[i]),
            "elem_at": "%s err %.2e ref %.2e scale %.2e" % (tuple(int(a) for a in at), d.flat[i], ref.flat[i],
                                                             scale.flat[i])}


def worst(e: dict) -> float:
    return max(e["norm"], e["row"], e["elem"])


def fmt(e: dict) -> str:
    return "norm %.2e row %.2e elem %.2e [%s]" % (e["norm"], e["row"], e["elem"], e.get("elem_at", ""))


def slice_rel(got: np.ndarray, ref: np.ndarray, token_major=True) -> float:
    """The worst of the three metrics (normwise per slice, per row, per
    element) for a [B, T, H, D] (token_major) or [B, H, D, D] tensor; compared
    against TOL by the tests."""
    return worst(errors(got, ref, "token" if token_major else "state"))


def inputs64(d: dict):
    """float64 copies of the stored inputs (exactly the values the GPU sees)."""
    dt = d["dtype"]
    out = {n: synth.to_f64(d[n], dt) for n in ("q", "k", "v", "log_f")}
    out["h0"] = None if d["h0"] is None else d["h0"].astype(np.float64)
    out["dy"] = None if d.get("dy") is None else synth.to_f64(d["dy"], dt)
    return out


def select_bh(x: np.ndarray | None, pairs, token_major=True):
    """Stack the chosen (b, h) slices into a [n, T, 1, D] (or [n, 1, D, D]) array."""
    if x is None:
        return None
    if token_major:
        return np.stack([x[b, :, h] for b, h in pairs])[:, :, None]
    return np.stack([x[b, h] for b, h in pairs])[:, None]
