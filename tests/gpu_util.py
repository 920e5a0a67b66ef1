"""Helpers shared by the GPU parity tests: move synthetic inputs to the GPU,
run the oracle on the same values, compare slice by slice."""

from __future__ import annotations

import numpy as np
import torch

import synth

TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_dev(a: np.ndarray | None, dtype: str):
    """Storage array (float32, or uint16 bfloat16 bits) -> CUDA tensor."""
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def slice_rel(got: np.ndarray, ref: np.ndarray, token_major=True) -> float:
    """Largest normwise relative error over (b, h) slices (inf if the GPU
    result holds a NaN or an infinity).

    token tensors are [B,T,H,D]; state tensors [B,H,D,D]."""
    if not np.all(np.isfinite(got)):
        return float("inf")
    worst = 0.0
    if token_major:
        B, _, H, _ = ref.shape
        for b in range(B):
            for h in range(H):
                r = ref[b, :, h]
                d = np.linalg.norm(got[b, :, h] - r)
                n = np.linalg.norm(r)
                worst = max(worst, d / n if n > 0 else d)
    else:
        B, H = ref.shape[:2]
        for b in range(B):
            for h in range(H):
                r = ref[b, h]
                d = np.linalg.norm(got[b, h] - r)
                n = np.linalg.norm(r)
                worst = max(worst, d / n if n > 0 else d)
    return float(worst)


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
