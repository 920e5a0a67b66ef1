"""Seeded synthetic inputs for the HGRN2 recurrence.

This module only draws random numbers and shapes them into the tensors the
recurrence consumes (q, k, v, log_f, initial state, upstream gradients).  It
holds none of the recurrence's arithmetic: the gate recipe below
(f = lam + (1 - lam) * sigmoid(z), k = 1 - f) is how a caller of the kernel
would produce its inputs (HGRN2 paper summary, paperlayer.ai, §2.1: input gate
tied to the forget gate as one minus it; §2.2: forget gate with an additive
lower bound and a learned residual above it).  Both the oracle tests and the
GPU path read these arrays; nothing here depends on either.

Recipe (fixed draw order per workload, numpy PCG64):
  1. z  ~ N(0, 1)          [B, T, H, D]   forget-gate pre-activation
  2. q  ~ N(0, 1) * qscale [B, T, H, D]
  3. v  ~ N(0, 1) * qscale [B, T, H, D]
  4. h0 ~ N(0, 1) * h0std  [B, H, D, D]   (only when the workload has one)
  5. dy ~ N(0, 1)          [B, T, H, D]   (only for training workloads)
  log_f = log(lam + (1 - lam) * sigmoid(z)) and k = (1 - lam) * sigmoid(-z),
  both evaluated in float64 without cancellation, then rounded to the
  workload dtype.  After rounding k and log_f are independent inputs.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "generate", "generate_decode", "to_f64",
           "bf16_round", "bf16_to_f32", "f32_to_bf16_bits"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    D: int
    chunk: int
    dtype: str            # "f32" or "bf16": storage type of q, k, v, log_f, y, grads
    lam: float            # forget-gate lower bound
    qscale: float         # std of q and v
    h0std: float          # std of the initial state (0 = zero state)
    train: bool           # draws dy as well
    seed: int
    decode: bool = False  # one-token decode step against a resident state


# The five synthetic workloads.  Sizes, distributions and gate bounds are the
# ones the benchmark suite fixes; the chunk of the training workload is ours.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, H=2, T=256, D=16, chunk=16, dtype="f32",
                         lam=0.0, qscale=1.0, h0std=0.0, train=False, seed=1000),
    "fwd_bf16": Workload("fwd_bf16", B=4, H=8, T=2048, D=128, chunk=64, dtype="bf16",
                         lam=0.5, qscale=1.0 / math.sqrt(128), h0std=0.0, train=False,
                         seed=1001),
    "train_bf16": Workload("train_bf16", B=8, H=16, T=4096, D=128, chunk=64, dtype="bf16",
                           lam=0.0, qscale=1.0 / math.sqrt(128), h0std=0.0, train=True,
                           seed=1002),
    "decode_f32": Workload("decode_f32", B=256, H=16, T=1, D=128, chunk=0, dtype="f32",
                           lam=0.9, qscale=1.0 / math.sqrt(128), h0std=0.1, train=False,
                           seed=1003, decode=True),
    "long_bf16": Workload("long_bf16", B=1, H=32, T=32768, D=128, chunk=64, dtype="bf16",
                          lam=0.97, qscale=1.0 / math.sqrt(128), h0std=0.1, train=False,
                          seed=1004),
}

# The training workload draws its lower bound per run from this set.
TRAIN_LAMBDAS = (0.0, 0.3, 0.6)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounding = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32 exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float -> nearest bfloat16 value, returned as float32."""
    return bf16_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 array to the storage dtype.

    f32 -> float32 array; bf16 -> uint16 array of bfloat16 bits (RNE from the
    float32 rounding; the values, not the rounding path, define the input)."""
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored input (bf16 bits are widened exactly)."""
    if dtype == "bf16" and x.dtype == np.uint16:
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _gates(z: np.ndarray, lam: float):
    """log f and k = 1 - f from the pre-activation z, in float64.

    f = lam + (1 - lam) * sigmoid(z)   and   1 - f = (1 - lam) * sigmoid(-z),
    so k never suffers the cancellation of 1 - f when f is close to one."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))            # in (0, 1], never overflows
    big = 1.0 / (1.0 + e)             # sigmoid(|z|)
    small = e / (1.0 + e)             # sigmoid(-|z|)
    sig_pos = np.where(z >= 0, big, small)    # sigmoid(z)
    sig_neg = np.where(z >= 0, small, big)    # sigmoid(-z)
    if lam == 0.0:
        # log sigmoid(z) = -softplus(-z), evaluated stably
        log_f = -(np.maximum(-z, 0.0) + np.log1p(np.exp(-np.abs(z))))
    else:
        log_f = np.log(lam + (1.0 - lam) * sig_pos)
    k = (1.0 - lam) * sig_neg
    return log_f, k


def generate(w: Workload | str, *, lam: float | None = None, seed: int | None = None,
             B: int | None = None, T: int | None = None, H: int | None = None,
             D: int | None = None) -> dict:
    """Draw one workload's inputs.  Sizes may be overridden for small parity cases.

    Returns a dict of numpy arrays in storage form (float32, or uint16 bfloat16
    bits) plus metadata: q, k, v, log_f [B,T,H,D]; z [B,T,H,D], the gate
    pre-activation that log_f and k were made from (rounded on its own, for
    callers that pass the pre-activation instead); h0 [B,H,D,D] float32 or
    None; dy [B,T,H,D] or None."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    D = w.D if D is None else D
    lam = w.lam if lam is None else lam
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, T, H, D)
    z = rng.standard_normal(shape)
    log_f, k = _gates(z, lam)
    q = rng.standard_normal(shape) * w.qscale
    v = rng.standard_normal(shape) * w.qscale
    h0 = None
    if w.h0std > 0:
        h0 = (rng.standard_normal((B, H, D, D)) * w.h0std).astype(np.float32)
    dy = None
    if w.train:
        dy = _store(rng.standard_normal(shape), w.dtype)
    return dict(q=_store(q, w.dtype), k=_store(k, w.dtype), v=_store(v, w.dtype),
                log_f=_store(log_f, w.dtype), z=_store(z, w.dtype), h0=h0, dy=dy, dtype=w.dtype,
                B=B, T=T, H=H, D=D, chunk=w.chunk, lam=lam, seed=seed, name=w.name)


def generate_decode(w: Workload | str = "decode_f32", *, seed: int | None = None,
                    B: int | None = None, H: int | None = None, D: int | None = None) -> dict:
    """One decode step: q, k, v, log_f [B,H,D] float32 and a state [B,H,D,D] float32.

    Draw order: z, q, v, state.  f = lam + (1 - lam) sigmoid(z), k = 1 - f."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    H = w.H if H is None else H
    D = w.D if D is None else D
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, D)
    z = rng.standard_normal(shape)
    log_f, k = _gates(z, w.lam)
    q = rng.standard_normal(shape) * w.qscale
    v = rng.standard_normal(shape) * w.qscale
    state = (rng.standard_normal((B, H, D, D)) * w.h0std).astype(np.float32)
    return dict(q=q.astype(np.float32), k=k.astype(np.float32), v=v.astype(np.float32),
                log_f=log_f.astype(np.float32), z=z.astype(np.float32), state=state, dtype="f32",
                B=B, H=H, D=D, seed=seed, name=w.name)


def lower_bounds(H: int, D: int, lam: float, spread: float = 0.0, seed: int = 7) -> np.ndarray:
    """A per-channel forget-gate lower bound [H, D] float32: lam everywhere, or
    lam + spread * U(-1, 1) clipped to [0, 0.99] when spread > 0 (a separate
    PCG64 stream, so the other inputs do not change)."""
    if spread <= 0.0:
        return np.full((H, D), lam, dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.clip(lam + spread * rng.uniform(-1.0, 1.0, (H, D)), 0.0, 0.99).astype(np.float32)


def large_device_inputs(B: int, T: int, H: int, D: int, *, seed: int, reset_every: int, device="cuda"):
    """bfloat16 token tensors too large to draw on the host, drawn on `device`
    with torch's seeded generator: q, k, v ~ N(0, 1)/sqrt(D), dy ~ N(0, 1),
    log_f ~ -U(0, 0.3), and log_f = -inf (a full reset, f = 0) on every channel
    of every token t with t % reset_every == 0, so that the sequence splits
    into independent windows that start from a zero state.  [B, T, H, D] each;
    returns a dict."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    shape = (B, T, H, D)
    out = {}
    for n in ("q", "k", "v"):
        out[n] = torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16).mul_(1.0 / math.sqrt(D))
    out["dy"] = torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
    lf = torch.rand(shape, generator=g, device=device, dtype=torch.bfloat16).mul_(-0.3)
    lf[:, ::reset_every] = float("-inf")
    out["log_f"] = lf
    return out
