"""Benchmark of the HGRN2 recurrence hot path on one MI355X.

One step = one training pass over one batch of the H16 d128 T4096 workload
(B8 H16 T4096, d_k = d_v = 128, bf16, chunk 64): hgrn2_fwd (saving the
chunk-boundary states) followed by hgrn2_bwd, issued as the four single
launches they are made of (state scan, per-chunk outputs, adjoint scan,
per-chunk gradients) so that HIP events on the launch stream bracket each
kernel.  Three resident input sets (forget-gate lower bound 0, 0.3, 0.6) are
rotated across steps.  The same step with tied gates (k = 1 - f formed in the
kernels, hgrn2_fwd_tied / hgrn2_bwd_tied) is timed next on the same inputs and
reported under "tied", then the step with the gate formed from its
pre-activation z and a per-channel lower bound (hgrn2_fwd_gate /
hgrn2_bwd_gate, its two calls timed) under "gate", the step with one decay per
head (hgrn2_fwd_scalar / hgrn2_bwd_scalar) under "scalar", and the HGRN1
elementwise recurrence on the same tensors read as [B, T, C] under "hgrn1";
the headline value is the untied step.  The decode step (B256 H16 d128,
float32 state) is timed as well and reported in HBM GB/s, and the two
forward-only workloads (B4 H8 T2048 and B1 H32 T32768 with an initial state,
both d128 bf16 chunk 64) under "fwd_bf16" and "long_bf16", each call after an
eviction of the caches.  Inputs are seeded synthetic data generated on the
host and copied to HBM before timing.  The float64 CPU oracle is timed on the
host cores on the same batches, and its outputs are compared with the GPU's.

Each leg first runs its own step untimed for SETTLE_S seconds of wall time
(the GPU's clocks ramp up over tens of milliseconds of sustained work), then
its W warmup steps, then exactly K timed steps.

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_SUMMARY = os.path.join(PROFILES, "hgrn2_traffic_train_bf16_B8H16T4096.txt")
CALIB_BYTES = 1 << 30          # the --calib-copy device copy: 1 GiB read, 1 GiB written

# the commands whose output --summarize turns into the files under profiles/
# (rocprofv3 writes under PROF_OUT, a directory relative to the repository root)
PROF_OUT = os.environ.get("HGRN2_PROF_OUT", "prof_out")
TRACE_CMD = ("rocprofv3 --kernel-trace --stats -d " + PROF_OUT + "/trace -o run --output-format csv "
             "-- python3 bench.py --steps 20 --warmup 3 --no-cpu")
PMC_CMD = ("rocprofv3 --pmc {ctr} -d " + PROF_OUT + "/{dir} -o run --output-format csv "
           "-- python3 bench.py --only train --steps 2 --warmup 1 --no-cpu --calib-copy")
MFMA_CMD = ("rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 MfmaUtil -d " + PROF_OUT + "/mfma -o run "
            "--output-format csv -- python3 bench.py --only train --steps 2 --warmup 1 --no-cpu")
MFMA_SUMMARY = os.path.join(PROFILES, "hgrn2_mfma_train_bf16_B8H16T4096.txt")
# the forward-only legs (the segmented forward), one trace and two counter runs each
FWD_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -d " + PROF_OUT + "/trace_{leg} -o run --output-format csv "
                 "-- python3 bench.py --only {leg} --steps 20 --warmup 3 --no-cpu")
FWD_PMC_CMD = ("rocprofv3 --pmc {ctr} -d " + PROF_OUT + "/{dir}_{leg} -o run --output-format csv "
               "-- python3 bench.py --only {leg} --steps 2 --warmup 1 --no-cpu --calib-copy")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--decode-steps", type=int, default=50)
    p.add_argument("--only", choices=["train", "decode", "fwd_bf16", "long_bf16", "all"], default="all",
                   help="run one leg only (train: the training step and its variants)")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB elementwise pass, read once and written once "
                        "(calibrates profiler byte counters)")
    p.add_argument("--summarize-fwd", nargs=4, metavar=("LEG", "TRACE", "FETCH", "WRITE"),
                   help="write the profiles/ summary of a forward-only leg from FWD_TRACE_CMD and FWD_PMC_CMD "
                        "output")
    p.add_argument("--summarize", nargs="+", metavar="DIR",
                   help="TRACE_DIR FETCH_DIR WRITE_DIR [MFMA_DIR]: write the profiles/ summaries "
                        "from rocprofv3 csv output and exit")
    return p.parse_args()


def kernel_source_digest() -> str:
    """Digest of the kernel sources and of their build options (build.py); a
    traffic figure taken on other sources or options is void."""
    import hashlib
    csrc = os.path.join(ROOT, "linear_attention_hgrn2_amd", "csrc")
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "linear_attention_hgrn2_amd", "build.py"), "rb") as f:
        h.update(f.read())
    for n in sorted(os.listdir(csrc)):
        if n.endswith((".h", ".hip", ".cpp")):
            h.update(n.encode())
            with open(os.path.join(csrc, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE) from the
    committed counter summary, or None if it is missing or was taken on other sources."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    kv = dict(l.split(": ", 1) for l in lines if ": " in l and not l.startswith(" "))
    if kv.get("source_digest") != kernel_source_digest():
        return None
    v = kv.get("traffic_bytes_per_launch " + kernel)
    return None if v is None else float(v)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_train_sets(torch, w, lams):
    import synth
    from tests.gpu_util import to_dev
    sets = []
    for i, lam in enumerate(lams):
        d = synth.generate(w, lam=lam, seed=w.seed + 10 * i)
        sets.append({n: to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f", "z", "dy")})
        sets[-1]["host"] = d if i == 0 else None
        log("inputs ready: lambda=%.1f" % lam)
    return sets


# untimed work of each leg before its warmup steps, in seconds of wall time
SETTLE_S = 0.3


def settle(torch, fn, seconds=SETTLE_S):
    """Runs fn(i) untimed for about `seconds` of wall time and returns the
    number of calls.  After an idle spell (host-side set-up, the oracle) the
    GPU's clocks ramp up over tens of milliseconds of sustained work: measured
    on the training step, the first timed steps after 3 warmup steps took
    1.05 ms, falling to a steady 0.89 ms after about 40 steps.  Each leg's
    timed steps are to see the sustained rate of its kernels, not that ramp;
    the timed region itself still holds exactly its K steps."""
    t0 = time.time()
    i = 0
    while True:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.time() - t0 >= seconds or i >= 4096:
            return i


class KernelTimer:
    """Events recorded on the stream the kernels run on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def start(self, name):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return (name, e)

    def stop(self, tok):
        name, s = tok
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(name, []).append((s, e))

    def times_ms(self, name):
        return [s.elapsed_time(e) for s, e in self.pairs[name]]

    def mean_ms(self, name):
        return float(np.mean(self.times_ms(name)))

    def stats(self, name):
        t = self.times_ms(name)
        return {"mean": float(np.mean(t)), "median": float(np.median(t)), "min": float(np.min(t)), "n": len(t)}


# the four launches of one training step, in order, with the kernel each one runs
TRAIN_KERNELS = (("scan", "hgrn2_scan_kernel (forward)"), ("cfwd", "hgrn2_chunk_fwd_kernel"),
                 ("scan_rev", "hgrn2_scan_kernel (reverse)"), ("cbwd", "hgrn2_chunk_bwd_res_kernel"))
# the same with tied gates (k = 1 - f formed in the kernels; the adjoint scan never reads k)
TIED_KERNELS = (("scan_tied", "hgrn2_scan_kernel (forward, tied)"),
                ("cfwd_tied", "hgrn2_chunk_fwd_kernel (tied)"),
                ("scan_rev", "hgrn2_scan_kernel (reverse)"),
                ("cbwd_tied", "hgrn2_chunk_bwd_res_kernel (tied)"))
# the gate-from-pre-activation step, as its two composite calls
GATE_CALLS = (("fwd_gate", "hgrn2_fwd_gate: state scan + per-chunk outputs"),
              ("bwd_gate", "hgrn2_bwd_gate: adjoint scan + per-chunk gradients + lower-bound sum"))
# the one-decay-per-head step, as its two composite calls
SCALAR_CALLS = (("fwd_scalar", "hgrn2_fwd_scalar: state scan + per-chunk outputs"),
                ("bwd_scalar", "hgrn2_bwd_scalar: adjoint scan + per-chunk gradients"))


def _template_args(n: str):
    if "<" not in n or ">" not in n:
        return []
    return [a.strip() for a in n[n.index("<") + 1:n.rindex(">")].split(",")]


GATE_SUFFIX = {"0": "", "1": "_tied", "2": "_gate", "3": "_scalar"}


def kernel_label(name: str):
    """rocprofv3 kernel name -> a label of TRAIN_KERNELS, TIED_KERNELS or GATE_KERNELS,
    "decode[_tied|_gate|_scalar]", "dlb", "seg_scan", "seg_fwd", "seg_carry", an
    HGRN1 label, or None.  The gate mode (0 untied, 1 tied, 2 gate, 3 per-head
    decay) is a template argument at a fixed place: scan <T, D, C, REV, GM, SEG>;
    chunk forward and generic backward <T, D, C, GM, TO>; resident backward
    <GM, TO>; segment walk <T, D, C, GM, TO>; decode <T, D, GM, TO>."""
    n = _short(name)
    a = _template_args(n)

    def sfx(i):
        return GATE_SUFFIX.get(a[i], "") if len(a) > i else ""
    if n.startswith("hgrn2_scan_kernel"):
        if len(a) > 5 and a[5] == "true":
            return "seg_scan" + sfx(4)
        return ("scan_rev" if len(a) > 3 and a[3] == "true" else "scan") + sfx(4)
    if n.startswith("hgrn2_chunk_fwd_kernel"):
        return "cfwd" + sfx(3)
    if n.startswith("hgrn2_chunk_bwd_res_kernel"):
        return "cbwd" + sfx(0)
    if n.startswith("hgrn2_chunk_bwd"):
        return "cbwd" + sfx(3)
    if n.startswith("hgrn2_seg_fwd_kernel"):
        return "seg_fwd" + sfx(3)
    if n.startswith("hgrn2_seg_carry_kernel"):
        return "seg_carry"
    if n.startswith("hgrn2_decode_kernel"):
        return "decode" + sfx(2)
    if n.startswith("hgrn2_dlb_reduce_kernel"):
        return "dlb"
    if n.startswith("hgrn1_"):
        rev = len(a) > 2 and a[2] == "true"
        for key, lab in (("summary", "h1_summary_rev" if rev else "h1_summary"), ("final_fwd", "h1_final_fwd"),
                         ("final_bwd", "h1_final_bwd")):
            if n.startswith("hgrn1_" + key):
                return lab
        if n.startswith("hgrn1_carry"):
            return "h1_carry_rev" if a and a[0] == "true" else "h1_carry"
    return None


def train_algorithmic_bytes(w):
    """Algorithmic HBM bytes per launch of each training kernel: every tensor
    the launch reads or writes, once.  tok = one bf16 [B,T,H,D] tensor; a
    state or adjoint entry is one bf16 [D,D] matrix per (b,h)."""
    tok = w.B * w.T * w.H * w.D * 2
    N = w.T // w.chunk
    ent = w.B * w.H * w.D * w.D * 2
    return {
        "scan": 3 * tok + (N + 1) * ent,                 # k, v, log_f in; states 0..N out
        "cfwd": 4 * tok + N * ent + tok,                 # q, k, v, log_f, states 0..N-1 in; y out
        "scan_rev": 3 * tok + N * ent,                   # q, dy, log_f in; adjoints 1..N out
        "cbwd": 5 * tok + 2 * N * ent + 4 * tok,         # q, k, v, log_f, dy, states, adjoints in; 4 grads out
        # tied gates: no k read, no dk written
        "scan_tied": 2 * tok + (N + 1) * ent,
        "cfwd_tied": 3 * tok + N * ent + tok,
        "cbwd_tied": 4 * tok + 2 * N * ent + 3 * tok,
        # gate from z: as tied (z in place of log f); the gradient launch also
        # writes one float per (b, h, chunk, channel) of lower-bound sums, which
        # the reduction reads back
        "scan_gate": 2 * tok + (N + 1) * ent,
        "cfwd_gate": 3 * tok + N * ent + tok,
        "scan_rev_gate": 3 * tok + N * ent,
        "cbwd_gate": 4 * tok + 2 * N * ent + 3 * tok + w.B * w.H * N * w.D * 4,
        "dlb": w.B * w.H * N * w.D * 4 + w.H * w.D * 4,
        # one decay per head: log a and dlog a are [B,T,H] (tok / D)
        "scan_scalar": 2 * tok + tok // w.D + (N + 1) * ent,
        "cfwd_scalar": 3 * tok + tok // w.D + N * ent + tok,
        "scan_rev_scalar": 2 * tok + tok // w.D + N * ent,
        "cbwd_scalar": 4 * tok + tok // w.D + 2 * N * ent + 3 * tok + tok // w.D,
    }


def train_abi_bytes(w):
    """Bytes per launch counted as the scope table's measurement section does:
    the tensors of the C ABI each launch reads or writes (q, k, v, log_f, dy,
    y and the four gradients, once each) plus the chunk-boundary states (an
    output of hgrn2_fwd, read by the chunk kernels); the adjoint workspace,
    which stays inside hgrn2_bwd, is left out."""
    tok = w.B * w.T * w.H * w.D * 2
    N = w.T // w.chunk
    ent = w.B * w.H * w.D * w.D * 2
    return {"scan": 3 * tok + (N + 1) * ent, "cfwd": 4 * tok + N * ent + tok, "scan_rev": 3 * tok,
            "cbwd": 5 * tok + N * ent + 4 * tok,
            "scan_tied": 2 * tok + (N + 1) * ent, "cfwd_tied": 3 * tok + N * ent + tok,
            "cbwd_tied": 4 * tok + N * ent + 3 * tok}


def train_step_flop(w):
    """Algorithmic flops of one training step (forward C(d_k + d_v) + 4 d_k d_v
    and backward 5 C d + 8 d^2 per token-head; no recompute, no masked work)."""
    th = w.B * w.T * w.H
    return th * (w.chunk * 2 * w.D + 4 * w.D * w.D) + th * (5 * w.chunk * w.D + 8 * w.D * w.D)


def train_compulsory_bytes(w):
    """The step's compulsory HBM bytes: the forward reads q, k, v, log_f and
    writes y; the backward reads q, k, v, log_f, dy and writes dq, dk, dv,
    dlog_f (14 bf16 token tensors)."""
    return 14 * w.B * w.T * w.H * w.D * 2


def hgrn1_algorithmic_bytes(B, T, C):
    """Bytes per launch of the HGRN1 kernels, tied, bf16, segment states saved by
    the forward: tok = one [B,T,C] tensor, seg = one float per (b, segment of 32
    tokens, channel), grp = one float per (b, group of 8 segments, channel)."""
    S = (T + 31) // 32
    tok = B * T * C * 2
    seg = B * S * C * 4
    grp = B * ((S + 7) // 8) * C * 4
    return {
        "h1_summary": 2 * tok + 2 * seg + 2 * grp,             # v, log_f in; in-group prefixes, group totals out
        "h1_carry": 2 * grp + grp,                             # group totals in; group carries out
        "h1_final_fwd": 3 * tok + 2 * seg + grp + tok + seg,   # q, v, log_f, prefixes, carries in; y, states out
        "h1_summary_rev": 3 * tok + 2 * seg + 2 * grp,         # q, dy, log_f in
        "h1_carry_rev": 2 * grp + grp,
        "h1_final_bwd": 4 * tok + seg + 2 * seg + grp + 3 * tok,  # q, v, log_f, dy, states, suffixes, carries in;
                                                                  # dq, dv, dlog_f out
    }


def bench_hgrn1(torch, m, args, sets):
    """The HGRN1 elementwise recurrence on the training workload's tensors read
    as [B, T, C] (C = H d channels), tied, bf16: hgrn1_fwd (saving the segment
    states) then hgrn1_bwd; each call event-timed."""
    import synth
    w = synth.WORKLOADS["train_bf16"]
    B, T, C = w.B, w.T, w.H * w.D
    dev = sets[0]["q"].device
    st = torch.empty((B, (T + 31) // 32, C), dtype=torch.float32, device=dev)
    y = torch.empty((B, T, C), dtype=torch.bfloat16, device=dev)
    g = [torch.empty((B, T, C), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    wsf = torch.empty(int(m.lib().hgrn1_fwd_workspace_bytes(B, T, C, 1)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(int(m.lib().hgrn1_bwd_workspace_bytes(B, T, C, 1)), dtype=torch.uint8, device=dev)
    views = [{n: s[n].view(B, T, C) for n in ("q", "v", "log_f", "dy")} for s in sets]
    calls = lambda s: (
        lambda: m.hgrn1_fwd(s["q"], None, s["v"], s["log_f"], None, tied=True, want_ht=False, y=y, states=st,
                            ws=wsf),
        lambda: m.hgrn1_bwd(s["q"], None, s["v"], s["log_f"], s["dy"], None, None, st, tied=True, want_dh0=False,
                            dq=g[0], dv=g[1], dlog_f=g[2], ws=wsb))
    labels = ("hgrn1_fwd", "hgrn1_bwd")

    def step(i, timer=None):
        for label, call in zip(labels, calls(views[i % len(views)])):
            t = timer.start(label) if timer else None
            call()
            if timer:
                timer.stop(t)

    settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the step time with nothing between the launches, then the per-call times
    # from a second pass with events around each call
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    timer = KernelTimer(torch)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, timer)
    torch.cuda.synchronize()
    kms = {label: timer.mean_ms(label) for label in labels}
    log("timed (hgrn1): %.3f ms/step (%s)" % (ms, ", ".join("%s %.3f ms" % kv for kv in kms.items())))
    alg = hgrn1_algorithmic_bytes(B, T, C)
    tok = B * T * C * 2
    return {"workload": "hgrn1_bf16: B8 T4096 C2048 (the training tensors read as [B, T, C]), tied, "
                        "fwd(states)+bwd", "value": B * T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "calls_ms": kms, "algorithmic_bytes_step": sum(alg.values()),
            "compulsory_bytes_step": 11 * tok,
            "GBps_step": sum(alg.values()) / (ms * 1e-3) / 1e9}


def bench_train(torch, m, args, sets, mode="untied"):
    """Times `args.steps` training steps (after `args.warmup` untimed ones) with
    untied gates (k an input), tied gates (k = 1 - f formed in the kernels; the
    four single launches are timed), or the gate formed from its pre-activation
    (the two composite calls are timed)."""
    import synth
    w = synth.WORKLOADS["train_bf16"]
    B, T, H, D, C = w.B, w.T, w.H, w.D, w.chunk
    dev = sets[0]["q"].device
    y = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    states = torch.empty(m.states_shape(B, T, H, D, C), dtype=torch.bfloat16, device=dev)
    lam = torch.empty(m.adjoints_shape(B, T, H, D, C), dtype=torch.bfloat16, device=dev)
    grads = [torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    kernels = {"untied": TRAIN_KERNELS, "tied": TIED_KERNELS, "gate": GATE_CALLS, "scalar": SCALAR_CALLS}[mode]
    lbd = dlbd = ws = dla = None   # gate mode: lower bound [H, D], its gradient; the workspace; dlog_a
    if mode == "scalar":
        for s_ in sets:
            s_.setdefault("log_a", s_["log_f"][..., 0].contiguous())
        dla = torch.empty((B, T, H), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(int(m.lib().hgrn2_bwd_workspace_bytes(B, T, H, D, D, C, 1, 1)), dtype=torch.uint8,
                         device=dev)
    if mode == "gate":
        import synth
        lbd = torch.from_numpy(synth.lower_bounds(H, D, 0.3, 0.25, seed=11)).to(dev)
        dlbd = torch.empty_like(lbd)
        ws = torch.empty(int(m.lib().hgrn2_bwd_gate_workspace_bytes(B, T, H, D, D, C, 1, 1)),
                         dtype=torch.uint8, device=dev)

    def calls_untied(s):
        return (
            lambda: m.fwd(s["q"], s["k"], s["v"], s["log_f"], None, chunk=C, want_ht=False, want_y=False,
                          states=states),
            lambda: m.fwd_chunk(s["q"], s["k"], s["v"], s["log_f"], states, chunk=C, y=y),
            lambda: m.bwd_adjoint(s["q"], s["log_f"], s["dy"], None, chunk=C, adjoints=lam),
            lambda: m.bwd_chunk(s["q"], s["k"], s["v"], s["log_f"], s["dy"], states, lam, chunk=C,
                                dq=grads[0], dk=grads[1], dv=grads[2], dlog_f=grads[3]),
        )

    def calls_tied(s):
        return (
            lambda: m.fwd_tied(s["q"], s["v"], s["log_f"], None, chunk=C, want_ht=False, want_y=False,
                               states=states),
            lambda: m.fwd_chunk_tied(s["q"], s["v"], s["log_f"], states, chunk=C, y=y),
            lambda: m.bwd_adjoint(s["q"], s["log_f"], s["dy"], None, chunk=C, adjoints=lam),
            lambda: m.bwd_chunk_tied(s["q"], s["v"], s["log_f"], s["dy"], states, lam, chunk=C,
                                     dq=grads[0], dv=grads[2], dlog_f=grads[3]),
        )

    def calls_gate(s):
        return (
            lambda: m.fwd_gate(s["q"], s["v"], s["z"], lbd, None, chunk=C, want_ht=False, states=states),
            lambda: m.bwd_gate(s["q"], s["v"], s["z"], lbd, s["dy"], None, None, states, chunk=C, want_dh0=False,
                               dq=grads[0], dv=grads[2], dz=grads[3], dlower_bound=dlbd, ws=ws),
        )

    def calls_scalar(s):
        return (
            lambda: m.fwd_scalar(s["q"], s["k"], s["v"], s["log_a"], None, chunk=C, want_ht=False, states=states),
            lambda: m.bwd_scalar(s["q"], s["k"], s["v"], s["log_a"], s["dy"], None, None, states, chunk=C,
                                 want_dh0=False, dq=grads[0], dk=grads[1], dv=grads[2], dlog_a=dla, ws=ws),
        )

    pick = {"untied": calls_untied, "tied": calls_tied, "gate": calls_gate, "scalar": calls_scalar}[mode]

    def step(i, timer=None):
        s = sets[i % len(sets)]
        st = timer.start("step") if timer else None
        for (label, _), call in zip(kernels, pick(s)):
            t = timer.start(label) if timer else None
            call()
            if timer:
                timer.stop(t)
        if timer:
            timer.stop(st)

    settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("warmup done (%s)" % mode)
    # timed region: exactly `steps` steps, bracketed by synchronisation, with
    # one event at each step boundary and nothing between a step's launches
    # (the per-step times give the median and the minimum)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    step_stats = {"mean": ms, "median": per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] +
                                                                                    per[len(per) // 2]),
                  "min": per[0], "n": args.steps}
    # the same steps again with events around each launch (on the stream the
    # kernels run on), for the per-kernel times; the events themselves sit
    # between the launches, so this pass's step time is reported beside
    timer = KernelTimer(torch)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i, timer)
    t1.record()
    torch.cuda.synchronize()
    ms_inst = t0.elapsed_time(t1) / args.steps
    kms = {label: timer.mean_ms(label) for label, _ in kernels}
    kstats = {label: timer.stats(label) for label, _ in kernels}
    log("timed (%s): %.3f ms/step; with events around each launch %.3f ms/step (%s)"
        % (mode, ms, ms_inst, ", ".join("%s %.3f ms" % kv for kv in kms.items())))
    out = None
    if mode == "untied":
        # after the timed region: one more step on the first input set, whose
        # outputs the CPU oracle checks
        step(0)
        torch.cuda.synchronize()
        out = {"y": y.clone(), "dq": grads[0].clone(), "dk": grads[1].clone(), "dv": grads[2].clone(),
               "dlog_f": grads[3].clone()}
    return dict(w=w, ms=ms, kernel_ms=kms, kernel_stats=kstats, step_stats=step_stats, ms_instrumented=ms_inst,
                host=sets[0]["host"], out=out)


def bench_decode(torch, m, args):
    import synth
    from tests.gpu_util import to_dev
    w = synth.WORKLOADS["decode_f32"]
    d = synth.generate_decode(w)
    q, k, v, lf = (to_dev(d[n], "f32") for n in ("q", "k", "v", "log_f"))
    S0 = to_dev(d["state"], "f32")
    states = [S0.clone(), S0.clone()]  # two resident states so the 256 MB cache never holds the one in use
    y = torch.empty_like(q)
    settle(torch, lambda i: m.decode_step(q, k, v, lf, states[i % 2], y=y))
    for i in range(5):
        m.decode_step(q, k, v, lf, states[i % 2], y=y)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    timer = KernelTimer(torch)
    a.record()
    for i in range(args.decode_steps):
        t = timer.start("decode")
        m.decode_step(q, k, v, lf, states[i % 2], y=y)
        timer.stop(t)
    b.record()
    torch.cuda.synchronize()
    ms_loop = a.elapsed_time(b) / args.decode_steps
    stats = timer.stats("decode")
    ms = stats["median"]   # one launch, between the events recorded around it on its stream
    state_bytes = w.B * w.H * w.D * w.D * 4
    vec_bytes = 5 * w.B * w.H * w.D * 4          # q, k, v, log_f read; y written
    gbs = (2 * state_bytes + vec_bytes) / (ms * 1e-3) / 1e9
    log("decode: median %.3f ms/launch (%.3f ms per step of the loop), %.1f GB/s" % (ms, ms_loop, gbs))
    return dict(ms=ms, ms_loop=ms_loop, gbs=gbs, bytes=2 * state_bytes + vec_bytes, stats=stats)


def _parity(got: dict, refs: dict, layouts: dict, tol: float):
    """errors() of each GPU output against the oracle's (every slice, row and
    element; tests/gpu_util.py), and whether all are within `tol`."""
    from tests.gpu_util import errors, to_host64, worst
    out = {}
    for n, r in refs.items():
        out[n] = errors(to_host64(got[n]), r, layouts.get(n, "token"))
    ok = all(worst(e) <= tol for e in out.values())
    return {"tolerance": tol, "pass": bool(ok), "errors": out}


def cpu_baseline(res, min_seconds=10.0, max_reps=8):
    """The float64 oracle on the host cores over the same training batch (all
    (b, h) sequences, all tokens, forward + backward), repeated until about
    `min_seconds` of CPU time has passed; the rate is the mean over
    repetitions.  The first repetition's outputs are compared with the GPU's
    outputs for the same batch (the first input set, lower bound 0)."""
    import oracle
    import synth
    w = res["w"]
    d = res["host"]
    threads = oracle.threads()
    x = {n: synth.to_f64(d[n], "bf16") for n in ("q", "k", "v", "log_f", "dy")}
    reps, t0, first = 0, time.time(), None
    while reps < max_reps and (reps == 0 or time.time() - t0 < min_seconds):
        yr, _ = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], None)
        gr = oracle.backward(x["q"], x["k"], x["v"], x["log_f"], x["dy"], None, None)
        if first is None:
            first = {"y": yr, "dq": gr[0], "dk": gr[1], "dv": gr[2], "dlog_f": gr[3]}
        del yr, gr
        reps += 1
    dt = time.time() - t0
    tokens_per_s = reps * w.B * w.T / dt
    log("cpu oracle: %d x the B%d T%d batch in %.2f s on %d threads" % (reps, w.B, w.T, dt, threads))
    out = {"value": tokens_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "the whole B%d H%d T%d batch (lower bound 0), fwd+bwd in float64, %d repetitions (%.1f s)"
                     % (w.B, w.H, w.T, reps, dt)}
    if res.get("out") is not None:
        del x
        out["parity"] = _parity(res["out"], first, {}, 2e-2)
        out["parity"]["compared"] = "y, dq, dk, dv, dlog_f of all %d (b, h) sequences" % (w.B * w.H)
        log("parity vs oracle: %s" % ("pass" if out["parity"]["pass"] else "FAIL"))
    return out


def bench_fwd_only(torch, m, args, name, cpu=True):
    """A forward-only workload (hgrn2_fwd: y and the final state, no states
    kept for a backward), one call per step.  Before each call a 512 MiB read
    evicts the inputs from L2 and the 256 MB last-level cache; events bracket
    the call alone.  The eviction only reads: a fill would leave its lines
    dirty in the last-level cache, and their write-back would land inside the
    timed call (measured: +60 to +85 us on the B1 H32 T32768 call).  The oracle then runs the same batch on the host cores and
    its outputs are compared with the GPU's."""
    import synth
    from tests.gpu_util import to_dev
    w = synth.WORKLOADS[name]
    d = synth.generate(w)
    B, T, H, D, C = w.B, w.T, w.H, w.D, w.chunk
    q, k, v, lf = (to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f"))
    h0 = to_dev(d["h0"], "f32")
    dev = q.device
    y = torch.empty_like(q)
    ht = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(int(m.lib().hgrn2_fwd_workspace_bytes(B, T, H, D, D, C, 1, 0)), dtype=torch.uint8, device=dev)
    flush = torch.ones(1 << 27, dtype=torch.float32, device=dev)   # 512 MiB, read before each call

    def call():
        m.fwd(q, k, v, lf, h0, chunk=C, y=y, ht=ht, ws=ws)

    def evicted_call(i):
        flush.sum()
        call()

    settle(torch, evicted_call)   # the same eviction as the timed calls
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    timer = KernelTimer(torch)
    for i in range(args.steps):
        evict = flush.sum()
        t = timer.start("call")
        call()
        timer.stop(t)
    torch.cuda.synchronize()
    del evict
    st = timer.stats("call")
    tok = B * T * H * D * 2
    sb = B * H * D * D * 4
    comp = 5 * tok + sb + (sb if h0 is not None else 0)   # q, k, v, log_f in, y out; ht out; h0 in
    flop = B * T * H * (C * 2 * D + 4 * D * D)
    log("timed (%s): median %.3f ms, min %.3f ms" % (name, st["median"], st["min"]))
    res = {"workload": "%s: B%d H%d T%d d%d chunk%d bf16, hgrn2_fwd (y and the final state)%s"
                       % (name, B, H, T, D, C, ", float32 initial state" if h0 is not None else ""),
           "value": B * T / (st["median"] * 1e-3), "unit": "tokens/s", "ms": st,
           "compulsory_bytes": comp, "GBps": comp / (st["median"] * 1e-3) / 1e9,
           "frac_hbm": comp / (st["median"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "mfma_frac": flop / (st["median"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)}
    if cpu:
        import oracle
        x = {n: synth.to_f64(d[n], "bf16") for n in ("q", "k", "v", "log_f")}
        h064 = None if d["h0"] is None else d["h0"].astype(np.float64)
        t0 = time.time()
        yr, htr = oracle.forward(x["q"], x["k"], x["v"], x["log_f"], h064)
        dt = time.time() - t0
        res["cpu_oracle"] = {"value": B * T / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
                             "sample": "the whole batch, forward in float64, one repetition (%.1f s)" % dt}
        del x
        res["parity"] = _parity({"y": y, "ht": ht}, {"y": yr, "ht": htr}, {"ht": "state"}, 2e-2)
        log("%s parity vs oracle: %s" % (name, "pass" if res["parity"]["pass"] else "FAIL"))
    return res


def _csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    n = name.split("(")[0]
    return n.replace("void ", "").replace("hgrn2::", "")


def summarize(trace_dir, fetch_dir, write_dir, mfma_dir=None):
    """profiles/ summaries from the csv output of TRACE_CMD, the two PMC_CMD runs
    and (optionally) the MFMA_CMD run."""
    digest = kernel_source_digest()
    os.makedirs(PROFILES, exist_ok=True)
    # kernel-trace statistics
    rows = _csv(os.path.join(trace_dir, "run_kernel_stats.csv"))
    out = ["rocprofv3 kernel-trace statistics, HGRN2 training step (B8 H16 T4096 d128 bf16 chunk64)",
           "and decode step (B256 H16 d128 fp32 state)",
           "command: " + TRACE_CMD, "source_digest: " + digest, "",
           "%-52s %6s %12s %10s %10s %10s %6s" % ("kernel", "calls", "total_us", "avg_us",
                                                    "min_us", "max_us", "pct")]
    _w = __import__("synth").WORKLOADS["train_bf16"]
    alg = train_algorithmic_bytes(_w)
    alg.update(hgrn1_algorithmic_bytes(_w.B, _w.T, _w.H * _w.D))
    rates = []
    for r in rows:
        out.append("%-52s %6d %12.1f %10.1f %10.1f %10.1f %6.2f" % (
            _short(r["Name"])[:52], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["Percentage"])))
        label = kernel_label(r["Name"])
        if label in alg:
            gbs = alg[label] / float(r["AverageNs"])
            rates.append("  %-9s algorithmic %7.1f MB per launch / average %8.1f us = %7.1f GB/s "
                         "(%.1f%% of %.0f GB/s)" % (label, alg[label] / 1e6, float(r["AverageNs"]) / 1e3,
                                                   gbs, 100 * gbs / HBM_PEAK_GBS, HBM_PEAK_GBS))
    out += [""] + rates
    kt = _csv(os.path.join(trace_dir, "run_kernel_trace.csv"))
    seen = set()
    out.append("")
    for r in kt:
        n = _short(r["Kernel_Name"])
        if n in seen or not n.startswith("hgrn2_"):
            continue
        seen.add(n)
        out.append("  %s: grid %s wg %s vgpr %s agpr %s sgpr %s lds %s scratch %s" % tuple(
            [n] + [r.get(c, "?") for c in ("Grid_Size_X", "Workgroup_Size_X", "VGPR_Count",
                                           "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size",
                                           "Scratch_Size")]))
    name = os.path.join(PROFILES, "hgrn2_kernels_train_bf16_B8H16T4096_decode_B256H16.txt")
    with open(name, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))

    # HBM traffic from FETCH_SIZE / WRITE_SIZE (KiB per dispatch)
    def per_kernel(d, ctr):
        acc = {}
        for r in _csv(os.path.join(d, "run_counter_collection.csv")):
            if r["Counter_Name"] == ctr:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "MulFunctor" in k and k in write]
    assert copy, "the counter runs need --calib-copy"
    f_fac = CALIB_BYTES / (fetch[copy[0]] * 1024)
    w_fac = CALIB_BYTES / (write[copy[0]] * 1024)
    out = ["HBM traffic per launch, HGRN2 training step (B8 H16 T4096 d128 bf16 chunk64)",
           "fetch command: " + PMC_CMD.format(ctr="FETCH_SIZE", dir="fetch"),
           "write command: " + PMC_CMD.format(ctr="WRITE_SIZE", dir="write"),
           "calibration: a 1 GiB elementwise pass (torch.mul, 1 GiB read, 1 GiB written) reads "
           "FETCH_SIZE %.0f KiB and WRITE_SIZE %.0f KiB" % (fetch[copy[0]], write[copy[0]]),
           "fetch_scale: %.4f" % f_fac, "write_scale: %.4f" % w_fac,
           "source_digest: " + digest, ""]
    for k in fetch:
        label = kernel_label(k)
        if label not in alg:
            continue
        fb, wb = fetch[k] * 1024 * f_fac, write[k] * 1024 * w_fac
        out.append("  %s (%s): read %.1f MB, written %.1f MB, total %.1f MB; algorithmic %.1f MB; "
                   "total / algorithmic = %.3f" % (_short(k), label, fb / 1e6, wb / 1e6, (fb + wb) / 1e6,
                                                   alg[label] / 1e6, (fb + wb) / alg[label]))
        out.append("traffic_bytes_per_launch %s: %.0f" % (label, fb + wb))
    with open(TRAFFIC_SUMMARY, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))
    if mfma_dir:
        summarize_mfma(mfma_dir, {kernel_label(r["Name"]): float(r["AverageNs"]) for r in rows}, digest)


def seg_plan(B, T, H, chunk, want_y=True, units=512):
    """The segment plan hgrn2_fwd uses without stored states: P segments of G
    chunks per (b, h), NSEG of them summarised (P - 1 when y is written), for
    about `units` walking workgroups (512 for bf16 at d 128: two per compute
    unit, unless that leaves segments of fewer than 8 chunks; then 256)."""
    BH, N = B * H, -(-T // chunk)

    def plan(u):
        pt = min(N, max(1, -(-u // BH)))
        G = -(-N // pt)
        return -(-N // G), G

    P, G = plan(units)
    if units > 256 and P > 1 and G < 8:
        P, G = plan(256)
    return P, G, (P - 1 if want_y else P)


def fwd_leg_bytes(w):
    """Algorithmic bytes per launch of the segmented forward's kernels (bf16
    tokens, float32 states): every tensor each launch reads or writes, once."""
    tok = w.B * w.T * w.H * w.D * 2
    BH, S = w.B * w.H, w.D * w.D * 4
    P, G, NSEG = seg_plan(w.B, w.T, w.H, w.chunk)
    N = -(-w.T // w.chunk)
    frac = min(1.0, NSEG * G / N)                     # the summarised share of each sequence
    h0 = BH * S if w.h0std > 0 else 0
    return {"seg_scan": 3 * tok * frac + BH * NSEG * (S + w.D * 4),      # k, v, log f in; end states, totals out
            "seg_carry": h0 + BH * NSEG * (S + w.D * 4) + BH * (NSEG + 1) * S,
            "seg_fwd": 5 * tok + BH * (P if P > 1 else 0) * S + (h0 if P == 1 else 0) + BH * S}, \
        5 * tok + h0 + BH * S, (P, G, NSEG)


def summarize_fwd(leg, trace_dir, fetch_dir, write_dir):
    """profiles/ summary of one forward-only leg: kernel-trace statistics, the
    algorithmic bytes of each launch, and the HBM bytes the counters saw."""
    import synth
    w = synth.WORKLOADS[leg]
    digest = kernel_source_digest()
    alg, comp, (P, G, NSEG) = fwd_leg_bytes(w)
    rows = _csv(os.path.join(trace_dir, "run_kernel_stats.csv"))

    def per_kernel(d, ctr):
        acc = {}
        for r in _csv(os.path.join(d, "run_counter_collection.csv")):
            if r["Counter_Name"] == ctr:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "MulFunctor" in k and k in write]
    assert copy, "the counter runs need --calib-copy"
    f_fac = CALIB_BYTES / (fetch[copy[0]] * 1024)
    w_fac = CALIB_BYTES / (write[copy[0]] * 1024)
    shape = "B%d H%d T%d d%d chunk%d bf16" % (w.B, w.H, w.T, w.D, w.chunk)
    out = ["rocprofv3 kernel trace and HBM traffic, %s: hgrn2_fwd (y and the final state, no stored "
           "states), %s" % (leg, shape),
           "segment plan: P = %d segments of G = %d chunks per (b, h), %d summarised" % (P, G, NSEG),
           "trace command: " + FWD_TRACE_CMD.format(leg=leg),
           "fetch command: " + FWD_PMC_CMD.format(ctr="FETCH_SIZE", dir="fetch", leg=leg),
           "write command: " + FWD_PMC_CMD.format(ctr="WRITE_SIZE", dir="write", leg=leg),
           "fetch_scale: %.4f (a 1 GiB torch.mul reads FETCH_SIZE %.0f KiB)" % (f_fac, fetch[copy[0]]),
           "write_scale: %.4f (and writes WRITE_SIZE %.0f KiB)" % (w_fac, write[copy[0]]),
           "source_digest: " + digest, "",
           "%-52s %6s %10s %10s %10s %10s %10s %8s" % ("kernel", "calls", "avg_us", "min_us", "alg_MB",
                                                     "hbm_MB", "GB/s_alg", "hbm/alg")]
    tot_us = tot_hbm = tot_alg = 0.0
    for r in rows:
        label = kernel_label(r["Name"])
        if label is None:
            continue
        base = label.split("_tied")[0].split("_gate")[0].split("_scalar")[0]
        a = alg.get(base)
        k = r["Name"]
        hb = None
        if k in fetch and k in write:
            hb = fetch[k] * 1024 * f_fac + write[k] * 1024 * w_fac
        avg = float(r["AverageNs"]) / 1e3
        out.append("%-52s %6d %10.1f %10.1f %10.1f %10s %10.1f %8s" % (
            _short(k)[:52], int(r["Calls"]), avg, float(r["MinNs"]) / 1e3, (a or 0) / 1e6,
            "%.1f" % (hb / 1e6) if hb is not None else "-", (a or 0) / (avg * 1e3),
            "%.3f" % (hb / a) if (hb is not None and a) else "-"))
        tot_us += avg
        tot_alg += a or 0
        tot_hbm += hb or 0
    out += ["",
            "per call: %.1f us of kernels; algorithmic %.1f MB, counted %.1f MB, compulsory %.1f MB "
            "(q, k, v, log f in, y out, h0 in, ht out); counted / compulsory = %.3f"
            % (tot_us, tot_alg / 1e6, tot_hbm / 1e6, comp / 1e6, tot_hbm / comp)]
    name = os.path.join(PROFILES, "hgrn2_kernels_%s_%s.txt" % (leg, shape.replace(" ", "_")))
    with open(name, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_mfma(mfma_dir, avg_ns, digest):
    """Matrix-core work the counters saw per launch: executed bf16 MFMA flops
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), the rate over the kernel-trace average
    duration against the dense bf16 peak, and MfmaUtil (busy share of the
    matrix cores while the kernel ran)."""
    acc = {}
    for r in _csv(os.path.join(mfma_dir, "run_counter_collection.csv")):
        label = kernel_label(r["Kernel_Name"])
        if label is None or label.startswith("decode"):
            continue
        acc.setdefault((label, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    w = __import__("synth").WORKLOADS["train_bf16"]
    th = w.B * w.T * w.H
    alg_flop = {"scan": th * 2 * w.D * w.D, "cfwd": th * (w.chunk * 2 * w.D + 2 * w.D * w.D),
                "scan_rev": th * 2 * w.D * w.D, "cbwd": th * (5 * w.chunk * w.D + 6 * w.D * w.D)}
    for label in ("scan", "cfwd", "cbwd", "scan_rev"):   # the gate modes change no contraction
        for sfx in ("_tied", "_gate", "_scalar"):
            alg_flop[label + sfx] = alg_flop[label]
    out = ["Matrix-core work per launch, HGRN2 training step (B8 H16 T4096 d128 bf16 chunk64)",
           "command: " + MFMA_CMD, "durations: the kernel-trace averages of " + TRACE_CMD,
           "peak: %.0f TFLOP/s dense bf16" % BF16_PEAK_TFLOPS, "source_digest: " + digest, "",
           "%-9s %14s %14s %10s %10s %10s" % ("kernel", "executed_GFLOP", "algorithmic", "TFLOP/s",
                                              "of_peak", "MfmaUtil")]
    for label in list(dict(TRAIN_KERNELS + TIED_KERNELS)) + ["scan_gate", "cfwd_gate", "scan_rev_gate", "cbwd_gate",
                                                          "scan_scalar", "cfwd_scalar", "scan_rev_scalar",
                                                          "cbwd_scalar"]:
        mops = acc.get((label, "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
        util = acc.get((label, "MfmaUtil"))
        if not mops or label not in avg_ns:
            continue
        flop = sum(mops) / len(mops) * 512
        rate = flop / (avg_ns[label] * 1e-9) / 1e12
        out.append("%-9s %14.2f %14.2f %10.1f %9.2f%% %9.2f%%" % (
            label, flop / 1e9, alg_flop[label] / 1e9, rate, 100 * rate / BF16_PEAK_TFLOPS,
            sum(util) / len(util) if util else float("nan")))
    with open(MFMA_SUMMARY, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def main():
    args = parse()
    if args.summarize:
        summarize(*args.summarize)
        return
    if args.summarize_fwd:
        summarize_fwd(*args.summarize_fwd)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_attention_hgrn2_amd as m
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    m.lib()
    out = {"metric": "fwd+bwd tokens/s (H16,d128,T4096)", "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "settle_s": SETTLE_S,
           "settle": "each leg first runs its own step untimed for settle_s seconds, then its warmup steps: "
                     "the GPU's clocks ramp up over the first tens of milliseconds of sustained work"}
    res = None
    dres = None
    if args.only in ("train", "all"):
        import synth
        sets = make_train_sets(torch, synth.WORKLOADS["train_bf16"], synth.TRAIN_LAMBDAS)
        res = bench_train(torch, m, args, sets)
        tres = bench_train(torch, m, args, sets, mode="tied")
        gres = bench_train(torch, m, args, sets, mode="gate")
        sres = bench_train(torch, m, args, sets, mode="scalar")
        h1res = bench_hgrn1(torch, m, args, sets)
        del sets
        w = res["w"]
        tokens = w.B * w.T
        out["value"] = tokens / (res["ms"] * 1e-3)
        out["ms_per_step"] = res["ms"]
        out["ms_per_step_stats"] = res["step_stats"]
        out["ms_per_step_with_kernel_events"] = res["ms_instrumented"]
        out["config"] = {"workload": "train_bf16: B8 H16 T4096 d128 chunk64 fwd(states)+bwd",
                         "global_batch": w.B, "seq_len": w.T, "heads": w.H, "head_dim": w.D,
                         "chunk": w.chunk, "parallelism": "none (1 GPU)"}
        alg = train_algorithmic_bytes(w)
        abi = train_abi_bytes(w)
        kms = res["kernel_ms"]
        step_flop = train_step_flop(w)
        comp = train_compulsory_bytes(w)
        dom = max(kms, key=kms.get)
        ach = abi[dom] / (kms[dom] * 1e-3) / 1e9
        kname = dict(TRAIN_KERNELS)[dom]
        out["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(dom),
                           "ms": kms[dom], "ms_stats": res["kernel_stats"][dom],
                           "algorithmic_bytes": abi[dom],
                           "algorithmic_bytes_counts": "the C-ABI tensors the launch reads or writes "
                                                       "(q, k, v, log_f, dy, dq, dk, dv, dlog_f) and the "
                                                       "chunk-boundary states",
                           "design_bytes": alg[dom],
                           "design_bytes_counts": "every byte the launch moves, the adjoint workspace included",
                           "design_frac": alg[dom] / (kms[dom] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "source_digest": kernel_source_digest()}
        step_s = res["ms"] * 1e-3
        out["step_roofline"] = {
            "compulsory_bytes": comp, "compulsory_bytes_counts": "14 bf16 token tensors: the forward reads "
                                                                 "q, k, v, log_f and writes y; the backward "
                                                                 "reads q, k, v, log_f, dy and writes the four "
                                                                 "gradients",
            "hbm_frac": comp / step_s / 1e9 / HBM_PEAK_GBS,
            "algorithmic_flop": step_flop,
            "mfma_frac": step_flop / step_s / (BF16_PEAK_TFLOPS * 1e12),
            "binding_frac": max(step_flop / (BF16_PEAK_TFLOPS * 1e12), comp / (HBM_PEAK_GBS * 1e9)) / step_s,
            "moved_bytes": sum(alg[k_] for k_, _ in TRAIN_KERNELS),
            # at 100% of HBM peak on the compulsory bytes, the MFMA fraction could be at most this
            "mfma_frac_cap_at_hbm_peak": (step_flop / (BF16_PEAK_TFLOPS * 1e12)) / (comp / (HBM_PEAK_GBS * 1e9))}
        out["kernels"] = {label: {"kernel": kn, "ms": kms[label], "ms_stats": res["kernel_stats"][label],
                                  "bytes": abi[label], "design_bytes": alg[label],
                                  "GBps": abi[label] / kms[label] / 1e6,
                                  "frac_hbm": abi[label] / kms[label] / 1e6 / HBM_PEAK_GBS}
                          for label, kn in TRAIN_KERNELS}
        out["mfma_frac_step"] = out["step_roofline"]["mfma_frac"]
        tk = tres["kernel_ms"]
        out["tied"] = {"workload": "train_bf16 with tied gates (k = 1 - f): fwd(states)+bwd, total dlog_f",
                       "value": tokens / (tres["ms"] * 1e-3), "unit": "tokens/s", "ms_per_step": tres["ms"],
                       "ms_per_step_stats": tres["step_stats"],
                       "ms_per_step_with_kernel_events": tres["ms_instrumented"],
                       "kernels": {label: {"kernel": kn, "ms": tk[label], "ms_stats": tres["kernel_stats"][label],
                                           "bytes": abi[label], "design_bytes": alg[label],
                                           "GBps": abi[label] / tk[label] / 1e6,
                                           "frac_hbm": abi[label] / tk[label] / 1e6 / HBM_PEAK_GBS}
                                   for label, kn in TIED_KERNELS}}
        gk = gres["kernel_ms"]
        out["gate"] = {"workload": "train_bf16 with the gate formed from its pre-activation z and a lower bound "
                                   "[H, D] (f = lb + (1 - lb) sigmoid(z), k = 1 - f): fwd(states)+bwd, dz and dlb",
                       "value": tokens / (gres["ms"] * 1e-3), "unit": "tokens/s", "ms_per_step": gres["ms"],
                       "ms_per_step_stats": gres["step_stats"],
                       "ms_per_step_with_kernel_events": gres["ms_instrumented"],
                       "calls_ms": {label: gk[label] for label, _ in GATE_CALLS}}
        sk_ = sres["kernel_ms"]
        out["scalar"] = {"workload": "train_bf16 with one decay per head (log_a [B,T,H] = the first channel's "
                                     "log f): fwd(states)+bwd, dlog_a",
                         "value": tokens / (sres["ms"] * 1e-3), "unit": "tokens/s", "ms_per_step": sres["ms"],
                         "ms_per_step_stats": sres["step_stats"],
                         "ms_per_step_with_kernel_events": sres["ms_instrumented"],
                         "calls_ms": {label: sk_[label] for label, _ in SCALAR_CALLS}}
        out["hgrn1"] = h1res
    if args.only in ("decode", "all"):
        dres = bench_decode(torch, m, args)
        out["decode"] = {"workload": "decode_f32: B256 H16 d128, float32 state", "ms": dres["ms"],
                         "ms_is": "the median of per-launch event times", "ms_stats": dres["stats"],
                         "ms_loop": dres["ms_loop"], "GBps": dres["gbs"], "frac_hbm": dres["gbs"] / HBM_PEAK_GBS,
                         "bytes": dres["bytes"]}
        if res is None:
            out["value"] = dres["gbs"]
            out["metric"] = "decode-step HBM GB/s"
            out["unit"] = "GB/s"
            out["ms_per_step"] = dres["ms"]
            out["config"] = {"workload": "decode_f32: B256 H16 d128"}
    for name in ("fwd_bf16", "long_bf16"):
        if args.only in (name, "all"):
            out[name] = bench_fwd_only(torch, m, args, name, cpu=not args.no_cpu)
            if res is None and dres is None and args.only == name:
                out["metric"] = "fwd tokens/s (%s)" % name
                out["value"] = out[name]["value"]
                out["ms_per_step"] = out[name]["ms"]["median"]
                out["config"] = {"workload": out[name]["workload"]}
    if res is not None:
        t = {"train_mfma_frac": {"want": 0.40, "got": out["step_roofline"]["mfma_frac"],
                                 "met": out["step_roofline"]["mfma_frac"] >= 0.40,
                                 "cap_at_hbm_peak": out["step_roofline"]["mfma_frac_cap_at_hbm_peak"],
                                 "why": "the step is bound by HBM bytes: even its compulsory bytes at 100% of "
                                        "HBM peak leave the matrix cores below the wanted fraction"}}
        if dres is not None:
            fr = dres["gbs"] / HBM_PEAK_GBS
            t["decode_hbm_frac"] = {"want": 0.70, "got": fr, "met": fr >= 0.70}
        out["target"] = t
    if args.calib_copy:
        # torch's elementwise multiply: a grid over every XCD reading 1 GiB and
        # writing 1 GiB (the runtime's copy kernel has been seen to spread over
        # fewer XCDs, which skews per-XCD counters)
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
    if res is not None and not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(res)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
