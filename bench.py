"""Benchmark of the HGRN2 recurrence hot path on one MI355X.

One step = one training pass over one batch of the H16 d128 T4096 workload
(B8 H16 T4096, d_k = d_v = 128, bf16, chunk 64): hgrn2_fwd (saving the
chunk-boundary states) followed by hgrn2_bwd.  Three resident input sets
(forget-gate lower bound 0, 0.3, 0.6) are rotated across steps.  The decode
step (B256 H16 d128, float32 state) is timed as well and reported in HBM
GB/s.  Inputs are seeded synthetic data generated on the host and copied to
HBM before timing.

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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--decode-steps", type=int, default=50)
    p.add_argument("--only", choices=["train", "decode", "all"], default="all")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (calibrates profiler byte counters)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_train_sets(torch, w, lams):
    import synth
    from tests.gpu_util import to_dev
    sets = []
    for i, lam in enumerate(lams):
        d = synth.generate(w, lam=lam, seed=w.seed + 10 * i)
        sets.append({n: to_dev(d[n], "bf16") for n in ("q", "k", "v", "log_f", "dy")})
        sets[-1]["host"] = d if i == 0 else None
        log("inputs ready: lambda=%.1f" % lam)
    return sets


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

    def mean_ms(self, name):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs[name]]))


def bench_train(torch, m, args):
    import synth
    w = synth.WORKLOADS["train_bf16"]
    B, T, H, D, C = w.B, w.T, w.H, w.D, w.chunk
    sets = make_train_sets(torch, w, synth.TRAIN_LAMBDAS)
    dev = sets[0]["q"].device
    y = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    states = torch.empty(m.states_shape(B, T, H, D, C), dtype=torch.bfloat16, device=dev)
    grads = [torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev) for _ in range(4)]

    def step(i, timer=None):
        s = sets[i % len(sets)]
        t = timer.start("fwd") if timer else None
        m.fwd(s["q"], s["k"], s["v"], s["log_f"], None, chunk=C, want_ht=False,
              y=y, states=states)
        if timer:
            timer.stop(t)
            t = timer.start("bwd")
        m.bwd(s["q"], s["k"], s["v"], s["log_f"], s["dy"], None, None, states, chunk=C,
              want_dh0=False, dq=grads[0], dk=grads[1], dv=grads[2], dlog_f=grads[3])
        if timer:
            timer.stop(t)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("warmup done")
    # timed region: exactly `steps` steps, bracketed by synchronisation
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    log("timed: %.3f ms/step" % ms)
    # per-kernel durations (separate pass with events between the two launches)
    timer = KernelTimer(torch)
    for i in range(args.steps):
        step(i, timer)
    torch.cuda.synchronize()
    fwd_ms, bwd_ms = timer.mean_ms("fwd"), timer.mean_ms("bwd")
    log("fwd %.3f ms, bwd %.3f ms" % (fwd_ms, bwd_ms))
    return dict(w=w, ms=ms, fwd_ms=fwd_ms, bwd_ms=bwd_ms, host=sets[0]["host"])


def bench_decode(torch, m, args):
    import synth
    from tests.gpu_util import to_dev
    w = synth.WORKLOADS["decode_f32"]
    d = synth.generate_decode(w)
    q, k, v, lf = (to_dev(d[n], "f32") for n in ("q", "k", "v", "log_f"))
    S0 = to_dev(d["state"], "f32")
    states = [S0.clone(), S0.clone()]  # two resident states so the 256 MB cache never holds the one in use
    y = torch.empty_like(q)
    for i in range(5):
        m.decode_step(q, k, v, lf, states[i % 2], y=y)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.decode_steps):
        m.decode_step(q, k, v, lf, states[i % 2], y=y)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.decode_steps
    state_bytes = w.B * w.H * w.D * w.D * 4
    vec_bytes = 5 * w.B * w.H * w.D * 4          # q, k, v, log_f read; y written
    gbs = (2 * state_bytes + vec_bytes) / (ms * 1e-3) / 1e9
    log("decode: %.3f ms/step, %.1f GB/s" % (ms, gbs))
    return dict(ms=ms, gbs=gbs, bytes=2 * state_bytes + vec_bytes)


def cpu_baseline(res):
    """The float64 oracle on a bounded sample of the same workload: whole
    sequences (all T tokens) of some (b, h) pairs, forward + backward."""
    import oracle
    import synth
    w = res["w"]
    d = res["host"]
    threads = oracle.threads()
    nslice = w.B * w.H                     # the whole batch: a few seconds of CPU time
    pairs = [(i // w.H, i % w.H) for i in range(nslice)]
    from tests.gpu_util import select_bh
    x = {n: synth.to_f64(d[n], "bf16") for n in ("q", "k", "v", "log_f", "dy")}
    sub = {n: select_bh(x[n], pairs) for n in x}
    t0 = time.time()
    oracle.forward(sub["q"], sub["k"], sub["v"], sub["log_f"], None)
    oracle.backward(sub["q"], sub["k"], sub["v"], sub["log_f"], sub["dy"], None, None)
    dt = time.time() - t0
    token_heads = nslice * w.T
    tokens_per_s = token_heads / w.H / dt
    log("cpu oracle: %d (b,h) sequences of T=%d in %.2f s on %d threads" % (nslice, w.T, dt, threads))
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d (b,h) sequences, all %d tokens each, fwd+bwd in float64 (%.1f s)"
                      % (nslice, w.B * w.H, w.T, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_attention_hgrn2_amd as m
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    m.lib()
    out = {"metric": "fwd+bwd tokens/s (H16,d128,T4096)", "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    res = None
    if args.only in ("train", "all"):
        res = bench_train(torch, m, args)
        w = res["w"]
        tokens = w.B * w.T
        out["value"] = tokens / (res["ms"] * 1e-3)
        out["ms_per_step"] = res["ms"]
        out["config"] = {"workload": "train_bf16: B8 H16 T4096 d128 chunk64 fwd(states)+bwd",
                         "global_batch": w.B, "seq_len": w.T, "heads": w.H, "head_dim": w.D,
                         "chunk": w.chunk, "parallelism": "none (1 GPU)"}
        tok = w.B * w.T * w.H * w.D * 2                 # one bf16 [B,T,H,D] tensor
        st = w.B * w.H * (w.T // w.chunk + 1) * w.D * w.D * 2   # bf16 chunk-boundary states
        fwd_bytes = 4 * tok + tok + st                  # q,k,v,log_f in; y, states out
        bwd_bytes = 5 * tok + st + 4 * tok              # q,k,v,log_f,dy,states in; 4 grads out
        th = w.B * w.T * w.H
        fwd_flop = th * (w.chunk * 2 * w.D + 4 * w.D * w.D)
        bwd_flop = th * (5 * w.chunk * w.D + 8 * w.D * w.D)
        dom = "bwd" if res["bwd_ms"] >= res["fwd_ms"] else "fwd"
        kms = res[dom + "_ms"]
        kbytes = bwd_bytes if dom == "bwd" else fwd_bytes
        ach = kbytes / (kms * 1e-3) / 1e9
        out["roofline"] = {"kernel": "hgrn2_%s_kernel" % dom, "bound": "hbm", "achieved": ach,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                           "traffic": None, "ms": kms, "algorithmic_bytes": kbytes}
        out["kernels"] = {
            "fwd": {"ms": res["fwd_ms"], "bytes": fwd_bytes, "GBps": fwd_bytes / res["fwd_ms"] / 1e6,
                    "TFLOPs": fwd_flop / res["fwd_ms"] / 1e9},
            "bwd": {"ms": res["bwd_ms"], "bytes": bwd_bytes, "GBps": bwd_bytes / res["bwd_ms"] / 1e6,
                    "TFLOPs": bwd_flop / res["bwd_ms"] / 1e9},
            "mfma_frac_step": (fwd_flop + bwd_flop) / (res["ms"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        }
    if args.only in ("decode", "all"):
        dres = bench_decode(torch, m, args)
        out["decode"] = {"workload": "decode_f32: B256 H16 d128, float32 state", "ms": dres["ms"],
                         "GBps": dres["gbs"], "frac_hbm": dres["gbs"] / HBM_PEAK_GBS,
                         "bytes": dres["bytes"]}
        if res is None:
            out["value"] = dres["gbs"]
            out["metric"] = "decode-step HBM GB/s"
            out["unit"] = "GB/s"
            out["ms_per_step"] = dres["ms"]
            out["config"] = {"workload": "decode_f32: B256 H16 d128"}
    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if res is not None and not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(res)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
