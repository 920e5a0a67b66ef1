"""Host logic of bench.py, on the CPU: the refusal of more than one GPU, the
settle helper that runs before each leg's warmup, the byte accounting behind
the roofline figures, and the bench's mirror of the library's segment plan,
checked against the workspace the library sizes for that plan."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    import linear_attention_hgrn2_amd as m
    return m.lib()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_settle_runs_whole_batches_until_its_time_is_up():
    calls, syncs = [], []

    class Cuda:
        @staticmethod
        def synchronize():
            syncs.append(len(calls))

    class Torch:
        cuda = Cuda

    n = bench.settle(Torch, calls.append, seconds=0.05)
    assert n == len(calls) and n >= 8 and n % 8 == 0
    assert calls == list(range(n))                  # each call gets its own index, in order
    assert syncs == list(range(8, n + 1, 8))        # a synchronisation after every batch of 8


def test_training_step_bytes():
    """The C-ABI bytes of the training launches (B8 H16 T4096 d128, chunk 64,
    bf16): 134217728 bytes per token tensor, 4 MiB per chunk-boundary state
    entry over the batch."""
    w = synth.WORKLOADS["train_bf16"]
    tok, ent, n = 134217728, 8 * 16 * 128 * 128 * 2, 64
    abi = bench.train_abi_bytes(w)
    assert abi["scan"] == 3 * tok + (n + 1) * ent
    assert abi["cfwd"] == 5 * tok + n * ent
    assert abi["scan_rev"] == 3 * tok
    assert abi["cbwd"] == 9 * tok + n * ent == 1476395008
    assert abi["cbwd_tied"] == 7 * tok + n * ent
    # the step's compulsory bytes: the forward reads q, k, v, log f and writes
    # y; the backward reads those and dy and writes four gradients
    assert 14 * tok == 1879048192


@pytest.mark.parametrize("leg,plan,compulsory", [("long_bf16", (16, 32, 15), 1346371584),
                                                  ("fwd_bf16", (8, 4, 7), 85983232)])
def test_forward_only_bytes(leg, plan, compulsory):
    w = synth.WORKLOADS[leg]
    alg, comp, got = bench.fwd_leg_bytes(w)
    assert got == plan and comp == compulsory
    assert set(alg) == {"seg_scan", "seg_carry", "seg_fwd"}
    assert all(v > 0 for v in alg.values())


@pytest.mark.parametrize("B,H,T", [(1, 32, 32768), (4, 8, 2048), (5, 13, 63 * 64 + 17), (8, 16, 4096),
                                   (1, 1, 100), (2, 3, 9 * 64 + 7), (16, 16, 3 * 64 + 1), (1, 4, 20 * 64)])
def test_segment_plan_matches_the_library(lib, B, H, T):
    """With only the final state wanted, the library's forward workspace holds
    P + 1 float32 states and P decay vectors per sequence for its plan of P
    segments; the bench's plan must give the same sizes."""
    D, C = 128, 64
    P, G, NSEG = bench.seg_plan(B, T, H, C, want_y=False)
    assert NSEG == P and (P - 1) * G < -(-T // C) <= P * G
    want = (B * H * (NSEG + 1) * D * D + B * H * NSEG * D) * 4
    assert lib.hgrn2_fwd_workspace_bytes(B, T, H, D, D, C, 1, 0) == want
