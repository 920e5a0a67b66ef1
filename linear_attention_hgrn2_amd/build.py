"""Build libhgrn2.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m linear_attention_hgrn2_amd.build

Each translation unit is compiled in parallel, then linked into
``linear_attention_hgrn2_amd/libhgrn2.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhgrn2.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("HGRN2_OFFLOAD_ARCH", "gfx950")

SOURCES = ["scan_inst.hip", "cfwd_inst.hip", "cbwd_inst.hip", "cbwd_f32out_inst.hip", "cbwd_res_inst.hip",
           "decode_inst.hip", "hgrn1_inst.hip", "sfwd_inst.hip", "api.cpp"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # packed float32 vector ops are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument", "-Wno-shadow",
]

# sources whose matrix-core accumulators stay in ordinary vector registers
# (their per-step float32 updates of the state would otherwise move it
# between register files twice per step)
VGPR_MFMA = {"scan_inst.hip", "cfwd_inst.hip", "sfwd_inst.hip"}

# per-source options: the resident backward (issue-bound, two lock-stepped
# waves per SIMD) is scheduled by the compiler's iterative ILP strategy, which
# measured 1.6% faster there (0.4224 -> 0.415-0.417 ms at B8 H16 T4096); it
# adds spills to the generic chunk-128 backward, which keeps the default
EXTRA = {"cbwd_res_inst.hip": ["-mllvm", "--amdgpu-sched-strategy=iterative-ilp"]}


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _compile(src: str) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS
    if src in VGPR_MFMA:
        cmd += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    cmd += EXTRA.get(src, [])
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stdout))
    return obj


def build(verbose: bool = False) -> str:
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
