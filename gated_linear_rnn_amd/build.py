"""Build librglru.so (all HIP kernels + the C ABI) in-tree for gfx950 with hipcc.

Every source under csrc/ is compiled to an object in parallel, then linked into
gated_linear_rnn_amd/librglru.so.  Run as ``python -m gated_linear_rnn_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "librglru.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.hip", "conv.hip", "gemm.hip", "lru.hip", "decode.hip", "scan.hip", "bwd.hip", "block.hip",
           "mqa.hip", "mqa_decode.hip"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                                   # only the explicit fmaf calls fuse
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed fp32 VALU ops
    # the only read-modify-write atomics are single-lane ticket counters: without the wave
    # reduction this pass adds, the wait for the returned value sits at its first use, so
    # loads issued in between stay in flight
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
