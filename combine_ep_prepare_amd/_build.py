"""Compile the HIP library for gfx950 in-tree (always rebuilds).

Produces ``combine_ep_prepare_amd/libcombine_ep_prepare_amd.so`` from the
sources under ``csrc/`` with hipcc. The flags keep IEEE fp32 semantics
(no fast-math, no contraction, no denormal flush) and disable the packed
fp32 instructions.

Also produces ``libep_ceilings.so`` from ``csrc/ep_ceilings.hip``: the
memory-pattern ceiling kernels the benchmark times beside the routing ops.
It is a separate object; the routing library neither links nor loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "ep_api.hip"), os.path.join(CSRC, "ep_kernels.hip")]
LIB_NAME = "libcombine_ep_prepare_amd.so"
LIB = os.path.join(HERE, LIB_NAME)
CEILINGS_SOURCE = os.path.join(CSRC, "ep_ceilings.hip")
CEILINGS_LIB = os.path.join(HERE, "libep_ceilings.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library needs ROCm's hipcc")


def _compile(sources, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile([CEILINGS_SOURCE], CEILINGS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
