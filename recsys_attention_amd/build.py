"""Build libhstu.so in-tree with hipcc for gfx950.

    python -m recsys_attention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
CSRC = os.path.join(_HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("hstu_fwd_kernels.hip", "hstu_layer_kernels.hip", "hstu_api.cpp",
                                             "hstu_layer_api.cpp")]
OUT = os.path.join(_HERE, "libhstu.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the work queues' atomics are single-lane already: the wave-aggregating
    # rewrite of atomics only adds a wait for the result right after each one
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I" + os.path.join(_ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libhstu.so")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
