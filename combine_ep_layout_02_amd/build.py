"""Build libep_mi355x.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m combine_ep_layout_02_amd.build`` or call ``build()``.  The
library is built in place next to this file; the Python binding loads it from
there and refuses to run without it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libep_mi355x.so")
SOURCES = ["ep_abi.hip", "layout.hip", "dispatch.hip", "combine.hip", "gate.hip", "logfmt.hip",
           "probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE fp32 in source order: no fused contraction of separate mul/add
    "-ffp-contract=off",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", output + ".tmp", *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; harmless
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
