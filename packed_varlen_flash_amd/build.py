"""Build libpfa.so (HIP, gfx950) in-tree with hipcc.

The library is compiled for gfx950 only, with packed-FP32 instruction selection
disabled, and placed next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
# forward (all kernel modes), backward, and the merge / V quantiser; pfa_common.h is shared
SRCS = [os.path.join(CSRC, n) for n in ("pfa_fwd.hip", "pfa_bwd.hip", "pfa_aux.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpfa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (need ROCm with gfx950 support)")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-fno-honor-nans", "-I", INCLUDE, "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
