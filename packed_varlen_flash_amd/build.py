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


# compiler options of every kernel (gfx950 code generation)
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden", "-fno-honor-nans",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# what the forward kernel's code depends on: a built library records its hash beside
# itself, so that a measurement taken on one build can be matched to a later build of the
# same forward kernel (the build is deterministic)
FWD_SOURCES = [os.path.join(CSRC, "pfa_fwd.hip"), os.path.join(CSRC, "pfa_common.h"),
               os.path.join(INCLUDE, "pfa.h")]


def forward_sources_sha() -> str:
    import hashlib
    h = hashlib.sha256(" ".join([ARCH, *FLAGS]).encode())
    for path in FWD_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def build(verbose: bool = False, sanitize_host: bool = False, path: str | None = None) -> str:
    """sanitize_host: compile the host code (argument checks, validators, launch setup)
    with AddressSanitizer and UndefinedBehaviorSanitizer; the GPU code is built as always.
    Loading such a library needs clang's ASan runtime preloaded.  path: output file."""
    out = path or LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", *FLAGS, "-I", INCLUDE, "-I", CSRC]
    if sanitize_host:
        cmd += ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    cmd += [*SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, out)
    with open(out + ".fwdsha", "w") as f:      # the forward sources this build came from
        f.write(forward_sources_sha() + "\n")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
