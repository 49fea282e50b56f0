"""Build libkq.so (HIP, gfx950) in-tree with hipcc.

    python -m mxfp4_activation_quantizer_amd.build

Always recompiles when called through ``build_library()``; ``ensure_built()``
only compiles when the library is missing or older than its sources.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every rounding step is written out explicitly (fmaf where a fused
    # multiply-add is wanted), so the compiler may not contract on its own
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def deps():
    return sources() + sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + \
        sorted(glob.glob(os.path.join(INCLUDE, "*.h")))


def build_library(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def ensure_built() -> str:
    if not os.path.exists(LIB) or any(os.path.getmtime(p) > os.path.getmtime(LIB) for p in deps()):
        build_library()
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
