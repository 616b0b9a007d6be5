"""Builds libspecverify.so (gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libspecverify.so")
CSRC = os.path.join(PKG, "csrc")
# (source, extra flags).  The streaming kernel is built with IEEE mode off and NaN-free
# arithmetic assumed (finite logits are part of the contract; its input checks work on
# bit patterns); the other kernels keep IEEE semantics.
SOURCES = [
    (os.path.join(CSRC, "sv_rowpair.hip"), ["-fno-honor-nans", "-mno-amdgpu-ieee"]),
    (os.path.join(CSRC, "sv_kernels.hip"), []),
    (os.path.join(CSRC, "sv_head.hip"), []),
    (os.path.join(CSRC, "sv_diag.hip"), []),
    (os.path.join(CSRC, "sv_noalloc.hip"), []),
    (os.path.join(CSRC, "sv_api.cpp"), []),
]
HEADERS = [os.path.join(CSRC, f) for f in ("sv_device.h", "sv_lanes.h", "sv_layout.h", "sv_launch.h")] + [
    os.path.join(ROOT, "include", "specverify.h")
]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE arithmetic as written: fused multiply-adds only where the source asks for them
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # the host pass does not know the device-only feature flag
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build_library(verbose: bool = False, out: str = LIB) -> str:
    """Compiles each source to an object (own flags), links the shared library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src, extra in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        _run([hipcc(), *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src,
              "-o", obj], verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
