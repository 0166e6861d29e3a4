"""Build libssm.so (HIP, gfx950) in-tree with hipcc.

Run ``python -m selective_state_space_79_amd.build``; ``__graft_entry__.build()``
calls ``build()`` as well.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "scan_fwd.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are switched off for all device code (see the design doc,
# "Build"): the compiler would otherwise pair independent fp32 ops by itself.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-I", INCLUDE,
]


def build(verbose: bool = False) -> str:
    """Compile the HIP library; always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stderr or "").splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
