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
SRCS = [os.path.join(PKG, "csrc", name) for name in ("scan_fwd.hip", "scan_bwd.hip", "ssd_fwd.hip", "scan_chunked.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are switched off for all device code: the compiler would
# otherwise pair independent fp32 operations into them by itself.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-fvisibility=hidden",
    "-I", INCLUDE,
]


def _errors(r):
    return "\n".join(line for line in (r.stderr or "").splitlines() if "packed-fp32-ops" not in line)


def build(verbose: bool = False) -> str:
    """Compile the HIP sources (in parallel) and link libssm.so; always recompiles."""
    objs = [src[: -len(".hip")] + ".o" for src in SRCS]
    procs = []
    for src, obj in zip(SRCS, objs):
        cmd = [HIPCC, *HIP_FLAGS, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for cmd, proc in procs:
        out, err = proc.communicate()
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}\n{_errors(subprocess.CompletedProcess(cmd, proc.returncode, out, err))}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{_errors(r)}")
    for obj in objs:
        os.remove(obj)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
