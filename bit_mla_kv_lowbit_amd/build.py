"""Compile the HIP kernels and the C-ABI host code into libmla_lowbit.so (gfx950)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_lowbit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
BASE = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions are generated for gfx950
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# MFMA results in VGPRs: the 16-head decode scales each group's product on the
# VALU; the 128-head decode keeps its PV accumulators in AGPRs instead
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCES = {"api.hip": VGPR_FORM, "write.hip": VGPR_FORM, "decode.hip": VGPR_FORM,
           "decode_wide.hip": []}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False) -> str:
    """Always recompiles every source; returns the path of the shared library."""
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(CSRC, src + ".o")
        _run([HIPCC, *BASE, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    for o in objs:
        os.remove(o)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
