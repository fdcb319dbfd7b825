"""Build the HIP library ``libmlstm.so`` in-tree for gfx950.

``python -m linear_recurrent_sequence_fwd_amd.build`` compiles every source
each time it runs (hipcc cross-compiles; no GPU is needed to build).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmlstm.so")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "mlstm_kernels.hip"), os.path.join(CSRC, "mlstm_bf16.hip"),
           os.path.join(CSRC, "mlstm_fused.hip"), os.path.join(CSRC, "mlstm_bwd.hip"),
           os.path.join(CSRC, "slstm.hip"), os.path.join(CSRC, "mlstm_block.hip"),
           os.path.join(CSRC, "mlstm_segments.hip"),
           os.path.join(CSRC, "mlstm_abi.cpp")]

# Packed-fp32 VALU instructions are turned off for all device code. MFMA
# builtins are compiled in the VGPR form: with accumulators in AGPRs this
# compiler copies loop-carried accumulators between registers around every
# MFMA. (The fused kernels keep their carried state in AGPRs through explicit
# in-place MFMAs.)
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False) -> str:
    """Compile libmlstm.so; returns its path. Raises on a compiler error."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
