"""Compile libfp8dp.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every call recompiles.  The library is written next to this file so that it
travels with the source tree.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp8dp.so")
ARCH = "gfx950"

# -ffp-contract=off: no multiply-add contraction anywhere (the quantizer's
#   binary32 products must round on their own; the GEMM asks for its
#   fused multiply-adds explicitly).
# -packed-fp32-ops disabled: no packed FP32 instructions are emitted.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile all csrc/*.hip into libfp8dp.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}",
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
