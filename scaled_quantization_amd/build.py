"""Compile libfp8dp.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every call recompiles: each csrc/*.hip becomes an object under _build/ (the
files compile in parallel), then one link writes the library next to this
file so that it travels with the source tree.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp8dp.so")
OBJ = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# -ffp-contract=off: no multiply-add contraction anywhere (the quantizer's
#   binary32 products must round on their own; the GEMM asks for its
#   fused multiply-adds explicitly).
# -packed-fp32-ops disabled: no packed FP32 instructions are emitted.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
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


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}) on {cmd[-3]}:\n{errs}")
    if verbose and errs.strip():
        print(errs)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile all csrc/*.hip into libfp8dp.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(OBJ, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([cc, *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}",
                                     f"-I{CSRC}", "-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
