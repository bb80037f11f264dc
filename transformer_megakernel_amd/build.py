"""Build the HIP library (libmk.so) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# the decode kernel + C ABI + scheduler, and the measurement kernels
SRCS = [os.path.join(PKG, "csrc", "mk_api.hip"), os.path.join(PKG, "csrc", "mk_measure.hip")]
LIB = os.path.join(PKG, "libmk.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep hipcc from forming packed fp32 arithmetic on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-inline-asm",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile csrc/mk_api.hip (kernel + C ABI + scheduler) and csrc/mk_measure.hip
    (measurement kernels) into ``out`` (libmk.so in the package); ``defines``: extra
    -D options (build variants for comparison); return the path."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"), "-o", tmp,
           *SRCS]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
