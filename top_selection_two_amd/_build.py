"""Build the HIP library libtopk.so for gfx950 (in-tree, no JIT cache).

One translation unit, csrc/libtopk.hip, holds the C entry points and
includes the kernel headers.  The flags disable packed-FP32 instruction
selection (nothing here uses floating point, but every HIP build in this
project carries the flag), emit code for gfx950 only, and pin code object
version 5, which both the ROCm runtime in /opt/rocm and the one bundled with
PyTorch load.  They also turn off the compiler's atomic optimizer: every
atomic here is issued by one lane or targets a distinct address per lane,
and the optimizer's wave-wide combining would only add a scalar loop.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SO = os.path.join(PKG, "libtopk.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_libtopk(extra_flags=(), out: str = SO) -> str:
    src = os.path.join(CSRC, "libtopk.hip")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC,
           src, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_libtopk())
