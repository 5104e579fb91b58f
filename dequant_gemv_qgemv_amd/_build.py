"""Compile the HIP library in-tree: csrc/qw3.hip -> libqw3.so (gfx950 only)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "qw3.hip")
LIB = os.path.join(HERE, "libqw3.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def compile_hip(src: str, lib: str, extra_flags=None) -> None:
    """hipcc `src` (gfx950, the flags above) into the shared library `lib`."""
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + HIP_FLAGS + list(extra_flags or []) + ["-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(extra_flags=None) -> str:
    """Always recompiles the library; returns its path."""
    compile_hip(SRC, LIB, extra_flags)
    return LIB


if __name__ == "__main__":
    print(build())
