"""Compile the HIP library in-tree: csrc/qw3_gemv.hip + csrc/qw3.hip -> libqw3.so (gfx950 only)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqw3.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# The library's translation units and the flags each adds.  The batch-1
# kernels take the max-ilp machine scheduler (faster on them); the batched and
# prefill kernels keep the default one (max-ilp measured slower there).
UNITS = [
    ("qw3_gemv.hip", ["-mllvm", "--amdgpu-sched-strategy=max-ilp"]),
    ("qw3.hip", []),
]


def compile_hip(src: str, lib: str, extra_flags=None) -> None:
    """hipcc one source `src` (gfx950, the flags above) into the shared library `lib`."""
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + HIP_FLAGS + ["-shared"] + list(extra_flags or []) + ["-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(extra_flags=None) -> str:
    """Always recompiles every unit (in parallel) and links the library; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs, objs = [], []
    for src, flags in UNITS:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + HIP_FLAGS + flags + list(extra_flags or []) + ["-c", "-o", obj, os.path.join(CSRC, src)]
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    failed = [cmd for p, cmd in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
