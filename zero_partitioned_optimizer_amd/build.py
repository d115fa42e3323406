"""Build libzero.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libzero.so")
SOURCES = ["abi.cpp", "layout.cpp", "step_kernels.hip", "gather_kernels.hip"]
# host-only C++ (no device pass), compiled to an object and linked in
HOST_SOURCES = ["offload.cpp"]
HOST_FLAGS = ["-x", "c++", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-c"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                                   # one rounding per source operation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + proc.stdout + proc.stderr)


def build(out: str = LIB, extra=()) -> str:
    """Compile every source into ``out`` (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for h in HOST_SOURCES:
        obj = out + "." + os.path.splitext(h)[0] + ".o"
        rocm = os.path.dirname(os.path.dirname(os.path.realpath(shutil.which(hipcc()) or hipcc())))
        _run([hipcc(), *HOST_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
              *inc, os.path.join(CSRC, h), "-o", obj])
        objs.append(obj)
    _run([hipcc(), *HIPCC_FLAGS, *extra, *inc, *srcs, "-x", "none", *objs, "-o", out + ".tmp"])
    for obj in objs:
        os.remove(obj)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
