"""Build the HIP library ``libfp8adam.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fp8adam.hip")
DEPS = [SRC, os.path.join(PKG, "csrc", "fp8_codec.h"), os.path.join(ROOT, "include", "fp8adam.h")]
LIB = os.path.join(PKG, "libfp8adam.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_command(out: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep hand-written fp32 code off the packed-FP32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-o", out, SRC,
    ]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in DEPS):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run(compile_command(tmp), check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
