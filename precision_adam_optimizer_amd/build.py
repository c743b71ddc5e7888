"""Build the HIP library ``libfp8adam.so`` in-tree for gfx950 with hipcc.

The step kernels are instantiated in one translation unit per (m, v) format
pair (``csrc/fp8adam_step_*.hip``) and the C ABI is in ``csrc/fp8adam.hip``;
the units compile in parallel, then link into one shared library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
UNITS = [os.path.join(CSRC, "fp8adam.hip")] + sorted(glob.glob(os.path.join(CSRC, "fp8adam_step_*.hip")))
DEPS = UNITS + [os.path.join(CSRC, "fp8_codec.h"), os.path.join(CSRC, "fp8adam_engine.h"),
                os.path.join(ROOT, "include", "fp8adam.h")]
LIB = os.path.join(PKG, "libfp8adam.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_command(src: str, out: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
        # keep the fp32 code off the packed-FP32 instructions.  The flag reaches the host
        # pass too, whose backend warns that it does not know the feature and ignores it:
        # clang forwards no -Xclang option through -Xarch_device, so it cannot be scoped.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-o", out, src,
    ]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs


def build(force: bool = True, jobs: int | None = None) -> str:
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in DEPS):
        return LIB
    jobs = jobs or max(1, min(len(UNITS), os.cpu_count() or 1))
    with tempfile.TemporaryDirectory(prefix="fp8adam_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(u) + ".o") for u in UNITS]
        with ThreadPoolExecutor(jobs) as ex:
            for r in ex.map(lambda a: subprocess.run(compile_command(*a), capture_output=True, text=True),
                            zip(UNITS, objs)):
                if r.returncode != 0:
                    raise RuntimeError(f"hipcc failed:\n{r.stderr}")
        tmp = LIB + ".tmp"
        subprocess.run(link_command(objs, tmp), check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
