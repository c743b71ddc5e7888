"""The C ABI's host code under AddressSanitizer (and LeakSanitizer).

The library's translation units are built again with the sanitizer on the host
side only (every -fsanitize flag behind -Xarch_host; the device code is
unchanged), and tests/abi_sanitize_driver.c, a C program built with the same
compiler's sanitizer runtime, calls every argument-checking path that returns
before device work: null and misaligned pointers, bad enums and option
combinations, contexts past the launch limit (including a list of 524,272
tensors), hyperparameter and codec-probe errors.  No GPU is needed."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from precision_adam_optimizer_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(CLANG) or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="ROCm compilers not available")
def test_abi_host_code_is_clean_under_asan(tmp_path):
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_unit(src):
        out = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = b.compile_command(src, out)
        cmd[cmd.index("-O3")] = "-O1"
        r = subprocess.run(cmd[:-3] + host_asan + cmd[-3:], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return out

    with ThreadPoolExecutor(len(b.UNITS)) as ex:
        objs = list(ex.map(compile_unit, b.UNITS))
    lib = str(tmp_path / "libfp8adam.so")
    r = subprocess.run(b.link_command(objs, lib)[:1] + ["-Xarch_host", "-fsanitize=address"]
                       + b.link_command(objs, lib)[1:], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([CLANG, "-std=c11", "-g", "-O1", "-fsanitize=address", "-fno-omit-frame-pointer",
                        "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include",
                        os.path.join(ROOT, "tests", "abi_sanitize_driver.c"), f"-L{tmp_path}", "-lfp8adam",
                        "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "abi driver done, 0 failures" in run.stdout
    assert "Sanitizer" not in run.stderr, run.stderr[-4000:]
