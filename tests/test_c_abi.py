"""The C ABI from a plain C11 program (tests/c_abi_demo.c): no torch and no
Python in the calling process.  It links against libfp8adam.so and the HIP
runtime only, allocates with hipMalloc, lets fp8adam_init write the fresh
state (zero_state), runs two AdamW steps and writes inputs and results to a
file; the test replays them through the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import precision_adam_optimizer_amd as pk  # noqa: F401  (the library is built)
from tests.gpu_util import OracleState, oracle_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "precision_adam_optimizer_amd")


def build_c_demo(tmp_path, name: str = "c_abi_demo") -> str:
    """Compile and link tests/<name>.c against the library and the HIP runtime."""
    exe = str(tmp_path / name)
    subprocess.run(["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include",
                    os.path.join(ROOT, "tests", f"{name}.c"), f"-L{PKG}", "-lfp8adam", "-L/opt/rocm/lib",
                    "-lamdhip64", f"-Wl,-rpath,{PKG}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def _build(tmp_path) -> str:
    return build_c_demo(tmp_path)


def test_c_caller_compiles_and_links(tmp_path):
    """The header is plain C and the library links into a C program with the
    HIP runtime as its only other dependency."""
    exe = _build(tmp_path)
    libs = subprocess.run(["ldd", exe], check=True, capture_output=True, text=True).stdout
    assert "libfp8adam.so" in libs and "libamdhip64" in libs
    assert "torch" not in libs and "python" not in libs


def test_c_graph_caller_of_the_allocation_free_step_compiles():
    """tests/c_noalloc_graph_demo.c (run on the GPU by the allocation-free
    step's tests) is plain C against the header and the HIP runtime."""
    import tempfile
    import pathlib
    with tempfile.TemporaryDirectory() as d:
        exe = build_c_demo(pathlib.Path(d), "c_noalloc_graph_demo")
        assert os.path.exists(exe)


@pytest.mark.gpu
def test_c_caller_matches_the_oracle(tmp_path):
    exe = _build(tmp_path)
    out = tmp_path / "result.bin"
    r = subprocess.run([exe, str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    buf = out.read_bytes()
    off = 0

    def take(dtype, count):
        nonlocal off
        a = np.frombuffer(buf, dtype=dtype, count=count, offset=off).copy()
        off += a.nbytes
        return a

    h = oracle.Hyper(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    ntensors = 0
    while off < len(buf):
        n = int(take(np.int64, 1)[0])
        p0, g1, g2 = take(np.float32, n), take(np.uint16, n), take(np.uint16, n)
        p, m, v = take(np.float32, n), take(np.uint8, n), take(np.uint8, n)
        sm, sv = take(np.float32, 1), take(np.float32, 1)
        st = OracleState(p0.copy(), np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.ones(1, np.float32),
                         np.ones(1, np.float32))
        for t, g in ((1, g1), (2, g2)):
            h.step = t
            st.step(oracle_config(h, "e4m3", "e5m2", "tensor", "pow2", "fp32"), g)
        assert np.array_equal(m, st.cm) and np.array_equal(v, st.cv), f"tensor {ntensors}: codes differ"
        assert sm.tobytes() == st.sm.tobytes() and sv.tobytes() == st.sv.tobytes(), f"tensor {ntensors}: scales"
        # two steps without re-synchronizing p: twice the one-step bound
        tol = 2e-6 * np.maximum(np.abs(st.p), np.abs(p0)).astype(np.float64)
        assert (np.abs(p.astype(np.float64) - st.p) <= tol).all(), f"tensor {ntensors}: weights"
        ntensors += 1
    assert ntensors == 2
