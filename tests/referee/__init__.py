"""Independent referees that pin the CPU oracle.

* ``encode_sweep.c``: brute-force nearest-value FP8 encoder, swept over all
  2^32 fp32 bit patterns against the oracle's bit-level encoder.
* ``rational``: the whole FP8-moment AdamW step in exact rational arithmetic
  (fp32 roundings emulated exactly, FP8 quantization by nearest-value search
  over torch's float8 decode tables, the parameter update in 60-digit decimal).

Neither shares code with the oracle; both are test infrastructure.
"""
import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def sweep_lib() -> ctypes.CDLL:
    src = os.path.join(_HERE, "encode_sweep.c")
    so = os.path.join(_HERE, "libencode_sweep.so")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        tmp = so + ".tmp"
        subprocess.run(["gcc", "-std=c11", "-O2", "-pthread", "-fPIC", "-shared", "-o", tmp,
                        src, "-lm"], check=True)
        os.replace(tmp, so)
    L = ctypes.CDLL(so)
    L.sweep_encoder.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                ctypes.c_uint64, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64),
                                ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    L.sweep_encoder.restype = ctypes.c_uint64
    return L
