"""ctypes shim over the CPU oracle (``fp8adam_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
cpu_baseline leg are the only callers.  The product path never imports this
package, and the oracle shares no code with the GPU library.

The oracle follows the pages cited in ``fp8adam_oracle.c``: the daoxuan.cc
explainer of arXiv 2409.12517 (section on why Adam keeps m in E4M3 and v in
E5M2), the shd-paper.top summary of arXiv 2409.12517v2 (method details), and
the zyxy.net FP8 mixed-precision article (formats, strategies, AdamW code).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8adam_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2 = 0, 1
SCALE_POW2, SCALE_AMAX = 0, 1
FORMAT_NAMES = {"e4m3": E4M3, "e5m2": E5M2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, no SIMD, no fp contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Config(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
        ("step", ctypes.c_int64),
        ("m_fmt", ctypes.c_int), ("v_fmt", ctypes.c_int),
        ("block", ctypes.c_int), ("scale_mode", ctypes.c_int), ("master_bf16", ctypes.c_int),
        ("l2_coupled", ctypes.c_int),
        ("history_len", ctypes.c_int), ("margin", ctypes.c_int), ("delayed_from", ctypes.c_int64),
        ("grad_factor", ctypes.c_float), ("sched_step", ctypes.c_int64),
        ("stochastic", ctypes.c_int), ("tensor_index", ctypes.c_uint32), ("seed", ctypes.c_uint64),
        ("update_from_codes", ctypes.c_int),
    ]


class AmpConfig(ctypes.Structure):
    _fields_ = [("max_norm", ctypes.c_float), ("growth_factor", ctypes.c_float),
                ("backoff_factor", ctypes.c_float), ("growth_interval", ctypes.c_int32)]


class AmpState(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("growth_tracker", ctypes.c_int32), ("step", ctypes.c_int64),
                ("found_inf", ctypes.c_int32), ("grad_norm", ctypes.c_float), ("clip_coef", ctypes.c_float),
                ("grad_factor", ctypes.c_float)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class Stats(ctypes.Structure):
    _fields_ = [
        ("underflow_m", ctypes.c_int64), ("underflow_v", ctypes.c_int64),
        ("saturated_m", ctypes.c_int64), ("saturated_v", ctypes.c_int64),
        ("nonfinite", ctypes.c_int64),
        ("amax_m", ctypes.c_float), ("amax_v", ctypes.c_float),
        ("scale_m", ctypes.c_float), ("scale_v", ctypes.c_float),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P, u8p, f32p, u16p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        L.ref_decode.argtypes = [ctypes.c_int, ctypes.c_uint8]
        L.ref_decode.restype = ctypes.c_float
        L.ref_encode.argtypes = [ctypes.c_int, ctypes.c_float]
        L.ref_encode.restype = ctypes.c_uint8
        L.ref_format_max.argtypes = [ctypes.c_int]
        L.ref_format_max.restype = ctypes.c_float
        L.ref_encode_array.argtypes = [ctypes.c_int, f32p, u8p, ctypes.c_int64]
        L.ref_decode_array.argtypes = [ctypes.c_int, u8p, f32p, ctypes.c_int64]
        L.ref_encode_bits_range.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_int64, u8p]
        L.ref_double_to_bf16.argtypes = [ctypes.c_double]
        L.ref_double_to_bf16.restype = ctypes.c_uint16
        L.ref_f32_to_bf16.argtypes = [ctypes.c_float]
        L.ref_f32_to_bf16.restype = ctypes.c_uint16
        L.ref_choose_scale.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                       ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]
        L.ref_step.argtypes = [ctypes.POINTER(Config), ctypes.c_int64, P, u16p, u8p, u8p,
                               f32p, f32p, ctypes.POINTER(Stats)]
        L.ref_step.restype = ctypes.c_int
        L.ref_step_hist.argtypes = [ctypes.POINTER(Config), ctypes.c_int64, P, u16p, u8p, u8p,
                                    f32p, f32p, f32p, ctypes.POINTER(Stats)]
        L.ref_step_hist.restype = ctypes.c_int
        L.ref_step_fp32_moments.argtypes = [ctypes.POINTER(Config), ctypes.c_int64, f32p, u16p,
                                            f32p, f32p]
        L.ref_step_fp32_moments.restype = ctypes.c_int
        L.ref_rounding_is_nearest.restype = ctypes.c_int
        L.ref_encode_sr.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_uint32]
        L.ref_encode_sr.restype = ctypes.c_uint8
        L.ref_philox4x32_10.argtypes = [P, P, P]
        L.ref_encode_sr_bits_range.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_int64, ctypes.c_uint32, u8p]
        L.ref_encode_sr_array.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, u8p]
        L.ref_sr_word.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64]
        L.ref_sr_word.restype = ctypes.c_uint32
        L.ref_grad_sumsq.argtypes = [u16p, ctypes.c_int64, P, ctypes.POINTER(ctypes.c_int64)]
        L.ref_sumsq_total.argtypes = [P]
        L.ref_sumsq_total.restype = ctypes.c_double
        L.ref_amp_control.argtypes = [P, ctypes.c_int64, ctypes.POINTER(AmpConfig), ctypes.POINTER(AmpState)]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def fmt_id(fmt) -> int:
    return FORMAT_NAMES[fmt] if isinstance(fmt, str) else int(fmt)


def decode(fmt, codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    lib().ref_decode_array(fmt_id(fmt), _ptr(c), _ptr(out), c.size)
    return out


def encode(fmt, x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    lib().ref_encode_array(fmt_id(fmt), _ptr(a), _ptr(out), a.size)
    return out


def encode_bits_range(fmt, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint8)
    lib().ref_encode_bits_range(fmt_id(fmt), start, count, _ptr(out))
    return out


def format_max(fmt) -> float:
    return lib().ref_format_max(fmt_id(fmt))


def choose_scale(fmt, amax: float, mode: int = SCALE_POW2) -> tuple[float, float]:
    s, inv = ctypes.c_float(), ctypes.c_float()
    lib().ref_choose_scale(fmt_id(fmt), mode, amax, ctypes.byref(s), ctypes.byref(inv))
    return s.value, inv.value


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (RNE) with the oracle's own rounding."""
    a = np.ascontiguousarray(x, dtype=np.float32).ravel()
    f = lib().ref_f32_to_bf16
    return np.array([f(float(v)) for v in a], dtype=np.uint16)


@dataclass
class Hyper:
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.0
    step: int = 1


def make_config(h: Hyper, m_fmt=E4M3, v_fmt=E5M2, block: int = 0,
                scale_mode: int = SCALE_POW2, master_bf16: bool = False, l2_coupled: bool = False,
                history_len: int = 0, margin: int = 0, delayed_from: int = 2, grad_factor: float = 1.0,
                sched_step: int = 0, stochastic: bool = False, tensor_index: int = 0, seed: int = 0,
                update_from_codes: bool = False) -> Config:
    """history_len > 0 selects delayed scaling (per-tensor scales only); grad_factor
    multiplies every gradient first; sched_step (0: h.step) is the step number
    compared with delayed_from; update_from_codes selects the other reading of the
    update order (p from the new codes instead of the fresh moments; study only)."""
    return Config(h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.step,
                  fmt_id(m_fmt), fmt_id(v_fmt), block, scale_mode, int(master_bf16), int(l2_coupled),
                  history_len, margin, delayed_from, grad_factor, sched_step, int(stochastic), tensor_index, seed,
                  int(update_from_codes))


def step(cfg: Config, p: np.ndarray, g_bits: np.ndarray, cm: np.ndarray, cv: np.ndarray,
         sm: np.ndarray, sv: np.ndarray) -> dict:
    """One FP8-moment AdamW step on host arrays, in place.

    p: float32 (or uint16 bf16 bits when cfg.master_bf16); g_bits: uint16 bf16 bits;
    cm, cv: uint8 codes; sm, sv: float32 scales (1, or ceil(n/block)).
    """
    n = p.size
    assert g_bits.dtype == np.uint16 and g_bits.size == n
    assert cm.dtype == np.uint8 and cv.dtype == np.uint8 and cm.size == n and cv.size == n
    assert sm.dtype == np.float32 and sv.dtype == np.float32
    nb = 1 if cfg.block == 0 else -(-n // cfg.block)
    assert sm.size >= nb and sv.size >= nb
    assert p.dtype == (np.uint16 if cfg.master_bf16 else np.float32)
    st = Stats()
    rc = lib().ref_step(ctypes.byref(cfg), n, _ptr(p), _ptr(g_bits), _ptr(cm), _ptr(cv),
                        _ptr(sm), _ptr(sv), ctypes.byref(st))
    if rc != 0:
        raise ValueError("oracle ref_step rejected its arguments")
    return st.as_dict()


def step_hist(cfg: Config, p: np.ndarray, g_bits: np.ndarray, cm: np.ndarray, cv: np.ndarray,
              sm: np.ndarray, sv: np.ndarray, hist: np.ndarray) -> dict:
    """A step with delayed scaling: as ``step``, plus hist (float32, 2 * history_len:
    the amax history of m then v), read for the scale and updated in place."""
    n = p.size
    assert cfg.history_len > 0 and hist.dtype == np.float32 and hist.size == 2 * cfg.history_len
    assert g_bits.dtype == np.uint16 and g_bits.size == n
    assert cm.dtype == np.uint8 and cv.dtype == np.uint8 and cm.size == n and cv.size == n
    assert sm.dtype == np.float32 and sv.dtype == np.float32 and sm.size >= 1 and sv.size >= 1
    assert p.dtype == (np.uint16 if cfg.master_bf16 else np.float32)
    st = Stats()
    rc = lib().ref_step_hist(ctypes.byref(cfg), n, _ptr(p), _ptr(g_bits), _ptr(cm), _ptr(cv),
                             _ptr(sm), _ptr(sv), _ptr(hist), ctypes.byref(st))
    if rc != 0:
        raise ValueError("oracle ref_step_hist rejected its arguments")
    return st.as_dict()


def step_fp32_moments(cfg: Config, p: np.ndarray, g_bits: np.ndarray, m: np.ndarray,
                      v: np.ndarray) -> None:
    """AdamW with fp32 moments (codec removed), in place."""
    rc = lib().ref_step_fp32_moments(ctypes.byref(cfg), p.size, _ptr(p), _ptr(g_bits),
                                     _ptr(m), _ptr(v))
    if rc != 0:
        raise ValueError("oracle ref_step_fp32_moments rejected its arguments")


class GradSums:
    """Exact sum of squares (per-exponent integer buckets) and non-finite count
    of bf16 gradients, accumulated tensor by tensor."""

    def __init__(self):
        self.acc = np.zeros(256, np.uint64)
        self.nonfinite = ctypes.c_int64(0)

    def add(self, g_bits: np.ndarray) -> "GradSums":
        g = np.ascontiguousarray(g_bits, dtype=np.uint16)
        lib().ref_grad_sumsq(_ptr(g), g.size, _ptr(self.acc), ctypes.byref(self.nonfinite))
        return self

    def total(self) -> float:
        """The exact sum of squares rounded once to double."""
        return lib().ref_sumsq_total(_ptr(self.acc))


def amp_control(sums: GradSums, cfg: AmpConfig, state: AmpState) -> AmpState:
    """One loss-scaler / clipping decision over the whole list; updates state in place."""
    lib().ref_amp_control(_ptr(sums.acc), sums.nonfinite.value, ctypes.byref(cfg), ctypes.byref(state))
    return state


def encode_sr(fmt, x: float, r16: int) -> int:
    """Stochastic rounding of one value with 16 random bits."""
    return lib().ref_encode_sr(fmt_id(fmt), x, r16)


def encode_sr_bits_range(fmt, start: int, count: int, r16: int, out: np.ndarray | None = None) -> np.ndarray:
    """Stochastic-rounding encode of the fp32 patterns start .. start+count-1 with one r16."""
    out = np.empty(count, dtype=np.uint8) if out is None else out
    assert out.dtype == np.uint8 and out.size >= count and out.flags["C_CONTIGUOUS"]
    lib().ref_encode_sr_bits_range(fmt_id(fmt), start, count, r16, _ptr(out))
    return out


def encode_sr_array(fmt, x: np.ndarray, r16: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Stochastic-rounding encode of x[i] (float32) with its own 16 random bits r16[i] (uint16)."""
    assert x.dtype == np.float32 and r16.dtype == np.uint16 and x.shape == r16.shape
    x, r16 = np.ascontiguousarray(x), np.ascontiguousarray(r16)
    out = np.empty(x.size, dtype=np.uint8) if out is None else out
    assert out.dtype == np.uint8 and out.size >= x.size and out.flags["C_CONTIGUOUS"]
    lib().ref_encode_sr_array(fmt_id(fmt), _ptr(x), _ptr(r16), x.size, _ptr(out))
    return out


def philox4x32_10(ctr, key) -> list:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().ref_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return [int(x) for x in out]


def sr_word(seed: int, tensor: int, t: int, i: int) -> int:
    return lib().ref_sr_word(seed, tensor, t, i)
