"""Python binding of the FP8-moment Adam/AdamW step for MI355X.

A thin ctypes layer over ``libfp8adam.so`` (C ABI in ``include/fp8adam.h``):
the functions below carry the C names and only marshal arguments; every step
of the optimizer runs in the library's HIP kernels.  PyTorch supplies device
memory and the stream.  There is no fallback: if the library is missing,
``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp8adam.so")

E4M3, E5M2 = 0, 1
SCALE_TENSOR, SCALE_BLOCK128 = 0, 1
SCALE_POW2, SCALE_AMAX = 0, 1
MASTER_FP32, MASTER_BF16 = 0, 1
SCHEDULE_TWO_PASS, SCHEDULE_SPECULATIVE = 0, 1
BLOCK = 128

_FORMATS = {"e4m3": E4M3, "e5m2": E5M2}
_GRAN = {"tensor": SCALE_TENSOR, "block128": SCALE_BLOCK128}
_SMODE = {"pow2": SCALE_POW2, "amax": SCALE_AMAX}
_SCHED = {"two_pass": SCHEDULE_TWO_PASS, "speculative": SCHEDULE_SPECULATIVE}
DECAY_DECOUPLED, DECAY_L2 = 0, 1
_DECAY = {"decoupled": DECAY_DECOUPLED, "l2": DECAY_L2}
SCALING_JUST_IN_TIME, SCALING_DELAYED = 0, 1
ROUND_NEAREST, ROUND_STOCHASTIC = 0, 1
_ROUNDING = {"nearest": ROUND_NEAREST, "stochastic": ROUND_STOCHASTIC}
_SCALING = {"just_in_time": SCALING_JUST_IN_TIME, "delayed": SCALING_DELAYED}
PREDICT_AUTO, PREDICT_PROBE, PREDICT_GROWTH = 0, 1, 2
_PREDICT = {"auto": PREDICT_AUTO, "probe": PREDICT_PROBE, "growth": PREDICT_GROWTH}

KERNEL_KINDS = ("amax_pass", "update_pass", "scale_reduce", "block128_pass", "stats_reset", "spec_pass",
                "spec_check", "fixup", "delayed_pass", "delayed_commit", "gradnorm_pass", "amp_decision",
                "scale_prepare", "spec_probe", "part_fold")

# names of every entry point the header declares
EXPORTS = ("fp8adam_init", "fp8adam_step", "fp8adam_stats", "fp8adam_destroy", "fp8adam_last_error",
           "fp8adam_encode", "fp8adam_decode", "fp8adam_encode_bits_range", "fp8adam_set_timing",
           "fp8adam_set_timing_kinds",
           "fp8adam_kernel_times", "fp8adam_runtime_version", "fp8adam_num_chunks", "fp8adam_current_buffer",
           "fp8adam_step_amp", "fp8adam_encode_sr_bits_range", "fp8adam_encode_sr", "fp8adam_stream_copy",
           "fp8adam_step_noalloc", "fp8adam_stream_mix", "fp8adam_stream_rw")

# limits of fp8adam_step_noalloc (the header's FP8ADAM_NOALLOC_* macros)
NOALLOC_MAX_TENSORS = 4096
NOALLOC_MAX_CHUNKS = 131072
NOALLOC_SCRATCH_BYTES = 2015232


class Fp8AdamError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fp8adam error {code}: {msg}")
        self.code = code


class TensorArg(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("m_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("numel", ctypes.c_int64), ("m_alt", ctypes.c_void_p), ("v_alt", ctypes.c_void_p),
                ("amax_history", ctypes.c_void_p)]


class ConfigArg(ctypes.Structure):
    _fields_ = [("m_format", ctypes.c_int32), ("v_format", ctypes.c_int32),
                ("granularity", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("master", ctypes.c_int32), ("collect_stats", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("speculate_from_step", ctypes.c_int32),
                ("decay_mode", ctypes.c_int32), ("scaling", ctypes.c_int32),
                ("amax_history_len", ctypes.c_int32), ("margin", ctypes.c_int32),
                ("delayed_from_step", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("zero_state", ctypes.c_int32), ("predictor", ctypes.c_int32)]


class HParamsArg(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64)]


class AmpConfigArg(ctypes.Structure):
    _fields_ = [("max_norm", ctypes.c_float), ("growth_factor", ctypes.c_float),
                ("backoff_factor", ctypes.c_float), ("growth_interval", ctypes.c_int32)]


# fp8adam_amp_state, as it lies in device memory (32 bytes)
AMP_STATE_DTYPE = np.dtype([("scale", "<f4"), ("growth_tracker", "<i4"), ("step", "<i8"), ("found_inf", "<i4"),
                            ("grad_norm", "<f4"), ("clip_coef", "<f4"), ("grad_factor", "<f4")])


class StatsArg(ctypes.Structure):
    _fields_ = [("amax_m", ctypes.c_float), ("amax_v", ctypes.c_float),
                ("scale_m", ctypes.c_float), ("scale_v", ctypes.c_float),
                ("underflow_m", ctypes.c_int64), ("underflow_v", ctypes.c_int64),
                ("saturated_m", ctypes.c_int64), ("saturated_v", ctypes.c_int64),
                ("nonfinite", ctypes.c_int64), ("requantized", ctypes.c_int64),
                ("probed", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m precision_adam_optimizer_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.fp8adam_init.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(TensorArg), i32, ctypes.POINTER(ConfigArg), vp]
    L.fp8adam_step.argtypes = [vp, ctypes.POINTER(HParamsArg), vp]
    L.fp8adam_stats.argtypes = [vp, ctypes.POINTER(StatsArg), i32, vp]
    L.fp8adam_step_amp.argtypes = [vp, ctypes.POINTER(HParamsArg), ctypes.POINTER(AmpConfigArg), vp, vp]
    L.fp8adam_destroy.argtypes = [vp]
    L.fp8adam_destroy.restype = None
    L.fp8adam_last_error.restype = ctypes.c_char_p
    L.fp8adam_encode.argtypes = [i32, vp, vp, i64, vp]
    L.fp8adam_decode.argtypes = [i32, vp, vp, i64, vp]
    L.fp8adam_encode_bits_range.argtypes = [i32, ctypes.c_uint32, i64, vp, vp]
    L.fp8adam_set_timing.argtypes = [vp, i32]
    L.fp8adam_set_timing_kinds.argtypes = [vp, ctypes.c_uint32]
    L.fp8adam_kernel_times.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32), i32]
    L.fp8adam_runtime_version.argtypes = [ctypes.POINTER(i32)]
    L.fp8adam_num_chunks.argtypes = [vp]
    L.fp8adam_num_chunks.restype = i64
    L.fp8adam_current_buffer.argtypes = [vp]
    L.fp8adam_current_buffer.restype = i32
    L.fp8adam_encode_sr_bits_range.argtypes = [i32, ctypes.c_uint32, i64, ctypes.c_uint32, vp, vp]
    L.fp8adam_encode_sr.argtypes = [i32, vp, vp, vp, i64, vp]
    L.fp8adam_stream_copy.argtypes = [vp, vp, i64, vp]
    L.fp8adam_stream_mix.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, vp]
    L.fp8adam_stream_rw.argtypes = [vp, i64, vp, i64, vp]
    L.fp8adam_step_noalloc.argtypes = [ctypes.POINTER(TensorArg), i32, ctypes.POINTER(ConfigArg),
                                       ctypes.POINTER(HParamsArg), vp]
    for name in ("fp8adam_init", "fp8adam_step", "fp8adam_stats", "fp8adam_encode", "fp8adam_decode",
                 "fp8adam_encode_bits_range", "fp8adam_set_timing", "fp8adam_set_timing_kinds",
                 "fp8adam_kernel_times",
                 "fp8adam_runtime_version", "fp8adam_step_amp", "fp8adam_encode_sr_bits_range",
                 "fp8adam_encode_sr", "fp8adam_stream_copy", "fp8adam_step_noalloc",
                 "fp8adam_stream_mix", "fp8adam_stream_rw"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        raise Fp8AdamError(rc, load().fp8adam_last_error().decode())


def current_stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------- C names

def fp8adam_init(tensors: list[TensorArg], cfg: ConfigArg, stream: int | None = None) -> int:
    arr = (TensorArg * len(tensors))(*tensors)
    h = ctypes.c_void_p()
    _check(load().fp8adam_init(ctypes.byref(h), arr, len(tensors), ctypes.byref(cfg),
                               current_stream() if stream is None else stream))
    return h.value


def fp8adam_step(ctx: int, hp: HParamsArg, stream: int | None = None) -> None:
    _check(load().fp8adam_step(ctx, ctypes.byref(hp), current_stream() if stream is None else stream))


def fp8adam_step_amp(ctx: int, hp: HParamsArg, amp: AmpConfigArg, state: int, stream: int | None = None) -> None:
    _check(load().fp8adam_step_amp(ctx, ctypes.byref(hp), ctypes.byref(amp), state,
                                   current_stream() if stream is None else stream))


def fp8adam_step_noalloc(tensors: list[TensorArg], cfg: ConfigArg, hp: HParamsArg, stream: int | None = None) -> None:
    arr = (TensorArg * len(tensors))(*tensors)
    _check(load().fp8adam_step_noalloc(arr, len(tensors), ctypes.byref(cfg), ctypes.byref(hp),
                                       current_stream() if stream is None else stream))


def amp_state(init_scale: float = 65536.0, device="cuda") -> torch.Tensor:
    """A fresh loss-scaler state (fp8adam_amp_state) in device memory: 32 bytes."""
    rec = np.zeros(1, AMP_STATE_DTYPE)
    rec["scale"] = init_scale
    rec["clip_coef"] = 1.0
    return torch.from_numpy(rec.view(np.uint8).copy()).to(device)


def read_amp_state(t: torch.Tensor) -> dict:
    """The fields of a device-side loss-scaler state (copies to the host)."""
    rec = t.detach().cpu().numpy().view(AMP_STATE_DTYPE)[0]
    return {k: rec[k].item() for k in AMP_STATE_DTYPE.names}


def fp8adam_stats(ctx: int, n: int, stream: int | None = None) -> list[dict]:
    out = (StatsArg * n)()
    _check(load().fp8adam_stats(ctx, out, n, current_stream() if stream is None else stream))
    return [s.as_dict() for s in out]


def fp8adam_destroy(ctx: int) -> None:
    load().fp8adam_destroy(ctx)


def fp8adam_last_error() -> str:
    return load().fp8adam_last_error().decode()


def fp8adam_encode(fmt: int, x: torch.Tensor, out: torch.Tensor, stream: int | None = None) -> None:
    assert x.dtype == torch.float32 and out.dtype == torch.uint8 and x.is_contiguous() and out.is_contiguous()
    assert out.numel() >= x.numel()
    _check(load().fp8adam_encode(fmt, _ptr(x), _ptr(out), x.numel(),
                                 current_stream() if stream is None else stream))


def fp8adam_decode(fmt: int, codes: torch.Tensor, out: torch.Tensor, stream: int | None = None) -> None:
    assert codes.dtype == torch.uint8 and out.dtype == torch.float32 and codes.is_contiguous() and out.is_contiguous()
    assert out.numel() >= codes.numel()
    _check(load().fp8adam_decode(fmt, _ptr(codes), _ptr(out), codes.numel(),
                                 current_stream() if stream is None else stream))


def fp8adam_encode_bits_range(fmt: int, start: int, count: int, out: torch.Tensor,
                              stream: int | None = None) -> None:
    assert out.dtype == torch.uint8 and out.is_contiguous() and out.numel() >= count
    _check(load().fp8adam_encode_bits_range(fmt, start, count, _ptr(out),
                                            current_stream() if stream is None else stream))


def fp8adam_encode_sr_bits_range(fmt: int, start: int, count: int, r16: int, out: torch.Tensor,
                                 stream: int | None = None) -> None:
    assert out.dtype == torch.uint8 and out.is_contiguous() and out.numel() >= count
    _check(load().fp8adam_encode_sr_bits_range(fmt, start, count, r16, _ptr(out),
                                               current_stream() if stream is None else stream))


def fp8adam_encode_sr(fmt: int, x: torch.Tensor, r16: torch.Tensor, out: torch.Tensor,
                      stream: int | None = None) -> None:
    assert x.dtype == torch.float32 and r16.dtype == torch.uint16 and out.dtype == torch.uint8
    assert x.is_contiguous() and r16.is_contiguous() and out.is_contiguous()
    assert r16.numel() == x.numel() and out.numel() >= x.numel()
    _check(load().fp8adam_encode_sr(fmt, _ptr(x), _ptr(r16), _ptr(out), x.numel(),
                                    current_stream() if stream is None else stream))


def fp8adam_stream_copy(src: torch.Tensor, dst: torch.Tensor, stream: int | None = None) -> None:
    assert src.is_contiguous() and dst.is_contiguous()
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nbytes
    _check(load().fp8adam_stream_copy(_ptr(src), _ptr(dst), nbytes, current_stream() if stream is None else stream))


def fp8adam_stream_rw(src: torch.Tensor | None, dst: torch.Tensor | None, stream: int | None = None) -> None:
    """Read all of src and write all of dst (a read-only stream if dst is None, a
    write-only one if src is None)."""
    nr = 0 if src is None else src.numel() * src.element_size()
    nw = 0 if dst is None else dst.numel() * dst.element_size()
    assert (src is None or src.is_contiguous()) and (dst is None or dst.is_contiguous())
    _check(load().fp8adam_stream_rw(_ptr(src), nr, _ptr(dst), nw, current_stream() if stream is None else stream))


def fp8adam_stream_mix(p: torch.Tensor, g: torch.Tensor, m_in: torch.Tensor, v_in: torch.Tensor,
                       m_out: torch.Tensor, v_out: torch.Tensor, stream: int | None = None) -> None:
    n = p.numel()
    assert p.dtype in (torch.float32, torch.bfloat16) and g.dtype == torch.bfloat16
    assert all(t.is_contiguous() for t in (p, g, m_in, v_in, m_out, v_out))
    assert g.numel() == n and all(t.dtype == torch.uint8 and t.numel() == n for t in (m_in, v_in, m_out, v_out))
    master = MASTER_BF16 if p.dtype == torch.bfloat16 else MASTER_FP32
    _check(load().fp8adam_stream_mix(master, _ptr(p), _ptr(g), _ptr(m_in), _ptr(v_in), _ptr(m_out), _ptr(v_out), n,
                                     current_stream() if stream is None else stream))


def fp8adam_set_timing(ctx: int, enable: bool) -> None:
    _check(load().fp8adam_set_timing(ctx, int(enable)))


def fp8adam_set_timing_kinds(ctx: int, kinds) -> None:
    """Time only the launches of the given kernel kinds (names of KERNEL_KINDS)."""
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS.index(k)
    _check(load().fp8adam_set_timing_kinds(ctx, mask))


def fp8adam_kernel_times(ctx: int) -> dict:
    n = len(KERNEL_KINDS)
    tot = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(load().fp8adam_kernel_times(ctx, tot, cnt, n))
    return {k: (tot[i], cnt[i]) for i, k in enumerate(KERNEL_KINDS)}


def fp8adam_runtime_version() -> int:
    v = ctypes.c_int32()
    _check(load().fp8adam_runtime_version(ctypes.byref(v)))
    return v.value


def fp8adam_num_chunks(ctx: int) -> int:
    return load().fp8adam_num_chunks(ctx)


def fp8adam_current_buffer(ctx: int) -> int:
    return load().fp8adam_current_buffer(ctx)


# ------------------------------------------------------------ torch wrapper

class FP8AdamW:
    """FP8-moment AdamW over lists of torch tensors on one GPU.

    params: fp32 or bf16 master weights (all the same dtype); grads: bf16, same
    numel as their parameter.  The moment codes (uint8) and scales (fp32) are
    allocated here and the library writes the fresh state into them (zero codes,
    unit scales, a zero amax history: the config's zero_state), unless ``state``
    supplies (m, v, m_scale, v_scale) lists.  With ``schedule="speculative"`` a second
    pair of code buffers is allocated and the moments alternate between the two;
    ``m`` and ``v`` always return the pair that holds them.  ``decay_mode="l2"``
    adds weight_decay * p to the gradient instead of decaying p (Adam on an
    L2-regularised loss); it cannot be combined with the speculative schedule.
    ``scaling="delayed"`` quantizes with the scale of the largest amax over the
    last ``amax_history_len`` steps (times 2^margin) in one pass; each tensor
    then carries a float32 history of 2 * amax_history_len entries
    (``amax_history``; a fifth ``state`` list supplies it).  ``rounding="stochastic"``
    rounds the moments stochastically with a Philox4x32-10 stream keyed by ``seed``.
    ``predictor`` chooses how the speculative schedule predicts each scale:
    ``"probe"`` (the exact amax over the parts that held the tensor's largest
    values at the step before), ``"growth"`` (the previous amax times its
    expected growth) or ``"auto"`` (the probe for lists of at least 2^28
    elements); the results are the same.  Every tensor must be
    contiguous and 16-byte aligned on the same device, and must stay alive with
    the same storage while this object exists.
    """

    def __init__(self, params, grads, *, m_format="e4m3", v_format="e5m2", granularity="tensor",
                 scale_mode="pow2", collect_stats=False, state=None, schedule="two_pass",
                 speculate_from_step=0, decay_mode="decoupled", scaling="just_in_time",
                 amax_history_len=16, margin=0, delayed_from_step=0, rounding="nearest", seed=0,
                 predictor="auto"):
        params, grads = list(params), list(grads)
        if len(params) != len(grads) or not params:
            raise ValueError("need one gradient per parameter and at least one parameter")
        master = params[0].dtype
        if master not in (torch.float32, torch.bfloat16):
            raise ValueError("master weights must be float32 or bfloat16")
        self.granularity = _GRAN[granularity]
        self.params, self.grads = params, grads
        fresh = state is None  # the library writes the fresh state (zero_state) into these buffers
        if fresh:
            m = [torch.empty(p.numel(), dtype=torch.uint8, device=p.device) for p in params]
            v = [torch.empty(p.numel(), dtype=torch.uint8, device=p.device) for p in params]
            # (the scales are written too; ones keep an empty tensor's unused slot defined)
            ms = [torch.ones(self.num_scales(p.numel()), dtype=torch.float32, device=p.device) for p in params]
            vs = [torch.ones(self.num_scales(p.numel()), dtype=torch.float32, device=p.device) for p in params]
            state = (m, v, ms, vs)
        m, v, self.m_scale, self.v_scale = [list(x) for x in state[:4]]
        delayed = _SCALING[scaling] == SCALING_DELAYED
        amax_history_len = int(amax_history_len) if int(amax_history_len) > 0 else 16  # the library's default
        if delayed and len(state) > 4:
            self.amax_history = list(state[4])
        elif delayed:
            self.amax_history = [(torch.empty if fresh else torch.zeros)(2 * amax_history_len, dtype=torch.float32,
                                                                         device=p.device) for p in params]
        else:
            self.amax_history = [None] * len(params)
        spec = _SCHED[schedule] == SCHEDULE_SPECULATIVE
        m_alt = [torch.empty_like(x) for x in m] if spec else [None] * len(m)
        v_alt = [torch.empty_like(x) for x in v] if spec else [None] * len(v)
        self._m, self._v = (m, m_alt), (v, v_alt)
        args = []
        for i, (p, g) in enumerate(zip(params, grads)):
            if p.dtype != master or g.dtype != torch.bfloat16 or p.numel() != g.numel():
                raise ValueError(f"tensor {i}: dtype or size mismatch")
            for t in (p, g, m[i], v[i], self.m_scale[i], self.v_scale[i]):
                if not t.is_contiguous() or t.device != p.device:
                    raise ValueError(f"tensor {i}: every buffer must be contiguous on one device")
            # the kernels read and write these sizes through plain pointers: check them here
            n, ns = p.numel(), self.num_scales(p.numel())
            if any(x.dtype != torch.uint8 or x.numel() != n for x in (m[i], v[i])):
                raise ValueError(f"tensor {i}: moment codes must be uint8 with one byte per element")
            if any(x.dtype != torch.float32 or x.numel() < ns for x in (self.m_scale[i], self.v_scale[i])):
                raise ValueError(f"tensor {i}: scales must be float32, at least {ns} of them")
            h = self.amax_history[i]
            if delayed and (h.dtype != torch.float32 or h.numel() != 2 * amax_history_len
                            or not h.is_contiguous() or h.device != p.device):
                raise ValueError(f"tensor {i}: amax_history must be {2 * amax_history_len} contiguous float32")
            args.append(TensorArg(p.data_ptr(), g.data_ptr(), m[i].data_ptr(), v[i].data_ptr(),
                                  self.m_scale[i].data_ptr(), self.v_scale[i].data_ptr(), p.numel(),
                                  _ptr(m_alt[i]), _ptr(v_alt[i]), _ptr(self.amax_history[i])))
        self.cfg = ConfigArg(_FORMATS[m_format], _FORMATS[v_format], self.granularity, _SMODE[scale_mode],
                             MASTER_BF16 if master == torch.bfloat16 else MASTER_FP32, int(collect_stats),
                             _SCHED[schedule], int(speculate_from_step), _DECAY[decay_mode],
                             _SCALING[scaling], int(amax_history_len), int(margin), int(delayed_from_step),
                             _ROUNDING[rounding], int(seed) & 0xFFFFFFFFFFFFFFFF, int(fresh), _PREDICT[predictor])
        self.n = len(params)
        self.device = params[0].device
        with torch.cuda.device(self.device):
            self._ctx = fp8adam_init(args, self.cfg)

    def num_scales(self, numel: int) -> int:
        return 1 if self.granularity == SCALE_TENSOR else max(1, -(-numel // BLOCK))

    @property
    def current_buffer(self) -> int:
        if getattr(self, "_ctx", None):
            self._last_cur = fp8adam_current_buffer(self._ctx)
        return getattr(self, "_last_cur", 0)

    @property
    def m(self) -> list:
        return self._m[self.current_buffer]

    @property
    def v(self) -> list:
        return self._v[self.current_buffer]

    def checkpoint(self) -> list:
        """Copies of the whole optimizer state in the form ``state=`` takes:
        [m, v, m_scale, v_scale] (m and v from the pair that holds the moments),
        plus the amax histories with delayed scaling.  Together with the master
        weights (and, for step_amp, the loss-scaler state) it resumes bit for bit."""
        with torch.cuda.device(self.device):
            torch.cuda.current_stream().synchronize()
            out = [[x.clone() for x in self.m], [x.clone() for x in self.v],
                   [x.clone() for x in self.m_scale], [x.clone() for x in self.v_scale]]
            if self.amax_history[0] is not None:
                out.append([x.clone() for x in self.amax_history])
        return out

    def step(self, *, lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
             weight_decay: float = 0.0, step: int) -> None:
        with torch.cuda.device(self.device):
            fp8adam_step(self._ctx, HParamsArg(lr, beta1, beta2, eps, weight_decay, step))

    def step_amp(self, amp_state: torch.Tensor, *, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                 eps: float = 1e-8, weight_decay: float = 0.0, step: int, max_norm: float = 0.0,
                 growth_factor: float = 2.0, backoff_factor: float = 0.5, growth_interval: int = 2000) -> None:
        """A step on gradients of (loss * scale): unscale, skip on Inf/NaN, clip the
        global norm to max_norm (if > 0), all on the device (``amp_state`` from
        ``amp_state()``).  ``step`` counts calls; the bias correction uses the
        state's count of taken steps."""
        if amp_state.dtype != torch.uint8 or amp_state.numel() != AMP_STATE_DTYPE.itemsize:
            raise ValueError("amp_state must be the 32-byte tensor from amp_state()")
        with torch.cuda.device(self.device):
            fp8adam_step_amp(self._ctx, HParamsArg(lr, beta1, beta2, eps, weight_decay, step),
                             AmpConfigArg(max_norm, growth_factor, backoff_factor, growth_interval),
                             amp_state.data_ptr())

    def stats(self) -> list[dict]:
        with torch.cuda.device(self.device):
            return fp8adam_stats(self._ctx, self.n)

    def set_timing(self, enable: bool, kinds=None) -> None:
        """Per-kernel timing of later steps: every kind, or only ``kinds`` (names of KERNEL_KINDS)."""
        if enable and kinds is not None:
            fp8adam_set_timing_kinds(self._ctx, kinds)
        else:
            fp8adam_set_timing(self._ctx, enable)

    def kernel_times(self) -> dict:
        return fp8adam_kernel_times(self._ctx)

    @property
    def num_chunks(self) -> int:
        return fp8adam_num_chunks(self._ctx)

    def close(self) -> None:
        if getattr(self, "_ctx", None):
            _ = self.current_buffer  # remember where the moments are
            torch.cuda.synchronize(self.device)
            fp8adam_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
