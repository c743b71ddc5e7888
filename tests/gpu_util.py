"""Helpers shared by the GPU tests: run the HIP step through the C ABI and the
CPU oracle on the same seeded inputs, and compare them.

Comparison bar (written out in the tests):
  * FP8 codes and scales: bit-exact;
  * fp32 master weights: |p_gpu - p_ref| <= 1e-6 * max(|p_ref|, |p_old|)
    (the error bound of p*(1-lr*wd) - update relative to its operands);
  * bf16 master weights: |p_gpu - p_ref| <= ulp_bf16(p_ref) + 1e-6 * max(|p_ref|,
    |p_old|), and at most 1e-3 of the elements not bit-equal (the fp32 update
    rounds to bf16 from a value within a few fp32 ulps of the oracle's fp64
    one, so it can land on the other side of a rounding midpoint);
  * stats counts and amax: equal.
Every comparison is of ONE step from a common state: after each step the
tests upload the oracle's weights into the GPU buffers (codes and scales are
already bit-equal), so rounding differences do not accumulate across steps.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle
import workloads

FMT_ID = {"e4m3": 0, "e5m2": 1}


def np_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def np_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return np_u16(t)
    return t.detach().cpu().contiguous().numpy().copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def pool_size() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class OracleState:
    """Host copy of one tensor's optimizer state, advanced by the oracle."""

    def __init__(self, p: np.ndarray, cm: np.ndarray, cv: np.ndarray, sm: np.ndarray, sv: np.ndarray,
                 hist: np.ndarray | None = None):
        self.p, self.cm, self.cv, self.sm, self.sv = p, cm, cv, sm, sv
        self.hist = hist  # delayed scaling: the amax history (2H float32), else None
        self.p_old = p.copy()
        self.stats = None

    def step(self, cfg: oracle.Config, g_bits: np.ndarray) -> dict:
        self.p_old = self.p.copy()
        if self.hist is not None:
            self.stats = oracle.step_hist(cfg, self.p, g_bits, self.cm, self.cv, self.sm, self.sv, self.hist)
        else:
            self.stats = oracle.step(cfg, self.p, g_bits, self.cm, self.cv, self.sm, self.sv)
        return self.stats


def oracle_config(h: oracle.Hyper, m_fmt: str, v_fmt: str, granularity: str, scale_mode: str,
                  master: str, decay_mode: str = "decoupled", history_len: int = 0, margin: int = 0,
                  delayed_from: int = 2) -> oracle.Config:
    return oracle.make_config(h, FMT_ID[m_fmt], FMT_ID[v_fmt], block=128 if granularity == "block128" else 0,
                              scale_mode=oracle.SCALE_AMAX if scale_mode == "amax" else oracle.SCALE_POW2,
                              master_bf16=(master == "bf16"), l2_coupled=(decay_mode == "l2"),
                              history_len=history_len, margin=margin, delayed_from=delayed_from)


def compare_tensor(name: str, st: OracleState, p_gpu: np.ndarray, cm_gpu: np.ndarray, cv_gpu: np.ndarray,
                   sm_gpu: np.ndarray, sv_gpu: np.ndarray, master: str) -> None:
    """Raise AssertionError with a description if the GPU result is off the bar."""
    n = st.p.size
    if not np.array_equal(cm_gpu, st.cm):
        bad = np.nonzero(cm_gpu != st.cm)[0]
        raise AssertionError(f"{name}: {bad.size}/{n} m codes differ, first at {bad[0]}: "
                             f"gpu {cm_gpu[bad[0]]:#04x} oracle {st.cm[bad[0]]:#04x}")
    if not np.array_equal(cv_gpu, st.cv):
        bad = np.nonzero(cv_gpu != st.cv)[0]
        raise AssertionError(f"{name}: {bad.size}/{n} v codes differ, first at {bad[0]}: "
                             f"gpu {cv_gpu[bad[0]]:#04x} oracle {st.cv[bad[0]]:#04x}")
    if not (np.array_equal(sm_gpu.view(np.uint32), st.sm.view(np.uint32))
            and np.array_equal(sv_gpu.view(np.uint32), st.sv.view(np.uint32))):
        raise AssertionError(f"{name}: scales differ: gpu {sm_gpu[:4]} {sv_gpu[:4]} oracle {st.sm[:4]} {st.sv[:4]}")
    if master == "bf16":
        got = bf16_to_f32(p_gpu).astype(np.float64)
        ref = bf16_to_f32(st.p).astype(np.float64)
        old = bf16_to_f32(st.p_old).astype(np.float64)
        ulp = np.spacing(np.abs(bf16_to_f32(st.p))).astype(np.float64) * 65536.0  # fp32 spacing * 2^16
        ulp = np.maximum(ulp, 2.0 ** -133)
        tol = ulp + 1e-6 * np.maximum(np.abs(ref), np.abs(old))
        err = np.abs(got - ref)
        if not (err <= tol).all():
            i = int(np.argmax(err - tol))
            raise AssertionError(f"{name}: bf16 weight off by {err[i]:.3e} (tol {tol[i]:.3e}) at {i}: "
                                 f"gpu {p_gpu[i]:#06x} oracle {st.p[i]:#06x} old {st.p_old[i]:#06x}")
        ndiff = int((p_gpu != st.p).sum())
        if ndiff > max(1, 1e-3 * n):
            raise AssertionError(f"{name}: {ndiff}/{n} bf16 weights not bit-equal (allowed 1e-3)")
    else:
        tol = 1e-6 * np.maximum(np.abs(st.p), np.abs(st.p_old))
        err = np.abs(p_gpu.astype(np.float64) - st.p.astype(np.float64))
        if not (err <= tol).all():
            i = int(np.argmax(err - tol))
            raise AssertionError(f"{name}: weights off by {err[i]:.3e} (tol {tol[i]:.3e}) at {i}: "
                                 f"gpu {p_gpu[i]!r} oracle {st.p[i]!r} old {st.p_old[i]!r}")


def upload_params(param: torch.Tensor, st: OracleState) -> None:
    """Put the oracle's weights into the GPU buffer (host -> device), so the
    next step of both sides starts from the same state."""
    src = torch.from_numpy(st.p.copy())
    if param.dtype == torch.bfloat16:
        src = src.view(torch.int16).view(torch.bfloat16)
    param.copy_(src.to(param.device))


def random_grad(n: int, seed: int, device, lo: float = -7.0, hi: float = 1.0) -> torch.Tensor:
    """bf16 gradient with a log-uniform scale per call, exact zeros and
    negative zeros mixed in."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn(n, generator=g, device=device)
    sc = 10.0 ** (lo + (hi - lo) * torch.rand(n, generator=g, device=device))
    x = z * sc
    u = torch.rand(n, generator=g, device=device)
    x = torch.where(u < 0.05, torch.zeros_like(x), x)
    x = torch.where(u > 0.97, -torch.zeros_like(x), x)
    return x.to(torch.bfloat16)


def run_pool(fn, items):
    with cf.ThreadPoolExecutor(pool_size()) as ex:
        return list(ex.map(fn, items))
