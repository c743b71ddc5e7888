"""Pins for the oracle's loss scaling, non-finite skip and global-norm clipping.

  * the sum of squares is exact: equal to the correctly rounded Fraction sum,
    including cases where plain fp64 accumulation is wrong;
  * the scaler's state machine (backoff on Inf/NaN, growth after
    growth_interval clean steps, a skipped step not counted as an Adam step)
    equals torch.amp.GradScaler on the CPU, step by step;
  * the clip coefficient and the whole AMP + clip + Adam trajectory (fp32
    moments) equal torch's clip_grad_norm_ + GradScaler + Adam in fp64.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def bf16_bits(x) -> np.ndarray:
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_vals(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def exact_sumsq(bits) -> float:
    return float(sum(Fraction(float(v)) ** 2 for v in bf16_vals(bits).astype(np.float64)))


@pytest.mark.parametrize("kind", ["all_patterns", "narrow", "subnormal", "cancel_free_tiny", "tie", "tie_odd", "tie_sticky"])
def test_sumsq_is_exact(kind):
    rng = np.random.default_rng(hash(kind) % 1000)
    if kind == "all_patterns":
        g = rng.integers(0, 65536, 3000).astype(np.uint16)
        g = g[((g >> 7) & 0xFF) != 0xFF]
    elif kind == "narrow":
        g = bf16_bits(rng.standard_normal(5000) * 1e-3)
    elif kind == "subnormal":
        g = rng.integers(0, 128, 500).astype(np.uint16) | (rng.integers(0, 2, 500).astype(np.uint16) << 15)
    elif kind == "tie":  # 1 + 2^-53: halfway between two doubles, rounds to the even one (1)
        g = bf16_bits([1.0, 2.0 ** -27, 2.0 ** -27])
    elif kind == "tie_odd":  # 1 + 2^-52 + 2^-53: halfway, the lower neighbour is odd: rounds up
        g = bf16_bits([1.0, 2.0 ** -26, 2.0 ** -27, 2.0 ** -27])
    elif kind == "tie_sticky":  # 1 + 2^-53 + 2^-70: just above halfway, rounds up
        g = bf16_bits([1.0, 2.0 ** -27, 2.0 ** -27, 2.0 ** -35])
    else:
        # one large value and many tiny ones: a plain fp64 running sum drops the tiny squares
        g = np.concatenate([bf16_bits([1.0]), bf16_bits(np.full(4096, 2.0 ** -30))])
    s = oracle.GradSums().add(g)
    assert s.total() == exact_sumsq(g)
    assert s.nonfinite.value == 0
    if kind == "tie":
        assert s.total() == 1.0
    if kind == "tie_odd":
        assert s.total() == 1.0 + 2.0 ** -51
    if kind == "tie_sticky":
        assert s.total() == 1.0 + 2.0 ** -52
    if kind == "cancel_free_tiny":
        naive = 0.0
        for v in bf16_vals(g).astype(np.float64):
            naive += v * v
        assert naive != s.total()  # 1 + 4096 * 2^-60 is not representable; exact rounding is 1 + 2^-48
        assert s.total() == 1.0 + 2.0 ** -48


def test_sumsq_accumulates_over_tensors_and_counts_nonfinite():
    rng = np.random.default_rng(4)
    a = bf16_bits(rng.standard_normal(300))
    b = bf16_bits(rng.standard_normal(200) * 1e4)
    b[[3, 77]] = [0x7F80, 0xFFC1]  # +Inf, a NaN
    s = oracle.GradSums().add(a).add(b)
    assert s.nonfinite.value == 2
    finite_b = np.delete(b, [3, 77])
    assert s.total() == exact_sumsq(np.concatenate([a, finite_b]))


def test_scaler_state_machine_matches_torch_gradscaler():
    """Same overflow pattern into torch.amp.GradScaler (CPU) and the oracle:
    scale and growth tracker equal after every step, and torch Adam's step
    count equals the oracle's (skipped steps do not count)."""
    pattern = [0, 1, 0, 0, 0, 0, 1, 1, 0, 0, 0, 0, 0, 0, 0]
    init, interval = 2.0 ** 16, 3
    ts = torch.amp.GradScaler("cpu", init_scale=init, growth_factor=2.0, backoff_factor=0.5,
                              growth_interval=interval)
    p = torch.nn.Parameter(torch.ones(4, dtype=torch.float64))
    opt = torch.optim.Adam([p], lr=1e-3)
    cfg = oracle.AmpConfig(0.0, 2.0, 0.5, interval)
    st = oracle.AmpState(scale=init)
    for bad in pattern:
        g = np.full(4, 1.0, np.float32) * float(ts.get_scale())
        if bad:
            g[1] = np.inf
        ts.scale(torch.tensor(1.0, dtype=torch.float64))
        p.grad = torch.tensor(g.astype(np.float64))
        ts.unscale_(opt)
        ts.step(opt)
        ts.update()
        # the oracle sees the same gradient as bf16 (the scale is a power of two: exact)
        oracle.amp_control(oracle.GradSums().add(bf16_bits(g)), cfg, st)
        assert st.found_inf == bad
        assert st.scale == ts.get_scale()
        assert st.growth_tracker == int(ts._growth_tracker.item())
        torch_steps = int(opt.state[p]["step"].item()) if "step" in opt.state.get(p, {}) else 0
        assert st.step == torch_steps


@pytest.mark.parametrize("max_norm", [1.0, 0.05, 1e6])
def test_clip_matches_torch_clip_grad_norm(max_norm):
    """Three tensors, scale 2^10: the oracle's norm of the unscaled gradients
    and its clip coefficient (fp32) equal torch's fp64 clip_grad_norm_ rounded
    to fp32; max_norm 1e6 does not clip (coefficient 1)."""
    rng = np.random.default_rng(int(max_norm * 10) % 97)
    S = 2.0 ** 10
    grads = [bf16_bits(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0, n) * S) for n in (100, 257, 33)]
    params = [torch.nn.Parameter(torch.zeros(len(g), dtype=torch.float64)) for g in grads]
    for p, g in zip(params, grads):
        p.grad = torch.tensor(bf16_vals(g).astype(np.float64) / S)
    tn = torch.nn.utils.clip_grad_norm_(params, max_norm)
    coef = min(1.0, max_norm / (float(tn) + 1e-6))
    sums = oracle.GradSums()
    for g in grads:
        sums.add(g)
    st = oracle.amp_control(sums, oracle.AmpConfig(max_norm, 2.0, 0.5, 2000), oracle.AmpState(scale=S))
    assert st.found_inf == 0 and st.step == 1
    assert st.grad_norm == np.float32(float(tn))
    assert st.clip_coef == np.float32(coef)
    assert st.grad_factor == np.float32(np.float32(coef) * np.float32(1.0 / S))
    if max_norm >= 1e6:
        assert st.clip_coef == 1.0


def test_amp_adam_trajectory_matches_torch():
    """AMP + clip + Adam end to end: 12 steps with two overflow steps, scale
    growth every 4 clean steps, clipping at 0.1.  torch: GradScaler (CPU),
    clip_grad_norm_, Adam, all fp64.  Oracle: amp_control, then (unless
    skipped) the fp32-moment step with the gradient factor and t = the
    scaler's step count.  Weights agree to fp32 accuracy."""
    n = 64
    rng = np.random.default_rng(8)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    lr, b1, b2, eps = 1e-3, 0.9, 0.95, 1e-8
    f32 = lambda x: float(np.float32(x))
    tp = torch.nn.Parameter(torch.tensor(p0.astype(np.float64)))
    opt = torch.optim.Adam([tp], lr=f32(lr), betas=(f32(b1), f32(b2)), eps=f32(eps))
    ts = torch.amp.GradScaler("cpu", init_scale=2.0 ** 12, growth_factor=2.0, backoff_factor=0.5,
                              growth_interval=4)
    cfg = oracle.AmpConfig(0.1, 2.0, 0.5, 4)
    st = oracle.AmpState(scale=2.0 ** 12)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    skipped = 0
    for k in range(12):
        raw = rng.standard_normal(n) * 10.0 ** rng.uniform(-3, -1, n)
        g = bf16_bits(raw * float(ts.get_scale()))
        if k in (2, 7):
            g[5] = 0x7F80
        ts.scale(torch.tensor(1.0, dtype=torch.float64))
        tp.grad = torch.tensor(bf16_vals(g).astype(np.float64))
        ts.unscale_(opt)
        torch.nn.utils.clip_grad_norm_([tp], 0.1)
        ts.step(opt)
        ts.update()
        oracle.amp_control(oracle.GradSums().add(g), cfg, st)
        if st.found_inf:
            skipped += 1
            continue
        h = oracle.Hyper(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=0.0, step=st.step)
        oracle.step_fp32_moments(oracle.make_config(h, grad_factor=st.grad_factor), p, g, m, v)
        assert st.scale == ts.get_scale()
    assert skipped == 2 and st.step == 10
    ref = tp.detach().numpy()
    assert np.allclose(p, ref, rtol=1e-5, atol=1e-6 * lr)
