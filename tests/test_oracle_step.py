"""Pins for the oracle's FP8-moment AdamW step (CPU only).

Pinned against:
  * closed forms of bias-corrected Adam/AdamW on a constant gradient, with the
    codec taken out (fp32 moments);
  * torch.optim.AdamW on the CPU in float64 (library), same codec-free mode;
  * an exact FP8 trajectory that follows from dyadic arithmetic (g = 1,
    betas 0.5): every moment is 1 - 2^-t, so the stored codes are known by hand;
  * the exact-rational referee (tests/referee/rational.py) on tiny tensors,
    over formats, scale modes, block and tensor granularity and bf16 master;
  * the worked example at step level, and the Fig. 5 direction (v in E4M3
    underflows far more than v in E5M2);
  * invariants: no saturation under just-in-time power-of-two scaling, the amax
    element lands in the top binade, v codes are non-negative, a 128-element
    tensor gives the same result in block and tensor mode.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.referee import rational

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_vals(bits) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32(x) -> float:
    return float(np.float32(x))


# ----------------------------------------------------------- closed forms

@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_fp32_moments_constant_gradient_closed_form(wd):
    """With constant g, the bias-corrected moments are g and g^2, so every step
    moves p by lr*g/(|g|+eps) (plus decoupled decay c = 1 - lr*wd):
    p_t = c^t p_0 - lr*u*(1 - c^t)/(1 - c)   (or p_0 - t*lr*u when wd = 0)."""
    n = 64
    rng = np.random.default_rng(0)
    g = bf16_bits(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0, n))
    gv = bf16_vals(g).astype(np.float64)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p = p0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    h = oracle.Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    T = 25
    for t in range(1, T + 1):
        h.step = t
        oracle.step_fp32_moments(oracle.make_config(h), p, g, m, v)
    lr, eps = f32(h.lr), f32(h.eps)
    u = gv / (np.abs(gv) + eps)
    c = 1.0 - lr * f32(wd)
    if wd == 0.0:
        want = p0.astype(np.float64) - T * lr * u
    else:
        want = c ** T * p0 - lr * u * (1 - c ** T) / (1 - c)
    # fp32 moment rounding only: a few parts in 1e7 of the accumulated update
    assert np.allclose(p, want, rtol=0, atol=2e-6 * T * lr)


def test_fp32_moments_match_torch_adamw():
    n = 300
    rng = np.random.default_rng(1)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    h = oracle.Hyper(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    tp = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=f32(h.lr), betas=(f32(h.beta1), f32(h.beta2)),
                            eps=f32(h.eps), weight_decay=f32(h.weight_decay))
    p = p0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 11):
        g = bf16_bits(rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 0, n))
        h.step = t
        oracle.step_fp32_moments(oracle.make_config(h), p, g, m, v)
        tp.grad = torch.tensor(bf16_vals(g).astype(np.float64))
        opt.step()
    ref = tp.detach().numpy()
    assert np.allclose(p, ref, rtol=1e-6, atol=1e-6 * f32(h.lr))


def test_fp32_moments_coupled_l2_match_torch_adam():
    """Coupled L2 (the L2-regularised objective): torch.optim.Adam's weight_decay
    adds wd*p to the gradient, as the oracle's l2_coupled variant does."""
    n = 300
    rng = np.random.default_rng(2)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    h = oracle.Hyper(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    tp = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.Adam([tp], lr=f32(h.lr), betas=(f32(h.beta1), f32(h.beta2)), eps=f32(h.eps),
                           weight_decay=f32(h.weight_decay))
    p = p0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 11):
        g = bf16_bits(rng.standard_normal(n) * 10.0 ** rng.uniform(-5, -1, n))
        h.step = t
        oracle.step_fp32_moments(oracle.make_config(h, l2_coupled=True), p, g, m, v)
        tp.grad = torch.tensor(bf16_vals(g).astype(np.float64))
        opt.step()
    ref = tp.detach().numpy()
    assert np.allclose(p, ref, rtol=1e-5, atol=1e-6 * f32(h.lr))
    # and it is not the decoupled update
    p2, m2, v2 = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    rng = np.random.default_rng(2)
    rng.standard_normal(n)
    for t in range(1, 11):
        g = bf16_bits(rng.standard_normal(n) * 10.0 ** rng.uniform(-5, -1, n))
        h.step = t
        oracle.step_fp32_moments(oracle.make_config(h), p2, g, m2, v2)
    assert not np.allclose(p2, ref, rtol=1e-5, atol=1e-6 * f32(h.lr))


def test_exact_fp8_trajectory_dyadic():
    """g = 1, beta1 = beta2 = 0.5: the fresh moments are 1 - 2^-t exactly and the
    power-of-two scale puts them just under the format maximum.
    t=3: m' = 0.875 = FMAX * 2^-9 exactly -> code 0x7E, no saturation.
    t=4: v' = 0.9375 needs 4 significant bits; E5M2 keeps 3 -> tie, rounds to even (1.0).
    t=5: m' = 0.96875 needs 5 bits; E4M3 keeps 4 -> tie, rounds to even (1.0)."""
    h = oracle.Hyper(lr=1e-3, beta1=0.5, beta2=0.5, eps=1e-8, weight_decay=0.0)
    p = np.zeros(1, np.float32)
    g = bf16_bits([1.0])
    cm, cv = np.zeros(1, np.uint8), np.zeros(1, np.uint8)
    sm, sv = np.ones(1, np.float32), np.ones(1, np.float32)
    seen = {}
    for t in range(1, 7):
        h.step = t
        st = oracle.step(oracle.make_config(h), p, g, cm, cv, sm, sv)
        seen[t] = (int(cm[0]), float(sm[0]), int(cv[0]), float(sv[0]), st)
    # t=1: 0.5 = 0.875*2^9 ... stored as 256 * 2^-9 -> E4M3 256 = 1.0*2^8 -> code 0x78
    assert seen[1][:4] == (0x78, 2.0 ** -9, 0x78, 2.0 ** -16)
    # t=2: 0.75 -> 384 * 2^-9 = 1.5*2^8 (0x7C);  E5M2 0.75*2^16 = 1.5*2^15 (0x7A)
    assert seen[2][:4] == (0x7C, 2.0 ** -9, 0x7A, 2.0 ** -16)
    # t=3: 0.875 -> 448 * 2^-9, exactly FMAX: code 0x7E and not saturated
    assert seen[3][0] == 0x7E and seen[3][1] == 2.0 ** -9 and seen[3][4]["saturated_m"] == 0
    assert seen[3][2:4] == (0x7B, 2.0 ** -16)
    # t=4: m' = 0.9375 > 0.875 -> scale 2^-8, 240 = 1.875*2^7 (0x77);
    #      v' = 0.9375 -> scale 2^-15: 30720 = 1.875*2^14, tie between 1.75 and 2.0 -> 2.0*2^14 (0x78)
    assert seen[4][:4] == (0x77, 2.0 ** -8, 0x78, 2.0 ** -15)
    # t=5: m (stored 0.9375) -> m' = 0.96875: 248 = 1.9375*2^7, tie -> 2.0*2^7 (0x78)
    assert seen[5][0] == 0x78 and seen[5][1] == 2.0 ** -8
    # stored v was 1.0 at t=4, so v' at t=5 is exactly 1.0
    assert seen[5][4]["amax_v"] == 1.0


def test_update_from_codes_reading_on_the_dyadic_trajectory():
    """The other reading of the update order (an oracle flag for study, outside
    the contract): p moves with the stored moments, code x new scale, instead
    of the fresh m', v'.  On the dyadic trajectory above the stored values are
    known by hand (m: 0.5, 0.75, 0.875, 0.9375, 1.0; v: 0.5, 0.75, 0.875, 1.0,
    1.0), so each update is lr * (m/(1-2^-t)) / (sqrt(v/(1-2^-t)) + eps); it
    equals the contract's reading while the moments are stored exactly (t <= 3)
    and departs from it once a tie rounds v (t = 4) and then m (t = 5)."""
    lr, eps = 1e-3, 1e-8
    stored_m = [0.5, 0.75, 0.875, 0.9375, 1.0]
    stored_v = [0.5, 0.75, 0.875, 1.0, 1.0]
    # the fresh moments: 0.5 * (stored value of the step before) + 0.5
    fresh_m = [0.5, 0.75, 0.875, 0.9375, 0.96875]
    fresh_v = [0.5, 0.75, 0.875, 0.9375, 1.0]
    runs = {}
    for flag in (False, True):
        h = oracle.Hyper(lr=lr, beta1=0.5, beta2=0.5, eps=eps, weight_decay=0.0)
        p = np.zeros(1, np.float32)
        g = bf16_bits([1.0])
        cm, cv = np.zeros(1, np.uint8), np.zeros(1, np.uint8)
        sm, sv = np.ones(1, np.float32), np.ones(1, np.float32)
        deltas = []
        for t in range(1, 6):
            h.step = t
            before = float(p[0])
            oracle.step(oracle.make_config(h, update_from_codes=flag), p, g, cm, cv, sm, sv)
            deltas.append(before - float(p[0]))
        runs[flag] = deltas
    for t in range(1, 6):
        bc = 1.0 - 0.5 ** t
        want_b = lr * (stored_m[t - 1] / bc) / (math.sqrt(stored_v[t - 1] / bc) + eps)
        want_a = lr * (fresh_m[t - 1] / bc) / (math.sqrt(fresh_v[t - 1] / bc) + eps)
        assert runs[True][t - 1] == pytest.approx(want_b, rel=1e-5), t
        assert runs[False][t - 1] == pytest.approx(want_a, rel=1e-5), t
    assert runs[True][:3] == pytest.approx(runs[False][:3], rel=1e-6)
    assert abs(runs[True][3] - runs[False][3]) > 0.02 * lr   # t = 4: v rounded up by a tie
    assert abs(runs[True][4] - runs[False][4]) > 0.01 * lr   # t = 5: m rounded up by a tie


# --------------------------------------------------- exact-rational referee

def _rand_case(n, seed, m_fmt, v_fmt, block, amax_mode, bf16_master):
    rng = np.random.default_rng(seed)
    mags = 10.0 ** rng.uniform(-9, 1, n)
    g = rng.standard_normal(n) * mags
    g[rng.random(n) < 0.1] = 0.0
    g[rng.random(n) < 0.05] = -0.0
    gb = bf16_bits(g)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p[rng.random(n) < 0.05] = 0.0
    if bf16_master:
        p = bf16_bits(p)
    nb = 1 if block == 0 else -(-n // block)
    cm, cv, sm, sv = workloads.random_state(n, "cpu", seed + 99, m_fmt, v_fmt, nblocks=nb,
                                            scale_exp=(-24, 2), pow2=not amax_mode)
    return p, gb, cm.numpy(), cv.numpy(), sm.numpy(), sv.numpy()


def _ulp_diff_f32(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


CASES = [
    # n, m_fmt, v_fmt, block, amax_mode, bf16_master, steps
    (1, 0, 1, 0, False, False, 3),
    (3, 0, 1, 0, False, False, 3),
    (37, 0, 1, 0, False, False, 3),
    (129, 0, 1, 0, False, False, 2),
    (129, 1, 1, 0, False, False, 2),
    (64, 1, 0, 0, False, False, 2),
    (64, 0, 0, 0, False, False, 2),
    (300, 0, 1, 128, False, False, 2),
    (200, 0, 1, 0, True, False, 2),
    (150, 0, 1, 128, True, False, 2),
    (96, 0, 1, 0, False, True, 2),
    (140, 0, 1, 0, False, False, 3, True),
    (130, 0, 1, 128, False, True, 2, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}_m{c[1]}v{c[2]}_b{c[3]}_{'amax' if c[4] else 'pow2'}_{'bf16' if c[5] else 'f32'}{'_l2' if len(c) > 7 else ''}" for c in CASES])
def test_oracle_equals_rational_referee(case):
    n, m_fmt, v_fmt, block, amax_mode, bf16_master, steps = case[:7]
    l2 = len(case) > 7 and case[7]
    p, g0, cm, cv, sm, sv = _rand_case(n, 11 + n, m_fmt, v_fmt, block, amax_mode, bf16_master)
    h = oracle.Hyper(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    rp = [float(x) for x in (bf16_vals(p) if bf16_master else p)]
    rcm, rcv = [int(x) for x in cm], [int(x) for x in cv]
    rsm, rsv = [float(x) for x in sm], [float(x) for x in sv]
    rng = np.random.default_rng(5 + n)
    for t in range(1, steps + 1):
        g = g0 if t == 1 else bf16_bits(rng.standard_normal(n) * 10.0 ** rng.uniform(-9, 1, n))
        h.step = t
        cfg = oracle.make_config(h, m_fmt, v_fmt, block=block,
                                 scale_mode=oracle.SCALE_AMAX if amax_mode else oracle.SCALE_POW2,
                                 master_bf16=bf16_master, l2_coupled=l2)
        oracle.step(cfg, p, g, cm, cv, sm, sv)
        rp, rcm, rcv, rsm, rsv = rational.step(
            rp, [float(x) for x in bf16_vals(g)], rcm, rcv, rsm, rsv,
            lr=f32(h.lr), b1=f32(h.beta1), b2=f32(h.beta2), eps=f32(h.eps),
            wd=f32(h.weight_decay), t=t, m_fmt=m_fmt, v_fmt=v_fmt, block=block,
            amax_mode=amax_mode, master_bf16=bf16_master, l2_coupled=l2)
        assert list(cm) == rcm, f"m codes differ at step {t}"
        assert list(cv) == rcv, f"v codes differ at step {t}"
        assert list(sm) == rsm and list(sv) == rsv, f"scales differ at step {t}"
        if bf16_master:
            got = bf16_vals(p)
            want = np.array(rp, np.float32)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        else:
            d = _ulp_diff_f32(p, np.array(rp, np.float32))
            assert d.max() <= 1, f"p differs by {d.max()} ulp at step {t}"
        # keep both sides on the same parameters so ulp-level drift cannot grow
        rp = [float(x) for x in (bf16_vals(p) if bf16_master else p)]


def test_referee_rejects_planted_moment_bug():
    """A dropped (1 - beta1) factor in the moment update must change codes."""
    n = 64
    p, g, cm, cv, sm, sv = _rand_case(n, 3, 0, 1, 0, False, False)
    rp = [float(x) for x in p]
    args = dict(lr=3e-4, b1=f32(0.9), b2=f32(0.95), eps=f32(1e-8), wd=0.0, t=1)
    good = rational.step(rp, [float(x) for x in bf16_vals(g)], list(map(int, cm)),
                         list(map(int, cv)), list(map(float, sm)), list(map(float, sv)), **args)
    orig = rational.mul32
    try:
        rational.mul32 = lambda a, b: orig(1.0, b) if a == rational.sub32(1.0, f32(0.9)) else orig(a, b)
        bad = rational.step(rp, [float(x) for x in bf16_vals(g)], list(map(int, cm)),
                            list(map(int, cv)), list(map(float, sm)), list(map(float, sv)), **args)
    finally:
        rational.mul32 = orig
    assert good[1] != bad[1]


# --------------------------------------------------- worked example, Fig. 5

def test_worked_example_at_step_level():
    """Two elements whose fresh v' are about 1e-4 and 100 (gradients 0.0447 and
    44.7 at t=1 with beta2 = 0.95): with v in E5M2 the small v survives the
    per-tensor scale (code nonzero, about 1e-4 after decode); with v in E4M3 it
    flushes to a zero code, so the next step sees v = 0 (the example's blow-up)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    g_small = math.sqrt(ex["v_small"] / 0.05)
    g = bf16_bits([g_small, math.sqrt(100.0 / 0.05)])
    res = {}
    for v_fmt in (oracle.E5M2, oracle.E4M3):
        p = np.zeros(2, np.float32)
        cm, cv = np.zeros(2, np.uint8), np.zeros(2, np.uint8)
        sm, sv = np.ones(1, np.float32), np.ones(1, np.float32)
        h = oracle.Hyper(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, step=1)
        st = oracle.step(oracle.make_config(h, oracle.E4M3, v_fmt), p, g, cm, cv, sm, sv)
        vstored = oracle.decode(v_fmt, cv) * sv[0]
        res[v_fmt] = (cv.copy(), vstored, st)
    cv5, vs5, st5 = res[oracle.E5M2]
    cv4, vs4, st4 = res[oracle.E4M3]
    assert cv5[0] != 0 and abs(vs5[0] - ex["v_small"]) / ex["v_small"] < 0.1
    assert cv4[0] == 0 and vs4[0] == 0.0 and st4["underflow_v"] == 1 and st5["underflow_v"] == 0
    # the stored second moments give 1/sqrt(v) ~ 100 vs a 1/(0+eps) blow-up
    assert abs(1.0 / math.sqrt(vs5[0]) - ex["inv_sqrt_v_small"]) < 5.0
    assert 1.0 / (math.sqrt(vs4[0]) + 1e-8) >= 1e7


def test_fig5_direction_v_underflow():
    """On a scaled-down Llama-2-100M-shaped list with the same gradient scales,
    v stored in E4M3 underflows far more elements than v stored in E5M2."""
    w = workloads.llama2_100m()
    shapes = workloads.scaled_llama(workloads.LLAMA2_100M, n_layers=2, d=128, ffn=344, vocab=1000)
    under = {}
    for m_fmt, v_fmt in [(0, 1), (1, 1), (1, 0), (0, 0)]:
        tot = 0
        for ti, (_, shape) in enumerate(shapes):
            n = workloads.numel(shape)
            p = workloads.make_param(w, ti, shape, "cpu").numpy().copy()
            cm, cv, sm, sv = [x.numpy().copy() for x in workloads.make_state(n, "cpu")]
            for t in range(1, 4):
                g = workloads.make_grad(w, ti, shape, t, "cpu").view(torch.int16).numpy().view(np.uint16).copy()
                h = oracle.Hyper(step=t)
                st = oracle.step(oracle.make_config(h, m_fmt, v_fmt), p, g, cm, cv, sm, sv)
                tot += st["underflow_v"]
        under[(m_fmt, v_fmt)] = tot
    assert under[(0, 0)] > 20 * max(1, under[(0, 1)])
    assert under[(1, 0)] > 20 * max(1, under[(1, 1)])


# ------------------------------------------------------------- invariants

def test_invariants_random_tensor():
    n = 50_000
    rng = np.random.default_rng(9)
    for v_fmt in (oracle.E5M2, oracle.E4M3):
        p = (rng.standard_normal(n) * 0.02).astype(np.float32)
        cm, cv, sm, sv = [x.numpy().copy() for x in workloads.make_state(n, "cpu")]
        for t in range(1, 5):
            g = bf16_bits(rng.standard_normal(n) * 10.0 ** rng.uniform(-7, 0, n))
            st = oracle.step(oracle.make_config(oracle.Hyper(step=t), oracle.E4M3, v_fmt),
                             p, g, cm, cv, sm, sv)
            assert st["saturated_m"] == 0 and st["saturated_v"] == 0
            assert (cv & 0x80).max() == 0  # v never negative
            # the largest element sits in the top binade: value >= FMAX/2
            assert oracle.decode(oracle.E4M3, cm).__abs__().max() >= oracle.format_max(0) / 2
            assert oracle.decode(v_fmt, cv).max() >= oracle.format_max(v_fmt) / 2
            assert st["scale_m"] == sm[0] and st["scale_v"] == sv[0]


def test_block_mode_on_one_block_equals_tensor_mode():
    n = 128
    rng = np.random.default_rng(4)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    outs = []
    for block in (0, 128):
        p = p0.copy()
        cm, cv, sm, sv = [x.numpy().copy() for x in workloads.make_state(n, "cpu")]
        for t in range(1, 4):
            g = bf16_bits(np.random.default_rng(t).standard_normal(n) * 1e-3)
            oracle.step(oracle.make_config(oracle.Hyper(step=t), block=block), p, g, cm, cv, sm, sv)
        outs.append((p, cm, cv, sm, sv))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def test_zero_gradient_first_step():
    n = 10
    p = np.full(n, 0.5, np.float32)
    cm, cv, sm, sv = [x.numpy().copy() for x in workloads.make_state(n, "cpu")]
    g = np.zeros(n, np.uint16)
    st = oracle.step(oracle.make_config(oracle.Hyper(step=1, weight_decay=0.0)), p, g, cm, cv, sm, sv)
    assert (cm == 0).all() and (cv == 0).all() and sm[0] == 1.0 and sv[0] == 1.0
    assert (p == 0.5).all() and st["amax_m"] == 0.0


def test_rejects_bad_arguments():
    cfg = oracle.make_config(oracle.Hyper(step=0))
    with pytest.raises(ValueError):
        oracle.step(cfg, np.zeros(1, np.float32), np.zeros(1, np.uint16), np.zeros(1, np.uint8),
                    np.zeros(1, np.uint8), np.ones(1, np.float32), np.ones(1, np.float32))


def test_nonfinite_count_closed_form():
    """An infinite gradient makes g*g and v' infinite (and m' infinite): exactly
    one non-finite element; the tensor's amax is then non-finite and the scale 1."""
    n = 8
    g = bf16_bits([1e-3] * n)
    g[3] = 0x7F80  # +Inf in bf16
    p = np.zeros(n, np.float32)
    cm, cv, sm, sv = [x.numpy().copy() for x in workloads.make_state(n, "cpu")]
    st = oracle.step(oracle.make_config(oracle.Hyper(step=1)), p, g, cm, cv, sm, sv)
    assert st["nonfinite"] == 1
    assert sm[0] == 1.0 and sv[0] == 1.0


# ------------------------------------------------------------ delayed scaling

DELAYED = [
    # H, margin, amax_mode, m_fmt, v_fmt, bf16_master
    (1, 0, False, 0, 1, False),
    (3, 0, False, 0, 1, False),
    (3, 2, False, 0, 1, True),
    (2, 1, True, 0, 1, False),
    (4, 0, False, 1, 0, False),
]


@pytest.mark.parametrize("case", DELAYED, ids=[f"H{c[0]}_margin{c[1]}_{'amax' if c[2] else 'pow2'}_m{c[3]}v{c[4]}{'_bf16' if c[5] else ''}" for c in DELAYED])
def test_delayed_scaling_equals_rational_referee(case):
    """Delayed scaling over 7 steps, step 1 just in time: the referee is told
    the reference amax (the max of its own record of the last H amaxes, times
    2^margin) and must agree with the oracle bit for bit, history included.
    The gradient grows 30x at step 4 (codes saturate) and shrinks at step 5."""
    H, margin, amax_mode, m_fmt, v_fmt, bf16_master = case
    n = 120
    p, _, cm, cv, sm, sv = _rand_case(n, 500 + H, m_fmt, v_fmt, 0, amax_mode, bf16_master)
    cm[:], cv[:], sm[:], sv[:] = 0, 0, 1.0, 1.0
    h = oracle.Hyper(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    hist = np.zeros(2 * H, np.float32)
    rhist = [0.0] * (2 * H)
    rp = [float(x) for x in (bf16_vals(p) if bf16_master else p)]
    rcm, rcv, rsm, rsv = [int(x) for x in cm], [int(x) for x in cv], [1.0], [1.0]
    rng = np.random.default_rng(H * 10 + margin)
    scales = [1e-3, 1e-3, 1e-3, 3e-2, 1e-4, 1e-3, 1e-3]
    saturated = 0
    for t, gs in enumerate(scales, start=1):
        g = bf16_bits(rng.standard_normal(n) * gs)
        h.step = t
        cfg = oracle.make_config(h, m_fmt, v_fmt, scale_mode=oracle.SCALE_AMAX if amax_mode else oracle.SCALE_POW2,
                                 master_bf16=bf16_master, history_len=H, margin=margin, delayed_from=2)
        st = oracle.step_hist(cfg, p, g, cm, cv, sm, sv, hist)
        saturated += st["saturated_m"] + st["saturated_v"]
        ref = None if t < 2 else (max(rhist[:H]) * 2.0 ** margin, max(rhist[H:]) * 2.0 ** margin)
        rp, rcm, rcv, rsm, rsv, am = rational.step(
            rp, [float(x) for x in bf16_vals(g)], rcm, rcv, rsm, rsv,
            lr=f32(h.lr), b1=f32(h.beta1), b2=f32(h.beta2), eps=f32(h.eps), wd=f32(h.weight_decay), t=t,
            m_fmt=m_fmt, v_fmt=v_fmt, amax_mode=amax_mode, master_bf16=bf16_master, scale_amax=ref,
            return_amax=True)
        slot = (t - 1) % H
        rhist[slot], rhist[H + slot] = am[0]
        assert list(cm) == rcm, f"m codes differ at step {t}"
        assert list(cv) == rcv, f"v codes differ at step {t}"
        assert list(sm) == rsm and list(sv) == rsv, f"scales differ at step {t}"
        assert list(hist) == rhist, f"history differs at step {t}"
        if bf16_master:
            assert np.array_equal(bf16_vals(p).view(np.uint32), np.array(rp, np.float32).view(np.uint32))
        else:
            assert _ulp_diff_f32(p, np.array(rp, np.float32)).max() <= 1
        rp = [float(x) for x in (bf16_vals(p) if bf16_master else p)]
    assert saturated > 0  # the growth step overran the delayed scale


def test_delayed_saturation_count_closed_form():
    """Zero moments, a history holding amax a: m' = (1-b1)*g exactly in fp32,
    the scale is POW2(a), and the saturated count is the number of |m'|/s above
    448 (counted here in numpy), the codes of those elements +-448."""
    n = 64
    rng = np.random.default_rng(1)
    g = bf16_bits(rng.standard_normal(n) * 1e-2)
    gv = bf16_vals(g)
    omb1 = np.float32(1.0) - np.float32(0.9)
    m1 = (omb1 * gv).astype(np.float32)
    a = np.float32(2e-4)
    k = math.frexp(float(a))[1] - 9 + (1 if math.frexp(float(a))[0] > 0.875 else 0)
    s = 2.0 ** k
    want_sat = int(np.sum(np.abs(m1.astype(np.float64)) / s > 448.0))
    assert 0 < want_sat < n
    p = np.zeros(n, np.float32)
    cm, cv = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    sm, sv = np.ones(1, np.float32), np.ones(1, np.float32)
    hist = np.array([a, 0.0, 1e30, 0.0], np.float32)  # H = 2: m history (a, 0), v history (1e30, 0)
    cfg = oracle.make_config(oracle.Hyper(step=5, lr=1e-3, weight_decay=0.0), history_len=2, delayed_from=2)
    st = oracle.step_hist(cfg, p, g, cm, cv, sm, sv, hist)
    assert st["saturated_m"] == want_sat and st["saturated_v"] == 0
    assert sm[0] == np.float32(s)
    top = np.abs(m1.astype(np.float64)) / s > 448.0
    assert np.all((cm[top] & 0x7F) == 0x7E)  # E4M3 448
    # slot (5-1) mod 2 = 0 now holds this step's amax, slot 1 is unchanged
    assert hist[0] == np.max(np.abs(m1)) and hist[1] == 0.0


def test_delayed_warmup_steps_are_just_in_time():
    """Steps before delayed_from equal the just-in-time step and record their
    amax; a delayed step whose history maximum equals its own amax is the
    just-in-time step too."""
    n = 257
    p, g, cm, cv, sm, sv = _rand_case(n, 77, 0, 1, 0, False, False)
    args = [x.copy() for x in (p, g, cm, cv, sm, sv)]
    h = oracle.Hyper(step=1, weight_decay=0.1)
    st = oracle.step(oracle.make_config(h), *args)
    hist = np.zeros(6, np.float32)
    b = [x.copy() for x in (p, g, cm, cv, sm, sv)]
    oracle.step_hist(oracle.make_config(h, history_len=3, delayed_from=3), *b, hist)
    for x, y in zip(args, b):
        assert np.array_equal(x, y)
    assert hist[0] == np.float32(st["amax_m"]) and hist[3] == np.float32(st["amax_v"])
    # same inputs at t = 4 (delayed), history preset to that step's own amax
    h.step = 4
    jit = [x.copy() for x in (p, g, cm, cv, sm, sv)]
    st4 = oracle.step(oracle.make_config(h), *jit)
    hist = np.array([0.0, st4["amax_m"], 0.0, 0.0, st4["amax_v"], 0.0], np.float32)
    d = [x.copy() for x in (p, g, cm, cv, sm, sv)]
    std = oracle.step_hist(oracle.make_config(h, history_len=3, delayed_from=2), *d, hist)
    for x, y in zip(jit, d):
        assert np.array_equal(x, y)
    assert std["saturated_m"] == 0 and std["saturated_v"] == 0


def test_delayed_rejects_block_mode_and_missing_history():
    cfg = oracle.make_config(oracle.Hyper(step=2), block=128, history_len=4)
    z = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        oracle.step_hist(cfg, np.zeros(8, np.float32), np.zeros(8, np.uint16), np.zeros(8, np.uint8),
                         np.zeros(8, np.uint8), np.ones(1, np.float32), np.ones(1, np.float32), np.zeros(8, np.float32))
    with pytest.raises(ValueError):
        oracle.step(oracle.make_config(oracle.Hyper(step=2), history_len=2), np.zeros(4, np.float32),
                    np.zeros(4, np.uint16), np.zeros(4, np.uint8), np.zeros(4, np.uint8), z[:1] + 1, z[:1] + 1)
