"""GPU parity for stochastic rounding of the moments: every schedule and
option with rounding="stochastic" against the oracle's stochastic mode (same
seed, Philox4x32-10 stream keyed by it, counter (i/4, t, tensor index)):
codes and scales bit-exact.  Also: the GPU's codes differ from round-to-
nearest, are unbiased on average, and depend on the seed.
"""
import numpy as np
import pytest
import torch

import precision_adam_optimizer_amd as pk
import workloads
from tests.gpu_util import np_host, random_grad
from tests.test_gpu_amp import run_amp
from tests.test_gpu_delayed import run_delayed
from tests.test_gpu_parity import FORMATS, SIZES, _layer_indices, run_full, run_small

pytestmark = pytest.mark.gpu

SEED = 0x5EED5EED12345678

CASES = [
    # fmts, granularity, scale_mode, master, schedule
    (FORMATS[0], "tensor", "pow2", "fp32", "two_pass"),
    (FORMATS[0], "tensor", "pow2", "bf16", "speculative"),
    (FORMATS[1], "tensor", "amax", "fp32", "two_pass"),
    (FORMATS[2], "block128", "pow2", "fp32", "two_pass"),
    (FORMATS[3], "block128", "amax", "bf16", "two_pass"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0][0]}-{c[0][1]}_{c[1]}_{c[2]}_{c[3]}_{c[4]}" for c in CASES])
def test_small_stochastic(case):
    fmts, gran, smode, master, schedule = case
    k = CASES.index(case)
    run_small(fmts, gran, smode, master, collect_stats=(k % 2 == 0), random_init=(k % 3 == 0), seed=500 + k,
              steps=5, schedule=schedule, speculate_from_step=2, rounding="stochastic", rng_seed=SEED + k)


def test_small_stochastic_l2_and_delayed_and_amp():
    run_small(FORMATS[0], "tensor", "pow2", "fp32", collect_stats=True, random_init=True, seed=510,
              decay_mode="l2", rounding="stochastic", rng_seed=SEED)
    run_delayed(SIZES, H=4, rounding="stochastic", rng_seed=SEED + 1, seed=511)
    run_amp(SIZES[:14], schedule="speculative", overflow_at=(2,), calls=5, rounding="stochastic", rng_seed=SEED + 2,
            seed=512)


def _one_step(rounding, seed, n=1 << 20, t=1):
    dev = torch.device("cuda")
    p = torch.zeros(n, device=dev)
    g = random_grad(n, 77, dev, lo=-4.0, hi=-2.0)
    opt = pk.FP8AdamW([p], [g], rounding=rounding, seed=seed)
    opt.step(lr=1e-3, beta1=0.9, beta2=0.95, weight_decay=0.0, step=t)
    torch.cuda.synchronize()
    out = np_host(opt.m[0]), np_host(opt.v[0]), float(opt.m_scale[0]), g.float().cpu().numpy()
    opt.close()
    return out


def test_stochastic_is_unbiased_and_seeded():
    """One step from zero moments: m' = 0.1 g exactly known.  The decoded
    stochastic codes average to m' (the round-to-nearest ones need not), the
    codes differ from round-to-nearest on about half the inexact elements,
    and another seed gives other codes."""
    cm_rn, _, s, g = _one_step("nearest", 0)
    cm_a, _, s2, _ = _one_step("stochastic", 11)
    cm_b, _, _, _ = _one_step("stochastic", 12)
    assert s == s2
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s
    omb1 = np.float32(1.0) - np.float32(0.9)
    m1 = (omb1 * g.astype(np.float32)).astype(np.float64)
    err_sr = dec(cm_a) - m1
    spacing = np.abs(dec(cm_a) - dec(cm_rn)).max()
    assert spacing > 0
    # mean error of SR is far below the quantization step (unbiased), 2^20 samples
    assert abs(err_sr.mean()) < 0.01 * np.abs(err_sr).mean()
    frac_diff = float(np.mean(cm_a != cm_rn))
    assert 0.2 < frac_diff < 0.6
    assert float(np.mean(cm_a != cm_b)) > 0.1


@pytest.mark.timeout(900)
def test_llama2_7b_stochastic_full_size():
    """The 7B list with stochastic rounding, speculative schedule as the
    benchmark runs it: sampled tensors against the oracle for 4 steps."""
    w = workloads.llama2_7b()
    n = len(w.shapes)
    run_full(w, steps=4, sample=_layer_indices(32, [3]) + [n - 1], schedule="speculative", speculate_from_step=2,
             rounding="stochastic", rng_seed=SEED)
