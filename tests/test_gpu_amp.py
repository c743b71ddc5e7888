"""GPU parity for the fused loss-scaling step (fp8adam_step_amp): one read of
every gradient for the global sum of squares and the Inf/NaN check, the
scaler's decision on the device, then the step with every gradient multiplied
by clip_coef / S and the bias corrections of the device-side step count.

Against the oracle: the scaler state after every call (scale, growth count,
step count, skip flag, clip coefficient, gradient factor and norm) equal;
a skipped call leaves every weight, code, scale and history as it was; the
taken ones meet the usual bar (codes and scales bit-exact).
"""
import numpy as np
import pytest
import torch

import oracle
import precision_adam_optimizer_amd as pk
import workloads
from tests.gpu_util import OracleState, compare_tensor, np_host, random_grad, run_pool, upload_params
from tests.test_gpu_delayed import compare_history
from tests.test_gpu_parity import SIZES, _compare_stats, _layer_indices

pytestmark = pytest.mark.gpu


def check_amp_state(name, got: dict, want: oracle.AmpState):
    for k in ("scale", "growth_tracker", "step", "found_inf", "clip_coef", "grad_factor"):
        g, w = got[k], getattr(want, k)
        assert np.float32(g).view(np.uint32) == np.float32(w).view(np.uint32) if isinstance(w, float) else g == w, \
            f"{name}: amp {k} gpu {g!r} oracle {w!r}"
    if not want.found_inf:
        assert np.float32(got["grad_norm"]) == np.float32(want.grad_norm), \
            f"{name}: grad_norm gpu {got['grad_norm']!r} oracle {want.grad_norm!r}"


def run_amp(sizes, *, schedule="two_pass", granularity="tensor", scaling="just_in_time", decay_mode="decoupled",
            master="fp32", max_norm=1.0, init_scale=2.0 ** 16, overflow_at=(3,), calls=7, growth_interval=3,
            seed=0, stats=True, speculate_from_step=2, rounding="nearest", rng_seed=0, predictor="auto"):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    params = []
    for n in sizes:
        p = torch.randn(n, generator=gen, device=dev) * 0.02
        params.append(p.to(torch.bfloat16) if master == "bf16" else p)
    grads = [torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    nb = [1 if granularity == "tensor" else -(-n // 128) for n in sizes]
    state = [list(x) for x in zip(*(workloads.make_state(n, dev, nblocks=k) for n, k in zip(sizes, nb)))]
    H = 4
    opt = pk.FP8AdamW(params, grads, granularity=granularity, collect_stats=stats, state=state, schedule=schedule,
                      speculate_from_step=speculate_from_step, decay_mode=decay_mode, scaling=scaling,
                      amax_history_len=H, rounding=rounding, seed=rng_seed, predictor=predictor)
    delayed = scaling == "delayed"
    host = [OracleState(np_host(params[i]), np_host(state[0][i]), np_host(state[1][i]), np_host(state[2][i]),
                        np_host(state[3][i]), np_host(opt.amax_history[i]) if delayed else None)
            for i in range(len(sizes))]
    amp = pk.amp_state(init_scale, dev)
    acfg = oracle.AmpConfig(max_norm, 2.0, 0.5, growth_interval)
    ast = oracle.AmpState(scale=init_scale, clip_coef=1.0)
    skipped = clipped = 0
    lr = 1e-3
    try:
        for t in range(1, calls + 1):
            S = float(ast.scale)
            for i, n in enumerate(sizes):
                g = random_grad(n, seed * 7919 + t * 101 + i, dev, lo=-6.0, hi=-1.0).float() * S
                if t in overflow_at and i == len(sizes) // 2 and n > 0:
                    g[n // 2] = float("inf")
                grads[i].copy_(g.to(torch.bfloat16))
            opt.step_amp(amp, lr=lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t, max_norm=max_norm,
                         growth_interval=growth_interval)
            torch.cuda.synchronize()
            sums = oracle.GradSums()
            gh = [np_host(x) for x in grads]
            for x in gh:
                sums.add(x)
            oracle.amp_control(sums, acfg, ast)
            got = pk.read_amp_state(amp)
            check_amp_state(f"call {t}", got, ast)
            gstats = opt.stats() if stats else None
            if ast.found_inf:
                skipped += 1
            else:
                clipped += ast.clip_coef < 1.0
                h = oracle.Hyper(lr=lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=ast.step)
                cfg = oracle.make_config(h, 0, 1, block=128 if granularity == "block128" else 0,
                                         master_bf16=(master == "bf16"), l2_coupled=(decay_mode == "l2"),
                                         history_len=H if delayed else 0, delayed_from=2,
                                         grad_factor=ast.grad_factor, sched_step=t,
                                         stochastic=(rounding == "stochastic"), seed=rng_seed)
            for i, n in enumerate(sizes):
                name = f"tensor {i} (numel {n}) call {t}"
                if not ast.found_inf:
                    cfg.tensor_index = i
                    host[i].step(cfg, gh[i])
                    if stats and granularity == "tensor":
                        _compare_stats(name, gstats[i], host[i].stats, granularity)
                else:
                    host[i].p_old = host[i].p.copy()
                compare_tensor(name, host[i], np_host(params[i]), np_host(opt.m[i]), np_host(opt.v[i]),
                               np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), master)
                if delayed:
                    compare_history(name, host[i], np_host(opt.amax_history[i]))
                upload_params(params[i], host[i])
    finally:
        opt.close()
    return skipped, clipped


CASES = [
    # schedule, granularity, scaling, decay, master, max_norm
    ("two_pass", "tensor", "just_in_time", "decoupled", "fp32", 1.0),
    ("speculative", "tensor", "just_in_time", "decoupled", "fp32", 1.0),
    ("two_pass", "block128", "just_in_time", "decoupled", "bf16", 1.0),
    ("two_pass", "tensor", "delayed", "decoupled", "fp32", 1.0),
    ("two_pass", "tensor", "just_in_time", "l2", "bf16", 0.0),
    ("speculative", "tensor", "just_in_time", "decoupled", "bf16", 1e6),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}_{c[1]}_{c[2]}_{c[3]}_{c[4]}_clip{c[5]:g}" for c in CASES])
def test_small_amp(case):
    schedule, gran, scaling, decay, master, max_norm = case
    k = CASES.index(case)
    skipped, clipped = run_amp(SIZES, schedule=schedule, granularity=gran, scaling=scaling, decay_mode=decay,
                               master=master, max_norm=max_norm, seed=400 + k, overflow_at=(3, 6))
    assert skipped == 2
    if max_norm == 1.0:
        assert clipped > 0


def test_small_amp_overflow_first_call_and_growth():
    """An overflow at call 1 (before any step: the speculative schedule's
    two-pass warm-up and the delayed warm-up see a skipped call) and growth
    of the scale every 2 taken steps."""
    skipped, _ = run_amp(SIZES[:12], schedule="speculative", overflow_at=(1, 5), calls=8, growth_interval=2,
                         seed=431, speculate_from_step=2)
    assert skipped == 2
    run_amp(SIZES[:12], scaling="delayed", overflow_at=(1,), calls=5, growth_interval=2, seed=432)


@pytest.mark.parametrize("master", ["fp32", "bf16"])
def test_small_amp_speculative_with_the_scale_probe(master):
    """The speculative schedule predicting from the scale probe through two
    skipped calls: a skipped step neither probes nor lists, and the next taken
    step probes the candidates listed before the skip."""
    skipped, clipped = run_amp(SIZES, schedule="speculative", master=master, seed=470 + (master == "bf16"),
                               overflow_at=(3, 6), predictor="probe")
    assert skipped == 2 and clipped > 0


def test_small_amp_overflow_first_call_with_the_scale_probe():
    """An overflow at call 1, the exact-scale step that would list the probe's
    first candidates: the first speculative step has none and takes the growth
    model, the later ones the probe."""
    skipped, _ = run_amp(SIZES[:12], schedule="speculative", overflow_at=(1, 5), calls=8, growth_interval=2,
                         seed=433, speculate_from_step=2, predictor="probe")
    assert skipped == 2


@pytest.mark.timeout(900)
def test_llama2_7b_amp_clip_full_size():
    """The 7B list with loss scale 2^16 and clipping at max_norm = 1.0 (the
    value in the pages' code example), speculative schedule as benchmarked:
    the scaler state from the oracle's exact sum over all 6.7e9 gradients, and
    sampled tensors against the oracle, for 4 calls with an overflow at call 3."""
    w = workloads.llama2_7b()
    dev = torch.device("cuda")
    shapes = w.shapes
    n_t = len(shapes)
    sample = _layer_indices(32, [0]) + [n_t - 1]
    params = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
    grads = [torch.empty(workloads.numel(s), dtype=torch.bfloat16, device=dev) for _, s in shapes]
    opt = pk.FP8AdamW(params, grads, schedule="speculative", speculate_from_step=2)
    host = {i: OracleState(np_host(params[i]), np.zeros(workloads.numel(shapes[i][1]), np.uint8),
                           np.zeros(workloads.numel(shapes[i][1]), np.uint8), np.ones(1, np.float32),
                           np.ones(1, np.float32)) for i in sample}
    S0 = 2.0 ** 16
    amp = pk.amp_state(S0, dev)
    acfg = oracle.AmpConfig(1.0, 2.0, 0.5, 2000)
    ast = oracle.AmpState(scale=S0, clip_coef=1.0)
    try:
        for t in range(1, 5):
            S = float(ast.scale)
            for i, (_, s) in enumerate(shapes):
                grads[i].copy_((workloads.make_grad(w, i, s, t, dev).float() * S).to(torch.bfloat16))
            if t == 3:
                grads[5][7] = float("nan")
            opt.step_amp(amp, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t,
                         max_norm=1.0)
            torch.cuda.synchronize()
            sums = oracle.GradSums()
            for i in range(n_t):
                sums.add(np_host(grads[i]))
            oracle.amp_control(sums, acfg, ast)
            print(f"7B amp call {t}: oracle sums done, found_inf {ast.found_inf}, clip {ast.clip_coef}", flush=True)
            check_amp_state(f"call {t}", pk.read_amp_state(amp), ast)
            if ast.found_inf:
                cfg = None
            else:
                assert ast.clip_coef < 1.0
                cfg = oracle.make_config(oracle.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                                                      weight_decay=w.weight_decay, step=ast.step),
                                         grad_factor=ast.grad_factor)

            def check(i):
                st = host[i]
                if cfg is not None:
                    st.step(cfg, np_host(grads[i]))
                else:
                    st.p_old = st.p.copy()
                compare_tensor(f"{shapes[i][0]} call {t}", st, np_host(params[i]), np_host(opt.m[i]),
                               np_host(opt.v[i]), np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), w.master)
                upload_params(params[i], st)

            run_pool(check, sample)
    finally:
        opt.close()
        del params, grads
        torch.cuda.empty_cache()
