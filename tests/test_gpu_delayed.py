"""GPU parity for delayed scaling: the scale of step t comes from the largest
amax of the previous H steps (times 2^margin); codes that no longer fit
saturate.  Compared with the oracle's delayed mode step by step: codes,
scales and the amax history bit-exact, weights to the usual bar, stats
(saturation and underflow counts, amax) equal.  The gradient is scaled up 30x
at one step (the delayed scale is too small: saturation) and down 100x at the
next (underflow), then back.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_adam_optimizer_amd as pk
import workloads
from tests.gpu_util import OracleState, compare_tensor, np_host, oracle_config, random_grad, run_pool, upload_params
from tests.test_gpu_parity import SIZES, _compare_stats, _layer_indices

pytestmark = pytest.mark.gpu

FACTORS = [1.0, 1.0, 1.0, 30.0, 0.01, 1.0, 1.0]


def compare_history(name, st: OracleState, hist_gpu: np.ndarray):
    if not np.array_equal(hist_gpu.view(np.uint32), st.hist.view(np.uint32)):
        bad = np.nonzero(hist_gpu.view(np.uint32) != st.hist.view(np.uint32))[0]
        raise AssertionError(f"{name}: amax history differs at {bad[:4]}: gpu {hist_gpu[bad[:4]]} "
                             f"oracle {st.hist[bad[:4]]}")


def run_delayed(sizes, *, H=16, margin=0, delayed_from=2, scale_mode="pow2", master="fp32", stats=True,
                decay_mode="decoupled", fmts=("e4m3", "e5m2"), seed=0, factors=FACTORS, lr=3e-4,
                preset_history=False, rounding="nearest", rng_seed=0):
    m_fmt, v_fmt = fmts
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    params = []
    for n in sizes:
        p = torch.randn(n, generator=gen, device=dev) * 0.02
        params.append(p.to(torch.bfloat16) if master == "bf16" else p)
    grads = [torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    state = [list(x) for x in zip(*(workloads.make_state(n, dev) for n in sizes))]
    if preset_history:  # a history carried over from earlier training
        hist = [(torch.rand(2 * H, generator=gen, device=dev) * 1e-3).contiguous() for _ in sizes]
        state.append(hist)
    opt = pk.FP8AdamW(params, grads, m_format=m_fmt, v_format=v_fmt, scale_mode=scale_mode, collect_stats=stats,
                      state=state, decay_mode=decay_mode, scaling="delayed", amax_history_len=H, margin=margin,
                      delayed_from_step=delayed_from, rounding=rounding, seed=rng_seed)
    host = [OracleState(np_host(params[i]), np_host(state[0][i]), np_host(state[1][i]), np_host(state[2][i]),
                        np_host(state[3][i]), np_host(opt.amax_history[i])) for i in range(len(sizes))]
    saturated = 0
    try:
        for t, f in enumerate(factors, start=1):
            for i, n in enumerate(sizes):
                g = random_grad(n, seed * 7919 + t * 101 + i, dev, lo=-6.0, hi=-2.0)
                grads[i].copy_((g.float() * f).to(torch.bfloat16))
            opt.step(lr=lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            torch.cuda.synchronize()
            h = oracle.Hyper(lr=lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            cfg = oracle_config(h, m_fmt, v_fmt, "tensor", scale_mode, master, decay_mode, history_len=H,
                                margin=margin, delayed_from=delayed_from)
            cfg.stochastic, cfg.seed = int(rounding == "stochastic"), rng_seed
            gstats = opt.stats() if stats else None
            for i, n in enumerate(sizes):
                cfg.tensor_index = i
                host[i].step(cfg, np_host(grads[i]))
                name = f"tensor {i} (numel {n}) step {t}"
                compare_tensor(name, host[i], np_host(params[i]), np_host(opt.m[i]), np_host(opt.v[i]),
                               np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), master)
                compare_history(name, host[i], np_host(opt.amax_history[i]))
                if stats:
                    _compare_stats(name, gstats[i], host[i].stats, "tensor")
                    saturated += gstats[i]["saturated_m"] + gstats[i]["saturated_v"]
                upload_params(params[i], host[i])
    finally:
        opt.close()
    return saturated


CASES = [
    # H, margin, scale_mode, master, decay_mode, fmts, delayed_from
    (16, 0, "pow2", "fp32", "decoupled", ("e4m3", "e5m2"), 2),
    (1, 0, "pow2", "fp32", "decoupled", ("e4m3", "e5m2"), 2),
    (3, 2, "pow2", "bf16", "decoupled", ("e4m3", "e5m2"), 2),
    (4, 1, "amax", "fp32", "decoupled", ("e4m3", "e5m2"), 3),
    (16, 0, "pow2", "fp32", "l2", ("e4m3", "e5m2"), 2),
    (5, 0, "amax", "bf16", "l2", ("e5m2", "e4m3"), 2),
    (100, 0, "pow2", "fp32", "decoupled", ("e5m2", "e5m2"), 1),
]


@pytest.mark.parametrize("case", CASES, ids=[f"H{c[0]}_margin{c[1]}_{c[2]}_{c[3]}_{c[4]}_{c[5][0]}-{c[5][1]}_from{c[6]}" for c in CASES])
def test_small_delayed(case):
    H, margin, smode, master, decay, fmts, dfrom = case
    k = CASES.index(case)
    sat = run_delayed(SIZES, H=H, margin=margin, delayed_from=dfrom, scale_mode=smode, master=master,
                      decay_mode=decay, fmts=fmts, seed=300 + k, stats=True)
    if margin == 0:
        assert sat > 0  # the 30x step overran the delayed scale


def test_small_delayed_preset_history_no_stats():
    run_delayed(SIZES, H=8, preset_history=True, stats=False, seed=317)


def test_delayed_warmup_steps_equal_just_in_time():
    """Steps before delayed_from_step run just in time: the delayed context
    gives bit-identical weights, codes and scales to a just-in-time one, and
    its history holds those steps' amax in slots 0..2 (slot 3 untouched)."""
    dev = torch.device("cuda")
    sizes = [1000, 4097, 70000]
    outs = []
    for scaling in ("just_in_time", "delayed"):
        params = [torch.linspace(-0.02, 0.02, n, device=dev) for n in sizes]
        grads = [random_grad(n, 5 + n, dev) for n in sizes]
        opt = pk.FP8AdamW(params, grads, scaling=scaling, amax_history_len=4, delayed_from_step=4)
        for t in (1, 2, 3):
            opt.step(lr=1e-3, weight_decay=0.1, step=t)
        torch.cuda.synchronize()
        outs.append([np_host(x) for x in params + opt.m + opt.v + opt.m_scale + opt.v_scale])
        if scaling == "delayed":
            hist = [np_host(x) for x in opt.amax_history]
        opt.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    for h in hist:
        assert (h[:3] > 0).all() and h[3] == 0.0 and (h[4:7] > 0).all() and h[7] == 0.0


@pytest.mark.timeout(900)
def test_llama2_7b_delayed_full_size():
    """The 7B list with delayed scaling (H = 16, margin 0) in the launch
    configuration the benchmark times; sampled tensors against the oracle,
    history included, for 4 steps (step 1 just in time)."""
    w = workloads.llama2_7b()
    dev = torch.device("cuda")
    shapes = w.shapes
    n_t = len(shapes)
    sample = _layer_indices(32, [0, 31]) + [n_t - 2, n_t - 1]
    params = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
    grads = [torch.empty(workloads.numel(s), dtype=torch.bfloat16, device=dev) for _, s in shapes]
    opt = pk.FP8AdamW(params, grads, scaling="delayed", amax_history_len=16, collect_stats=True)
    host = {}
    for i in sample:
        n = workloads.numel(shapes[i][1])
        host[i] = OracleState(np_host(params[i]), np.zeros(n, np.uint8), np.zeros(n, np.uint8),
                              np.ones(1, np.float32), np.ones(1, np.float32), np.zeros(32, np.float32))
    try:
        for t in range(1, 5):
            for i, (_, s) in enumerate(shapes):
                grads[i].copy_(workloads.make_grad(w, i, s, t, dev))
            opt.step(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
            torch.cuda.synchronize()
            cfg = oracle_config(oracle.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                                             weight_decay=w.weight_decay, step=t),
                                w.m_fmt, w.v_fmt, "tensor", "pow2", w.master, history_len=16)
            gstats = opt.stats()

            def check(i):
                st = host[i]
                st.step(cfg, np_host(grads[i]))
                name = f"{shapes[i][0]} step {t}"
                compare_tensor(name, st, np_host(params[i]), np_host(opt.m[i]), np_host(opt.v[i]),
                               np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), w.master)
                compare_history(name, st, np_host(opt.amax_history[i]))
                upload_params(params[i], st)
                return st.stats

            ostats = dict(zip(sample, run_pool(check, sample)))
            for i in sample:
                _compare_stats(f"{shapes[i][0]} step {t}", gstats[i], ostats[i], "tensor")
            # every tensor: the history slot of this step holds its amax
            for i in range(n_t):
                hs = opt.amax_history[i]
                assert float(hs[(t - 1) % 16]) == gstats[i]["amax_m"]
                assert float(hs[16 + (t - 1) % 16]) == gstats[i]["amax_v"]
    finally:
        opt.close()
        del params, grads
        torch.cuda.empty_cache()
