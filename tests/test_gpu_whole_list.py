"""Whole-list parity at full size: every tensor of the Llama-2-7B list (per
tensor and block-128) and of the Llama-2-13B bf16 list against the oracle for
one step in the launch configuration the benchmark times, and the whole 13B
list under both schedules bit for bit.

A checked step starts from a device-side snapshot of the whole optimizer state
(weights, the codes of the buffer that holds the moments, scales) taken after
the earlier steps; then every tensor's pre-step state, gradient and result go
to the host one tensor per worker thread (16), where the oracle takes the same
step and the result is compared (bar of tests/gpu_util.py: codes and scales bit
for bit, weights within 1e-6 of max(|p_ref|, |p_old|), bf16 weights within one
ulp on at most 1e-3 of the elements).  Host memory stays at one tensor per
worker.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_adam_optimizer_amd as pk
import workloads
from tests.gpu_util import OracleState, compare_tensor, np_host, oracle_config, run_pool

pytestmark = pytest.mark.gpu


def whole_list_step(w: workloads.Workload, t_check: int, schedule: str = "two_pass", speculate_from_step: int = 0):
    """Steps 1..t_check of workload w (fresh gradients, stats off), then every
    tensor of step t_check against the oracle.  Returns the number of
    (element, moment) pairs the speculative fix-up moved in that step."""
    dev = torch.device("cuda")
    shapes = w.shapes
    params = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
    grads = [torch.empty(workloads.numel(s), dtype=torch.bfloat16, device=dev) for _, s in shapes]
    opt = pk.FP8AdamW(params, grads, m_format=w.m_fmt, v_format=w.v_fmt, granularity=w.granularity,
                      schedule=schedule, speculate_from_step=speculate_from_step, decay_mode=w.decay_mode)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    snap = None
    try:
        for t in range(1, t_check + 1):
            for i, (_, s) in enumerate(shapes):
                grads[i].copy_(workloads.make_grad(w, i, s, t, dev))
            if t == t_check:
                torch.cuda.synchronize()
                snap = [(params[i].clone(), opt.m[i].clone(), opt.v[i].clone(), opt.m_scale[i].clone(),
                         opt.v_scale[i].clone()) for i in range(len(shapes))]
            opt.step(step=t, **hp)
            torch.cuda.synchronize()
            print(f"{w.name}: step {t} done", flush=True)
        moved = sum(s["requantized"] for s in opt.stats())
        h = oracle.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                         step=t_check)
        cfg = oracle_config(h, w.m_fmt, w.v_fmt, w.granularity, "pow2", w.master, w.decay_mode)

        def check(i):
            st = OracleState(*[np_host(x) for x in snap[i]])
            st.step(cfg, np_host(grads[i]))
            compare_tensor(f"{shapes[i][0]} step {t_check}", st, np_host(params[i]), np_host(opt.m[i]),
                           np_host(opt.v[i]), np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), w.master)
            return workloads.numel(shapes[i][1])

        order = sorted(range(len(shapes)), key=lambda i: -workloads.numel(shapes[i][1]))
        checked = sum(run_pool(check, order))
        assert checked == w.total_params
        print(f"{w.name}: step {t_check}, all {len(shapes)} tensors ({checked} params) equal to the oracle; "
              f"fix-up moved {moved} (element, moment) pairs", flush=True)
        return moved
    finally:
        opt.close()
        del params, grads, snap
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_llama2_7b_every_tensor_speculative_step():
    """The 7B list as benchmarked (speculative from step 4, stats off): every
    one of its 291 tensors against the oracle at step 5, a speculative step
    whose fix-up moves the moments of the tensors whose predicted scale was off."""
    moved = whole_list_step(workloads.llama2_7b(), 5, schedule="speculative", speculate_from_step=4)
    assert moved > 0  # the checked step exercised the fix-up


@pytest.mark.timeout(900)
def test_llama2_7b_block128_every_tensor():
    """The block-128 7B list as benchmarked (one pass, stats off, Student-t
    gradients with 1% zeros): every tensor against the oracle at step 2."""
    whole_list_step(workloads.llama2_7b_block128(), 2)


@pytest.mark.timeout(900)
def test_llama2_13b_bf16_every_tensor_speculative_step():
    """The 13B bf16-master list as benchmarked (speculative from step 4, stats
    off, 2048-element parts): every one of its 363 tensors against the oracle at
    step 5."""
    whole_list_step(workloads.llama2_13b_bf16(), 5, schedule="speculative", speculate_from_step=4)


@pytest.mark.timeout(900)
def test_llama2_13b_bf16_speculative_equals_two_pass_whole_list():
    """The whole 13B bf16 list (1.3e10 parameters) under both schedules from the
    same state and the same fresh gradients for 12 steps, stats off: weights,
    codes and scales of every tensor bit-identical after steps 4, 8 and 12."""
    w = workloads.llama2_13b_bf16()
    dev = torch.device("cuda")
    shapes = w.shapes
    grads = [torch.empty(workloads.numel(s), dtype=torch.bfloat16, device=dev) for _, s in shapes]
    pa = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
    pb = [p.clone() for p in pa]
    a = pk.FP8AdamW(pa, grads, schedule="two_pass")
    b = pk.FP8AdamW(pb, grads, schedule="speculative")
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    moved = 0
    try:
        for t in range(1, 13):
            for i, (_, s) in enumerate(shapes):
                grads[i].copy_(workloads.make_grad(w, i, s, t, dev))
            a.step(step=t, **hp)
            b.step(step=t, **hp)
            moved += sum(s["requantized"] for s in b.stats())
            if t in (4, 8, 12):
                torch.cuda.synchronize()
                for i, (name, _) in enumerate(shapes):
                    for kind, x, y in (("p", pa[i], pb[i]), ("m", a.m[i], b.m[i]), ("v", a.v[i], b.v[i]),
                                       ("m_scale", a.m_scale[i], b.m_scale[i]),
                                       ("v_scale", a.v_scale[i], b.v_scale[i])):
                        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"step {t}: {kind} of {name}"
                print(f"13B bf16 list: step {t} bit-identical under both schedules", flush=True)
        assert moved > 0
    finally:
        a.close()
        b.close()
        del pa, pb, grads
        torch.cuda.empty_cache()
