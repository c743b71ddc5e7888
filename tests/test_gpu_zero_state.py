"""fp8adam_config.zero_state: fp8adam_init writes a fresh optimizer state (zero
codes, unit scales, zero amax history) into buffers that start with arbitrary
content.  Three steps from such buffers must equal, bit for bit, three steps
from buffers the caller cleared itself, in every schedule and granularity."""
import ctypes

import numpy as np
import pytest
import torch

import precision_adam_optimizer_amd as pk
from tests.gpu_util import np_host, random_grad

pytestmark = pytest.mark.gpu

SIZES = [40_000, 0, 4097, 129, 1]
HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
H = 4

CASES = {
    "two_pass": dict(schedule=pk.SCHEDULE_TWO_PASS, scaling=pk.SCALING_JUST_IN_TIME, gran=pk.SCALE_TENSOR),
    "speculative": dict(schedule=pk.SCHEDULE_SPECULATIVE, scaling=pk.SCALING_JUST_IN_TIME, gran=pk.SCALE_TENSOR),
    "delayed": dict(schedule=pk.SCHEDULE_TWO_PASS, scaling=pk.SCALING_DELAYED, gran=pk.SCALE_TENSOR),
    "block128": dict(schedule=pk.SCHEDULE_TWO_PASS, scaling=pk.SCALING_JUST_IN_TIME, gran=pk.SCALE_BLOCK128),
}


def _state(case, garbage, seed):
    """Per-tensor buffers: p, g, m, v, m_scale, v_scale, m_alt, v_alt, history."""
    gen = torch.Generator(device="cuda")  # the garbage only: both runs get the same weights
    gen.manual_seed(seed)
    out = []
    for i, n in enumerate(SIZES):
        ns = max(1, -(-n // 128)) if case["gran"] == pk.SCALE_BLOCK128 else 1
        pg = torch.Generator(device="cuda")
        pg.manual_seed(seed * 1000 + i)
        p = torch.randn(max(n, 1), generator=pg, device="cuda")[:n].contiguous() * 0.02
        g = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        if garbage:
            m = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
            v = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
            ms = torch.full((ns,), 8.0, device="cuda")
            vs = torch.full((ns,), 0.25, device="cuda")
            hist = torch.rand(2 * H, device="cuda", generator=gen) * 100
        else:
            m = torch.zeros(n, dtype=torch.uint8, device="cuda")
            v = torch.zeros(n, dtype=torch.uint8, device="cuda")
            ms = torch.ones(ns, device="cuda")
            vs = torch.ones(ns, device="cuda")
            hist = torch.zeros(2 * H, device="cuda")
        m_alt = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
        v_alt = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
        out.append([p, g, m, v, ms, vs, m_alt, v_alt, hist])
    return out


def _run(case, garbage):
    torch.manual_seed(0)
    bufs = _state(case, garbage, seed=11)
    args = []
    for p, g, m, v, ms, vs, ma, va, h in bufs:
        n = p.numel()
        ptr = (lambda x: x.data_ptr()) if n > 0 else (lambda x: 0)
        args.append(pk.TensorArg(ptr(p), ptr(g), ptr(m), ptr(v), ms.data_ptr(), vs.data_ptr(), n,
                                 ptr(ma), ptr(va), h.data_ptr()))
    cfg = pk.ConfigArg(pk.E4M3, pk.E5M2, case["gran"], pk.SCALE_POW2, pk.MASTER_FP32, 0, case["schedule"], 2,
                       pk.DECAY_DECOUPLED, case["scaling"], H, 0, 2, pk.ROUND_NEAREST, 0, int(garbage))
    ctx = pk.fp8adam_init(args, cfg)
    try:
        if garbage:  # the fresh state is in place once init returns
            for i, (p, g, m, v, ms, vs, ma, va, h) in enumerate(bufs):
                assert not m.any() and not v.any(), f"tensor {i}: codes not cleared"
                if SIZES[i] > 0 or case["gran"] == pk.SCALE_TENSOR:
                    assert bool((ms == 1.0).all()) and bool((vs == 1.0).all()), f"tensor {i}: scales not 1"
                if case["scaling"] == pk.SCALING_DELAYED and SIZES[i] > 0:
                    assert not h.any(), f"tensor {i}: history not cleared"
        for t in range(1, 4):
            for i, (p, g, *_rest) in enumerate(bufs):
                if SIZES[i] > 0:
                    g.copy_(random_grad(SIZES[i], 1000 * t + i, "cuda", lo=-6.0, hi=-1.0))
            hp = pk.HParamsArg(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], t)
            pk.fp8adam_step(ctx, hp)
        torch.cuda.synchronize()
        cur = pk.fp8adam_current_buffer(ctx)
    finally:
        pk.fp8adam_destroy(ctx)
    out = []
    for i, (p, g, m, v, ms, vs, ma, va, h) in enumerate(bufs):
        if SIZES[i] == 0:
            continue
        cm, cv = (ma, va) if cur == 1 else (m, v)
        out += [np_host(p), np_host(cm), np_host(cv), np_host(ms), np_host(vs)]
        if case["scaling"] == pk.SCALING_DELAYED:
            out.append(np_host(h))
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_zero_state_equals_a_cleared_state(name):
    case = CASES[name]
    want = _run(case, garbage=False)
    got = _run(case, garbage=True)
    assert len(got) == len(want)
    for k, (a, b) in enumerate(zip(got, want)):
        assert a.tobytes() == b.tobytes(), f"{name}: array {k} differs"
