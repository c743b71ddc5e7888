"""The paired code layout (per run of 1024 elements, their m codes and then
their v codes, in one buffer per tensor) against the split layout (separate m
and v arrays): only where the codes live differs, so every schedule and option
must give the same weights, codes, scales and stats, bit for bit."""
import numpy as np
import pytest
import torch

import precision_adam_optimizer_amd as pk
import workloads
from tests.gpu_util import np_host, random_grad
from tests.test_gpu_parity import SIZES

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)

CASES = {
    "two_pass": dict(),
    "speculative": dict(schedule="speculative", speculate_from_step=2),
    "speculative_bf16": dict(schedule="speculative", speculate_from_step=2, master=torch.bfloat16),
    "speculative_sr": dict(schedule="speculative", speculate_from_step=2, rounding="stochastic", seed=5),
    "delayed": dict(scaling="delayed", amax_history_len=4),
    "block128": dict(granularity="block128"),
    "block128_sr_bf16": dict(granularity="block128", rounding="stochastic", seed=9, master=torch.bfloat16),
}


def _run(layout, sizes, steps, base_seed, collect_stats, master=torch.float32, **kw):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(base_seed)
    params = [(torch.randn(n, generator=gen, device=dev) * 0.02).to(master) for n in sizes]
    grads = [torch.empty(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    opt = pk.FP8AdamW(params, grads, code_layout=layout, collect_stats=collect_stats, **kw)
    out = []
    try:
        for t in range(1, steps + 1):
            for i, n in enumerate(sizes):
                grads[i].copy_(random_grad(n, base_seed * 100 + t * 7 + i, dev))
            opt.step(step=t, **HP)
            torch.cuda.synchronize()
            out.append(([np_host(p) for p in params], [np_host(m) for m in opt.m], [np_host(v) for v in opt.v],
                        [np_host(s) for s in opt.m_scale], [np_host(s) for s in opt.v_scale],
                        opt.stats() if collect_stats else None))
    finally:
        opt.close()
    return out


@pytest.mark.parametrize("case", list(CASES))
def test_paired_layout_equals_split(case):
    kw = dict(CASES[case])
    sizes = SIZES + [300_001, 2048, 1025]
    stats = case in ("two_pass", "speculative", "block128")
    a = _run("split", sizes, 6, base_seed=17, collect_stats=stats, **kw)
    b = _run("paired", sizes, 6, base_seed=17, collect_stats=stats, **kw)
    for t, (x, y) in enumerate(zip(a, b), start=1):
        for kind, xs, ys in zip(("p", "m", "v", "m_scale", "v_scale"), x[:5], y[:5]):
            for i, (u, w) in enumerate(zip(xs, ys)):
                assert np.array_equal(u.view(np.uint8), w.view(np.uint8)), f"{case} step {t}: {kind} of tensor {i}"
        if stats:
            assert x[5] == y[5], f"{case} step {t}: stats differ"


def test_paired_buffer_padding_and_size_checks():
    """The paired buffer of a tensor is 2 * ceil(n/1024) * 1024 bytes; the
    binding refuses a state for it and the init a missing m buffer."""
    assert pk.paired_code_bytes(1) == 2048 and pk.paired_code_bytes(1024) == 2048
    assert pk.paired_code_bytes(1025) == 4096 and pk.paired_code_bytes(0) == 0
    dev = torch.device("cuda")
    p = [torch.zeros(10, device=dev)]
    g = [torch.zeros(10, dtype=torch.bfloat16, device=dev)]
    with pytest.raises(ValueError):
        pk.FP8AdamW(p, g, code_layout="paired", state=([torch.zeros(2048, dtype=torch.uint8, device=dev)], [None],
                                                        [torch.ones(1, device=dev)], [torch.ones(1, device=dev)]))
    opt = pk.FP8AdamW(p, g, code_layout="paired")
    assert opt._m[0][0].numel() == 2048 and opt.m[0].numel() == 10 and opt.v[0].numel() == 10
    opt.close()


@pytest.mark.timeout(900)
def test_llama2_7b_paired_equals_split_as_benchmarked():
    """The whole 7B list, speculative from step 4, stats off: the paired layout
    gives the split layout's weights, codes and scales bit for bit over 6 steps."""
    w = workloads.llama2_7b()
    dev = torch.device("cuda")
    shapes = w.shapes
    grads = [torch.empty(workloads.numel(s), dtype=torch.bfloat16, device=dev) for _, s in shapes]
    pa = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
    pb = [p.clone() for p in pa]
    a = pk.FP8AdamW(pa, grads, schedule="speculative")
    b = pk.FP8AdamW(pb, grads, schedule="speculative", code_layout="paired")
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    try:
        for t in range(1, 7):
            for i, (_, s) in enumerate(shapes):
                grads[i].copy_(workloads.make_grad(w, i, s, t, dev))
            a.step(step=t, **hp)
            b.step(step=t, **hp)
        torch.cuda.synchronize()
        bm, bv = b.m, b.v
        for i, (name, _) in enumerate(shapes):
            assert torch.equal(pa[i].view(torch.uint8), pb[i].view(torch.uint8)), f"p of {name}"
            assert torch.equal(a.m[i], bm[i]) and torch.equal(a.v[i], bv[i]), f"codes of {name}"
            assert torch.equal(a.m_scale[i], b.m_scale[i]) and torch.equal(a.v_scale[i], b.v_scale[i]), name
    finally:
        a.close()
        b.close()
        del pa, pb, grads
        torch.cuda.empty_cache()
