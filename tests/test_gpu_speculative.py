"""The speculative schedule (one update pass quantizing with a predicted
power-of-two scale into the other code buffer, then a per-tensor check and a
fix-up that brings the moments whose true scale differs to it, by moving
exponent fields or recomputing) against the two-pass schedule (bit for bit)
and against the CPU oracle."""
import itertools

import numpy as np
import pytest
import torch

import precision_adam_optimizer_amd as pk
import workloads
from tests.gpu_util import np_host, random_grad
from tests.test_gpu_parity import FORMATS, SIZES, run_full, run_small

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def drifting_grad(n, seed, t, i, dev):
    """Gradient whose tensor-level scale jumps by a random power of two (-2..+2
    binades) from step to step, so the per-tensor scales both keep and change."""
    g = torch.Generator()
    g.manual_seed(seed * 1000 + t * 31 + i)
    shift = int(torch.randint(-2, 3, (1,), generator=g))
    return (random_grad(n, seed * 7 + t * 13 + i, dev).float() * 2.0 ** shift).to(torch.bfloat16)


def sparse_drifting_grad(n, seed, t, i, dev):
    """drifting_grad with a wide spread of magnitudes (a factor 10^U(-6, 0) per
    element) and 2% exact zeros, so the moments hold zero, subnormal and
    smallest-normal codes as well as ordinary ones."""
    g = torch.Generator()
    g.manual_seed(seed * 1000 + t * 37 + i + 5)
    spread = torch.pow(10.0, -6.0 * torch.rand(n, generator=g))
    keep = (torch.rand(n, generator=g) >= 0.02).float()
    return (drifting_grad(n, seed, t, i, dev).float() * (spread * keep).to(dev)).to(torch.bfloat16)


def _run(schedule, sizes, steps, seed, master=torch.float32, spec_from=2, collect_stats=True, grad_fn=None,
         rounding="nearest", predictor="probe"):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    params = [(torch.randn(n, generator=gen, device=dev) * 0.02).to(master) for n in sizes]
    grads = [torch.empty(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    opt = pk.FP8AdamW(params, grads, collect_stats=collect_stats, schedule=schedule, speculate_from_step=spec_from,
                      rounding=rounding, seed=11, predictor=predictor)
    grad_fn = grad_fn or drifting_grad
    hist = []
    for t in range(1, steps + 1):
        for i, n in enumerate(sizes):
            grads[i].copy_(grad_fn(n, seed, t, i, dev))
        opt.step(step=t, **HP)
        torch.cuda.synchronize()
        st = opt.stats() if collect_stats else None
        hist.append(([np_host(p) for p in params], [np_host(m) for m in opt.m], [np_host(v) for v in opt.v],
                     [np_host(s) for s in opt.m_scale], [np_host(s) for s in opt.v_scale], st))
    opt.close()
    return hist


# The growth model mispredicts often on these small tensors, which keeps the
# fix-up's every path busy; the probe predicts most of them exactly.
PREDICTORS = ["growth", "probe"]


@pytest.mark.parametrize("predictor", PREDICTORS)
@pytest.mark.parametrize("master", [torch.float32, torch.bfloat16])
def test_speculative_equals_two_pass_bitwise(master, predictor):
    sizes = SIZES + [300_001]
    a = _run("two_pass", sizes, 10, seed=3, master=master)
    b = _run("speculative", sizes, 10, seed=3, master=master, predictor=predictor)
    requant_steps, clean_steps = 0, 0
    for t, (x, y) in enumerate(zip(a, b), start=1):
        for kind, xs, ys in zip(("p", "m", "v", "m_scale", "v_scale"), x[:5], y[:5]):
            for i, (u, w) in enumerate(zip(xs, ys)):
                assert np.array_equal(u.view(np.uint8), w.view(np.uint8)), f"step {t}: {kind} of tensor {i} differs"
        for i, (sa, sb) in enumerate(zip(x[5], y[5])):
            for k in ("amax_m", "amax_v", "scale_m", "scale_v", "underflow_m", "underflow_v", "saturated_m",
                      "saturated_v", "nonfinite"):
                assert np.float64(sa[k]) == np.float64(sb[k]) or (np.isnan(sa[k]) and np.isnan(sb[k])), \
                    f"step {t} tensor {i}: stat {k} {sa[k]} vs {sb[k]}"
            assert sa["requantized"] == 0 and sa["probed"] == 0
        if predictor == "growth":
            assert all(sb["probed"] == 0 for sb in y[5])  # no probe runs
        rq = sum(s["requantized"] for s in y[5])
        if t >= 2:
            requant_steps += rq > 0
            clean_steps += rq < 2 * sum(sizes)  # (element, moment) pairs
    # both paths of the speculative schedule ran
    assert clean_steps > 0
    assert requant_steps > 0 or predictor == "probe"


@pytest.mark.parametrize("predictor", PREDICTORS)
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
@pytest.mark.parametrize("master", [torch.float32, torch.bfloat16])
def test_speculative_equals_two_pass_without_stats(master, rounding, predictor):
    """The fix-up without the stats counters (where a zero code of a shrinking
    moment is kept as it is under round-to-nearest), on moments full of zero,
    subnormal and smallest-normal codes: bit-identical to the two-pass
    schedule in every step."""
    sizes = SIZES + [300_001, 65_536]
    a = _run("two_pass", sizes, 10, seed=8, master=master, collect_stats=False, grad_fn=sparse_drifting_grad,
             rounding=rounding)
    b = _run("speculative", sizes, 10, seed=8, master=master, collect_stats=False, grad_fn=sparse_drifting_grad,
             rounding=rounding, predictor=predictor)
    moved = 0
    for t, (x, y) in enumerate(zip(a, b), start=1):
        for kind, xs, ys in zip(("p", "m", "v", "m_scale", "v_scale"), x[:5], y[:5]):
            for i, (u, w) in enumerate(zip(xs, ys)):
                assert np.array_equal(u.view(np.uint8), w.view(np.uint8)), f"step {t}: {kind} of tensor {i} differs"
        if t >= 2:  # scales that changed from step to step: the fix-up's cases
            moved += sum(int(x[3][i][0] != a[t - 2][3][i][0]) + int(x[4][i][0] != a[t - 2][4][i][0])
                         for i in range(len(sizes)))
    assert moved > 0
    # the moments hold the codes the fix-up must recompute rather than move
    m_all = np.concatenate(b[-1][1])
    assert (m_all & 0x7F == 0).any() and ((m_all & 0x7F) < 8).any()


SPEC_COMBOS = list(itertools.product(FORMATS, ["fp32", "bf16"]))


@pytest.mark.parametrize("predictor", PREDICTORS)
@pytest.mark.parametrize("combo", SPEC_COMBOS, ids=[f"{a}-{b}_{m}" for (a, b), m in SPEC_COMBOS])
def test_speculative_vs_oracle_ragged(combo, predictor):
    fmts, master = combo
    k = SPEC_COMBOS.index(combo)
    # random mid-training state (predictions mostly wrong) and zero state (mixed)
    rq = run_small(fmts, "tensor", "pow2", master, collect_stats=True, random_init=(k % 2 == 0), steps=5,
                   seed=40 + k, schedule="speculative", speculate_from_step=2, predictor=predictor)
    assert rq > 0 or predictor == "probe"


@pytest.mark.parametrize("predictor", PREDICTORS)
def test_speculative_resume_is_bit_exact(predictor):
    """A context rebuilt from the state after step 4 (no probe candidates yet,
    so its first speculative step predicts from the growth model) continues
    bit for bit like the uninterrupted run."""
    sizes = [50_001, 4096, 3]
    ref = _run("speculative", sizes, 7, seed=5, predictor=predictor)
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    params = [torch.randn(n, generator=gen, device=dev) * 0.02 for n in sizes]
    grads = [torch.empty(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    opt = pk.FP8AdamW(params, grads, collect_stats=True, schedule="speculative", speculate_from_step=2,
                      predictor=predictor)
    for t in range(1, 5):
        for i, n in enumerate(sizes):
            grads[i].copy_(drifting_grad(n, 5, t, i, dev))
        opt.step(step=t, **HP)
    torch.cuda.synchronize()
    state = ([m.clone() for m in opt.m], [v.clone() for v in opt.v], [s.clone() for s in opt.m_scale],
             [s.clone() for s in opt.v_scale])
    opt.close()
    opt2 = pk.FP8AdamW(params, grads, collect_stats=True, schedule="speculative", speculate_from_step=2, state=state,
                       predictor=predictor)
    for t in range(5, 8):
        for i, n in enumerate(sizes):
            grads[i].copy_(drifting_grad(n, 5, t, i, dev))
        opt2.step(step=t, **HP)
    torch.cuda.synchronize()
    final = ([np_host(p) for p in params], [np_host(m) for m in opt2.m], [np_host(v) for v in opt2.v])
    opt2.close()
    for xs, ys in zip(ref[-1][:3], final):
        for u, w in zip(xs, ys):
            assert np.array_equal(u.view(np.uint8), w.view(np.uint8))


@pytest.mark.timeout(900)
def test_llama2_7b_bench_configuration_full_size():
    """The 7B list exactly as the benchmark runs it: speculative schedule from
    step 4 (steps 1-3 two-pass), stats off (the kernels without counters, where
    the fix-up keeps a shrinking zero code as it is), fresh gradients per step;
    sampled tensors against the oracle at every step."""
    w = workloads.llama2_7b()
    n = len(w.shapes)
    sample = [0] + list(range(1 + 9 * 15, 1 + 9 * 16)) + [n - 2, n - 1]
    run_full(w, steps=7, sample=sample, collect_stats=False, schedule="speculative", speculate_from_step=4)


@pytest.mark.timeout(900)
def test_llama2_7b_speculative_full_size():
    w = workloads.llama2_7b()
    n = len(w.shapes)
    sample = [0] + list(range(1 + 9 * 31, 1 + 9 * 32)) + [n - 2, n - 1]
    run_full(w, steps=4, sample=sample, collect_stats=True, schedule="speculative", speculate_from_step=2)


@pytest.mark.timeout(900)
def test_llama2_7b_speculative_equals_two_pass_over_60_steps():
    """The whole 7B list (6.7e9 parameters) under both schedules from the same
    state and the same fresh gradients for 60 steps, stats off as benchmarked:
    weights, codes and scales of every tensor bit-identical after steps 4, 20
    and 60, so no fix-up case anywhere in the list over a long run leaves a
    code that the true scale would not give."""
    w = workloads.llama2_7b()
    dev = torch.device("cuda")
    shapes = w.shapes
    grads = [torch.empty(workloads.numel(s), dtype=torch.bfloat16, device=dev) for _, s in shapes]
    pa = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
    pb = [p.clone() for p in pa]
    a = pk.FP8AdamW(pa, grads, schedule="two_pass")
    b = pk.FP8AdamW(pb, grads, schedule="speculative")
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    try:
        for t in range(1, 61):
            for i, (_, s) in enumerate(shapes):
                grads[i].copy_(workloads.make_grad(w, i, s, t, dev))
            a.step(step=t, **hp)
            b.step(step=t, **hp)
            if t in (4, 20, 60):
                torch.cuda.synchronize()
                for i, (name, _) in enumerate(shapes):
                    for kind, x, y in (("p", pa[i], pb[i]), ("m", a.m[i], b.m[i]), ("v", a.v[i], b.v[i]),
                                       ("m_scale", a.m_scale[i], b.m_scale[i]),
                                       ("v_scale", a.v_scale[i], b.v_scale[i])):
                        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"step {t}: {kind} of {name}"
    finally:
        a.close()
        b.close()
        del pa, pb, grads
        torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_llama2_7b_rank0_of_8_bench_configuration():
    """One data-parallel rank's real share of the 7B list (842M parameters,
    ending in a cut piece of layers.3.w_gate), speculative from step 4 with
    stats off as benchmarked; the embedding, a whole layer tensor and the cut
    piece against the oracle at every step."""
    w = workloads.llama2_7b_rank0_of_8()
    n = len(w.shapes)
    run_full(w, steps=6, sample=[0, 10, n - 1], collect_stats=False, schedule="speculative",
             speculate_from_step=4)


@pytest.mark.timeout(600)
def test_llama2_100m_speculative_all_format_pairs():
    """The Llama-2-100M-shaped list as benchmarked (speculative from step 4,
    stats off) in all four (m, v) format pairs: every tensor against the oracle
    at every one of 7 steps."""
    for m_fmt, v_fmt in FORMATS:
        w = workloads.llama2_100m(m_fmt, v_fmt)
        run_full(w, steps=7, sample=list(range(len(w.shapes))), collect_stats=False, schedule="speculative",
                 speculate_from_step=4)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
def test_llama2_100m_speculative_equals_two_pass_over_100_steps(rounding):
    """The Llama-2-100M list (110 tensors, 1.1e8 parameters) under both
    schedules from the same state and the same fresh gradients for 100 steps,
    stats off as benchmarked: on a list this short the growth model predicts
    and the fix-up splits its work into pieces, and every tensor's weights,
    codes and scales stay bit-identical to the two-pass schedule's after steps
    4, 30 and 100."""
    w = workloads.llama2_100m()
    dev = torch.device("cuda")
    shapes = w.shapes
    grads = [torch.empty(workloads.numel(s), dtype=torch.bfloat16, device=dev) for _, s in shapes]
    pa = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
    pb = [p.clone() for p in pa]
    a = pk.FP8AdamW(pa, grads, schedule="two_pass", rounding=rounding, seed=3)
    b = pk.FP8AdamW(pb, grads, schedule="speculative", rounding=rounding, seed=3)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    try:
        for t in range(1, 101):
            for i, (_, s) in enumerate(shapes):
                grads[i].copy_(workloads.make_grad(w, i, s, t, dev))
            a.step(step=t, **hp)
            b.step(step=t, **hp)
            if t in (4, 30, 100):
                torch.cuda.synchronize()
                for i, (name, _) in enumerate(shapes):
                    for kind, x, y in (("p", pa[i], pb[i]), ("m", a.m[i], b.m[i]), ("v", a.v[i], b.v[i]),
                                       ("m_scale", a.m_scale[i], b.m_scale[i]),
                                       ("v_scale", a.v_scale[i], b.v_scale[i])):
                        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"step {t}: {kind} of {name}"
    finally:
        a.close()
        b.close()


@pytest.mark.timeout(300)
def test_flat_1m_speculative_ten_steps():
    """The 1M flat tensor (per-row gradient scales) as benchmarked: speculative
    from step 4, stats off, ten steps against the oracle."""
    run_full(workloads.flat_1m(), steps=10, sample=[0], collect_stats=False, schedule="speculative",
             speculate_from_step=4)


@pytest.mark.timeout(300)
def test_scale_probe_lists_candidates_and_cuts_mispredictions():
    """The speculative schedule's scale probe on Llama-2-7B-sized tensors
    (Gaussian gradients with a fixed per-tensor scale, a fresh draw per step):
    from the first speculative step on (the step before it lists the first
    candidates) it reads the parts that held values near each tensor's amax, at
    most 1/32 of a large tensor (and at least 8 parts), and predicts the
    power-of-two scales well enough that at most 3% of the (element, moment)
    pairs need the fix-up (the growth model alone mispredicts 6-8% of them on
    such gradients)."""
    dev = torch.device("cuda")
    sizes = [16_777_216] * 6 + [45_088_768] * 2 + [4096, 1001]
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    params = [torch.randn(n, generator=gen, device=dev) * 0.02 for n in sizes]
    grads = [torch.empty(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    scales = [10.0 ** float(-6.0 + 5.0 * torch.rand(1, generator=gen, device=dev)) for _ in sizes]
    opt = pk.FP8AdamW(params, grads, schedule="speculative", speculate_from_step=4, predictor="probe")
    moved = pairs = 0
    listed = big = 0
    try:
        for t in range(1, 17):
            for i, n in enumerate(sizes):
                grads[i].copy_((torch.randn(n, generator=gen, device=dev) * scales[i]).to(torch.bfloat16))
            opt.step(step=t, **HP)
            st = opt.stats()
            for i, n in enumerate(sizes):
                nparts = -(-n // 1024)
                cap = min(nparts, max(8, nparts >> 5)) * 1024
                assert 0 <= st[i]["probed"] <= min(cap, n), (t, i, st[i]["probed"])
                if t < 4:
                    assert st[i]["probed"] == 0  # two-pass steps, and the step that lists the first candidates
                elif n >= 1 << 24:
                    big += 1
                    listed += st[i]["probed"] > 0
            if t >= 4:
                moved += sum(s["requantized"] for s in st)
                pairs += 2 * sum(sizes)
        print(f"probe active on {listed}/{big} (tensor, step) pairs; fix-up moved {moved / pairs:.2%} of the pairs")
        assert listed >= 0.9 * big
        assert moved <= 0.03 * pairs
    finally:
        opt.close()
        del params, grads
        torch.cuda.empty_cache()


def _edge_grad(n, seed, t, i, dev):
    """Gradients that exercise the probe's candidate list: tensor 0 constant
    (every part equal: more candidates than the cap, the growth model
    predicts), tensor 1 zero (amax 0: no candidates), tensor 2 one spike that
    moves every step (one candidate part, never the new maximum's), the rest
    drifting noise."""
    if i == 0:
        return torch.full((n,), 0.01 * (1 + t % 3), dtype=torch.bfloat16, device=dev)
    if i == 1:
        return torch.zeros(n, dtype=torch.bfloat16, device=dev)
    g = drifting_grad(n, seed, t, i, dev)
    if i == 2:
        g = g.float() * 1e-3
        g[(7919 * t + 13) % n] = 4.0
        g = g.to(torch.bfloat16)
    return g


@pytest.mark.parametrize("master", [torch.float32, torch.bfloat16])
def test_scale_probe_edge_cases_equal_two_pass(master):
    """The probe's candidate list at its edges (a tensor over the cap, one
    with amax 0, one whose single candidate never holds the new maximum)
    changes predictions only: weights, codes, scales and stats stay equal to
    the two-pass schedule's bit for bit."""
    sizes = [300_001, 65_536, 1 << 20, 5_000, 12_289]
    a = _run("two_pass", sizes, 9, seed=21, master=master, grad_fn=_edge_grad)
    b = _run("speculative", sizes, 9, seed=21, master=master, grad_fn=_edge_grad, predictor="probe")
    for t, (x, y) in enumerate(zip(a, b), start=1):
        for kind, xs, ys in zip(("p", "m", "v", "m_scale", "v_scale"), x[:5], y[:5]):
            for i, (u, w) in enumerate(zip(xs, ys)):
                assert np.array_equal(u.view(np.uint8), w.view(np.uint8)), f"step {t}: {kind} of tensor {i} differs"
        for i, (sa, sb) in enumerate(zip(x[5], y[5])):
            for k in ("underflow_m", "underflow_v", "saturated_m", "saturated_v", "nonfinite"):
                assert sa[k] == sb[k], f"step {t} tensor {i}: stat {k}"
    st = b[-1][5]
    assert st[0]["probed"] == 0  # over the cap: no list
    assert st[1]["probed"] == 0  # amax 0: nothing to list
    # the parts of the last few spikes (v decays by beta2 a step, and its E5M2 codes may round a decayed
    # spike up): listed, within the cap of 1/32 of the tensor's parts
    assert 0 < st[2]["probed"] <= (1 << 20) // 32
