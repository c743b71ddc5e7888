"""GPU parity: the HIP step (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar (see tests/gpu_util.py): FP8 codes and scales bit-exact; fp32 weights
within 1e-6 of max(|p_ref|, |p_old|); bf16 weights equal except <= 1 ulp on
<= 1e-3 of the elements; stats counts and amax equal.

Sizes: small ragged multi-tensor lists (1 element up to several chunks, tails
of 1-3 elements, partial 128-blocks) over every format pair, granularity,
scale mode, master dtype and stats setting; then the five synthetic workloads
at full size (flat 1M, Llama-2-100M, 7B per-tensor, 7B block-128, 13B bf16)
in the launch configuration the benchmark times, checked tensor by tensor on
a sample of whole tensors plus size-independent properties on every tensor.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import precision_adam_optimizer_amd as pk
import workloads
from tests.gpu_util import (OracleState, compare_tensor, np_host, oracle_config, random_grad, run_pool,
                            upload_params)

pytestmark = pytest.mark.gpu

SIZES = [1, 2, 3, 4, 5, 7, 127, 128, 129, 255, 1000, 1023, 1024, 1025, 2047, 2049, 4095, 4096, 4097, 16383,
         16384, 16385, 16387, 40000, 65539]
FORMATS = [("e4m3", "e5m2"), ("e5m2", "e5m2"), ("e5m2", "e4m3"), ("e4m3", "e4m3")]
COMBOS = list(itertools.product(FORMATS, ["tensor", "block128"], ["pow2", "amax"], ["fp32", "bf16"]))


def _compare_stats(name, got: dict, want: dict, granularity: str):
    for k in ("underflow_m", "underflow_v", "saturated_m", "saturated_v", "nonfinite"):
        if k not in want:
            continue
        assert got[k] == want[k], f"{name}: stat {k} gpu {got[k]} oracle {want[k]}"
    for k in ("amax_m", "amax_v", "scale_m", "scale_v"):
        assert np.float32(got[k]).view(np.uint32) == np.float32(want[k]).view(np.uint32), \
            f"{name}: stat {k} gpu {got[k]!r} oracle {want[k]!r}"


def run_small(fmts, granularity, scale_mode, master, collect_stats, random_init, sizes=SIZES, steps=3,
              lr=3e-4, seed=0, schedule="two_pass", speculate_from_step=0, decay_mode="decoupled", wd=0.1,
              rounding="nearest", rng_seed=0, predictor="probe"):
    m_fmt, v_fmt = fmts
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    params = []
    for n in sizes:
        p = torch.randn(n, generator=gen, device=dev) * 0.02
        params.append(p.to(torch.bfloat16) if master == "bf16" else p)
    grads = [torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    nb = [1 if granularity == "tensor" else -(-n // 128) for n in sizes]
    state = ([], [], [], [])
    for i, n in enumerate(sizes):
        if random_init:
            cm, cv, sm, sv = workloads.random_state(n, dev, seed * 1000 + i, workloads_fmt(m_fmt),
                                                    workloads_fmt(v_fmt), nblocks=nb[i], scale_exp=(-24, 2),
                                                    pow2=(scale_mode == "pow2"))
        else:
            cm, cv, sm, sv = workloads.make_state(n, dev, nblocks=nb[i])
        for lst, x in zip(state, (cm, cv, sm, sv)):
            lst.append(x)
    host = [OracleState(np_host(params[i]), np_host(state[0][i]), np_host(state[1][i]), np_host(state[2][i]),
                        np_host(state[3][i])) for i in range(len(sizes))]
    opt = pk.FP8AdamW(params, grads, m_format=m_fmt, v_format=v_fmt, granularity=granularity,
                      scale_mode=scale_mode, collect_stats=collect_stats, state=state, schedule=schedule,
                      speculate_from_step=speculate_from_step, decay_mode=decay_mode, rounding=rounding,
                      seed=rng_seed, predictor=predictor)
    requantized = 0
    try:
        for t in range(1, steps + 1):
            for i, n in enumerate(sizes):
                grads[i].copy_(random_grad(n, seed * 7919 + t * 101 + i, dev))
            opt.step(lr=lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=wd, step=t)
            torch.cuda.synchronize()
            h = oracle.Hyper(lr=lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=wd, step=t)
            cfg = oracle_config(h, m_fmt, v_fmt, granularity, scale_mode, master, decay_mode)
            cfg.stochastic, cfg.seed = int(rounding == "stochastic"), rng_seed
            gstats = opt.stats() if collect_stats else None
            for i, n in enumerate(sizes):
                cfg.tensor_index = i
                host[i].step(cfg, np_host(grads[i]))
                name = f"tensor {i} (numel {n}) step {t}"
                compare_tensor(name, host[i], np_host(params[i]), np_host(opt.m[i]), np_host(opt.v[i]),
                               np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), master)
                if collect_stats:
                    _compare_stats(name, gstats[i], host[i].stats, granularity)
                    requantized += gstats[i]["requantized"]
                upload_params(params[i], host[i])
    finally:
        opt.close()
    return requantized


def workloads_fmt(f):
    return 0 if f == "e4m3" else 1


@pytest.mark.parametrize("combo", COMBOS, ids=[f"{a}-{b}_{g}_{s}_{m}" for (a, b), g, s, m in COMBOS])
def test_small_ragged_lists(combo):
    fmts, gran, smode, master = combo
    k = COMBOS.index(combo)
    run_small(fmts, gran, smode, master, collect_stats=(k % 2 == 0), random_init=(k % 4 < 2), seed=k)


@pytest.mark.parametrize("gran", ["tensor", "block128"])
def test_small_large_learning_rate_and_stats(gran):
    """Big updates (lr 1e-2) from a random mid-training state, stats on."""
    run_small(("e4m3", "e5m2"), gran, "pow2", "fp32", collect_stats=True, random_init=True, lr=1e-2,
              steps=4, seed=99)


L2_COMBOS = list(itertools.product(["tensor", "block128"], ["pow2", "amax"], ["fp32", "bf16"]))


@pytest.mark.parametrize("combo", L2_COMBOS, ids=[f"{g}_{s}_{m}" for g, s, m in L2_COMBOS])
def test_small_coupled_l2(combo):
    """Coupled L2 (weight_decay * p added to the gradient, no separate decay):
    wd = 0.1 with |p| ~ 0.02 makes the L2 term dominate the smaller gradients."""
    gran, smode, master = combo
    k = L2_COMBOS.index(combo)
    run_small(("e4m3", "e5m2"), gran, smode, master, collect_stats=(k % 2 == 0), random_init=(k % 4 < 2),
              seed=200 + k, decay_mode="l2")


def test_small_coupled_l2_other_formats_and_zero_decay():
    run_small(("e5m2", "e4m3"), "tensor", "pow2", "fp32", collect_stats=True, random_init=True, seed=211,
              decay_mode="l2", wd=0.5)
    # weight_decay 0 is plain Adam in both modes (a -0 gradient stays -0)
    run_small(("e4m3", "e5m2"), "block128", "pow2", "bf16", collect_stats=True, random_init=False, seed=212,
              decay_mode="l2", wd=0.0)


def test_zero_sized_tensor_in_list():
    dev = torch.device("cuda")
    sizes = [10, 0, 5]
    params = [torch.randn(n, device=dev) * 0.02 for n in sizes]
    grads = [random_grad(n, 3 + n, dev) for n in sizes]
    host = [OracleState(np_host(p), np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.ones(1, np.float32),
                        np.ones(1, np.float32)) for p, n in zip(params, sizes)]
    opt = pk.FP8AdamW(params, grads)
    opt.step(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, step=1)
    torch.cuda.synchronize()
    cfg = oracle_config(oracle.Hyper(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, step=1), "e4m3", "e5m2",
                        "tensor", "pow2", "fp32")
    for i, n in enumerate(sizes):
        host[i].step(cfg, np_host(grads[i]))
        compare_tensor(f"tensor {i}", host[i], np_host(params[i]), np_host(opt.m[i]), np_host(opt.v[i]),
                       np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), "fp32")
    opt.close()


# ------------------------------------------------------------ full-size lists

def _top_code(fmt: str) -> int:
    """Code of FMAX/2: the amax element of a tensor must land at or above it."""
    return int(oracle.encode(fmt, [oracle.format_max(fmt) / 2])[0])


def run_full(w: workloads.Workload, steps: int, sample: list, base_seed: int = 0, collect_stats: bool = False,
             schedule: str = "two_pass", speculate_from_step: int = 0, rounding: str = "nearest", rng_seed: int = 0):
    dev = torch.device("cuda")
    shapes = w.shapes
    params = [workloads.make_param(w, i, s, dev, base_seed) for i, (_, s) in enumerate(shapes)]
    grads = [torch.empty(workloads.numel(s), dtype=torch.bfloat16, device=dev) for _, s in shapes]
    host = {}
    for i in sample:
        n = workloads.numel(shapes[i][1])
        nb = 1 if w.granularity == "tensor" else -(-n // 128)
        host[i] = OracleState(np_host(params[i]), np.zeros(n, np.uint8), np.zeros(n, np.uint8),
                              np.ones(nb, np.float32), np.ones(nb, np.float32))
    opt = pk.FP8AdamW(params, grads, m_format=w.m_fmt, v_format=w.v_fmt, granularity=w.granularity,
                      collect_stats=collect_stats, schedule=schedule, speculate_from_step=speculate_from_step,
                      decay_mode=w.decay_mode, rounding=rounding, seed=rng_seed)
    top_m, top_v = _top_code(w.m_fmt), _top_code(w.v_fmt)
    all_stats = []
    try:
        for t in range(1, steps + 1):
            for i, (_, s) in enumerate(shapes):
                grads[i].copy_(workloads.make_grad(w, i, s, t, dev, base_seed))
            opt.step(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
            torch.cuda.synchronize()
            h = oracle.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
            cfg = oracle_config(h, w.m_fmt, w.v_fmt, w.granularity, "pow2", w.master, w.decay_mode)

            def check(i):
                st = host[i]
                cfg_i = oracle.Config.from_buffer_copy(cfg)
                cfg_i.stochastic, cfg_i.seed, cfg_i.tensor_index = int(rounding == "stochastic"), rng_seed, i
                st.step(cfg_i, np_host(grads[i]))
                compare_tensor(f"{shapes[i][0]} step {t}", st, np_host(params[i]), np_host(opt.m[i]),
                               np_host(opt.v[i]), np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), w.master)
                upload_params(params[i], st)
                return st.stats

            ostats = dict(zip(sample, run_pool(check, sample)))
            gstats = opt.stats() if collect_stats else None
            if collect_stats:
                for i in sample:
                    _compare_stats(f"{shapes[i][0]} step {t}", gstats[i], ostats[i], w.granularity)
                all_stats.append(gstats)
            # properties of every tensor at any size
            for i in range(len(shapes)):
                assert not bool((opt.v[i] & 0x80).any()), f"{shapes[i][0]}: negative v code"
                if w.granularity == "tensor":
                    mm = int((opt.m[i] & 0x7F).max())
                    vv = int((opt.v[i] & 0x7F).max())
                    # skipped only for an all-zero moment (scale 1) or a clamped tiny scale
                    if float(opt.m_scale[i]) > 2.0 ** -126 and not (mm == 0 and float(opt.m_scale[i]) == 1.0):
                        assert mm >= top_m, f"{shapes[i][0]}: m amax not in the top binade"
                    if float(opt.v_scale[i]) > 2.0 ** -126 and not (vv == 0 and float(opt.v_scale[i]) == 1.0):
                        assert vv >= top_v, f"{shapes[i][0]}: v amax not in the top binade"
    finally:
        opt.close()
        del params, grads
        torch.cuda.empty_cache()
    return all_stats


def _layer_indices(n_layers: int, layers: list) -> list:
    idx = [0]
    for L in layers:
        idx += list(range(1 + 9 * L, 1 + 9 * (L + 1)))
    return idx


@pytest.mark.timeout(300)
def test_flat_1m_ten_steps():
    run_full(workloads.flat_1m(), steps=10, sample=[0], collect_stats=True)


@pytest.mark.timeout(900)
def test_llama2_100m_all_format_pairs():
    """The Llama-2-100M-shaped list in all four (m, v) format pairs, 20 steps
    each, stats on: every tensor against the oracle at every step (codes,
    scales, weights, and the underflow / saturation counts equal); v in E4M3
    underflows far more than v in E5M2 over the 20 steps and in each of the
    first three (with fresh zero-mean gradients every step, a moment that once
    held a representable value rarely falls back below the smallest code, so the
    E4M3 underflow of v dies out after a few steps)."""
    under_v = {}
    for m_fmt, v_fmt in FORMATS:
        w = workloads.llama2_100m(m_fmt, v_fmt)
        print(f"llama2_100m {m_fmt}/{v_fmt}: 20 steps, every tensor", flush=True)
        stats = run_full(w, steps=20, sample=list(range(len(w.shapes))), collect_stats=True)
        under_v[(m_fmt, v_fmt)] = [sum(s["underflow_v"] for s in st) for st in stats]
        assert all(s["saturated_m"] == 0 and s["saturated_v"] == 0 for st in stats for s in st)
    for a, b in ((("e4m3", "e4m3"), ("e4m3", "e5m2")), (("e5m2", "e4m3"), ("e5m2", "e5m2"))):
        assert sum(under_v[a]) > 20 * max(1, sum(under_v[b])), (a, under_v[a], b, under_v[b])
        for t in range(3):
            assert under_v[a][t] > 20 * max(1, under_v[b][t]), (t + 1, a, under_v[a], b, under_v[b])


@pytest.mark.timeout(900)
def test_llama2_7b_per_tensor_full_size():
    w = workloads.llama2_7b()
    n = len(w.shapes)
    sample = _layer_indices(32, [0, 17, 31]) + [n - 2, n - 1]
    run_full(w, steps=2, sample=sample)


@pytest.mark.timeout(900)
def test_llama2_7b_coupled_l2_full_size():
    w = workloads.llama2_7b_l2()
    n = len(w.shapes)
    sample = _layer_indices(32, [0, 31]) + [n - 2, n - 1]
    run_full(w, steps=2, sample=sample, collect_stats=True)


@pytest.mark.timeout(900)
def test_llama2_7b_block128_full_size():
    w = workloads.llama2_7b_block128()
    n = len(w.shapes)
    sample = _layer_indices(32, [0, 31]) + [n - 2, n - 1]
    run_full(w, steps=2, sample=sample, collect_stats=True)


@pytest.mark.timeout(900)
def test_llama2_7b_block128_as_benchmarked():
    """The block-128 list in the benchmark's launch configuration (stats off:
    the kernel instantiation the benchmark times), three steps."""
    w = workloads.llama2_7b_block128()
    n = len(w.shapes)
    sample = _layer_indices(32, [5]) + [n - 1]
    run_full(w, steps=3, sample=sample, collect_stats=False)


@pytest.mark.timeout(1200)
def test_llama2_13b_bf16_master_full_size():
    """The 13B list as benchmarked: bf16 master, speculative schedule (step 1
    two-pass, steps 2-5 speculative, with the bf16 master's 2048-element parts)."""
    w = workloads.llama2_13b_bf16()
    n = len(w.shapes)
    sample = _layer_indices(40, [0]) + [n - 2, n - 1]
    run_full(w, steps=5, sample=sample, schedule="speculative", speculate_from_step=2)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("sizes,chunk", [([1_048_576], 4096), ([9_000_001, 11_000_003], 8192),
                                          ([30_000_005, 5_000_000, 3], 16384), ([70_000_000], 32768)])
def test_chunk_size_choice_and_parity(sizes, chunk):
    """The context picks the largest chunk (4096..32768) that still gives at
    least 2048 amax-pass work-groups; each choice is checked against the oracle."""
    dev = torch.device("cuda")
    params = [torch.randn(n, device=dev) * 0.02 for n in sizes]
    grads = [random_grad(n, 77 + i, dev) for i, n in enumerate(sizes)]
    host = [OracleState(np_host(p), np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.ones(1, np.float32),
                        np.ones(1, np.float32)) for p, n in zip(params, sizes)]
    opt = pk.FP8AdamW(params, grads, collect_stats=True)
    assert opt.num_chunks == sum(-(-n // chunk) for n in sizes)
    try:
        for t in (1, 2):
            opt.step(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            torch.cuda.synchronize()
            cfg = oracle_config(oracle.Hyper(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t),
                                "e4m3", "e5m2", "tensor", "pow2", "fp32")
            gstats = opt.stats()

            def check(i):
                host[i].step(cfg, np_host(grads[i]))
                compare_tensor(f"tensor {i} step {t}", host[i], np_host(params[i]), np_host(opt.m[i]),
                               np_host(opt.v[i]), np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), "fp32")
                _compare_stats(f"tensor {i} step {t}", gstats[i], host[i].stats, "tensor")
                upload_params(params[i], host[i])

            run_pool(check, list(range(len(sizes))))
    finally:
        opt.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("master", ["fp32", "bf16"])
def test_flat_block128_tensor_past_2_to_32_elements(master):
    """One flat tensor of 2^32 + 2^20 + 333 elements with per-128 block scales
    (a flat optimizer buffer, as sharded optimizers keep one): element, block,
    part and chunk indices all pass 2^31 and 2^32.  Block scales are local, so
    a block-aligned window is an exact sub-problem: windows at the start,
    around 2^31 and from just below 2^32 to the ragged end are checked
    against the oracle over two steps; the stats counters cover the whole
    tensor (no saturation with power-of-two scales)."""
    dev = torch.device("cuda")
    n = (1 << 32) + (1 << 20) + 333
    piece = 1 << 28
    gen = torch.Generator(device=dev)
    gen.manual_seed(21)
    param = torch.empty(n, device=dev, dtype=torch.bfloat16 if master == "bf16" else torch.float32)
    grad = torch.empty(n, dtype=torch.bfloat16, device=dev)
    for k, a in enumerate(range(0, n, piece)):
        b = min(n, a + piece)
        param[a:b].normal_(0.0, 0.02, generator=gen)
    windows = [(0, 1 << 20), ((1 << 31) - (1 << 19), (1 << 31) + (1 << 19)), ((1 << 32) - (1 << 19), n)]
    host = [OracleState(np_host(param[a:b]), np.zeros(b - a, np.uint8), np.zeros(b - a, np.uint8),
                        np.ones(-(-(b - a) // 128), np.float32), np.ones(-(-(b - a) // 128), np.float32))
            for a, b in windows]
    opt = pk.FP8AdamW([param], [grad], granularity="block128", collect_stats=True)
    try:
        for t in (1, 2):
            for k, a in enumerate(range(0, n, piece)):
                b = min(n, a + piece)
                grad[a:b].copy_(random_grad(b - a, 1000 * t + k, dev))
            opt.step(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            torch.cuda.synchronize()
            h = oracle.Hyper(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            cfg = oracle_config(h, "e4m3", "e5m2", "block128", "pow2", master)
            for (a, b), st in zip(windows, host):
                st.step(cfg, np_host(grad[a:b]))
                compare_tensor(f"window [{a}, {b}) step {t}", st, np_host(param[a:b]), np_host(opt.m[0][a:b]),
                               np_host(opt.v[0][a:b]), np_host(opt.m_scale[0][a // 128:-(-b // 128)]),
                               np_host(opt.v_scale[0][a // 128:-(-b // 128)]), master)
                st.p = np_host(param[a:b]).copy()  # continue from the device's weights (within the bar)
            s = opt.stats()[0]
            assert s["saturated_m"] == 0 and s["saturated_v"] == 0 and s["nonfinite"] == 0
            assert s["underflow_m"] > 0  # the gradients span 8 decades: some moments flush in every step
    finally:
        opt.close()
        del param, grad
        torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("schedule,master", [("two_pass", "fp32"), ("speculative", "fp32"), ("speculative", "bf16")])
def test_flat_per_tensor_past_2_to_32_elements(schedule, master):
    """One flat tensor of 2^32 + 2^20 + 333 elements with one scale per moment,
    in both schedules (stats off, as benchmarked).  The same large gradient
    (2^13, far above every other one) is planted at the first element of each
    checked window in every step, so each window's amax of the new moments is
    the whole tensor's: each window is then an exact sub-problem for the
    oracle, which is checked over three steps (the speculative schedule from
    step 2, with the fix-up of the moments whose predicted scale was off)."""
    dev = torch.device("cuda")
    n = (1 << 32) + (1 << 20) + 333
    piece = 1 << 28
    gen = torch.Generator(device=dev)
    gen.manual_seed(22)
    param = torch.empty(n, device=dev, dtype=torch.bfloat16 if master == "bf16" else torch.float32)
    grad = torch.empty(n, dtype=torch.bfloat16, device=dev)
    for a in range(0, n, piece):
        param[a:min(n, a + piece)].normal_(0.0, 0.02, generator=gen)
    windows = [(0, 1 << 20), ((1 << 31) - (1 << 19), (1 << 31) + (1 << 19)), ((1 << 32) - (1 << 19), n)]
    host = [OracleState(np_host(param[a:b]), np.zeros(b - a, np.uint8), np.zeros(b - a, np.uint8),
                        np.ones(1, np.float32), np.ones(1, np.float32)) for a, b in windows]
    opt = pk.FP8AdamW([param], [grad], schedule=schedule, speculate_from_step=2)
    try:
        for t in (1, 2, 3):
            for k, a in enumerate(range(0, n, piece)):
                b = min(n, a + piece)
                grad[a:b].copy_(random_grad(b - a, 2000 * t + k, dev))
            for a, _ in windows:
                grad[a] = 8192.0
            opt.step(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            torch.cuda.synchronize()
            h = oracle.Hyper(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            cfg = oracle_config(h, "e4m3", "e5m2", "tensor", "pow2", master)
            for (a, b), st in zip(windows, host):
                st.step(cfg, np_host(grad[a:b]))
                compare_tensor(f"{schedule} {master} window [{a}, {b}) step {t}", st, np_host(param[a:b]),
                               np_host(opt.m[0][a:b]), np_host(opt.v[0][a:b]), np_host(opt.m_scale[0]),
                               np_host(opt.v_scale[0]), master)
                st.p = np_host(param[a:b]).copy()  # continue from the device's weights (within the bar)
    finally:
        opt.close()
        del param, grad
        torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["two_pass", "speculative", "block128"])
def test_zero_gradient_tensors_and_transitions(mode):
    """Degenerate amax cases in one list, against the oracle at every step:
    a tensor whose gradient is zero in every step (amax 0: scale 1, zero
    codes, weights only decayed), one whose gradient is zero for steps 1-4 and
    random afterwards (under the speculative schedule, from step 2, the first
    nonzero step is predicted from an amax of 0, so the fix-up recomputes the
    zero codes), and one that is random for steps 1-3 and zero afterwards (the
    moments decay)."""
    dev = torch.device("cuda")
    sizes = [4099, 70001, 1000]
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    params = [torch.randn(n, generator=gen, device=dev) * 0.02 for n in sizes]
    grads = [torch.zeros(n, dtype=torch.bfloat16, device=dev) for n in sizes]
    gran = "block128" if mode == "block128" else "tensor"
    nb = [1 if gran == "tensor" else -(-n // 128) for n in sizes]
    host = [OracleState(np_host(p), np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.ones(k, np.float32),
                        np.ones(k, np.float32)) for p, n, k in zip(params, sizes, nb)]
    opt = pk.FP8AdamW(params, grads, granularity=gran, collect_stats=True,
                      schedule="speculative" if mode == "speculative" else "two_pass", speculate_from_step=2)
    try:
        for t in range(1, 8):
            grads[0].zero_()
            grads[1].copy_(random_grad(sizes[1], 500 + t, dev) if t >= 5 else torch.zeros_like(grads[1]))
            grads[2].copy_(random_grad(sizes[2], 600 + t, dev) if t <= 3 else torch.zeros_like(grads[2]))
            opt.step(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            torch.cuda.synchronize()
            h = oracle.Hyper(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
            cfg = oracle_config(h, "e4m3", "e5m2", gran, "pow2", "fp32")
            gstats = opt.stats()
            for i, n in enumerate(sizes):
                host[i].step(cfg, np_host(grads[i]))
                name = f"{mode} tensor {i} step {t}"
                compare_tensor(name, host[i], np_host(params[i]), np_host(opt.m[i]), np_host(opt.v[i]),
                               np_host(opt.m_scale[i]), np_host(opt.v_scale[i]), "fp32")
                _compare_stats(name, gstats[i], host[i].stats, gran)
                upload_params(params[i], host[i])
            assert (opt.m_scale[0] == 1.0).all() and not opt.m[0].any() and not opt.v[0].any()
    finally:
        opt.close()
