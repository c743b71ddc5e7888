"""fp8adam_step_noalloc, the step for callers that cannot allocate device
memory, against fp8adam_init + fp8adam_step on the same inputs.

Both run the same kernels, so every output is compared bit for bit (weights,
codes and scales), which is stricter than the oracle bar the context path is
held to; the second call of each sequence also goes through the oracle.  The
calls come in a row on one process's scratch array: a large ragged list, then
a smaller one (fewer tensors, fewer chunks), so stale descriptors, chunk
entries and partials of the first call are left behind for the second.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_adam_optimizer_amd as pk
import workloads
from tests.gpu_util import OracleState, compare_tensor, np_host, oracle_config, random_grad

pytestmark = pytest.mark.gpu

LARGE = [1, 3, 127, 128, 129, 1000, 4097, 65539, 262_147, 1_048_576 + 5, 3_000_001, 16385, 0, 70_001]
SMALL = [5, 4096, 129, 33_333, 7]


def _lists(sizes, master, granularity, seed, dev):
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    out = {"p": [], "g": [], "m": [], "v": [], "sm": [], "sv": []}
    for i, n in enumerate(sizes):
        p = torch.randn(n, generator=gen, device=dev) * 0.02
        out["p"].append(p.to(torch.bfloat16) if master == "bf16" else p)
        out["g"].append(random_grad(n, seed * 131 + i, dev))
        nb = 1 if granularity == "tensor" else max(1, -(-n // 128))
        cm, cv, sm, sv = workloads.random_state(n, dev, seed * 1000 + i, 0, 1, nblocks=nb, scale_exp=(-24, 2))
        for k, x in zip(("m", "v", "sm", "sv"), (cm, cv, sm, sv)):
            out[k].append(x)
    return out


def _clone(lists):
    return {k: [x.clone() for x in v] for k, v in lists.items()}


def _args(L):
    return [pk.TensorArg(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), sm.data_ptr(), sv.data_ptr(),
                         p.numel()) for p, g, m, v, sm, sv in zip(L["p"], L["g"], L["m"], L["v"], L["sm"], L["sv"])]


def _config(granularity, scale_mode, master, decay_mode, rounding):
    cfg = pk.ConfigArg()
    cfg.m_format, cfg.v_format = pk.E4M3, pk.E5M2
    cfg.granularity = pk._GRAN[granularity]
    cfg.scale_mode = pk._SMODE[scale_mode]
    cfg.master = pk.MASTER_BF16 if master == "bf16" else pk.MASTER_FP32
    cfg.schedule = pk.SCHEDULE_TWO_PASS
    cfg.decay_mode = pk._DECAY[decay_mode]
    cfg.rounding = pk._ROUNDING[rounding]
    cfg.seed = 77
    return cfg


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (t.view(torch.int32) if t.dtype == torch.float32 else t)


def _run_pair(sizes, granularity, scale_mode, master, decay_mode, rounding, seed, t):
    """One call of each entry point on copies of the same state; returns both lists."""
    dev = torch.device("cuda")
    A = _lists(sizes, master, granularity, seed, dev)
    B = _clone(A)
    cfg = _config(granularity, scale_mode, master, decay_mode, rounding)
    hp = pk.HParamsArg(3e-4, 0.9, 0.95, 1e-8, 0.1, t)
    torch.cuda.synchronize()
    ctx = pk.fp8adam_init(_args(A), cfg)
    try:
        pk.fp8adam_step(ctx, hp)
        pk.fp8adam_step_noalloc(_args(B), cfg, hp)
        torch.cuda.synchronize()
    finally:
        pk.fp8adam_destroy(ctx)
    for k in A:
        for i, (a, b) in enumerate(zip(A[k], B[k])):
            assert torch.equal(_bits(a), _bits(b)), f"{k} of tensor {i} (numel {sizes[i]}) differs"
    return A, B


def _check_oracle(sizes, granularity, scale_mode, master, decay_mode, rounding, seed, t):
    """The allocation-free step against the oracle (the bar of the parity tests)."""
    dev = torch.device("cuda")
    L = _lists(sizes, master, granularity, seed, dev)
    host = [OracleState(np_host(L["p"][i]), np_host(L["m"][i]), np_host(L["v"][i]), np_host(L["sm"][i]),
                        np_host(L["sv"][i])) for i in range(len(sizes))]
    cfg = _config(granularity, scale_mode, master, decay_mode, rounding)
    pk.fp8adam_step_noalloc(_args(L), cfg, pk.HParamsArg(3e-4, 0.9, 0.95, 1e-8, 0.1, t))
    torch.cuda.synchronize()
    ocfg = oracle_config(oracle.Hyper(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t),
                         "e4m3", "e5m2", granularity, scale_mode, master, decay_mode)
    ocfg.stochastic, ocfg.seed = int(rounding == "stochastic"), 77
    for i, n in enumerate(sizes):
        ocfg.tensor_index = i
        host[i].step(ocfg, np_host(L["g"][i]))
        compare_tensor(f"noalloc tensor {i} (numel {n})", host[i], np_host(L["p"][i]), np_host(L["m"][i]),
                       np_host(L["v"][i]), np_host(L["sm"][i]), np_host(L["sv"][i]), master)


CASES = [("tensor", "pow2", "fp32", "decoupled", "nearest"),
         ("block128", "amax", "bf16", "l2", "stochastic"),
         ("tensor", "amax", "bf16", "decoupled", "stochastic")]


@pytest.mark.parametrize("case", CASES, ids=["-".join(c) for c in CASES])
def test_noalloc_equals_the_context_step_twice_in_a_row(case):
    print(f"noalloc case {case}: large list", flush=True)
    _run_pair(LARGE, *case, seed=5, t=3)
    print(f"noalloc case {case}: smaller list", flush=True)
    _run_pair(SMALL, *case, seed=6, t=4)
    print(f"noalloc case {case}: smaller list against the oracle", flush=True)
    _check_oracle(SMALL, *case, seed=7, t=2)


def test_noalloc_a_list_whose_chunks_grow_to_fit_the_table():
    """A list of more than 131072 chunks at the context's chunk size (32768
    elements) takes larger chunks here: same results bit for bit."""
    sizes = [131_072 * 32_768 // 3 + 5, 131_072 * 32_768 // 3 + 77, 131_072 * 32_768 // 3 + 1000]
    assert sum(-(-n // 32768) for n in sizes) > pk.NOALLOC_MAX_CHUNKS
    print("noalloc: 4.3e9-element list", flush=True)
    dev = torch.device("cuda")
    A = {"p": [], "g": [], "m": [], "v": [], "sm": [], "sv": []}
    for i, n in enumerate(sizes):
        A["p"].append(torch.full((n,), 0.01 * (i + 1), device=dev))
        g = torch.empty(n, dtype=torch.bfloat16, device=dev)
        piece = 1 << 28
        for k, a in enumerate(range(0, n, piece)):
            g[a:min(n, a + piece)].copy_(random_grad(min(n, a + piece) - a, 40 * i + k, dev))
        A["g"].append(g)
        cm, cv, sm, sv = workloads.make_state(n, dev)
        for k, x in zip(("m", "v", "sm", "sv"), (cm, cv, sm, sv)):
            A[k].append(x)
    B = {k: [x.clone() for x in v] for k, v in A.items() if k != "g"}
    B["g"] = A["g"]  # read only
    cfg = _config("tensor", "pow2", "fp32", "decoupled", "nearest")
    hp = pk.HParamsArg(3e-4, 0.9, 0.95, 1e-8, 0.1, 1)
    ctx = pk.fp8adam_init(_args(A), cfg)
    try:
        pk.fp8adam_step(ctx, hp)
        pk.fp8adam_step_noalloc(_args(B), cfg, hp)
        torch.cuda.synchronize()
    finally:
        pk.fp8adam_destroy(ctx)
    for k in ("p", "m", "v", "sm", "sv"):
        for i in range(len(sizes)):
            assert torch.equal(_bits(A[k][i]), _bits(B[k][i])), f"{k} of tensor {i} differs"
    del A, B
    torch.cuda.empty_cache()


def test_noalloc_at_the_tensor_limit():
    """FP8ADAM_NOALLOC_MAX_TENSORS (4096) small ragged tensors, some empty: 128
    set-up launches fill the descriptor table; the same results as a context."""
    n = pk.NOALLOC_MAX_TENSORS
    sizes = [(k * 37) % 301 for k in range(n)]  # 0..300 elements, zeros included
    print(f"noalloc: {n} tensors", flush=True)
    _run_pair(sizes, "tensor", "pow2", "fp32", "decoupled", "nearest", seed=8, t=2)
    _run_pair(sizes, "block128", "pow2", "bf16", "decoupled", "stochastic", seed=9, t=5)


def test_noalloc_refuses_what_it_cannot_do():
    dev = torch.device("cuda")
    L = _lists([100, 200], "fp32", "tensor", 3, dev)
    hp = pk.HParamsArg(3e-4, 0.9, 0.95, 1e-8, 0.1, 1)
    for field, value, text in (("schedule", pk.SCHEDULE_SPECULATIVE, "TWO_PASS"),
                               ("scaling", pk.SCALING_DELAYED, "just-in-time"),
                               ("collect_stats", 1, "collect_stats"), ("zero_state", 1, "zero_state")):
        cfg = _config("tensor", "pow2", "fp32", "decoupled", "nearest")
        setattr(cfg, field, value)
        with pytest.raises(pk.Fp8AdamError, match=text):
            pk.fp8adam_step_noalloc(_args(L), cfg, hp)
    cfg = _config("tensor", "pow2", "fp32", "decoupled", "nearest")
    too_many = _args(L) * (pk.NOALLOC_MAX_TENSORS // 2 + 1)
    with pytest.raises(pk.Fp8AdamError, match="NOALLOC_MAX_TENSORS"):
        pk.fp8adam_step_noalloc(too_many, cfg, hp)
    # nothing was enqueued: the state is untouched
    torch.cuda.synchronize()
    assert torch.equal(L["p"][0], _lists([100, 200], "fp32", "tensor", 3, dev)["p"][0])


@pytest.mark.parametrize("granularity", ["tensor", "block128"])
def test_noalloc_step_replayed_from_a_graph(granularity):
    """The allocation-free step captured in a HIP graph (through torch's graph
    capture) and replayed three times, with eager work and synchronizations
    between the replays: after every replay the state equals, bit for bit, the
    one that as many eager calls of the same step reach.  (The captured kernels
    use no memset nodes; the scratch array's address is set up by an eager call
    before the capture.)"""
    dev = torch.device("cuda")
    sizes = SMALL + [300_001]
    A = _lists(sizes, "fp32", granularity, 91, dev)
    B = _clone(A)
    W = _clone(A)
    cfg = _config(granularity, "pow2", "fp32", "decoupled", "nearest")
    hp = pk.HParamsArg(3e-4, 0.9, 0.95, 1e-8, 0.1, 5)
    args_a = _args(A)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pk.fp8adam_step_noalloc(_args(W), cfg, hp)  # an eager call first (sets up this device's scratch)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pk.fp8adam_step_noalloc(args_a, cfg, hp)
    torch.cuda.synchronize()
    for k in A:  # capture records the launches without running them
        for x, y in zip(A[k], B[k]):
            assert torch.equal(_bits(x), _bits(y)), f"capture changed {k}"
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        pk.fp8adam_step_noalloc(_args(B), cfg, hp)
        torch.cuda.synchronize()
        _ = float(torch.randn(1 << 20, device=dev).abs().sum())  # eager work between the replays
        for k in A:
            for i, (x, y) in enumerate(zip(A[k], B[k])):
                assert torch.equal(_bits(x), _bits(y)), f"replay {r + 1}: {k} of tensor {i} (numel {sizes[i]})"
    del g
    torch.cuda.synchronize()


def test_noalloc_step_in_a_graph_from_plain_c(tmp_path):
    """The allocation-free step from a plain C program with no torch and no
    Python in the process (tests/c_noalloc_graph_demo.c): after one eager call
    that sets up the device's scratch address, a step is captured with the HIP
    graph API (the capture leaves the state untouched) and replayed three
    times, bit for bit against the same step called eagerly on a copy."""
    import subprocess

    from tests.test_c_abi import build_c_demo
    exe = build_c_demo(tmp_path, "c_noalloc_graph_demo")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
