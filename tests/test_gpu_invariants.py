"""GPU invariants and ABI behaviour of the HIP step (through the C ABI):
determinism, tensor-order invariance, block mode on one block == tensor mode,
checkpoint/resume, guard bands after every buffer, error codes, runtime."""
import ctypes

import numpy as np
import pytest
import torch

import precision_adam_optimizer_amd as pk
from tests.gpu_util import np_host, random_grad

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _make(sizes, seed, device="cuda", master=torch.float32):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    params = [(torch.randn(n, generator=g, device=device) * 0.02).to(master) for n in sizes]
    return params


def _run(sizes, steps, seed=0, order=None, granularity="tensor"):
    params = _make(sizes, seed)
    grads = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
    order = list(range(len(sizes))) if order is None else order
    opt = pk.FP8AdamW([params[i] for i in order], [grads[i] for i in order], granularity=granularity)
    for t in range(1, steps + 1):
        for i, n in enumerate(sizes):
            grads[i].copy_(random_grad(n, 1000 * seed + 10 * t + i, "cuda"))
        opt.step(step=t, **HP)
    torch.cuda.synchronize()
    inv = {o: k for k, o in enumerate(order)}
    out = [(np_host(params[i]), np_host(opt.m[inv[i]]), np_host(opt.v[inv[i]]), np_host(opt.m_scale[inv[i]]),
            np_host(opt.v_scale[inv[i]])) for i in range(len(sizes))]
    opt.close()
    return out


def _same(a, b):
    for x, y in zip(a, b):
        for u, v in zip(x, y):
            assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def test_deterministic_bitwise():
    sizes = [100_003, 4096, 77]
    _same(_run(sizes, 3), _run(sizes, 3))


def test_tensor_order_invariance():
    sizes = [100_003, 4096, 77, 16384 * 3 + 5]
    _same(_run(sizes, 2), _run(sizes, 2, order=[3, 1, 0, 2]))


def test_block_mode_on_one_block_equals_tensor_mode():
    a = _run([128], 4, granularity="tensor")
    b = _run([128], 4, granularity="block128")
    _same(a, b)


def test_resume_is_bit_exact():
    """Run 5 steps; separately run 3, copy the state, build a new context from
    the copy and run steps 4-5: identical bits."""
    sizes = [50_001, 4096]
    ref = _run(sizes, 5)
    params = _make(sizes, 0)
    grads = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
    opt = pk.FP8AdamW(params, grads)
    for t in range(1, 4):
        for i, n in enumerate(sizes):
            grads[i].copy_(random_grad(n, 10 * t + i, "cuda"))
        opt.step(step=t, **HP)
    torch.cuda.synchronize()
    ckpt = ([p.clone() for p in params], [m.clone() for m in opt.m], [v.clone() for v in opt.v],
            [s.clone() for s in opt.m_scale], [s.clone() for s in opt.v_scale])
    opt.close()
    p2 = ckpt[0]
    opt2 = pk.FP8AdamW(p2, grads, state=ckpt[1:])
    for t in range(4, 6):
        for i, n in enumerate(sizes):
            grads[i].copy_(random_grad(n, 10 * t + i, "cuda"))
        opt2.step(step=t, **HP)
    torch.cuda.synchronize()
    out = [(np_host(p2[i]), np_host(opt2.m[i]), np_host(opt2.v[i]), np_host(opt2.m_scale[i]),
            np_host(opt2.v_scale[i])) for i in range(len(sizes))]
    opt2.close()
    _same(ref, out)


@pytest.mark.parametrize("granularity,schedule,predictor", [("tensor", "two_pass", None), ("block128", "two_pass", None),
                                                            ("tensor", "speculative", "growth"),
                                                            ("tensor", "speculative", "probe")])
@pytest.mark.parametrize("master", [torch.float32, torch.bfloat16])
def test_guard_bands_untouched(granularity, schedule, predictor, master):
    """Every buffer is a view into a larger allocation whose bytes after the
    tensor (up to the next 16-byte boundary and 64 bytes more) hold a canary;
    ragged sizes must not write past their end.  Under the speculative
    schedule the second code buffers are guarded too; with the growth model's
    predictions the fix-up (16 codes per lane, then groups of 4, then single
    codes at a tensor's end) runs whenever a tensor's scale moves between
    steps, and with the probe's the probe reads the candidate parts, ragged
    last parts included."""
    sizes = [1, 3, 129, 1025, 16387]
    pad = 128
    canary = 0x5A
    bufs, views = [], []

    def alloc(n, dtype):
        esz = torch.tensor([], dtype=dtype).element_size()
        nbytes = n * esz
        raw = torch.full((nbytes + pad,), canary, dtype=torch.uint8, device="cuda")
        bufs.append((raw, nbytes))
        return raw[:nbytes].view(dtype)

    params = [alloc(n, master) for n in sizes]
    for p in params:
        p.copy_((torch.randn(p.numel(), device="cuda") * 0.02).to(master))
    grads = [alloc(n, torch.bfloat16) for n in sizes]
    nb = [1 if granularity == "tensor" else -(-n // 128) for n in sizes]
    m = [alloc(n, torch.uint8) for n in sizes]
    v = [alloc(n, torch.uint8) for n in sizes]
    ms = [alloc(k, torch.float32) for k in nb]
    vs = [alloc(k, torch.float32) for k in nb]
    for x in m + v:
        x.zero_()
    for x in ms + vs:
        x.fill_(1.0)
    if schedule == "speculative":
        # the binding makes the second code buffers with torch.empty_like: hand it guarded ones
        alts = iter([alloc(n, torch.uint8) for n in sizes] + [alloc(n, torch.uint8) for n in sizes])
        orig = torch.empty_like
        torch.empty_like = lambda x, *a, **k: next(alts)
        try:
            opt = pk.FP8AdamW(params, grads, granularity=granularity, collect_stats=True, state=(m, v, ms, vs),
                              schedule="speculative", speculate_from_step=2, predictor=predictor)
        finally:
            torch.empty_like = orig
    else:
        opt = pk.FP8AdamW(params, grads, granularity=granularity, collect_stats=True, state=(m, v, ms, vs))
    requantized = 0
    for t in range(1, 7):
        for i, n in enumerate(sizes):
            grads[i].copy_((random_grad(n, t * 31 + i, "cuda").float() * 4.0 ** (t % 3)).to(torch.bfloat16))
        opt.step(step=t, **HP)
        requantized += sum(s["requantized"] for s in opt.stats())
    torch.cuda.synchronize()
    opt.close()
    if predictor == "growth":
        assert requantized > 0  # the fix-up ran
    for raw, nbytes in bufs:
        tail = raw[nbytes:].cpu().numpy()
        assert (tail == canary).all(), "write past the end of a buffer"


def test_abi_errors_on_device():
    L = pk.load()
    p = torch.zeros(64, device="cuda")
    g = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(64, dtype=torch.uint8, device="cuda")
    s = torch.ones(1, device="cuda")
    good = pk.TensorArg(p.data_ptr(), g.data_ptr(), c.data_ptr(), c.data_ptr(), s.data_ptr(), s.data_ptr(), 64)
    cfg = pk.ConfigArg(0, 1, 0, 0, 0, 0)
    h = ctypes.c_void_p()
    arr = (pk.TensorArg * 1)(good)
    assert L.fp8adam_init(ctypes.byref(h), arr, 1, ctypes.byref(cfg), None) == 0
    for bad in (pk.HParamsArg(1e-3, 0.9, 0.999, 1e-8, 0.0, 0),      # t = 0
                pk.HParamsArg(1e-3, 1.0, 0.999, 1e-8, 0.0, 1),      # beta1 = 1
                pk.HParamsArg(1e-3, 0.9, -0.1, 1e-8, 0.0, 1),       # beta2 < 0
                pk.HParamsArg(1e-3, 0.9, 0.999, -1e-8, 0.0, 1),     # eps < 0
                pk.HParamsArg(float("nan"), 0.9, 0.999, 1e-8, 0.0, 1)):
        assert L.fp8adam_step(h, ctypes.byref(bad), None) == -1
        assert pk.fp8adam_last_error()
    out = (pk.StatsArg * 2)()
    assert L.fp8adam_stats(h, out, 2, None) == -1
    L.fp8adam_destroy(h)
    L.fp8adam_destroy(None)
    mis = pk.TensorArg(p.data_ptr() + 4, g.data_ptr(), c.data_ptr(), c.data_ptr(), s.data_ptr(), s.data_ptr(), 60)
    arr = (pk.TensorArg * 1)(mis)
    assert L.fp8adam_init(ctypes.byref(h), arr, 1, ctypes.byref(cfg), None) == -2
    assert h.value is None


def test_nonfinite_gradient_is_counted_and_isolated():
    sizes = [1000, 1000]
    params = _make(sizes, 5)
    grads = [random_grad(n, 7 + i, "cuda") for i, n in enumerate(sizes)]
    grads[0][10] = float("inf")
    grads[0][11] = float("nan")
    before1 = params[1].clone()
    opt = pk.FP8AdamW(params, grads, collect_stats=True)
    opt.step(step=1, **HP)
    st = opt.stats()
    assert st[0]["nonfinite"] >= 2 and st[1]["nonfinite"] == 0
    assert torch.isfinite(params[1]).all() and not torch.equal(params[1], before1)
    assert opt.m_scale[0].item() == 1.0  # non-finite amax -> unit scale
    opt.close()


def test_runtime_is_torchs():
    v = pk.fp8adam_runtime_version()
    major, minor = (int(x) for x in torch.version.hip.split(".")[:2])
    assert v // 10_000_000 == major and (v // 100_000) % 100 == minor


def test_device_is_gfx950():
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName


def test_timing_only_the_chosen_kernel_kinds():
    """fp8adam_set_timing_kinds: only launches of the chosen kinds are timed
    (the benchmark times the dominant pass and leaves the small kernels'
    launches untimed, free of the gap a timed launch adds)."""
    sizes = [70_001, 4096]
    params = [torch.randn(n, device="cuda") * 0.02 for n in sizes]
    grads = [random_grad(n, 5 + i, "cuda") for i, n in enumerate(sizes)]
    opt = pk.FP8AdamW(params, grads, schedule="speculative", speculate_from_step=2)
    try:
        opt.step(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
        opt.set_timing(True, kinds=["spec_pass", "fixup"])
        for t in (2, 3, 4):
            opt.step(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
        kt = opt.kernel_times()
        assert kt["spec_pass"][1] == 3 and kt["fixup"][1] == 3
        assert all(cnt == 0 for k, (_, cnt) in kt.items() if k not in ("spec_pass", "fixup"))
        opt.set_timing(True)
        opt.step(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=5)
        kt = opt.kernel_times()
        assert kt["spec_pass"][1] == 1 and kt["spec_check"][1] == 1 and kt["scale_prepare"][1] == 1
        opt.set_timing(False)
    finally:
        opt.close()


def test_timed_step_captured_in_a_graph_is_untimed_and_replays_exactly():
    """A two-pass step captured in a HIP graph (torch's capture) while timing
    is on: the captured launches are not timed (a captured kernel runs only
    when the graph replays), and every replay, with eager work and
    synchronizations between the replays, leaves the same state, bit for bit,
    as the same step called eagerly on a copy."""
    dev = torch.device("cuda")
    sizes = [70_001, 4096, 33]
    pa = [torch.randn(n, device=dev) * 0.02 for n in sizes]
    pb = [x.clone() for x in pa]
    grads = [random_grad(n, 11 + i, "cuda") for i, n in enumerate(sizes)]
    hp = HP
    A = pk.FP8AdamW(pa, grads)
    B = pk.FP8AdamW(pb, grads)
    try:
        A.step(**hp, step=1)
        B.step(**hp, step=1)
        torch.cuda.synchronize()
        A.set_timing(True)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            A.step(**hp, step=2)
        torch.cuda.synchronize()
        assert all(cnt == 0 for _, cnt in A.kernel_times().values())
        for r in range(3):
            g.replay()
            torch.cuda.synchronize()
            B.step(**hp, step=2)
            torch.cuda.synchronize()
            _ = float(torch.randn(1 << 20, device=dev).abs().sum())  # eager work between the replays
            for name, xa, xb in (("p", pa, pb), ("m", A.m, B.m), ("v", A.v, B.v),
                                 ("m_scale", A.m_scale, B.m_scale), ("v_scale", A.v_scale, B.v_scale)):
                for i, (x, y) in enumerate(zip(xa, xb)):
                    assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"replay {r + 1}: {name} {i}"
        A.set_timing(False)
        del g
        torch.cuda.synchronize()
    finally:
        A.close()
        B.close()
