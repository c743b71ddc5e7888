"""Benchmark of the FP8-moment AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama2_7b]
                    [--schedule two_pass|speculative]

Times K whole optimizer steps (every tensor of the list, one fp8adam_step
each) after W warm-up steps, with inputs resident in HBM, and prints one JSON
line: params updated/s, the roofline of the dominant kernel (algorithmic
bytes / its HIP-event duration, against 8 TB/s, and beside it against a plain
2 GiB device copy timed on the same GPU), and the CPU oracle timed on a
bounded sample of the same workload.  Every step gets a fresh gradient draw
(generated into the bound gradient buffers between steps, outside the timed
events), so the moments and their scales evolve as in training.

Other modes (used to make the committed profiles):
    --calibrate-copy   a plain device copy of 2 GiB, for HBM counter scaling
    --same-grad        reuse step 1's gradient every step (profiler runs: drawing
                       fresh gradients under counter collection is very slow; the
                       optimizer kernels do the same work either way)
    --no-cpu-baseline  skip the oracle timing
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# algorithmic HBM bytes per parameter of the dominant kernel (one launch covers every parameter)
#   update pass, fp32 master: read p4 g2 m1 v1, write p4 m1 v1                 = 14
#   update pass, bf16 master: read p2 g2 m1 v1, write p2 m1 v1                 = 10
#   block-128 pass, fp32 master: 14 + 2 scales * (read 4 + write 4) / 128      = 14.125
BYTES_PER_PARAM = {("tensor", "fp32"): 14.0, ("tensor", "bf16"): 10.0,
                   ("block128", "fp32"): 14.125, ("block128", "bf16"): 10.125}
KERNEL_SOURCES = ["precision_adam_optimizer_amd/csrc/fp8adam.hip", "precision_adam_optimizer_amd/csrc/fp8adam_engine.h",
                  "precision_adam_optimizer_amd/csrc/fp8_codec.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def calibrate_copy():
    import torch
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {n} bytes 5 times")


def copy_bandwidth(stream) -> float:
    """GB/s (bytes read + bytes written) of a plain 2 GiB device-to-device
    streaming copy on this GPU (the library's fp8adam_stream_copy: the step
    kernels' access pattern), timed with HIP events: the practical ceiling the
    step's kernels are compared with beside the nominal peak."""
    import torch

    import precision_adam_optimizer_amd as pk
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        a.fill_(1)
        for _ in range(2):
            pk.fp8adam_stream_copy(a, b, stream.cuda_stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            pk.fp8adam_stream_copy(a, b, stream.cuda_stream)
        e1.record(stream)
    torch.cuda.synchronize()
    gbps = 2 * n * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    return gbps


def cpu_baseline(w, shapes, idx, threads: int = 1):
    """The oracle on step 1 of the tensors `idx` (inputs drawn with the same
    generators on the GPU, copied to the host): one oracle call per tensor, on
    `threads` host threads (the calls release the GIL).  Returns (params, wall s)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle
    import workloads

    h = oracle.Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=1)
    cfg = oracle.make_config(h, 0 if w.m_fmt == "e4m3" else 1, 0 if w.v_fmt == "e4m3" else 1,
                             block=128 if w.granularity == "block128" else 0, master_bf16=(w.master == "bf16"),
                             l2_coupled=(w.decay_mode == "l2"))
    jobs = []
    for i in idx:
        name, s = shapes[i]
        n = workloads.numel(s)
        p = workloads.make_param(w, i, s, "cuda").cpu()
        p = p.view(torch.int16).numpy().view(np.uint16).copy() if w.master == "bf16" else p.numpy().copy()
        g = workloads.make_grad(w, i, s, 1, "cuda").cpu().view(torch.int16).numpy().view(np.uint16).copy()
        nb = 1 if w.granularity == "tensor" else -(-n // 128)
        jobs.append((p, g, np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.ones(nb, np.float32),
                     np.ones(nb, np.float32)))
    jobs.sort(key=lambda j: -j[0].size)  # largest first: better balance over the threads
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda j: oracle.step(cfg, *j), jobs))
    return sum(j[0].size for j in jobs), time.perf_counter() - t0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama2_7b",
                    choices=["flat_1m", "llama2_100m", "llama2_7b", "llama2_7b_block128", "llama2_7b_l2",
                             "llama2_13b_bf16", "llama2_7b_rank0_of_8"])
    ap.add_argument("--schedule", default="speculative", choices=["two_pass", "speculative"])
    ap.add_argument("--scaling", default="just_in_time", choices=["just_in_time", "delayed"],
                    help="delayed: scale from a 16-step amax history, one pass (per-tensor lists)")
    ap.add_argument("--rounding", default="nearest", choices=["nearest", "stochastic"],
                    help="stochastic: moments rounded with a Philox4x32-10 stream (seed 1234)")
    ap.add_argument("--amp", action="store_true",
                    help="loss-scaled gradients (scale 2^16) through the fused unscale / Inf-NaN skip / "
                         "global-norm clip (max_norm 1.0) step")
    ap.add_argument("--same-grad", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the sharding design is described in the design notes); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch

    import precision_adam_optimizer_amd as pk
    import workloads

    w = workloads.WORKLOADS[args.workload]()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shapes = w.shapes
    total = w.total_params
    log(f"workload {w.name}: {len(shapes)} tensors, {total} params; generating inputs")
    params = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
    grads = [workloads.make_grad(w, i, s, 1, dev) for i, (_, s) in enumerate(shapes)]
    torch.cuda.synchronize()
    # one-pass block scales; coupled L2 needs the old p in the amax pass, so two passes
    scaling = args.scaling if w.granularity == "tensor" else "just_in_time"
    schedule = args.schedule if (w.granularity == "tensor" and w.decay_mode == "decoupled"
                                 and scaling == "just_in_time") else "two_pass"
    opt = pk.FP8AdamW(params, grads, m_format=w.m_fmt, v_format=w.v_fmt, granularity=w.granularity,
                      schedule=schedule, decay_mode=w.decay_mode, scaling=scaling, rounding=args.rounding,
                      seed=1234)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    stream = torch.cuda.current_stream()

    loss_scale = 2.0 ** 16
    amp = pk.amp_state(loss_scale, dev) if args.amp else None

    def load_grads(t):
        if args.same_grad and (t > 1 or not args.amp):  # (--amp: step 1 draws the scaled gradient)
            return
        for i, (_, shp) in enumerate(shapes):
            g = workloads.make_grad(w, i, shp, t, dev)
            grads[i].copy_((g.float() * loss_scale).to(torch.bfloat16) if args.amp else g)

    def opt_step(t):
        if args.amp:
            opt.step_amp(amp, step=t, max_norm=1.0, **hp)
        else:
            opt.step(step=t, **hp)

    log(f"context: {opt.num_chunks} chunks, schedule {schedule}, scaling {scaling}; warmup {args.warmup} steps")
    t = 0
    for _ in range(args.warmup):
        t += 1
        load_grads(t)
        opt_step(t)
        torch.cuda.synchronize()
        log(f"warm-up step {t} done")

    opt.set_timing(True)
    evs = []
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        t += 1
        load_grads(t)  # not timed
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        opt_step(t)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = sum(a.elapsed_time(b) for a, b in evs)
    ktimes = opt.kernel_times()
    opt.set_timing(False)
    ms_per_step = ms_total / args.steps
    value = total / (ms_per_step / 1e3)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (wall incl. gradient generation {wall / args.steps * 1e3:.3f} ms/step)")
    for k, (tot, cnt) in ktimes.items():
        if cnt:
            log(f"  {k}: {cnt} launches, avg {tot / cnt * 1e3:.1f} us")

    kernel = "block128_pass" if w.granularity == "block128" else (
        "delayed_pass" if scaling == "delayed" else "spec_pass" if schedule == "speculative" else "update_pass")
    ktot, kcnt = ktimes[kernel]
    kavg_s = ktot / kcnt / 1e3
    bpp = BYTES_PER_PARAM[(w.granularity, w.master)]
    alg_bytes = bpp * total
    achieved = alg_bytes / kavg_s / 1e9
    # the counters are per kernel instantiation: stochastic rounding has its own
    traffic = load_traffic(w.name, kernel + ("_sr" if args.rounding == "stochastic" else ""))
    # bytes the whole step moved: + the amax pass (g, m, v; and p with coupled L2) in the
    # two-pass schedule; the speculative schedule's fix-up (the codes of mispredicted moments
    # read and written) is timed separately and reported as fixup_avg_us
    fix_ms, fix_n = ktimes.get("fixup", (0.0, 0))
    amax_bpp = 4.0 + ((4.0 if w.master == "fp32" else 2.0) if w.decay_mode == "l2" else 0.0)
    step_bytes = alg_bytes + (amax_bpp * total if (w.granularity == "tensor" and schedule == "two_pass"
                                                   and scaling == "just_in_time") else 0.0)
    if args.amp:  # + the gradient-norm pass (g read once)
        step_bytes += 2.0 * total
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                "kernel_avg_us": round(kavg_s * 1e6, 2), "algorithmic_bytes_per_launch": alg_bytes,
                "bytes_per_param": bpp,
                "whole_step_GBps_excluding_fixup": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1)}
    if schedule == "speculative":
        roofline["fixup_avg_us"] = round(fix_ms / max(fix_n, 1) * 1e3, 2)

    copy_gbps = copy_bandwidth(stream)
    log(f"device copy: {copy_gbps:.0f} GB/s (read + write); {kernel} at {achieved / copy_gbps:.1%} of it")
    roofline["copy_GBps"] = round(copy_gbps, 1)
    roofline["frac_of_copy"] = round(achieved / copy_gbps, 4)

    cpu = None
    if not args.no_cpu_baseline:
        # step 1 of layer 0 (its nine tensors) on one thread, then of layers 0-3 on the
        # host's cores, one oracle call per tensor (the box gives a job 16 cores)
        layered = any(n.startswith("layers.0.") for n, _ in shapes)
        idx1 = [i for i, (n, _) in enumerate(shapes) if n.startswith("layers.0.")] or [0]
        n1, s1 = cpu_baseline(w, shapes, idx1, threads=1)
        log(f"cpu oracle, 1 thread: {n1 / s1:.3e} params/s over {n1} params")
        threads = max(1, min(16, os.cpu_count() or 1))
        idxn = [i for i, (n, _) in enumerate(shapes)
                if any(n.startswith(f"layers.{k}.") for k in range(4))] or [0]
        nn, sn = cpu_baseline(w, shapes, idxn, threads=threads)
        log(f"cpu oracle, {threads} threads: {nn / sn:.3e} params/s over {nn} params")
        cpu = {"value": round(nn / sn, 1), "unit": "params/s", "cores": threads, "kind": "oracle",
               "sample": (f"step 1 of the {len(idxn)} tensors of layers 0-3 ({nn} params) of the same list, "
                          if layered else f"step 1 of the whole list ({len(idxn)} tensor, {nn} params), ") +
                         f"C oracle, one call per tensor on {threads} threads, {sn:.1f} s wall; " +
                         (f"single thread on layer 0 ({n1} params)" if layered else "single thread") +
                         f": {n1 / s1:.4g} params/s",
               "value_1_thread": round(n1 / s1, 1)}

    out = {
        "metric": "params updated/sec + achieved HBM GB/s (% of peak), 7B-shaped FP8-moment Adam step",
        "value": round(value, 1),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.master == "fp32" else "bf16-master/f32-math",
        "data": "synthetic",
        "config": {"workload": w.name, "tensors": len(shapes), "params": total, "m_format": w.m_fmt,
                   "v_format": w.v_fmt, "scale": w.granularity, "master": w.master,
                   "weight_decay": w.weight_decay, "decay_mode": w.decay_mode, "schedule": schedule,
                   "scaling": scaling if scaling == "just_in_time" else "delayed (amax history 16, margin 0)",
                   "loss_scaling": "scale 2^16, Inf/NaN skip, clip to global norm 1.0" if args.amp else None,
                   "rounding": args.rounding,
                   "grad": "bf16, step 1's draw every step" if args.same_grad else "fresh bf16 draw per step",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    opt.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
