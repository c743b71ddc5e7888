"""Benchmark of the FP8-moment AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama2_7b]
                    [--schedule two_pass|speculative] [--predictor auto|probe|growth]
                    [--m-format e4m3|e5m2] [--v-format e4m3|e5m2]

Times K whole optimizer steps (every tensor of the list, one fp8adam_step
each) after W warm-up steps, with inputs resident in HBM, and prints one JSON
line: params updated/s; the roofline of the dominant kernel (algorithmic bytes
/ its HIP-event duration, against 8 TB/s, and beside it against the pass's own
byte mix streamed with trivial arithmetic by fp8adam_stream_mix on the same
GPU, and against the time its bytes would take at the GPU's read-only and
write-only rates, fp8adam_stream_rw); the bytes and rate of the whole step, the
speculative schedule's scale probe and fix-up included;
and the CPU oracle timed on the same workload (the whole list for the flat 1M
tensor and the Llama-2-100M list, a bounded sample of the larger lists).  Every
step gets a fresh gradient draw (generated into the bound gradient buffers
between steps, outside the timed events), so the moments and their scales
evolve as in training.

Other modes:
    --format-sweep     Llama-2-100M list: all four (m, v) format pairs over 20 steps with the
                       stats counters on; one JSON line with each pair's underflow and
                       saturation counts (the pages' Fig. 5 format experiment)
    --collect-stats    count underflow / saturation in the timed steps too (another kernel
                       instantiation than the default line's)
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
# of which written: p (4 or 2 bytes) and the two codes, plus the two block scales per 128 elements
WRITE_BYTES_PER_PARAM = {("tensor", "fp32"): 6.0, ("tensor", "bf16"): 4.0,
                         ("block128", "fp32"): 6.0625, ("block128", "bf16"): 4.0625}
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


def rw_bandwidth(stream) -> tuple[float, float]:
    """GB/s of a read-only and of a write-only stream of 4 GiB (fp8adam_stream_rw: the
    step kernels' access pattern), median of three rounds on fresh allocations, five
    launches each: the two rates that bound any mix of reads and writes."""
    import torch

    import precision_adam_optimizer_amd as pk
    n = 4 << 30
    reads, writes = [], []
    with torch.cuda.stream(stream):
        for _ in range(3):
            a = torch.ones(n, dtype=torch.uint8, device="cuda")
            b = torch.empty(n, dtype=torch.uint8, device="cuda")
            for src, dst, out in ((a, None, reads), (None, b, writes)):
                for _ in range(2):
                    pk.fp8adam_stream_rw(src, dst, stream.cuda_stream)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(5):
                    pk.fp8adam_stream_rw(src, dst, stream.cuda_stream)
                e1.record(stream)
                e1.synchronize()
                out.append(n * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9)
            del a, b
            torch.cuda.empty_cache()
    torch.cuda.synchronize()
    return sorted(reads)[1], sorted(writes)[1]


def mix_bandwidth(stream, master: str) -> tuple[float, float]:
    """GB/s of the update pass's own byte mix (fp8adam_stream_mix: read p, g and two
    code streams, write p and two code streams, with the pass's instructions,
    work-group shape and order, trivial arithmetic) over 2^29 elements (7.5 GB per
    launch with an fp32 master), timed with HIP events on this GPU.  Where the six
    buffers land in HBM moves the rate by a few percent, so each of three rounds
    allocates them anew and times five launches: (best, median) of the rounds."""
    import torch

    import precision_adam_optimizer_amd as pk
    n = 1 << 29
    pdt = torch.bfloat16 if master == "bf16" else torch.float32
    bpe = 10.0 if master == "bf16" else 14.0
    rates = []
    with torch.cuda.stream(stream):
        for _ in range(3):
            p = torch.zeros(n, dtype=pdt, device="cuda")
            g = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
            codes = [torch.zeros(n, dtype=torch.uint8, device="cuda") for _ in range(4)]
            for _ in range(2):
                pk.fp8adam_stream_mix(p, g, *codes, stream=stream.cuda_stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                pk.fp8adam_stream_mix(p, g, *codes, stream=stream.cuda_stream)
            e1.record(stream)
            e1.synchronize()
            rates.append(bpe * n * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9)
            del p, g, codes
            torch.cuda.empty_cache()
    torch.cuda.synchronize()
    rates.sort()
    return rates[-1], rates[1]


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


FORMATS = [("e4m3", "e5m2"), ("e5m2", "e5m2"), ("e5m2", "e4m3"), ("e4m3", "e4m3")]


def format_sweep(args):
    """The Llama-2-100M list in all four (m, v) format pairs, 20 steps each from a
    fresh state with the stats counters on: per pair, the underflow and saturation
    counts summed over the steps and at the last step, and the share of moments
    stored as zero although nonzero (the pages' Fig. 5 format experiment: v in
    E4M3 loses small second moments to zero)."""
    import torch

    import precision_adam_optimizer_amd as pk
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pairs = {}
    for m_fmt, v_fmt in FORMATS:
        w = workloads.llama2_100m(m_fmt, v_fmt)
        shapes = w.shapes
        params = [workloads.make_param(w, i, s, dev) for i, (_, s) in enumerate(shapes)]
        grads = [workloads.make_grad(w, i, s, 1, dev) for i, (_, s) in enumerate(shapes)]
        opt = pk.FP8AdamW(params, grads, m_format=m_fmt, v_format=v_fmt, collect_stats=True,
                          schedule=args.schedule)
        keys = ("underflow_m", "underflow_v", "saturated_m", "saturated_v", "nonfinite")
        total = dict.fromkeys(keys, 0)
        last = None
        for t in range(1, w.steps + 1):
            for i, (_, shp) in enumerate(shapes):
                grads[i].copy_(workloads.make_grad(w, i, shp, t, dev))
            opt.step(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=t)
            st = opt.stats()
            last = {k: sum(x[k] for x in st) for k in keys}
            for k in keys:
                total[k] += last[k]
        opt.close()
        n = w.total_params
        pairs[f"{m_fmt}/{v_fmt}"] = {
            "steps": w.steps, "params": n, "total_over_steps": total, "at_last_step": last,
            "underflow_v_share_last_step": round(last["underflow_v"] / n, 6),
            "underflow_m_share_last_step": round(last["underflow_m"] / n, 6)}
        log(f"{m_fmt}/{v_fmt}: over {w.steps} steps {total}; last step {last}")
        del params, grads, opt
        torch.cuda.empty_cache()
    out = {"metric": "underflow and saturation counts of the FP8 moments, Llama-2-100M list, four format pairs",
           "unit": "elements", "n_gpus": 1, "data": "synthetic",
           "config": {"workload": "llama2_100m", "tensors": len(workloads.llama2_100m().shapes),
                      "params": workloads.llama2_100m().total_params, "steps": 20, "schedule": args.schedule,
                      "grad": "fresh bf16 draw per step, per-tensor scale 10^U(-7,-1)"},
           "pairs": pairs}
    print(json.dumps(out), flush=True)


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
    ap.add_argument("--predictor", default="auto", choices=["auto", "probe", "growth"],
                    help="how the speculative schedule predicts each scale (auto: the probe on lists of "
                         "at least 2^28 elements)")
    ap.add_argument("--m-format", choices=["e4m3", "e5m2"], default=None,
                    help="format of the first moment (default: the workload's, E4M3)")
    ap.add_argument("--v-format", choices=["e4m3", "e5m2"], default=None,
                    help="format of the second moment (default: the workload's, E5M2)")
    ap.add_argument("--amp", action="store_true",
                    help="loss-scaled gradients (scale 2^16) through the fused unscale / Inf-NaN skip / "
                         "global-norm clip (max_norm 1.0) step")
    ap.add_argument("--collect-stats", action="store_true")
    ap.add_argument("--format-sweep", action="store_true")
    ap.add_argument("--same-grad", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the step has no multi-GPU path; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.format_sweep:
        format_sweep(args)
        return

    import torch

    import precision_adam_optimizer_amd as pk
    import workloads

    w = workloads.WORKLOADS[args.workload]()
    if args.m_format or args.v_format:
        w.m_fmt = args.m_format or w.m_fmt
        w.v_fmt = args.v_format or w.v_fmt
        if args.workload == "llama2_100m":
            w.name = f"llama2_100m_{w.m_fmt}_{w.v_fmt}"
        else:
            w.name = f"{w.name}_{w.m_fmt}_{w.v_fmt}"
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
                      predictor=args.predictor,
                      seed=1234, collect_stats=args.collect_stats)
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

    kernel = "block128_pass" if w.granularity == "block128" else (
        "delayed_pass" if scaling == "delayed" else "spec_pass" if schedule == "speculative" else "update_pass")
    # HIP events on the dominant kernel's launches (the roofline's duration) and, in the
    # speculative schedule, the fix-up's and the probe's (reported below); every timed launch adds
    # a gap of a few microseconds to the stream, so the small kernels that are not reported go untimed
    opt.set_timing(True, kinds=[kernel] + (["fixup", "spec_probe"] if schedule == "speculative" else []))
    evs = []
    spacer = torch.zeros(1 << 26, dtype=torch.float32, device=dev)  # 256 MB: ~0.1 ms of streaming
    requant = []  # per timed step: (element, moment) pairs brought to the true scale by the fix-up
    probed = []   # per timed step: elements the speculative schedule's scale probe read
    stat_keys = ("underflow_m", "underflow_v", "saturated_m", "saturated_v", "nonfinite")
    stat_sum = dict.fromkeys(stat_keys, 0)
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        t += 1
        load_grads(t)  # not timed
        # untimed work queued ahead of the step keeps the GPU busy while the host enqueues the step's
        # launches, as the backward pass would in training (else a short step would include the
        # host's launch latency: the stats read below leaves the stream idle)
        spacer.mul_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        opt_step(t)
        e1.record(stream)
        evs.append((e0, e1))
        # read outside the events (this synchronizes the stream between steps)
        st = opt.stats()
        requant.append(sum(x["requantized"] for x in st))
        probed.append(sum(x["probed"] for x in st))
        if args.collect_stats:
            for k in stat_keys:
                stat_sum[k] += sum(x[k] for x in st)
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

    ktot, kcnt = ktimes[kernel]
    kavg_s = ktot / kcnt / 1e3
    bpp = BYTES_PER_PARAM[(w.granularity, w.master)]
    alg_bytes = bpp * total
    achieved = alg_bytes / kavg_s / 1e9
    # the counters are per kernel instantiation: stochastic rounding has its own
    traffic = load_traffic(w.name, kernel + ("_sr" if args.rounding == "stochastic" else ""))
    # bytes the whole step moved:
    #   the dominant pass (algorithmic bytes);
    #   + the amax pass (g, m, v; and p with coupled L2) in the two-pass schedule;
    #   + the per-part amax partials the speculative and delayed passes write and the
    #     check / commit reads (8 bytes each way per part of 1024 elements, 2048 with bf16),
    #     and in the speculative schedule their per-chunk maxima (8 bytes each way per chunk);
    #   + the scale probe: g and both codes of the candidate parts it reads (4 bytes per
    #     element);
    #   + the fix-up: the codes of every mispredicted moment, read and written (2 bytes per
    #     (element, moment) pair; the rare groups it recomputes read 3 bytes more, not counted);
    #   + the gradient-norm pass with loss scaling (g read once).
    two_pass = w.granularity == "tensor" and schedule == "two_pass" and scaling == "just_in_time"
    amax_bpp = 4.0 + ((4.0 if w.master == "fp32" else 2.0) if w.decay_mode == "l2" else 0.0)
    part = 2048 if w.master == "bf16" else 1024
    step_bytes = alg_bytes + (amax_bpp * total if two_pass else 0.0)
    if schedule == "speculative" or scaling == "delayed":
        step_bytes += 16.0 * -(-total // part)
    if schedule == "speculative":
        step_bytes += 16.0 * opt.num_chunks
    fix_ms, fix_n = ktimes.get("fixup", (0.0, 0))
    fix_pairs = sum(requant) / max(len(requant), 1)
    fix_bytes = 2.0 * fix_pairs
    step_bytes += fix_bytes
    probe_ms, probe_n = ktimes.get("spec_probe", (0.0, 0))
    probe_elems = sum(probed) / max(len(probed), 1)
    probe_bytes = 4.0 * probe_elems
    step_bytes += probe_bytes
    if args.amp:
        step_bytes += 2.0 * total
    step_gbps = step_bytes / (ms_per_step / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                "kernel_avg_us": round(kavg_s * 1e6, 2), "algorithmic_bytes_per_launch": alg_bytes,
                "bytes_per_param": bpp,
                "whole_step_bytes": round(step_bytes), "whole_step_GBps": round(step_gbps, 1),
                "whole_step_frac": round(step_gbps / HBM_PEAK_GBS, 4)}
    if schedule == "speculative":
        fix_us = fix_ms / max(fix_n, 1) * 1e3
        roofline.update({
            "fixup_avg_us": round(fix_us, 2),
            "fixup_pairs_per_step": round(fix_pairs),
            "fixup_pair_share": round(fix_pairs / (2.0 * total), 5),
            "fixup_bytes_per_step": round(fix_bytes),
            "fixup_GBps": round(fix_bytes / (fix_us / 1e6) / 1e9, 1) if fix_us > 0 else None,
            "fixup_pairs_each_step": requant})
        probe_us = probe_ms / max(probe_n, 1) * 1e3
        roofline.update({
            "probe_avg_us": round(probe_us, 2),
            "probe_elements_per_step": round(probe_elems),
            "probe_bytes_per_step": round(probe_bytes),
            "probe_GBps": round(probe_bytes / (probe_us / 1e6) / 1e9, 1) if probe_us > 0 else None})

    mix_best, mix_med = mix_bandwidth(stream, w.master)
    copy_gbps = copy_bandwidth(stream)
    log(f"pass byte mix: {mix_med:.0f} GB/s (median; best {mix_best:.0f}); {kernel} at {achieved / mix_med:.1%} of it; "
        f"device copy {copy_gbps:.0f} GB/s")
    roofline["mix_GBps"] = round(mix_med, 1)
    roofline["mix_GBps_best"] = round(mix_best, 1)
    roofline["frac_of_mix"] = round(achieved / mix_med, 4)
    roofline["copy_GBps"] = round(copy_gbps, 1)
    # the kernel's bytes at the read-only and the write-only rates, one after the other: the
    # bound its read/write mix would reach if the two streams did not slow each other down
    read_gbps, write_gbps = rw_bandwidth(stream)
    wpp = WRITE_BYTES_PER_PARAM[(w.granularity, w.master)]
    rw_bound = bpp / ((bpp - wpp) / read_gbps + wpp / write_gbps)
    log(f"read-only stream {read_gbps:.0f} GB/s, write-only {write_gbps:.0f} GB/s: {kernel}'s "
        f"{bpp - wpp:g} B read + {wpp:g} B written per param at those rates {rw_bound:.0f} GB/s; "
        f"{kernel} at {achieved / rw_bound:.1%} of it")
    roofline["read_GBps"] = round(read_gbps, 1)
    roofline["write_GBps"] = round(write_gbps, 1)
    roofline["rw_bound_GBps"] = round(rw_bound, 1)
    roofline["frac_of_rw_bound"] = round(achieved / rw_bound, 4)

    cpu = None
    if not args.no_cpu_baseline:
        threads = max(1, min(16, os.cpu_count() or 1))
        if total <= 250_000_000:
            # small lists: step 1 of the whole list, on one thread and on the host's cores
            idx1 = idxn = list(range(len(shapes)))
            what = f"step 1 of the whole list ({len(shapes)} tensors, {total} params)"
            what1 = "single thread on the whole list"
        else:
            # step 1 of layer 0 (its nine tensors) on one thread, then of layers 0-3 on the
            # host's cores, one oracle call per tensor (the box gives a job 16 cores)
            idx1 = [i for i, (n, _) in enumerate(shapes) if n.startswith("layers.0.")] or [0]
            idxn = [i for i, (n, _) in enumerate(shapes)
                    if any(n.startswith(f"layers.{k}.") for k in range(4))] or [0]
            what = f"step 1 of the {len(idxn)} tensors of layers 0-3 of the same list"
            what1 = "single thread on layer 0"
        n1, s1 = cpu_baseline(w, shapes, idx1, threads=1)
        log(f"cpu oracle, 1 thread: {n1 / s1:.3e} params/s over {n1} params")
        nn, sn = cpu_baseline(w, shapes, idxn, threads=threads)
        log(f"cpu oracle, {threads} threads: {nn / sn:.3e} params/s over {nn} params")
        cpu = {"value": round(nn / sn, 1), "unit": "params/s", "cores": threads, "kind": "oracle",
               "sample": f"{what} ({nn} params), C oracle, one call per tensor on {threads} threads, "
                         f"{sn:.1f} s wall; {what1} ({n1} params): {n1 / s1:.4g} params/s",
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
                   "predictor": args.predictor if schedule == "speculative" else None,
                   "grad": "bf16, step 1's draw every step" if args.same_grad else "fresh bf16 draw per step",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if args.collect_stats:
        out["stats_over_timed_steps"] = stat_sum
    opt.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
