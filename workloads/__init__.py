"""Tensor-list shapes and seeded synthetic inputs for the FP8-moment Adam step.

This module holds no optimizer arithmetic: it only lists parameter shapes and
draws seeded random tensors (PyTorch generators, on whichever device the caller
names).  The GPU path, the oracle and the benchmark all take their inputs from
here, so both sides of every parity check see the same numbers.

The pages train Llama-2-style models (a 100M-parameter model for the format
sweep of Fig. 5 and a 7B model on Gaudi2); no dataset or trained weights are
available, so these synthetic lists with the same shapes stand in for them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


# --------------------------------------------------------------------- shapes

def llama_shapes(n_layers: int, d: int, ffn: int, vocab: int, tied: bool) -> list[tuple[str, tuple]]:
    """Parameter list of a Llama-2-style decoder (no biases, RMSNorm weights)."""
    out = [("tok_embeddings", (vocab, d))]
    for i in range(n_layers):
        p = f"layers.{i}."
        out += [(p + "wq", (d, d)), (p + "wk", (d, d)), (p + "wv", (d, d)), (p + "wo", (d, d)),
                (p + "w_gate", (ffn, d)), (p + "w_up", (ffn, d)), (p + "w_down", (d, ffn)),
                (p + "attn_norm", (d,)), (p + "ffn_norm", (d,))]
    out.append(("norm", (d,)))
    if not tied:
        out.append(("lm_head", (vocab, d)))
    return out


def numel(shape) -> int:
    return int(math.prod(shape))


@dataclass
class Workload:
    """One synthetic optimizer workload.

    grad_dist: "normal" or "student_t3"; grad_scale: (lo, hi) of the log-uniform
    scale; grad_scale_per: "row" (first dim) or "tensor"; zero_frac: fraction of
    gradient entries set to exactly zero.
    """
    name: str
    shapes: list
    master: str = "fp32"           # "fp32" or "bf16"
    grad_dist: str = "normal"
    grad_scale: tuple = (1e-6, 1e-1)
    grad_scale_per: str = "tensor"
    zero_frac: float = 0.0
    granularity: str = "tensor"    # "tensor" or "block128"
    m_fmt: str = "e4m3"
    v_fmt: str = "e5m2"
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.0
    decay_mode: str = "decoupled"  # "decoupled" (AdamW) or "l2" (wd * p added to the gradient)
    steps: int = 10
    param_std: float = 0.02
    extra: dict = field(default_factory=dict)

    @property
    def total_params(self) -> int:
        return sum(numel(s) for _, s in self.shapes)


LLAMA2_100M = dict(n_layers=12, d=768, ffn=2048, vocab=32000, tied=True)
LLAMA2_7B = dict(n_layers=32, d=4096, ffn=11008, vocab=32000, tied=False)
LLAMA2_13B = dict(n_layers=40, d=5120, ffn=13824, vocab=32000, tied=False)


def flat_1m() -> Workload:
    """1,048,576 fp32 weights as one 1024x1024 tensor; per-row gradient scales
    log-uniform in [1e-6, 1]; Adam without weight decay; 10 steps."""
    return Workload("flat_1m", [("flat", (1024, 1024))], grad_scale=(1e-6, 1.0),
                    grad_scale_per="row", steps=10)


def llama2_100m(m_fmt="e4m3", v_fmt="e5m2") -> Workload:
    """Llama-2-100M-shaped list (tied embedding, 109.5M params), gradient scales
    per tensor in [1e-7, 1e-1], 20 steps, any of the four (m, v) format pairs."""
    return Workload(f"llama2_100m_{m_fmt}_{v_fmt}", llama_shapes(**LLAMA2_100M),
                    grad_scale=(1e-7, 1e-1), steps=20, m_fmt=m_fmt, v_fmt=v_fmt)


def llama2_7b() -> Workload:
    """Llama-2-7B-shaped list (291 tensors, 6.74B params), per-tensor scales,
    Gaussian gradients with per-tensor scale in [1e-6, 1e-1], AdamW wd=0.1."""
    return Workload("llama2_7b_pertensor", llama_shapes(**LLAMA2_7B), grad_scale=(1e-6, 1e-1),
                    weight_decay=0.1, steps=20)


def llama2_7b_block128() -> Workload:
    """Same list with one scale per 128 elements; Student-t(3) gradients with 1%
    exact zeros."""
    return Workload("llama2_7b_block128", llama_shapes(**LLAMA2_7B), grad_dist="student_t3",
                    grad_scale=(1e-6, 1e-1), zero_frac=0.01, granularity="block128",
                    weight_decay=0.1, steps=20)


def llama2_7b_l2() -> Workload:
    """The 7B per-tensor list with coupled L2 (wd=0.1 enters the gradient)
    instead of AdamW's decoupled decay."""
    w = llama2_7b()
    w.name = "llama2_7b_pertensor_l2"
    w.decay_mode = "l2"
    return w


def llama2_13b_bf16() -> Workload:
    """Llama-2-13B-shaped list (363 tensors, 13.0B params) with bf16 master
    weights, gradient scales in [1e-7, 1], Adam as for the 1M case, 5 steps."""
    return Workload("llama2_13b_bf16master", llama_shapes(**LLAMA2_13B), master="bf16",
                    grad_scale=(1e-7, 1.0), steps=5)


def shard_shapes(shapes: list, rank: int, world: int, align: int = 128) -> list:
    """One data-parallel rank's share of a tensor list: the list flattened in
    order and cut into `world` contiguous slices at multiples of `align`
    elements (the last slice takes the rest).  A tensor cut by a slice boundary
    contributes the 1-D piece inside the slice, named name[a:b]."""
    total = sum(numel(s) for _, s in shapes)
    cut = [(total * r // world) // align * align for r in range(world)] + [total]
    lo, hi = cut[rank], cut[rank + 1]
    out, off = [], 0
    for name, s in shapes:
        n = numel(s)
        a, b = max(lo, off), min(hi, off + n)
        if a < b:
            out.append((name, s) if (a, b) == (off, off + n) else (f"{name}[{a - off}:{b - off}]", (b - a,)))
        off += n
    return out


def llama2_7b_rank0_of_8() -> Workload:
    """Rank 0's share of the 7B per-tensor list when eight data-parallel ranks
    each own a contiguous eighth of the flattened parameters (842,301,952
    params: the embedding, layers 0-2, and layer 3 up to part of w_gate).  The
    cut piece of w_gate carries its own scales here; across ranks its amax
    would be reduced first."""
    w = llama2_7b()
    w.name = "llama2_7b_rank0_of_8"
    w.shapes = shard_shapes(w.shapes, 0, 8)
    return w


def scaled_llama(base: dict, **over) -> list:
    """A smaller list with the same structure, for tests that must run on a CPU."""
    kw = dict(base)
    kw.update(over)
    return llama_shapes(**kw)


WORKLOADS = {
    "flat_1m": flat_1m,
    "llama2_100m": llama2_100m,
    "llama2_7b": llama2_7b,
    "llama2_7b_block128": llama2_7b_block128,
    "llama2_7b_l2": llama2_7b_l2,
    "llama2_13b_bf16": llama2_13b_bf16,
    "llama2_7b_rank0_of_8": llama2_7b_rank0_of_8,
}


# ------------------------------------------------------------------ generators

_ROLE = {"param": 1, "grad": 2, "gscale": 3, "zero": 4, "state": 5}


def seed_for(base: int, tensor: int, step: int, role: str) -> int:
    """Deterministic 63-bit seed for one (tensor, step, role) draw."""
    x = (base * 0x9E3779B97F4A7C15 + tensor * 0xBF58476D1CE4E5B9 + step * 0x94D049BB133111EB
         + _ROLE[role] * 0x2545F4914F6CDD1D) & 0xFFFFFFFFFFFFFFFF
    x ^= x >> 31
    return x & 0x7FFFFFFFFFFFFFFF


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_param(w: Workload, tidx: int, shape, device, base_seed: int = 0) -> torch.Tensor:
    """Master weights ~ N(0, param_std), fp32 or rounded to bf16."""
    g = _gen(device, seed_for(base_seed, tidx, 0, "param"))
    p = torch.randn(numel(shape), generator=g, device=device, dtype=torch.float32) * w.param_std
    return p.to(torch.bfloat16) if w.master == "bf16" else p


def make_grad(w: Workload, tidx: int, shape, step: int, device, base_seed: int = 0) -> torch.Tensor:
    """BF16 gradient for one tensor at one step (step is 1-based)."""
    n = numel(shape)
    g = _gen(device, seed_for(base_seed, tidx, step, "grad"))
    z = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    if w.grad_dist == "student_t3":
        c = torch.randn(3, n, generator=g, device=device, dtype=torch.float32)
        z = z / torch.sqrt((c * c).sum(0) / 3.0)
    lo, hi = math.log10(w.grad_scale[0]), math.log10(w.grad_scale[1])
    gs = _gen(device, seed_for(base_seed, tidx, 0, "gscale"))  # a property of the tensor, fixed across steps
    if w.grad_scale_per == "row" and len(shape) == 2:
        rows = shape[0]
        sc = 10.0 ** (lo + (hi - lo) * torch.rand(rows, generator=gs, device=device, dtype=torch.float64))
        z = (z.view(rows, -1) * sc.to(torch.float32)[:, None]).reshape(-1)
    else:
        sc = 10.0 ** (lo + (hi - lo) * torch.rand(1, generator=gs, device=device, dtype=torch.float64))
        z = z * sc.to(torch.float32)
    if w.zero_frac > 0:
        gz = _gen(device, seed_for(base_seed, tidx, step, "zero"))
        mask = torch.rand(n, generator=gz, device=device) < w.zero_frac
        z = torch.where(mask, torch.zeros_like(z), z)
    return z.to(torch.bfloat16)


def make_state(n: int, device, nblocks: int = 1):
    """Zero moments (codes 0) with unit scales: the state before step 1."""
    cm = torch.zeros(n, dtype=torch.uint8, device=device)
    cv = torch.zeros(n, dtype=torch.uint8, device=device)
    sm = torch.ones(nblocks, dtype=torch.float32, device=device)
    sv = torch.ones(nblocks, dtype=torch.float32, device=device)
    return cm, cv, sm, sv


def random_state(n: int, device, seed: int, m_fmt: int, v_fmt: int, nblocks: int = 1,
                 scale_exp=(-30, 4), pow2: bool = True):
    """Random finite FP8 moment codes (v non-negative) and random scales: the
    state a step would see mid-training.  Formats: 0 = E4M3, 1 = E5M2."""
    g = _gen(device, seed)
    cm = torch.randint(0, 256, (n,), generator=g, device=device, dtype=torch.int32)
    cv = torch.randint(0, 128, (n,), generator=g, device=device, dtype=torch.int32)

    def finite(c, fmt):
        mag = c & 0x7F
        top = 0x7E if fmt == 0 else 0x7B
        mag = torch.where(mag > top, mag - (top + 1), mag)
        return (c & 0x80) | mag

    cm = finite(cm, m_fmt).to(torch.uint8)
    cv = finite(cv, v_fmt).to(torch.uint8)
    e = torch.randint(scale_exp[0], scale_exp[1] + 1, (2, nblocks), generator=g, device=device)
    s = torch.pow(2.0, e.to(torch.float32))
    if not pow2:
        s = s * (1.0 + torch.rand(2, nblocks, generator=g, device=device))
    return cm, cv, s[0].contiguous(), s[1].contiguous()
