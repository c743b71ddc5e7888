"""Device FP8 codec (the gfx950 packed converts with the saturating clamp, as
used by the step kernels) against the oracle codec: all 256 codes decoded,
all 2^32 fp32 bit patterns encoded, through the C ABI."""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
import precision_adam_optimizer_amd as pk
from tests.gpu_util import pool_size

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [0, 1])
def test_decode_all_codes(fmt):
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    pk.fp8adam_decode(fmt, codes, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.decode(fmt, np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))


@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_special_values(fmt):
    vals = np.array([0.0, -0.0, 1e-45, -1e-45, 0.96875, 0.9375, 1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9,
                     1e-4, 448.0, 449.0, 464.0, 480.0, 57344.0, 61440.0, 1e30, -1e30, np.inf, -np.inf,
                     2.0 ** -17, 3 * 2.0 ** -17, 1.17549435e-38, -1.17549435e-38], dtype=np.float32)
    x = torch.from_numpy(vals).cuda()
    out = torch.empty(vals.size, dtype=torch.uint8, device="cuda")
    pk.fp8adam_encode(fmt, x, out)
    torch.cuda.synchronize()
    assert list(out.cpu().numpy()) == list(oracle.encode(fmt, vals))


NAN_RANGES = ((0x7F800001, 0x80000000), (0xFF800001, 0x100000000))  # [lo, hi) of NaN bit patterns


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_all_fp32_bit_patterns(fmt):
    """Every fp32 pattern except NaNs (outside the contract): device code ==
    oracle code.  Covers rounding, ties, subnormals, signed zeros, saturation
    and the byte order of the packed converts."""
    slice_len = 1 << 28
    dev = torch.empty(slice_len, dtype=torch.uint8, device="cuda")
    host = torch.empty(slice_len, dtype=torch.uint8, pin_memory=True)
    parts = 16  # slices of the oracle's share, run on pool_size() threads
    step = slice_len // parts

    def oracle_part(start):
        return oracle.encode_bits_range(fmt, start, step)

    mismatches, first = 0, None
    for s in range(0, 1 << 32, slice_len):
        pk.fp8adam_encode_bits_range(fmt, s, slice_len, dev)
        host.copy_(dev)
        torch.cuda.synchronize()
        got = host.numpy()
        with cf.ThreadPoolExecutor(pool_size()) as ex:
            want = np.concatenate(list(ex.map(oracle_part, [s + k * step for k in range(parts)])))
        diff = got != want
        for lo, hi in NAN_RANGES:
            a, b = max(lo, s) - s, min(hi, s + slice_len) - s
            if a < b:
                diff[a:b] = False
        if diff.any():
            mismatches += int(diff.sum())
            if first is None:
                i = int(np.nonzero(diff)[0][0])
                first = (s + i, int(got[i]), int(want[i]))
    assert mismatches == 0, f"{mismatches} mismatches; first bits {first[0]:#010x}: gpu {first[1]:#04x} oracle {first[2]:#04x}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_sr_matches_oracle_over_the_fp8_range(fmt):
    """The device's stochastic-rounding encode (the one the step kernels use)
    equals the oracle's for every fp32 pattern from 2^-24 to just past FMAX,
    both signs, for five values of the 16 random bits; and for the smallest
    patterns (fp32 subnormals) with all random bits set."""
    lo = 0x33800000                                   # 2^-24
    hi = {0: 0x43E40000, 1: 0x47680000}[fmt]          # a little above 448 / 57344
    threads = max(1, min(16, os.cpu_count() or 1))
    ranges = [(s | lo, hi - lo, r) for s in (0, 0x80000000) for r in (0, 0x3A5C, 0x7FFF, 0x8000, 0xFFFF)]
    ranges += [(0, 1 << 20, 0xFFFF), (0x80000000, 1 << 20, 0xFFFF)]
    out = torch.empty(max(c for _, c, _ in ranges), dtype=torch.uint8, device="cuda")
    for start, count, r16 in ranges:
        pk.fp8adam_encode_sr_bits_range(fmt, start, count, r16, out)
        got = out[:count].cpu().numpy()
        want = np.empty(count, np.uint8)
        step = -(-count // threads)

        def work(k):
            a = k * step
            b = min(count, a + step)
            if a < b:
                oracle.encode_sr_bits_range(fmt, start + a, b - a, r16, want[a:b])

        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(threads)))
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (f"fmt {fmt} r16 {r16:#06x}: {bad.size} codes differ, first at pattern "
                               f"{start + int(bad[0]):#010x}: gpu {got[bad[0]]:#04x} oracle {want[bad[0]]:#04x}")
        print(f"sr sweep fmt {fmt} start {start:#010x} count {count} r16 {r16:#06x}: equal", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", [0, 1])
def test_encode_sr_every_r16_on_sampled_values(fmt):
    """Each of 512 values, spread over every FP8 binade (normal, subnormal,
    below the smallest subnormal, the top binade up to FMAX, exact FP8 values
    and the midpoints between neighbours), both signs, stochastically rounded
    with every one of the 2^16 random values: device code == oracle code.  For
    each value this pins the exact r16 threshold at which it rounds up."""
    rng = np.random.default_rng(2409 + fmt)
    lo_e, hi_e = (-12, 8) if fmt == 0 else (-19, 15)
    k = 384
    vals = np.ldexp(1.0 + rng.random(k), rng.integers(lo_e, hi_e + 1, size=k)).astype(np.float32)
    fp8 = oracle.decode(fmt, np.arange(0, 127, dtype=np.uint8)).astype(np.float64)
    fp8 = fp8[np.isfinite(fp8)]
    exact = rng.choice(fp8, 64)
    mids = (fp8[1:] + fp8[:-1]) / 2
    vals = np.concatenate([vals, exact.astype(np.float32), rng.choice(mids, 64).astype(np.float32)])
    vals = np.clip(vals, 0.0, {0: 448.0, 1: 57344.0}[fmt]).astype(np.float32)
    vals[rng.random(vals.size) < 0.5] *= -1
    assert vals.size == 512
    r16 = np.arange(1 << 16, dtype=np.uint16)
    x_all = np.repeat(vals, r16.size)
    r_all = np.tile(r16, vals.size)
    out = torch.empty(x_all.size, dtype=torch.uint8, device="cuda")
    pk.fp8adam_encode_sr(fmt, torch.from_numpy(x_all).cuda(), torch.from_numpy(r_all).cuda(), out)
    got = out.cpu().numpy()
    want = np.empty_like(got)
    threads = max(1, min(16, os.cpu_count() or 1))
    step = -(-x_all.size // threads)

    def work(t):
        a, b = t * step, min(x_all.size, (t + 1) * step)
        if a < b:
            oracle.encode_sr_array(fmt, x_all[a:b], r_all[a:b], want[a:b])

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(threads)))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"{bad.size} codes differ; first x={x_all[bad[0]]!r} r16={int(r_all[bad[0]]):#06x}: "
                           f"gpu {got[bad[0]]:#04x} oracle {want[bad[0]]:#04x}")


def test_stream_copy_copies_every_byte():
    """The bandwidth probe the benchmark compares the step with is a real copy:
    sizes around its 16 KiB work-group tile, and the destination's bytes past
    the copied range stay untouched."""
    for nbytes in (16, 4096, 16384 - 16, 16384, 16384 + 16, 3 * 16384 + 4096 + 48, 1 << 22):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
        dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
        pk.fp8adam_stream_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes], src), nbytes
        assert bool((dst[nbytes:] == 0xA5).all()), nbytes


def test_stream_rw_reads_and_writes_what_it_counts():
    """The read and write streams the benchmark decomposes the byte mix with:
    equal sizes copy; a longer destination gets zeros past the source; a
    read-only call leaves memory untouched; a write-only call writes zeros; bytes
    past the written range stay untouched.  Sizes around the 16 KiB tile."""
    for nr, nw in ((16384, 16384), (16, 4096), (3 * 16384 + 48, 3 * 16384 + 48 + 4096 + 16), (1 << 22, 0),
                   (0, 16384 + 16), (4096, 16)):
        src = torch.randint(0, 256, (max(nr, 16),), dtype=torch.uint8, device="cuda")
        dst = torch.full((nw + 64,), 0xA5, dtype=torch.uint8, device="cuda")
        src0 = src.clone()
        pk.fp8adam_stream_rw(src[:nr] if nr else None, dst[:nw] if nw else None)
        torch.cuda.synchronize()
        k = min(nr, nw)
        assert torch.equal(dst[:k], src[:k]), (nr, nw)
        assert bool((dst[k:nw] == 0).all()), (nr, nw)
        assert bool((dst[nw:] == 0xA5).all()), (nr, nw)
        assert torch.equal(src, src0), (nr, nw)


@pytest.mark.parametrize("master", ["fp32", "bf16"])
def test_stream_mix_reads_and_writes_every_element(master):
    """The byte-mix probe the benchmark uses as the update pass's ceiling moves
    every byte it counts: p += g in place (fp32, or rounded to nearest-even
    bf16), each output code word = the input code word xor the word of two bf16
    gradients at the same position; bytes past the range stay untouched."""
    part = 2048 if master == "bf16" else 1024
    n = part * 37
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    pdt = torch.bfloat16 if master == "bf16" else torch.float32
    p = torch.empty(n + 64, dtype=pdt, device="cuda")
    p.copy_(torch.randn(n + 64, generator=gen, device="cuda"))
    g = torch.randn(n, generator=gen, device="cuda").to(torch.bfloat16)
    m_in = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
    v_in = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen)
    m_out = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    v_out = torch.full((n + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    p0 = p.cpu()
    pk.fp8adam_stream_mix(p[:n], g, m_in, v_in, m_out[:n], v_out[:n])
    torch.cuda.synchronize()
    want_p = (p0[:n].float() + g.cpu().float()).to(pdt)
    assert torch.equal(p[:n].cpu().view(torch.int16 if master == "bf16" else torch.int32),
                       want_p.view(torch.int16 if master == "bf16" else torch.int32))
    assert torch.equal(p[n:].cpu().view(torch.uint8), p0[n:].view(torch.uint8))
    gw = g.cpu().view(torch.int16).numpy().view(np.uint32)  # two bf16 per word, little-endian
    cm = m_in.cpu().numpy().view(np.uint32)
    cv = v_in.cpu().numpy().view(np.uint32)
    assert np.array_equal(m_out[:n].cpu().numpy().view(np.uint32), cm ^ gw[0::2])
    assert np.array_equal(v_out[:n].cpu().numpy().view(np.uint32), cv ^ gw[1::2])
    assert bool((m_out[n:] == 0xA5).all()) and bool((v_out[n:] == 0x5A).all())
