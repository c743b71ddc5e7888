"""Pins for the oracle's bit-level FP8 codec (CPU only).

Pinned against things other than the oracle itself:
  * torch's float8_e4m3fn / float8_e5m2 decode of all 256 codes (library);
  * the bit splits and the E4M3 smallest normal printed on the pages
    (tests/golden/formats.json);
  * a brute-force nearest-value encoder swept over all 2^32 fp32 patterns
    (tests/referee/encode_sweep.c);
  * torch's float8 cast for in-range inputs (library; it does not saturate);
  * hand-derived tie cases and the worked example (tests/golden/worked_example.json).
"""
import ctypes
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.referee import sweep_lib

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TD = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def torch_decode(fmt):
    return torch.arange(256, dtype=torch.uint8).view(TD[fmt]).to(torch.float32).numpy()


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_all_codes_match_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode(fmt, codes)
    want = torch_decode(fmt)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    # bit-for-bit, so the sign of zero and the infinities count too
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))


def test_format_facts_from_pages():
    facts = json.load(open(os.path.join(GOLDEN, "formats.json")))
    e4 = oracle.decode(oracle.E4M3, np.arange(128, dtype=np.uint8))
    e5 = oracle.decode(oracle.E5M2, np.arange(128, dtype=np.uint8))
    # bit splits: number of distinct binades and of mantissa steps per binade
    assert facts["e4m3"]["exponent_bits"] + facts["e4m3"]["mantissa_bits"] == 7
    # E4M3: 8 codes per binade (3 mantissa bits); E5M2: 4 (2 mantissa bits)
    assert e4[0x09] - e4[0x08] == e4[0x08] / 8
    assert e5[0x05] - e5[0x04] == e5[0x04] / 4
    # smallest normal of E4M3 printed as ~0.0156 = 2^-6
    assert e4[0x08] == facts["e4m3"]["min_normal"] == 2.0 ** -6
    # one more exponent bit roughly doubles the dynamic range in binades
    fin4 = e4[np.isfinite(e4) & (e4 > 0)]
    fin5 = e5[np.isfinite(e5) & (e5 > 0)]
    b4 = math.log2(fin4.max() / fin4.min())
    b5 = math.log2(fin5.max() / fin5.min())
    assert 1.6 < b5 / b4 < 2.0


def test_format_constants():
    assert oracle.format_max(oracle.E4M3) == 448.0
    assert oracle.format_max(oracle.E5M2) == 57344.0
    e4 = oracle.decode(oracle.E4M3, np.arange(256, dtype=np.uint8))
    e5 = oracle.decode(oracle.E5M2, np.arange(256, dtype=np.uint8))
    assert np.isnan(e4).sum() == 2 and np.isinf(e4).sum() == 0
    assert np.isnan(e5).sum() == 6 and np.isinf(e5).sum() == 2
    assert e4[1] == 2.0 ** -9 and e5[1] == 2.0 ** -16
    assert e5[0x04] == 2.0 ** -14


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_exhaustive_vs_bruteforce(fmt):
    """Every fp32 bit pattern (NaNs excepted): oracle encode == nearest value,
    ties to the even code, saturating."""
    L = sweep_lib()
    values = torch_decode(fmt).astype(np.float64)
    enc_addr = ctypes.cast(oracle.lib().ref_encode, ctypes.c_void_p).value
    bad = ctypes.c_uint64()
    got, want = ctypes.c_int(), ctypes.c_int()
    threads = max(1, min(16, os.cpu_count() or 1))
    n = L.sweep_encoder(values.ctypes.data, enc_addr, fmt, 0, 1 << 32, threads,
                        ctypes.byref(bad), ctypes.byref(got), ctypes.byref(want))
    assert n == 0, f"{n} mismatches; first at bits {bad.value:#010x}: got {got.value:#04x} want {want.value:#04x}"


def test_referee_catches_a_planted_encoder_bug():
    """The sweep must notice a plausible mistake: round-half-up instead of
    ties-to-even (planted in a Python encoder, on the CPU)."""
    L = sweep_lib()
    values = torch_decode(oracle.E4M3).astype(np.float64)
    ENC = ctypes.CFUNCTYPE(ctypes.c_uint8, ctypes.c_int, ctypes.c_float)

    def half_up(fmt, x):
        c = oracle.lib().ref_encode(fmt, x)
        # for an exact tie that went down to an even code, go up instead
        v = float(x)
        if v > 0 and (c & 0x7F) < 0x7E:
            lo, hi = values[c & 0x7F], values[(c & 0x7F) + 1]
            if v - lo == hi - v:
                return c + 1
        return c

    cb = ENC(half_up)
    addr = ctypes.cast(cb, ctypes.c_void_p).value
    bad = ctypes.c_uint64()
    got, want = ctypes.c_int(), ctypes.c_int()
    # bit patterns around 1.0625, a tie between 1.0 (even code) and 1.125
    center = int(np.float32(1.0625).view(np.uint32))
    n = L.sweep_encoder(values.ctypes.data, addr, oracle.E4M3, center - 4, center + 4, 1,
                        ctypes.byref(bad), ctypes.byref(got), ctypes.byref(want))
    assert n == 1 and bad.value == center


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_matches_torch_cast_in_range(fmt):
    rng = np.random.default_rng(1234 + fmt)
    fm = oracle.format_max(fmt)
    # log-uniform magnitudes over the whole format range and beyond its bottom
    mags = 10.0 ** rng.uniform(-12, math.log10(fm), size=2_000_000)
    x = (mags * rng.choice([-1.0, 1.0], size=mags.size)).astype(np.float32)
    x = x[np.abs(x) <= fm]
    got = oracle.encode(fmt, x)
    want = torch.from_numpy(x).to(TD[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_encode_ties_to_even():
    # E4M3 near 1: 0.9375 (0x37) and 1.0 (0x38); midpoint 0.96875 -> even 0x38
    assert oracle.encode("e4m3", [0.96875])[0] == 0x38
    # E4M3 1.0 (0x38) and 1.125 (0x39); midpoint 1.0625 -> even 0x38
    assert oracle.encode("e4m3", [1.0625])[0] == 0x38
    # 1.125 (0x39), 1.25 (0x3A); midpoint 1.1875 -> even 0x3A
    assert oracle.encode("e4m3", [1.1875])[0] == 0x3A
    # E5M2 0.875 (0x3B) and 1.0 (0x3C); midpoint 0.9375 -> even 0x3C
    assert oracle.encode("e5m2", [0.9375])[0] == 0x3C
    # subnormal tie: half the smallest E4M3 subnormal rounds to zero (even)
    assert oracle.encode("e4m3", [2.0 ** -10])[0] == 0x00
    assert oracle.encode("e4m3", [-(2.0 ** -10)])[0] == 0x80
    # 1.5 * 2^-9 is a tie between codes 1 and 2 -> even code 2
    assert oracle.encode("e4m3", [1.5 * 2.0 ** -9])[0] == 0x02


def test_encode_saturates_and_keeps_sign():
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e30, np.inf, -500.0, -np.inf], dtype=np.float32)
    assert list(oracle.encode("e4m3", big)) == [0x7E] * 6 + [0xFE] * 2
    big5 = np.array([57344.0, 61440.0, 1e38, np.inf, -np.inf], dtype=np.float32)
    assert list(oracle.encode("e5m2", big5)) == [0x7B] * 4 + [0xFB]
    z = np.array([0.0, -0.0, 1e-45, -1e-45], dtype=np.float32)
    assert list(oracle.encode("e4m3", z)) == [0x00, 0x80, 0x00, 0x80]
    assert list(oracle.encode("e5m2", z)) == [0x00, 0x80, 0x00, 0x80]


def test_worked_example_codec():
    """The numerical example: 1e-4 survives in E5M2 (1/sqrt about 100), but is
    below E4M3's range (flush to 0 -> 1/(0+eps); or the smallest normal -> 8)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    v = np.float32(ex["v_small"])
    c5 = oracle.encode("e5m2", [v])[0]
    assert c5 == 0x07
    v5 = float(oracle.decode("e5m2", [c5])[0])
    assert v5 == 1.068115234375e-4
    inv = 1.0 / (math.sqrt(v5) + 1e-8)
    assert abs(inv - ex["inv_sqrt_v_small"]) / ex["inv_sqrt_v_small"] < 0.05  # "about 100"
    c4 = oracle.encode("e4m3", [v])[0]
    assert c4 == 0x00 and oracle.decode("e4m3", [c4])[0] == 0.0
    assert 1.0 / (0.0 + 1e-8) == 1e8  # the blow-up
    mn = float(oracle.decode("e4m3", [0x08])[0])
    assert mn == ex["e4m3_min_normal"] and round(mn, 4) == ex["e4m3_min_normal_printed"]
    assert math.sqrt(mn) == ex["sqrt_e4m3_min_normal_printed"]
    assert 1.0 / math.sqrt(mn) == ex["inv_sqrt_e4m3_min_normal"]
    assert round(ex["inv_sqrt_v_small"] / (1.0 / math.sqrt(mn))) == ex["error_factor_printed"]
    # the normal-sized second moment is exact in both formats
    assert oracle.decode("e5m2", oracle.encode("e5m2", [1.0]))[0] == 1.0
    assert oracle.decode("e4m3", oracle.encode("e4m3", [1.0]))[0] == 1.0


def test_encode_bits_range_matches_scalar():
    start = int(np.float32(0.5).view(np.uint32))
    codes = oracle.encode_bits_range("e5m2", start, 1000)
    x = (np.arange(1000, dtype=np.uint64) + start).astype(np.uint32).view(np.float32)
    assert np.array_equal(codes, oracle.encode("e5m2", x))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-40, 38, 200_000)).astype(np.float32)
    x = x[np.isfinite(x)]
    got = oracle.f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
