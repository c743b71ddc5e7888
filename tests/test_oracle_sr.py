"""Pins for the oracle's stochastic rounding and its generator.

  * Philox4x32-10 equals the known-answer vectors published with the
    generator (Salmon et al., SC 2011; the Random123 distribution's KAT list);
  * ref_encode_sr keeps exact FP8 values, saturates like round-to-nearest,
    and over all 2^16 random inputs rounds up exactly floor(f * 2^16) times,
    f = the distance to the lower neighbour as a fraction of the spacing
    (neighbours and f found here by a search of torch's float8 decode table
    with exact fractions), so its mean is within 2^-16 of a spacing of x;
  * a whole step with stochastic rounding equals the exact-rational referee
    fed the same random words.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.referee import rational

KAT = [  # counter, key, output (Philox4x32-10)
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("kat", KAT, ids=["zeros", "ones", "pi"])
def test_philox_known_answers(kat):
    ctr, key, out = kat
    assert oracle.philox4x32_10(ctr, key) == list(out)


def test_sr_word_layout():
    seed = 0x0123456789ABCDEF
    for tensor, t, i in [(0, 1, 0), (3, 7, 5), (290, 20, (1 << 33) + 6), (1, 2, 1023)]:
        g = i >> 2
        words = oracle.philox4x32_10((g & 0xFFFFFFFF, g >> 32, t, tensor), (seed & 0xFFFFFFFF, seed >> 32))
        assert oracle.sr_word(seed, tensor, t, i) == words[i & 3]


def _table(fmt):
    dt = torch.float8_e4m3fn if fmt == 0 else torch.float8_e5m2
    return [float(v) for v in torch.arange(256, dtype=torch.uint8).view(dt).to(torch.float64)]


@pytest.mark.parametrize("fmt", [0, 1])
def test_sr_keeps_exact_values_and_saturates(fmt):
    tab = _table(fmt)
    for code in range(256):
        x = tab[code]
        if not math.isfinite(x):
            continue
        for r in (0, 1, 0x7FFF, 0x8000, 0xFFFF):
            got = oracle.encode_sr(fmt, np.float32(x), r)
            want = oracle.encode(fmt, [x])[0]
            assert got == want, (code, r)
    fmax = oracle.format_max(fmt)
    for x in (fmax * 1.001, fmax * 4, float("inf"), -fmax * 2):
        for r in (0, 0xFFFF):
            assert oracle.encode_sr(fmt, np.float32(x), r) == oracle.encode(fmt, [x])[0]


@pytest.mark.parametrize("fmt", [0, 1])
def test_sr_up_count_and_mean_exhaustive(fmt):
    """For each x, all 65536 random inputs: the up count is floor(f * 2^16)."""
    tab = _table(fmt)
    finite = sorted({abs(v) for v in tab if math.isfinite(v)})
    rng = np.random.default_rng(fmt)
    xs = list(np.float32(rng.uniform(-1, 1, 12) * 10.0 ** rng.uniform(-6, 2, 12)))
    xs += [np.float32(finite[1] * 0.3), np.float32(finite[5] * 1.01), np.float32(-finite[-2] * 1.0001)]
    for x in xs:
        a = Fraction(float(abs(x)))
        if a == 0 or a >= Fraction(finite[-1]):
            continue
        lo = max(v for v in finite if Fraction(v) <= a)
        hi = min(v for v in finite if Fraction(v) > a)
        f = (a - Fraction(lo)) / (Fraction(hi) - Fraction(lo))
        d = math.floor(f * 65536)
        codes = np.array([oracle.encode_sr(fmt, x, r) for r in range(65536)], np.uint8)
        vals = np.abs(oracle.decode(fmt, codes).astype(np.float64))
        ups = int(np.sum(vals == hi))
        assert ups == d and int(np.sum(vals == lo)) == 65536 - d, (x, ups, d)
        mean = Fraction(lo) + (Fraction(hi) - Fraction(lo)) * Fraction(d, 65536)
        assert abs(mean - a) < (Fraction(hi) - Fraction(lo)) / 65536
        # the sign is kept
        assert np.all((codes & 0x80) == (0x80 if x < 0 else 0))


@pytest.mark.parametrize("m_fmt,v_fmt,block", [(0, 1, 0), (1, 0, 128), (0, 1, 128)])
def test_stochastic_step_equals_rational_referee(m_fmt, v_fmt, block):
    n = 150
    rng = np.random.default_rng(31 + block)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    nb = 1 if block == 0 else -(-n // block)
    cm, cv, sm, sv = [x.numpy() for x in workloads.random_state(n, "cpu", 5, m_fmt, v_fmt, nblocks=nb,
                                                                 scale_exp=(-24, 2))]
    h = oracle.Hyper(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    rp, rcm, rcv = [float(x) for x in p], [int(x) for x in cm], [int(x) for x in cv]
    rsm, rsv = [float(x) for x in sm], [float(x) for x in sv]
    seed, tensor = 0xDEADBEEF12345678, 7
    for t in (1, 2, 3):
        g = torch.tensor(rng.standard_normal(n) * 10.0 ** rng.uniform(-7, 0, n), dtype=torch.float32)
        gb = g.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
        h.step = t
        cfg = oracle.make_config(h, m_fmt, v_fmt, block=block, stochastic=True, tensor_index=tensor, seed=seed)
        oracle.step(cfg, p, gb, cm, cv, sm, sv)
        words = [oracle.sr_word(seed, tensor, t, i) for i in range(n)]
        gv = (gb.astype(np.uint32) << 16).view(np.float32)
        rp, rcm, rcv, rsm, rsv = rational.step(
            rp, [float(x) for x in gv], rcm, rcv, rsm, rsv, lr=float(np.float32(h.lr)),
            b1=float(np.float32(h.beta1)), b2=float(np.float32(h.beta2)), eps=float(np.float32(h.eps)),
            wd=float(np.float32(h.weight_decay)), t=t, m_fmt=m_fmt, v_fmt=v_fmt, block=block, sr_words=words)
        assert list(cm) == rcm and list(cv) == rcv, f"codes differ at step {t}"
        assert list(sm) == rsm and list(sv) == rsv
        rp = [float(x) for x in p]
    # and stochastic rounding is not round-to-nearest on this data
    p2, cm2, cv2, sm2, sv2 = p.copy(), cm.copy(), cv.copy(), sm.copy(), sv.copy()
    oracle.step(oracle.make_config(h, m_fmt, v_fmt, block=block), p2, gb, cm2, cv2, sm2, sv2)
    oracle.step(oracle.make_config(h, m_fmt, v_fmt, block=block, stochastic=True, tensor_index=tensor, seed=seed),
                p, gb, cm, cv, sm, sv)
    assert not (np.array_equal(cm, cm2) and np.array_equal(cv, cv2))
