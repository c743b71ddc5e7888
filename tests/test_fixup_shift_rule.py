"""The speculative schedule's fix-up moves the exponent field of a code written
with one power-of-two scale to express it in another (the device helper
shift_codes4).  That is exact only under conditions: the code strictly between
the smallest normal and FMAX before and after the move, or a zero code that
shrinks under round-to-nearest.  These tests check that claim against the
oracle's own encoders (round to nearest even, and stochastic rounding with the
same 16 random bits): wherever the rule accepts a code, the moved code equals
the encoding of the value at the other scale.  They also show that the cases
the rule refuses are really needed (a smallest-normal code rounded up from a
subnormal value moves to the wrong code)."""
import numpy as np
import pytest

import oracle

MANT = {"e4m3": 3, "e5m2": 2}
TOP = {"e4m3": 0x7E, "e5m2": 0x7B}


def shift_rule(codes: np.ndarray, fmt: str, d: int, zero_ok: bool):
    """Restatement of the fix-up's rule: (accepted mask, moved codes)."""
    mn, top = 1 << MANT[fmt], TOP[fmt]
    mag = (codes & 0x7F).astype(np.int64)
    nm = mag - d * mn
    keep_zero = zero_ok & (mag == 0)
    normal = (mag > mn) & (mag < top) & (nm > mn) & (nm < top)
    moved = (codes & 0x80) | np.where(keep_zero, 0, nm & 0x7F)
    return keep_zero | normal, moved.astype(np.uint8)


def sample_values(fmt: str, rng: np.random.Generator) -> np.ndarray:
    """fp32 values over the whole FP8 range and beyond, dense around every
    representable value and every rounding midpoint (both signs)."""
    fmax = oracle.format_max(fmt)
    lo, hi = np.float32(2.0 ** -30), np.float32(fmax * 64)
    bits = rng.integers(lo.view(np.uint32), hi.view(np.uint32), size=1 << 20, dtype=np.uint32)
    grid = oracle.decode(fmt, np.arange(0, 0x80, dtype=np.uint8)).astype(np.float64)
    grid = grid[np.isfinite(grid)]
    mids = (grid[1:] + grid[:-1]) / 2
    anchors = np.concatenate([grid, mids]).astype(np.float32)
    near = [anchors]
    for k in range(1, 4):  # a few fp32 ulps either side
        near.append((anchors.view(np.uint32) + np.uint32(k)).view(np.float32))
        near.append((anchors.view(np.uint32) - np.uint32(k)).view(np.float32))
    x = np.concatenate([bits.view(np.float32)] + near)
    x = x[np.isfinite(x) & (x >= 2.0 ** -100)]  # no fp32 subnormals: scaling them is not exact
    return np.concatenate([x, -x]).astype(np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("d", [-5, -2, -1, 1, 2, 5])
def test_moved_codes_equal_the_encoding_at_the_other_scale(fmt, d):
    rng = np.random.default_rng(100 + 10 * d + len(fmt))
    x = sample_values(fmt, rng)
    y = (x.astype(np.float64) * 2.0 ** -d).astype(np.float32)  # exact: a power of two, no fp32 underflow here
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) * 2.0 ** -d)
    ca, cb = oracle.encode(fmt, x), oracle.encode(fmt, y)
    ok, moved = shift_rule(ca, fmt, d, zero_ok=d > 0)
    bad = ok & (moved != cb)
    assert not bad.any(), f"{int(bad.sum())} moved codes differ, e.g. x={x[bad][:4]}"
    # every value that is at least twice the smallest normal and at most FMAX/2 at
    # both scales is accepted: the fix-up recomputes only the rare others
    min_normal = float(oracle.decode(fmt, np.array([1 << MANT[fmt]], np.uint8))[0])
    half_max = oracle.format_max(fmt) / 2
    inside = ((np.abs(x) >= 2 * min_normal) & (np.abs(x) <= half_max) & (np.abs(y) >= 2 * min_normal)
              & (np.abs(y) <= half_max))
    assert inside.sum() > 1000 and ok[inside].all()

    r16 = rng.integers(0, 1 << 16, size=x.size, dtype=np.uint16)
    sa, sb = oracle.encode_sr_array(fmt, x, r16), oracle.encode_sr_array(fmt, y, r16)
    ok, moved = shift_rule(sa, fmt, d, zero_ok=False)
    bad = ok & (moved != sb)
    assert not bad.any(), f"stochastic rounding: {int(bad.sum())} moved codes differ, e.g. x={x[bad][:4]}"


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_refused_cases_are_needed(fmt):
    """A subnormal value rounded up to the smallest normal, moved up a binade,
    is not the value's code there; zero codes of growing values, and the FMAX
    code of a saturated value, are not either."""
    mb = MANT[fmt]
    mn_code = 1 << mb
    min_normal = float(oracle.decode(fmt, np.array([mn_code], np.uint8))[0])
    # between the last rounding midpoint below the smallest normal (1 - 2^-(mb+1)
    # of it) and the point whose double rounds up to the next binade: it rounds
    # up to the smallest normal, its double rounds down inside the binade
    x = np.float32(min_normal * (1 - 3 * 2.0 ** -(mb + 3)))
    assert oracle.encode(fmt, [x])[0] == mn_code
    y = np.float32(x * 2.0)  # the same value at half the scale (d = -1)
    moved = mn_code + (1 << mb)
    assert oracle.encode(fmt, [y])[0] != moved
    ok, _ = shift_rule(np.array([mn_code], np.uint8), fmt, -1, zero_ok=False)
    assert not ok[0]
    # a value that rounds to zero can become nonzero when the values grow
    tiny = np.float32(float(oracle.decode(fmt, np.array([1], np.uint8))[0]) * 0.4)
    assert oracle.encode(fmt, [tiny])[0] == 0 and oracle.encode(fmt, [np.float32(tiny * 4)])[0] != 0
    ok, _ = shift_rule(np.array([0], np.uint8), fmt, -2, zero_ok=False)
    assert not ok[0]
    # a saturated value: FMAX code at one scale, but not FMAX/2 at twice the scale
    fmax = oracle.format_max(fmt)
    big = np.float32(fmax * 1.9)
    assert oracle.encode(fmt, [big])[0] == TOP[fmt]
    assert oracle.encode(fmt, [np.float32(big / 2)])[0] != TOP[fmt] - (1 << mb)
    ok, _ = shift_rule(np.array([TOP[fmt]], np.uint8), fmt, 1, zero_ok=True)
    assert not ok[0]


def _loose_rule(codes: np.ndarray, fmt: str, d: int, zero_ok: bool):
    """The rule with the smallest-normal code accepted (a plausible mistake)."""
    mn, top = 1 << MANT[fmt], TOP[fmt]
    mag = (codes & 0x7F).astype(np.int64)
    nm = mag - d * mn
    keep_zero = zero_ok & (mag == 0)
    normal = (mag >= mn) & (mag < top) & (nm >= mn) & (nm < top)
    moved = (codes & 0x80) | np.where(keep_zero, 0, nm & 0x7F)
    return keep_zero | normal, moved.astype(np.uint8)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_the_check_rejects_a_looser_rule(fmt):
    """Accepting the smallest-normal code (or moving codes into it) gives wrong
    codes when the values grow by a binade: the comparison above catches it."""
    rng = np.random.default_rng(7)
    x = sample_values(fmt, rng)
    y = (x.astype(np.float64) * 2.0).astype(np.float32)
    ca, cb = oracle.encode(fmt, x), oracle.encode(fmt, y)
    ok, moved = _loose_rule(ca, fmt, -1, zero_ok=False)
    assert (ok & (moved != cb)).any()
    ok, moved = shift_rule(ca, fmt, -1, zero_ok=False)
    assert not (ok & (moved != cb)).any()
