"""Exact-rational referee for the FP8-moment AdamW step (tiny tensors only).

Independent of the oracle: fp32 operations are emulated as an exact rational
result followed by one round-to-nearest-even to binary32 (signed zeros kept),
FP8 quantization is a nearest-value search over torch's float8 decode table
(ties to the even code, saturating above the largest finite value), the
power-of-two scale is found by searching exponents, and the parameter update
is evaluated with 60-digit decimals and rounded once.

The step it computes is the one the oracle documents: dequantize (code times
scale), m' = b1*m + (1-b1)*g and v' = b2*v + (1-b2)*g*g in fp32 with one
rounding for the multiply-add, new scale from the amax of m' / v', requantize
with x * inv_scale, and p' = p*(1 - lr*wd) - lr/(1-b1^t) * m' / (sqrt(v'/(1-b2^t)) + eps).
With l2_coupled the gradient is g + wd*p (one fp32 rounding) and there is no
decoupled decay.  With scale_amax the scales are chosen from the given amax
values (delayed scaling) instead of this step's.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import torch

getcontext().prec = 60

_TORCH_DTYPES = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


def decode_table(fmt: int) -> list[float]:
    codes = torch.arange(256, dtype=torch.uint8)
    return [float(x) for x in codes.view(_TORCH_DTYPES[fmt]).to(torch.float64)]


_TABLES = {f: decode_table(f) for f in (0, 1)}


def fmax(fmt: int) -> float:
    return max(v for v in _TABLES[fmt] if math.isfinite(v))


def _sign(x: float) -> int:
    return -1 if math.copysign(1.0, x) < 0 else 1


def _round_binary(a: Fraction, sig_bits: int, min_exp: int) -> Fraction:
    """Round a positive rational to `sig_bits` significant bits, RNE, with the
    spacing floored at 2^(min_exp - sig_bits + 1) (gradual underflow)."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    q = max(e, min_exp) - (sig_bits - 1)
    unit = Fraction(2) ** q
    n, r = divmod(a, unit)
    n = int(n)
    if r * 2 > unit or (r * 2 == unit and n % 2 == 1):
        n += 1
    return n * unit


def round_f32(x: Fraction, sign_if_zero: int = 1) -> float:
    if x == 0:
        return math.copysign(0.0, sign_if_zero)
    s = -1 if x < 0 else 1
    r = _round_binary(abs(x), 24, -126)
    if r >= Fraction(2) ** 128:
        return s * math.inf
    return math.copysign(float(r), s)


def round_bf16(x: Fraction, sign_if_zero: int = 1) -> float:
    if x == 0:
        return math.copysign(0.0, sign_if_zero)
    s = -1 if x < 0 else 1
    r = _round_binary(abs(x), 8, -126)
    if r >= Fraction(2) ** 128:
        return s * math.inf
    return math.copysign(float(r), s)


def mul32(a: float, b: float) -> float:
    exact = Fraction(a) * Fraction(b)
    return round_f32(exact, _sign(a) * _sign(b))


def fma32(a: float, b: float, c: float) -> float:
    prod = Fraction(a) * Fraction(b)
    exact = prod + Fraction(c)
    if exact == 0:
        # IEEE: an exact zero sum is -0 only when both addends are -0
        both_neg = (prod == 0 and _sign(a) * _sign(b) < 0) and (c == 0 and _sign(c) < 0)
        return -0.0 if both_neg else 0.0
    return round_f32(exact)


def sub32(a: float, b: float) -> float:
    exact = Fraction(a) - Fraction(b)
    if exact == 0:
        return -0.0 if (a == 0 and b == 0 and _sign(a) < 0 < _sign(b)) else 0.0
    return round_f32(exact)


def div32(a: float, b: float) -> float:
    exact = Fraction(a) / Fraction(b)
    return round_f32(exact, _sign(a) * _sign(b))


def quantize(fmt: int, x: float) -> int:
    """Nearest FP8 code by search, ties to the even code, saturating."""
    tab = _TABLES[fmt]
    sign = 0x80 if _sign(x) < 0 else 0
    a = abs(x)
    best, best_d = None, None
    top = max(c for c in range(128) if math.isfinite(tab[c]))
    if a >= tab[top]:
        return sign | top
    for c in range(128):
        v = tab[c]
        if not math.isfinite(v):
            continue
        d = abs(Fraction(a) - Fraction(v))
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return sign | best


def quantize_sr(fmt: int, x: float, r16: int) -> int:
    """Stochastic rounding by table search: the FP8 neighbours lo <= |x| < hi,
    f = (|x| - lo) / (hi - lo) exactly, up iff floor(f * 2^16) + r16 >= 2^16.
    Saturation, zeros and exact values as in quantize()."""
    tab = _TABLES[fmt]
    a = abs(x)
    top = max(c for c in range(128) if math.isfinite(tab[c]))
    if a == 0 or a >= tab[top]:
        return quantize(fmt, x)
    sign = 0x80 if _sign(x) < 0 else 0
    lo_c = max(c for c in range(top + 1) if tab[c] <= a)
    lo, hi = Fraction(tab[lo_c]), Fraction(tab[lo_c + 1])
    f = (Fraction(a) - lo) / (hi - lo)
    d = math.floor(f * 65536)
    return sign | (lo_c + 1 if d + r16 >= 65536 else lo_c)


def dequant(fmt: int, code: int) -> float:
    return _TABLES[fmt][code]


def pow2_scale(fmt: int, amax: float) -> tuple[float, float]:
    if not (amax > 0) or not math.isfinite(amax):
        return 1.0, 1.0
    fm = Fraction(fmax(fmt))
    for k in range(-126, 127):
        if Fraction(amax) / Fraction(2) ** k <= fm:
            return float(Fraction(2) ** k), float(Fraction(2) ** -k)
    return float(Fraction(2) ** 126), float(Fraction(2) ** -126)


def amax_scale(fmt: int, amax: float) -> tuple[float, float]:
    if not (amax > 0) or not math.isfinite(amax):
        return 1.0, 1.0
    fm = fmax(fmt)
    s = div32(amax, fm)
    if s < 2.0 ** -126:
        return 2.0 ** -126, 2.0 ** 126
    return s, div32(fm, amax)


def _dec(x: Fraction) -> Decimal:
    return Decimal(x.numerator) / Decimal(x.denominator)


def param_update(p: float, m1: float, v1: float, lr: float, b1: float, b2: float, eps: float,
                 wd: float, t: int) -> Fraction:
    """p*(1-lr*wd) - lr/(1-b1^t) * m1/(sqrt(v1/(1-b2^t)) + eps), 60 digits."""
    F = Fraction
    bc1 = 1 - F(b1) ** t
    bc2 = 1 - F(b2) ** t
    decay = _dec(1 - F(lr) * F(wd))
    step_size = _dec(F(lr) / bc1)
    vhat = _dec(F(v1) / bc2)
    denom = vhat.sqrt() + _dec(F(eps))
    res = _dec(F(p)) * decay - step_size * _dec(F(m1)) / denom
    return Fraction(res)


def step(p: list[float], g: list[float], cm: list[int], cv: list[int], sm: list[float],
         sv: list[float], *, lr: float, b1: float, b2: float, eps: float, wd: float, t: int,
         m_fmt: int = 0, v_fmt: int = 1, block: int = 0, amax_mode: bool = False,
         master_bf16: bool = False, l2_coupled: bool = False, scale_amax=None, return_amax: bool = False,
         sr_words=None):
    """Returns new (p, cm, cv, sm, sv), plus the per-block (amax m', amax v')
    list with return_amax. All floats are values already exact in their storage
    type (fp32, or bf16 for g and a bf16 master).  scale_amax: (am, av) to
    choose a per-tensor step's scales from.  sr_words: one random 32-bit word
    per element for stochastic rounding (m takes the low 16 bits, v the high)."""
    assert scale_amax is None or block == 0
    n = len(p)
    blen = block if block > 0 else max(n, 1)
    omb1 = sub32(1.0, b1)
    omb2 = sub32(1.0, b2)
    p2, cm2, cv2 = list(p), list(cm), list(cv)
    sm2, sv2 = list(sm), list(sv)
    choose = amax_scale if amax_mode else pow2_scale
    amaxes = []
    for bi, lo in enumerate(range(0, n, blen)):
        hi = min(lo + blen, n)
        si = bi if block > 0 else 0
        m1s, v1s = [], []
        for i in range(lo, hi):
            m = mul32(dequant(m_fmt, cm[i]), sm[si])
            v = mul32(dequant(v_fmt, cv[i]), sv[si])
            gi = fma32(wd, p[i], g[i]) if l2_coupled else g[i]
            m1 = fma32(b1, m, mul32(omb1, gi))
            v1 = fma32(b2, v, mul32(omb2, mul32(gi, gi)))
            m1s.append(m1)
            v1s.append(v1)
        am = max((abs(x) for x in m1s), default=0.0)
        av = max((abs(x) for x in v1s), default=0.0)
        amaxes.append((am, av))
        if scale_amax is not None:
            am, av = scale_amax
        nsm, nism = choose(m_fmt, am)
        nsv, nisv = choose(v_fmt, av)
        for j, i in enumerate(range(lo, hi)):
            if sr_words is not None:
                cm2[i] = quantize_sr(m_fmt, mul32(m1s[j], nism), sr_words[i] & 0xFFFF)
                cv2[i] = quantize_sr(v_fmt, mul32(v1s[j], nisv), sr_words[i] >> 16)
            else:
                cm2[i] = quantize(m_fmt, mul32(m1s[j], nism))
                cv2[i] = quantize(v_fmt, mul32(v1s[j], nisv))
            exact = param_update(p[i], m1s[j], v1s[j], lr, b1, b2, eps, 0.0 if l2_coupled else wd, t)
            p2[i] = round_bf16(exact) if master_bf16 else round_f32(exact)
        sm2[si], sv2[si] = nsm, nsv
    if return_amax:
        return p2, cm2, cv2, sm2, sv2, amaxes
    return p2, cm2, cv2, sm2, sv2
