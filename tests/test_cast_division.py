"""The divisions the fp8 cast kernels use, restated with exact rational
arithmetic and compared bit for bit with IEEE float32 division.

* Scale: s = RN(ap / 448) with ap = max(amax, 1e-4f), computed as q =
  RN(ap * c) with c = RN(1/448), then one residual correction
  q + RN(ap - 448 q) * c (Markstein's refinement, P. Markstein, IBM J. Res.
  Dev. 34(1), 1990).
* Quotient: x / s computed as y = RN(1/s) once per scale group, then per
  element q = RN(x*y) and one correction q = RN(q + y*RN(x - s*q)), with x's
  sign.

Both are asked to equal IEEE division on every input the kernels can meet:
x is a bf16 value and amax the largest |x| of its group (a bf16 value, or
the 1e-4f floor), so the dividends take 128 significands (129 with 1e-4f)
and s one of 129; every pair of significands is checked, at more than one
exponent (the steps scale with the operands' exponents while they stay
normal).  Quotients below 2^-12 have e4m3 code +-0: there only the sign and
the magnitude class are asked for."""
from fractions import Fraction

import numpy as np

import ep_inputs


def _rn32(v: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # subnormals share the minimum exponent
    scaled = a / Fraction(2) ** (e - 23)  # 24-bit significand range
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(sign * float(Fraction(m) * Fraction(2) ** (e - 23)))


def _fma32(a, b, c):
    return _rn32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


C448 = np.float32(1.0) / np.float32(448.0)          # RN(1/448)
FLOOR = np.float32(1e-4)


def _scale_kernel(amax):
    ap = max(np.float32(amax), FLOOR)
    q = np.float32(ap * C448)
    return _fma32(_fma32(-q, np.float32(448.0), ap), C448, q)


def _div_kernel(x, s):
    y = np.float32(1.0) / s
    q = np.float32(x * y)
    r = _fma32(-q, s, x)
    q = _fma32(r, y, q)
    return np.copysign(q, x).astype(np.float32)


def _check_div(x, s):
    x, s = np.float32(x), np.float32(s)
    ref = x / s
    got = _div_kernel(x, s)
    if abs(ref) >= np.float32(2.0 ** -12):
        assert got.view(np.uint32) == ref.view(np.uint32), (x, s, got, ref)
    else:
        assert np.signbit(got) == np.signbit(ref) and abs(got) < 2.0 ** -10


def _bf16_significands():
    """The 128 bf16 significands as float32 values in [1, 2)."""
    return ((np.arange(128, dtype=np.uint32) | 0x3F80) << 16).view(np.float32)


def test_scale_matches_ieee_for_every_amax_significand():
    amaxes = [m * np.float32(2.0 ** e) for e in (-13, -3, 0, 7, 40, 126) for m in _bf16_significands()]
    amaxes += [np.float32(0.0), FLOOR, np.float32(9.9e-5), np.float32(3.3895314e38)]
    for a in amaxes:
        a = np.float32(a)
        ref = np.float32(max(a, FLOOR) / np.float32(448.0))
        got = _scale_kernel(a)
        assert got.view(np.uint32) == ref.view(np.uint32), (a, got, ref)


def test_division_matches_ieee_for_every_significand_pair():
    sig = _bf16_significands()
    scales = [np.float32(m / np.float32(448.0)) for m in sig] + [np.float32(FLOOR / np.float32(448.0))]
    for s in scales:
        for shift in (np.float32(0.5), np.float32(2.0 ** -9)):
            for X in sig:
                x = np.float32(X * shift)
                _check_div(x, s)
                _check_div(-x, s)


def test_division_at_scale_exponents_and_tiny_quotients():
    """The same significand pairs with the scale far from 1 (amax 2^-13 ..
    2^126) and dividends down to the tiny-quotient region."""
    rng = ep_inputs.make_rng(22)
    sig = _bf16_significands()
    for e in (-13, 40, 126):
        for m in sig[rng.choice(128, 16, replace=False)]:
            amax = np.float32(m * np.float32(2.0 ** e))
            s = _scale_kernel(amax)
            for X in sig[rng.choice(128, 24, replace=False)]:
                for d in (0, 3, 11, 20, 40):
                    x = np.float32(X * np.float32(2.0 ** (e - 1 - d)))
                    if abs(x) <= amax:
                        _check_div(x, s)
                        _check_div(-x, s)
    # +-0 and the smallest bf16 magnitudes
    for x in (0.0, -0.0, 9.2e-41, -9.2e-41, 1.18e-38):
        _check_div(np.float32(x), _scale_kernel(FLOOR))


def test_division_on_cast_workload_inputs():
    """bf16 N(0,1) rows in groups of 128: each element against its group's
    scale, as the cast computes them."""
    rng = ep_inputs.make_rng(21)
    x = ep_inputs.bf16_normal(rng, (48, 128))
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    for row in xf:
        s = _scale_kernel(np.abs(row).max())
        for v in row:
            _check_div(v, s)
