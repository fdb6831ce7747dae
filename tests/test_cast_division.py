"""The division the fp8 cast kernels use: y = RN(1/s) once per scale group,
then per element q = RN(x*y) and two corrections q = RN(q + y*RN(x - s*q))
(Markstein's refinement, P. Markstein, IBM J. Res. Dev. 34(1), 1990), with
x's sign.  Restated here with exact rational FMAs and compared bit for bit
with IEEE float32 division on sampled inputs of the cast's range: bf16 x,
s = max(amax, 1e-4) / 448 for the group's amax >= |x|.  Bitwise equality is
asked wherever an e4m3 code can be non-zero or sit on a rounding boundary
(|x/s| >= 2^-12, with margin); below that, the codes are signed zeros."""
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


def _div_kernel(x, s):
    y = np.float32(1.0) / s
    q = np.float32(x * y)
    r = _fma32(-q, s, x)
    q = _fma32(r, y, q)
    r = _fma32(-q, s, x)
    q = _fma32(r, y, q)
    return np.copysign(q, x).astype(np.float32)


def _check(xs, ss):
    for x, s in zip(xs, ss):
        x, s = np.float32(x), np.float32(s)
        ref = x / s
        got = _div_kernel(x, s)
        if abs(ref) >= np.float32(2.0 ** -12):
            assert got.view(np.uint32) == ref.view(np.uint32), (x, s, got, ref)
        else:
            # Every e4m3 code of |q| < 2^-10 is a signed zero.  Down here the
            # residual of a tiny x can fall below fp32's normal range, where
            # the corrections are no longer exact: only sign and magnitude class
            # are asked for.
            assert np.signbit(got) == np.signbit(ref) and abs(got) < 2.0 ** -10


def test_division_matches_ieee_on_cast_inputs():
    rng = ep_inputs.make_rng(21)
    n = 6000
    x = ep_inputs.bf16_normal(rng, (n,))
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    # group amax at or above |x|: |x| times a factor in [1, 2^12]
    amax = np.abs(xf) * np.exp2(rng.uniform(0, 12, n)).astype(np.float32)
    s = (np.maximum(amax, np.float32(1e-4)) / np.float32(448)).astype(np.float32)
    _check(xf, s)


def test_division_matches_ieee_on_all_bf16_magnitudes():
    """Every bf16 exponent and several significands, against a few scales."""
    rng = ep_inputs.make_rng(22)
    bits = np.concatenate([np.arange(0, 0x7F80, 97), [0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F]])
    bits = np.concatenate([bits, bits | 0x8000]).astype(np.uint16)
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    for lead in (np.float32(448.0), np.float32(3.0e38), np.float32(0.37), np.float32(1e-4)):
        a = np.maximum(np.abs(xf).max(initial=0), lead) if lead > 1 else lead
        keep = np.abs(xf) <= a
        s = np.float32(max(a, np.float32(1e-4)) / np.float32(448))
        _check(xf[keep][:1500], np.full(min(keep.sum(), 1500), s, np.float32))
    # random scales
    s = (np.exp2(rng.uniform(-20, 20, 3000)) / 448).astype(np.float32)
    x = np.clip(rng.standard_normal(3000).astype(np.float32) * s * 448, -448 * s, 448 * s)
    _check(x.astype(np.float32), s)
