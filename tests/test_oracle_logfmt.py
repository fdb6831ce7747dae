"""Pins for the oracle's 10-bit logarithmic combine payload ("DeepEP test
target API reference" sec. 3.4, low_latency_combine's use_logfmt: the page
names a 10-bit log format and defines nothing else of it).

The reading under test: groups of 128 channels; a magnitude's log is its bf16
magnitude bits read as a fixed-point base-2 logarithm (exponent field, then
the mantissa as fraction), rounded half to even to five fractional bits and
held at the largest finite value; one sign bit over a 9-bit index measured
down from the group's largest log (largest magnitude = 511, 0 = zero, which
keeps the input's sign); groups with an infinity or NaN decode to NaN.

Every pin below states the expected result in the value domain (frexp,
ldexp, rint in float64) or by hand, not with the oracle's integer steps:
* the round trip of every bf16 pattern equals rounding to six significant
  bits (five fraction bits) with the bf16 subnormal quantum, saturated;
* the window: with a group maximum of 2^k the smallest value kept is
  1.0625 * 2^(k-16) (worked by hand); with a maximum whose log is below 511
  nothing nonzero is flushed;
* the relative error bound 2^-6, monotonicity and odd symmetry;
* hand-worked codes of a small group, and the byte layout of the packing;
* a payload of values already in the format is lossless through the combine,
  and the combine's error against float64 stays inside the codec's bound."""
import numpy as np
import pytest

import ep_inputs
import oracle

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE = ALL[(ALL & 0x7FFF) < 0x7F80]


def _val(bits):
    return oracle.bf16_to_float(bits).astype(np.float64)


def _round6(v):
    """|v| rounded half to even to 1 + 5 significant bits with the quantum of
    its binade (at least that of 2^-126), saturated at (2 - 2^-5) * 2^127;
    sign kept, also on a zero result."""
    a = np.abs(v)
    _, e = np.frexp(a)                       # a = f * 2^e, f in [0.5, 1)
    qe = np.maximum(e - 1, -126) - 5
    q = np.ldexp(np.rint(np.ldexp(a, -qe)), qe)
    q = np.minimum(q, (2.0 - 2.0 ** -5) * 2.0 ** 127)
    return np.copysign(np.where(a == 0, 0.0, q), v)


def _same(got, want):
    """Equal values with equal signs (so -0 differs from +0)."""
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(want))


def _groups_with(first, xs):
    """One 128-channel row per x: [first, x, 0, ...]; first=None puts x alone."""
    rows = np.zeros((xs.size, 128), np.uint16)
    if first is None:
        rows[:, 0] = xs
    else:
        rows[:, 0] = first
        rows[:, 1] = xs
    return rows


def test_round_trip_of_every_pattern_alone_in_its_group():
    rows = _groups_with(None, ALL)
    codes, refs = oracle.logfmt_encode(rows)
    dec = oracle.logfmt_decode(codes, refs)
    fin = (ALL & 0x7FFF) < 0x7F80
    # non-finite: the group is marked and every channel decodes to NaN
    assert np.all(refs[~fin, 0] == oracle.LOGFMT_POISON)
    assert np.all(codes[~fin] == 0)
    assert np.all(np.isnan(_val(dec[~fin])))
    # finite: rounding to five fraction bits, and the value alone is the
    # group's largest, index 511 (unless it rounds to zero)
    got = _val(dec[fin, 0])
    want = _round6(_val(ALL[fin]))
    _same(got, want)
    nz = want != 0
    assert np.all(codes[fin, 0][nz] & 511 == 511)
    assert np.all((codes[fin, 0] >> 9) == (ALL[fin] >> 15))
    assert np.all(codes[fin, 0][~nz] & 511 == 0)
    assert np.all(dec[fin, 1:] == 0)


@pytest.mark.parametrize("k", [0, 7, -20, 100, -110, 127])
def test_window_below_a_power_of_two_maximum(k):
    top = _val(oracle.bf16_from_float(np.float32(2.0 ** k)))[0]
    xs = FINITE[np.abs(_val(FINITE)) <= top]
    rows = _groups_with(oracle.bf16_from_float(np.float32(2.0 ** k))[0], xs)
    codes, refs = oracle.logfmt_encode(rows)
    dec = _val(oracle.logfmt_decode(codes, refs)[:, 1])
    # the log of 2^k is 32 (127 + k) units; 510 units below it is
    # 32 (111 + k) + 2 units: the pattern of 2^(k-16) * (1 + 2/32)
    smallest = 1.0625 * 2.0 ** (k - 16)
    q = _round6(_val(xs))
    want = np.where(np.abs(q) >= smallest, q, np.copysign(0.0, q))
    _same(dec, want)
    assert np.all(codes[:, 0] == 511)


def test_nothing_is_flushed_below_a_small_maximum():
    # a maximum of 2^-130 (a bf16 subnormal, log 2 units): every value at or
    # below it keeps its rounding
    top_bits = np.uint16(0x0008)
    xs = FINITE[(FINITE & 0x7FFF) <= 0x0008]
    codes, refs = oracle.logfmt_encode(_groups_with(top_bits, xs))
    _same(_val(oracle.logfmt_decode(codes, refs)[:, 1]), _round6(_val(xs)))
    assert np.all(refs[:, 0] == 2)


def test_error_bound_monotone_and_odd():
    rng = ep_inputs.make_rng(77)
    y = ep_inputs.make_y_wide(rng, 400, 1024, specials=False)
    codes, refs = oracle.logfmt_encode(y)
    dec = _val(oracle.logfmt_decode(codes, refs))
    x = _val(y)
    gmax = np.abs(x).reshape(400, 8, 128).max(axis=2).repeat(128, axis=1)
    kept = dec != 0
    normal = np.abs(x) >= 2.0 ** -126
    sel = kept & normal
    assert np.all(np.abs(dec[sel] - x[sel]) <= 2.0 ** -6 * np.abs(x[sel]))
    assert np.all(np.sign(dec[kept]) == np.sign(x[kept]))
    # flushed values lie more than 15 octaves under the group maximum; kept
    # ones fewer than 17
    flushed = (dec == 0) & (x != 0) & normal
    assert np.all(np.abs(x[flushed]) < 2.0 ** -15 * gmax[flushed])
    assert np.all(np.abs(x[sel]) > 2.0 ** -17 * gmax[sel])
    assert flushed.sum() > 1000 and sel.sum() > 100000
    # monotone and odd over all patterns under one maximum
    pos = FINITE[(FINITE < 0x8000) & (FINITE <= 0x4780)]      # up to 2^16
    pos = pos[np.argsort(_val(pos))]
    for s in (0, 0x8000):
        c, r = oracle.logfmt_encode(_groups_with(np.uint16(0x4780), pos | np.uint16(s)))
        d = _val(oracle.logfmt_decode(c, r)[:, 1])
        if s == 0:
            assert np.all(np.diff(d) >= 0)
            d_pos = d
        else:
            np.testing.assert_array_equal(d, -d_pos)


def test_hand_worked_group():
    # 1.0 = 0x3F80: log 0x3F80/4 = 0xFE0, the reference; index 511
    # -0.5 = 0xBF00: log 0xFC0, one octave (32) down: 479 = 0x1DF, sign: 0x3DF
    # 0.75 = 0x3F40: log 0xFD0: 495 = 0x1EF
    # 0x3EAB (0.333984375): 0x3EAB/4 = 0xFAA.C -> 0xFAB: 458 = 0x1CA, decodes
    #   to 0xFAB*4 = 0x3EAC (0.3359375)
    # 2^-16 = 0x3780: log 0xDE0 = 0xFE0 - 512: index -1, flushed
    # 1.0625 * 2^-16 = 0x3788: log 0xDE2: index 1
    # +0 and -0: index 0, the sign kept: 0x000 and 0x200
    # -2^-16 = 0xB780: flushed like 2^-16, the sign kept: 0x200, decodes to -0
    # 0x3F83 (1.0234375): 0x3F83/4 = 0xFE0.C -> 0xFE1 becomes the reference:
    #   every other index above drops by one
    row = np.zeros((1, 128), np.uint16)
    row[0, :9] = [0x3F80, 0xBF00, 0x3F40, 0x3EAB, 0x3780, 0x3788, 0x0000, 0x8000, 0xB780]
    codes, refs = oracle.logfmt_encode(row)
    assert refs.tolist() == [[0x0FE0]]
    assert codes[0, :9].tolist() == [0x1FF, 0x3DF, 0x1EF, 0x1CA, 0, 0x001, 0, 0x200, 0x200]
    dec = oracle.logfmt_decode(codes, refs)
    assert dec[0, :9].tolist() == [0x3F80, 0xBF00, 0x3F40, 0x3EAC, 0, 0x3788, 0, 0x8000, 0x8000]
    row[0, 100] = 0x3F83
    codes, refs = oracle.logfmt_encode(row)
    assert refs.tolist() == [[0x0FE1]]
    assert codes[0, :9].tolist() == [0x1FE, 0x3DE, 0x1EE, 0x1C9, 0, 0, 0, 0x200, 0x200]
    assert codes[0, 100] == 0x1FF
    # ties to even: 0x3F82 / 4 = 0xFE0.8 -> 0xFE0; 0x3F86 / 4 = 0xFE1.8 -> 0xFE2
    row2 = np.zeros((2, 128), np.uint16)
    row2[0, 0], row2[1, 0] = 0x3F82, 0x3F86
    _, refs = oracle.logfmt_encode(row2)
    assert refs[:, 0].tolist() == [0x0FE0, 0x0FE2]
    # saturation: the top of the bf16 range holds at 0x1FDF (0x7F7C)
    row2[0, 0], row2[1, 0] = 0x7F7F, 0xFF7E
    codes, refs = oracle.logfmt_encode(row2)
    assert refs[:, 0].tolist() == [0x1FDF, 0x1FDF]
    assert oracle.logfmt_decode(codes, refs)[:, 0].tolist() == [0x7F7C, 0xFF7C]


def test_packed_byte_layout():
    codes = np.zeros((1, 256), np.uint16)
    codes[0, 0] = 0x155          # bit 8 set, positive
    codes[0, 17] = 0x3FF         # bits 8 and 9 (sign) set
    codes[0, 255] = 0x2AA        # bit 9 only
    refs = np.array([[0x0ABC, 0x1234]], np.uint16)
    p = oracle.logfmt_pack(codes, refs)
    H = 256
    assert oracle.logfmt_row_bytes(H) == 384 and p.shape == (1, 384)
    assert p[0, 0] == 0x55 and p[0, 17] == 0xFF and p[0, 255] == 0xAA
    # channel 16v + 2p + e: bit 8 of the code at bit 7 - p + 16e of word v,
    # the sign at bit 15 - p + 16e
    assert p[0, H:H + 4].tolist() == [0x80, 0x00, 0x00, 0x00]          # channel 0: bit 7
    assert p[0, H + 4:H + 8].tolist() == [0x00, 0x00, 0x80, 0x80]      # channel 17: 23, 31
    assert p[0, H + 60:H + 64].tolist() == [0x00, 0x00, 0x00, 0x01]    # channel 255: 24
    assert p[0, H + 64:H + 68].tolist() == [0xBC, 0x0A, 0x34, 0x12]
    assert not p[0, H + 68:].any()
    assert np.count_nonzero(p[0, :H]) == 3
    assert oracle.logfmt_row_bytes(7168) == 9088 and oracle.logfmt_row_bytes(128) == 256
    rng = ep_inputs.make_rng(5)
    c, r = oracle.logfmt_encode(ep_inputs.make_y_wide(rng, 50, 384))
    c2, r2 = oracle.logfmt_unpack(oracle.logfmt_pack(c, r), 384)
    np.testing.assert_array_equal(c2, c)
    np.testing.assert_array_equal(r2, r)


def test_codes_are_ten_bits_and_decode_rejects_others():
    rng = ep_inputs.make_rng(6)
    y = ep_inputs.make_y_wide(rng, 300, 512)
    codes, refs = oracle.logfmt_encode(y)
    assert codes.max() < 1024
    assert np.any(refs == oracle.LOGFMT_POISON)
    with pytest.raises(ValueError):
        bad = refs.copy()
        bad[0, 0] = 0x2000             # no finite log is that large
        oracle.logfmt_decode(codes, bad)
    with pytest.raises(ValueError):
        r, g = np.argwhere(refs == oracle.LOGFMT_POISON)[0]
        bad = codes.copy()
        bad[r, g * 128] = 0x001        # a marked group holds only zero codes
        oracle.logfmt_decode(bad, refs)
    with pytest.raises(ValueError):
        oracle.logfmt_encode(np.zeros((2, 100), np.uint16))


def test_combine_over_exact_values_is_lossless():
    # values with at most five fraction bits in a narrow range pass unchanged,
    # so the combine over the payload equals the bf16 combine bit for bit
    rng = ep_inputs.make_rng(8)
    T, K, R, H = 200, 4, 600, 256
    mant = rng.integers(32, 64, (R, H))
    expo = rng.integers(-3, 4, (R, H))
    sign = np.where(rng.random((R, H)) < 0.5, -1.0, 1.0)
    y = oracle.bf16_from_float((sign * np.ldexp(mant / 32.0, expo)).astype(np.float32))
    y = y.reshape(R, H)
    codes, refs = oracle.logfmt_encode(y)
    np.testing.assert_array_equal(oracle.logfmt_decode(codes, refs), y)
    dst = rng.integers(-1, R, (T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    np.testing.assert_array_equal(oracle.combine_logfmt_f32(codes, refs, dst, w),
                                  oracle.combine_f32(y, dst, w))


def test_combine_error_within_the_codec_bound():
    w = ep_inputs.make_workload("tiny")
    lay = oracle.get_layout(w.topk_idx, w.num_experts, w.expert_alignment)
    rng = ep_inputs.make_rng(9)
    y = ep_inputs.make_y(rng, lay.R, 256)
    codes, refs = oracle.logfmt_encode(y)
    got = _val(oracle.combine_logfmt_f32(codes, refs, lay.dst, w.topk_weights))
    exact = oracle.combine_f64(y, lay.dst, w.topk_weights)
    # |sum w y - sum w dec(y)| <= sum |w| (2^-6 |y| for a kept value, or
    # 2^-15 of its group's maximum for a flushed one), then one bf16
    # rounding of the result
    absw = np.abs(w.topk_weights.astype(np.float64))
    mag = np.zeros_like(exact)
    top = np.zeros_like(exact)
    yv = np.abs(_val(y))
    gm = np.repeat(yv.reshape(lay.R, 2, 128).max(axis=2), 128, axis=1)
    for k in range(w.num_topk):
        d = lay.dst[:, k]
        ok = d >= 0
        mag[ok] += absw[ok, k, None] * yv[d[ok]]
        top[ok] += absw[ok, k, None] * gm[d[ok]]
    bound = 2.0 ** -6 * mag + 2.0 ** -15 * top + 2.0 ** -8 * np.abs(exact)
    assert np.all(np.abs(got - exact) <= bound * 1.0001)
    assert np.any(got != _val(oracle.combine_f32(y, lay.dst, w.topk_weights)))
