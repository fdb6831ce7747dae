"""Pins for the oracle's floating-point steps: bf16 rounding, OCP e4m3
encoding, the per-(token, group) fp8 cast, and the combine reduction.

References used (none of them is the oracle itself): torch's CPU casts to
bfloat16 and float8_e4m3fn (library special cases), numpy's IEEE fp32
division, exact rational arithmetic (fractions), closed-form error bounds, and
the method's invariants.
"""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from oracle import brute


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return bits, oracle.bf16_to_float(bits)


def _torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 1.0 / 448.0, 0.0013, 37.25, 2.0 ** -12])
def test_e4m3_exhaustive_vs_torch(scale):
    """Every bf16 pattern divided (fp32) by a scale: oracle E4M3 == torch."""
    _, v = _all_bf16_values()
    with np.errstate(all="ignore"):
        d = (v / np.float32(scale)).astype(np.float32)
    ours = oracle.e4m3_from_float(d)
    ref = _torch_e4m3(d)
    nan = np.isnan(d)
    # NaN payload/sign conventions aside, NaN maps to a NaN code
    assert ((ours[nan] & 0x7F) == 0x7F).all()
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_e4m3_midpoints_ties_to_even():
    """Exact midpoints between neighbouring e4m3 magnitudes round to the even
    mantissa; one fp32 ulp either side rounds to the nearer neighbour."""
    mags = np.array([oracle.e4m3_to_float(c)[0] for c in range(0x7F)], np.float64)
    mids = (mags[:-1] + mags[1:]) / 2
    for sgn in (1.0, -1.0):
        m32 = (sgn * mids).astype(np.float32)
        assert np.array_equal(m32.astype(np.float64), sgn * mids)  # exact in fp32
        got = oracle.e4m3_from_float(m32) & 0x7F
        lo = np.arange(0x7E)
        expect = np.where(lo % 2 == 0, lo, lo + 1)
        np.testing.assert_array_equal(got, expect)
        up = np.nextafter(m32, np.float32(sgn * np.inf))
        dn = np.nextafter(m32, np.float32(0))
        np.testing.assert_array_equal(oracle.e4m3_from_float(up) & 0x7F, lo + 1)
        np.testing.assert_array_equal(oracle.e4m3_from_float(dn) & 0x7F, lo)
        np.testing.assert_array_equal(got, _torch_e4m3(m32) & 0x7F)


def test_e4m3_round_trip_and_signed_zero():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert len(codes) == 254
    vals = oracle.e4m3_to_float(codes)
    np.testing.assert_array_equal(oracle.e4m3_from_float(vals), codes)
    assert oracle.e4m3_to_float([0x7E])[0] == 448.0
    assert oracle.e4m3_to_float([0x01])[0] == 2.0 ** -9
    assert oracle.e4m3_to_float([0x08])[0] == 2.0 ** -6
    np.testing.assert_array_equal(oracle.e4m3_from_float(np.array([-1e-9, 1e-9, 464.0, -464.0], np.float32)),
                                  [0x80, 0x00, 0x7E, 0xFE])
    assert (oracle.e4m3_from_float(np.array([465.0, 1e30, -500.0], np.float32)) & 0x7F == 0x7F).all()


def _bf16_torch(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, size=100000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near = np.array([0x7F7F8000, 0x7F7FFFFF, 0x00008000, 0x00018000, 0x80008000, 0x3F808000,
                     0x3F818000, 0x00000001, 0x7F800000, 0xFF800000], np.uint32)
    v = np.concatenate([bits, ties, near]).view(np.float32)
    v = v[~np.isnan(v)]
    np.testing.assert_array_equal(oracle.bf16_from_float(v), _bf16_torch(v))


def test_div_f32_is_ieee():
    rng = np.random.default_rng(2)
    a = rng.standard_normal(100000).astype(np.float32)
    b = (np.abs(rng.standard_normal(100000)) + 1e-3).astype(np.float32)
    np.testing.assert_array_equal(oracle.div_f32(a, b), a / b)


def _cast_reference(x_bits, G):
    """Library composition: amax and division in numpy fp32, e4m3 by torch."""
    x = oracle.bf16_to_float(x_bits)
    T, H = x.shape
    g = x.reshape(T, H // G, G)
    amax = np.abs(g).max(axis=2)
    s = (np.maximum(amax, np.float32(1e-4)) / np.float32(448.0)).astype(np.float32)
    d = (g / s[:, :, None]).astype(np.float32)
    return _torch_e4m3(d.reshape(T, H)).reshape(T, H), s


@pytest.mark.parametrize("G", [128, 32, 256])
def test_cast_fp8_vs_library_composition(G):
    rng = ep_inputs.make_rng(3)
    x = ep_inputs.bf16_normal(rng, (64, 1024))
    x[3, :G] = 0                       # all-zero group hits the 1e-4 floor
    x[5, G:2 * G] = 0x0001             # tiny subnormal bf16 values
    x[7, 5] = 0x7F7F                   # the largest finite bf16 in one group
    q, s = oracle.cast_fp8(x, G)
    rq, rs = _cast_reference(x, G)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)


def test_cast_fp8_per_token_whole_row():
    """G = H reproduces the page's per-token formula (one scale per row)."""
    x = ep_inputs.bf16_normal(ep_inputs.make_rng(4), (16, 7168))
    q, s = oracle.cast_fp8(x, 7168)
    rq, rs = _cast_reference(x, 7168)
    assert s.shape == (16, 1)
    np.testing.assert_array_equal(q, rq)
    np.testing.assert_array_equal(s, rs)


def test_cast_fp8_error_bound_and_amax_code():
    x = ep_inputs.bf16_normal(ep_inputs.make_rng(5), (128, 7168))
    q, s = oracle.cast_fp8(x, 128)
    xf = oracle.bf16_to_float(x).astype(np.float64)
    back = oracle.cast_back(q, s, 128).astype(np.float64)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * srep) * (1 + 2.0 ** -22)
    assert (np.abs(back - xf) <= bound + 1e-30).all()
    g = np.abs(xf).reshape(128, 56, 128)
    pos = g.argmax(axis=2)
    codes = np.take_along_axis(q.reshape(128, 56, 128), pos[:, :, None], axis=2)[..., 0]
    assert ((codes & 0x7F) == 0x7E).all()


def test_cast_fp8_negative_underflow_keeps_sign():
    x = np.zeros((1, 128), np.uint16)
    x[0, 0] = oracle.bf16_from_float(np.array([100.0], np.float32))[0]
    x[0, 1] = oracle.bf16_from_float(np.array([-1e-4], np.float32))[0]
    x[0, 2] = oracle.bf16_from_float(np.array([1e-4], np.float32))[0]
    q, _ = oracle.cast_fp8(x, 128)
    assert q[0, 1] == 0x80 and q[0, 2] == 0x00 and q[0, 0] == 0x7E


# ---------------------------------------------------------------- combine


def _tiny_case(seed, T=6, K=3, E=5, H=16, bias=0):
    rng = ep_inputs.make_rng(seed)
    idx, w = ep_inputs.routing_uniform(rng, T, E, K)
    idx[rng.random((T, K)) < 0.2] = -1
    lay = oracle.get_layout(idx, E, 2)
    y = ep_inputs.bf16_normal(rng, (lay.R, H))
    b = [ep_inputs.bf16_normal(rng, (T, H)) for _ in range(bias)]
    return idx, w, lay, y, b


@pytest.mark.parametrize("bias", [0, 1, 2])
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_vs_exact_rationals(bias, weighted):
    idx, w, lay, y, b = _tiny_case(7 + bias, bias=bias)
    yf = oracle.bf16_to_float(y)
    bf = [oracle.bf16_to_float(bb) for bb in b]
    exact = brute.combine_exact(yf.tolist(), lay.dst.tolist(), w.tolist() if weighted else None,
                                bf[0].tolist() if bias > 0 else None,
                                bf[1].tolist() if bias > 1 else None)
    ex = np.array([[float(v) for v in row] for row in exact])
    args = dict(topk_weights=w if weighted else None, bias0=b[0] if bias > 0 else None,
                bias1=b[1] if bias > 1 else None)
    f64 = oracle.combine_f64(y, lay.dst, **args)
    np.testing.assert_allclose(f64, ex, rtol=1e-14, atol=1e-14)
    f32 = oracle.bf16_to_float(oracle.combine_f32(y, lay.dst, **args)).astype(np.float64)
    # fp32 accumulation of <= 5 terms, then bf16 rounding
    err = np.abs(f32 - ex)
    scale = np.abs(ex) + sum(np.abs(bb) for bb in bf) + np.abs(yf).max() * 3
    assert (err <= 2.0 ** -8 * np.abs(ex) + 2.0 ** -20 * scale).all()


def test_combine_of_dispatch_is_x_times_weight_sum():
    """combine(dispatch(x)) = x * sum_k w[t,k] (the invariant the method fixes)."""
    w = ep_inputs.make_workload("prefill", T=300, H=512)
    lay = oracle.get_layout(w.topk_idx, 256, 128)
    recv, _, _ = oracle.dispatch(w.x, lay, w.topk_weights)
    out = oracle.combine_f64(recv, lay.dst, w.topk_weights)
    wsum = np.where(w.topk_idx >= 0, w.topk_weights.astype(np.float64), 0).sum(axis=1)
    expect = oracle.bf16_to_float(w.x).astype(np.float64) * wsum[:, None]
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=1e-30)
    f32 = oracle.bf16_to_float(oracle.combine_f32(recv, lay.dst, w.topk_weights))
    np.testing.assert_allclose(f32, expect, rtol=2.0 ** -8 + 1e-6, atol=1e-30)


def test_combine_k1_unit_weight_is_exact_gather():
    rng = ep_inputs.make_rng(11)
    idx, _ = ep_inputs.routing_uniform(rng, 50, 16, 1)
    lay = oracle.get_layout(idx, 16, 4)
    y = ep_inputs.bf16_normal(rng, (lay.R, 64))
    out = oracle.combine_f32(y, lay.dst)
    np.testing.assert_array_equal(out, y[lay.dst[:, 0]])


def test_combine_k1_weighted_single_rounding():
    """K = 1, no bias: fmaf(w, y, 0) = fp32 rounding of the exact product, then
    bf16 (numpy float32 product and torch's bf16 cast)."""
    rng = ep_inputs.make_rng(12)
    idx, w = ep_inputs.routing_uniform(rng, 64, 8, 1)
    w = rng.standard_normal((64, 1)).astype(np.float32)
    lay = oracle.get_layout(idx, 8, 1)
    y = ep_inputs.bf16_normal(rng, (lay.R, 128))
    prod = (w * oracle.bf16_to_float(y[lay.dst[:, 0]])).astype(np.float32)
    np.testing.assert_array_equal(oracle.combine_f32(y, lay.dst, w), _bf16_torch(prod))


def test_combine_bias_only():
    """No valid pair: out = bf16(bias0 + bias1) in fp32."""
    rng = ep_inputs.make_rng(13)
    b0 = ep_inputs.bf16_normal(rng, (4, 64))
    b1 = ep_inputs.bf16_normal(rng, (4, 64))
    dst = np.full((4, 2), -1, np.int32)
    y = np.zeros((1, 64), np.uint16)
    s = (oracle.bf16_to_float(b0) + oracle.bf16_to_float(b1)).astype(np.float32)
    np.testing.assert_array_equal(oracle.combine_f32(y, dst, None, b0, b1), _bf16_torch(s))
    np.testing.assert_array_equal(oracle.combine_f32(y, dst, None, b0), b0)


def test_combine_token_subset_matches_full():
    idx, w, lay, y, b = _tiny_case(21, T=20, bias=2)
    full = oracle.combine_f32(y, lay.dst, w, b[0], b[1])
    sub = oracle.combine_f32(y, lay.dst, w, b[0], b[1], tokens=np.array([19, 0, 7]))
    np.testing.assert_array_equal(sub, full[[19, 0, 7]])


def test_dispatch_rows_and_zero_padding():
    w = ep_inputs.make_workload("decode", T=40, H=64)
    lay = oracle.get_layout(w.topk_idx, 256, 1, 1, 4)
    junk = np.full((lay.R, 64), 0x1234, np.uint16)
    recv, _, rw = oracle.dispatch(w.x, lay, w.topk_weights, zero_padding=False, recv_init=junk)
    for t in range(40):
        for k in range(8):
            s = lay.dst[t, k]
            if s >= 0:
                np.testing.assert_array_equal(recv[s], w.x[t])
                assert rw[s] == w.topk_weights[t, k]
    pad = lay.src_of_slot < 0
    assert (recv[pad] == 0x1234).all() and (rw[pad] == 0).all()
    recvz, _, _ = oracle.dispatch(w.x, lay, w.topk_weights, zero_padding=True, recv_init=junk)
    assert (recvz[pad] == 0).all()
    np.testing.assert_array_equal(recvz[~pad], recv[~pad])
    cw = oracle.combined_weights(rw, lay.dst)
    np.testing.assert_array_equal(cw, np.where(lay.dst >= 0, w.topk_weights, 0))
