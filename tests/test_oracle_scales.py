"""Pins for the oracle's power-of-two ("round_scale") and UE8M0 scale
formats of the low-latency fp8 path: closed-form values, the defining
inequalities, a float64 ceil(log2) reference, and codes equal to torch's
float8_e4m3fn cast of the exactly scaled values."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle


def test_pow2_ceil_values():
    cases = {1.0: 1.0, 0.75: 1.0, 0.5: 0.5, 1.0000001: 2.0, 3.0: 4.0, 2.0 ** -22: 2.0 ** -22,
             1e-4 / 448: 2.0 ** -22, 448.0 / 448: 1.0, 449.0 / 448: 2.0, 2.0 ** 100 * 1.5: 2.0 ** 101}
    for v, expect in cases.items():
        assert oracle.pow2_ceil(np.float32(v))[0] == np.float32(expect), v


def test_pow2_ceil_matches_float64_log2():
    rng = ep_inputs.make_rng(11)
    v = np.exp(rng.uniform(-40, 40, 5000)).astype(np.float32)
    v[:20] = 2.0 ** np.arange(-10, 10)                  # exact powers stay put
    got = oracle.pow2_ceil(v)
    ref = (2.0 ** np.ceil(np.log2(v.astype(np.float64)))).astype(np.float32)
    np.testing.assert_array_equal(got, ref)
    assert np.all(got >= v) and np.all(got < 2 * v.astype(np.float64))


def test_ue8m0_encoding():
    assert oracle.ue8m0_of(np.float32(1.0))[0] == 127
    assert oracle.ue8m0_of(np.float32(2.0))[0] == 128
    assert oracle.ue8m0_of(np.float32(2.0 ** -22))[0] == 105
    b = np.arange(0, 255, dtype=np.uint8)
    dec = oracle.ue8m0_to_float(b)
    np.testing.assert_array_equal(dec, np.ldexp(np.float32(1.0), b.astype(np.int32) - 127))
    np.testing.assert_array_equal(oracle.ue8m0_of(dec[1:]), b[1:])   # 2^-127 is subnormal


@pytest.mark.parametrize("G", [128, 32, 7168])
def test_pow2_cast_against_torch(G):
    w = ep_inputs.make_workload("fp8", T=64)
    x = w.x.copy()
    x[3, :G] = 0                                     # an all-zero group: floor 1e-4
    x[5, 0] = 0x4380                                 # 256.0 in bf16
    q, s, e8 = oracle.cast_fp8_pow2(x, G, ue8m0=True)
    xf = oracle.bf16_to_float(x).reshape(64, -1, G)
    amax = np.maximum(np.abs(xf).max(axis=2), np.float32(1e-4))
    s0 = (amax / np.float32(448)).astype(np.float32)
    assert np.all(s >= s0) and np.all(s < 2 * s0.astype(np.float64))
    np.testing.assert_array_equal(s, oracle.pow2_ceil(s0).reshape(s.shape))
    np.testing.assert_array_equal(oracle.ue8m0_to_float(e8).reshape(s.shape), s)
    assert np.all(amax / s <= 448)
    scaled = (xf / s[:, :, None]).astype(np.float32)     # exact: s is a power of two
    ref = torch.from_numpy(scaled.reshape(64, -1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, ref)
    # without UE8M0 the codes and fp32 scales are the same
    q2, s2, none = oracle.cast_fp8_pow2(x, G)
    assert none is None
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s)


def test_pow2_cast_reduces_to_plain_cast_on_power_of_two_amax():
    """When amax/448 is already a power of two the two casts agree."""
    rng = ep_inputs.make_rng(12)
    xf = rng.uniform(-1, 1, (16, 128)).astype(np.float32)
    xf[:, 0] = 448.0 * 2.0 ** -3                      # amax = 56 exactly -> scale 1/8
    x = oracle.bf16_from_float(xf).reshape(16, 128)
    q, s, _ = oracle.cast_fp8_pow2(x, 128)
    qp, sp = oracle.cast_fp8(x, 128)
    np.testing.assert_array_equal(s, sp)
    np.testing.assert_array_equal(q, qp)
    assert np.all(s == np.float32(0.125))
