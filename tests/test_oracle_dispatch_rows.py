"""Pins for the oracle's row copies: oracle_dispatch and
oracle_dispatch_partitioned, the bytes of each row, its scale row (fp32
scales and UE8M0 bytes, "DeepEP test target API reference" sec. 2.1: fp8 x
travels as (codes, scales); sec. 3.3 use_ue8m0), the receive weights, and the
padding rows (left as they were, or zeroed with their scales under
do_zero_padding).

The expected buffers are built here with numpy indexing from layouts of the
pure-Python brute force (oracle/brute.py), so neither the slot map nor the
copy shares code with the C oracle.  Row and scale-row widths differ and
every token's rows, scales and weights are distinct, so a wrong stride, a
swapped token or a missed padding row changes the result."""
import numpy as np
import pytest

import oracle
from oracle import brute


def _routing(rng, T, K, E, drop):
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx[rng.random((T, K)) < drop] = -1
    return idx


def _layout_from_brute(idx, E, A, C=0):
    T, K = idx.shape
    b = brute.layout(idx.tolist(), E, A, 1, C)
    return oracle.Layout(dst=np.array(b["dst"], np.int32).reshape(T, K),
                         src_of_slot=np.array(b["src_of_slot"], np.int32), R=b["R"],
                         count=np.array(b["count"], np.int32), offset=np.array(b["offset"], np.int32))


def _scales(rng, T, ng, fmt):
    if fmt == "ue8m0":
        return rng.permutation(np.arange(256, dtype=np.uint8).repeat(-(-T * ng // 256)))[:T * ng] \
            .reshape(T, ng)
    return (rng.uniform(0.001, 1.0, size=(T, ng)) * (1 + np.arange(T)[:, None])).astype(np.float32)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("zero_padding", [False, True])
@pytest.mark.parametrize("C", [0, 24])
def test_dispatch_rows_scales_weights_padding(fmt, zero_padding, C):
    rng = np.random.default_rng(3 + C)
    T, K, E, A, H, G = 40, 4, 8, 4, 96, 32
    idx = _routing(rng, T, K, E, 0.2)
    lay = _layout_from_brute(idx, E, A, C)
    q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    s = _scales(rng, T, H // G, fmt)
    w = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    R = lay.R
    q_init = np.full((R, H), 0xA5, np.uint8)
    s_init = np.full((R, H // G), 0x7B, np.uint8) if fmt == "ue8m0" else \
        np.full((R, H // G), -7.5, np.float32)
    recv, recv_s, recv_w = oracle.dispatch(q, lay, w, x_scales=s, zero_padding=zero_padding,
                                           recv_init=q_init, scales_init=s_init)
    exp, exp_s = q_init.copy(), s_init.copy()
    exp_w = np.zeros(R, np.float32)
    t_of, k_of = np.nonzero(lay.dst >= 0)
    slots = lay.dst[t_of, k_of]
    exp[slots] = q[t_of]
    exp_s[slots] = s[t_of]
    exp_w[slots] = w[t_of, k_of]
    pad = np.setdiff1d(np.arange(R), slots)
    assert len(pad) > 0
    if zero_padding:
        exp[pad] = 0
        exp_s[pad] = 0
    np.testing.assert_array_equal(recv, exp)
    np.testing.assert_array_equal(recv_s.view(np.uint8), exp_s.view(np.uint8))
    np.testing.assert_array_equal(recv_w, exp_w)
    if zero_padding and fmt == "fp32":
        assert not np.signbit(recv_s[pad]).any()     # +0.0f, not -0.0f


def test_dispatch_unweighted_rows_get_weight_one():
    rng = np.random.default_rng(8)
    idx = _routing(rng, 12, 3, 6, 0.3)
    lay = _layout_from_brute(idx, 6, 2)
    x = rng.integers(0, 1 << 16, size=(12, 8), dtype=np.uint16)
    recv, recv_s, recv_w = oracle.dispatch(x, lay)
    used = lay.src_of_slot >= 0
    np.testing.assert_array_equal(recv_w[used], 1.0)
    np.testing.assert_array_equal(recv_w[~used], 0.0)
    np.testing.assert_array_equal(recv[used], x[lay.src_of_slot[used] // 3])
    assert recv_s is None


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_dispatch_partitioned_rows_scales_metadata(fmt):
    rng = np.random.default_rng(5)
    T, K, E, P, H, G = 30, 5, 24, 6, 64, 16
    idx = _routing(rng, T, K, E, 0.15)
    b = brute.partition_layout(idx.tolist(), E, P)
    ts = np.array(b["token_slot"], np.int32).reshape(T, P)
    play = oracle.Layout(token_slot=ts, Rp=b["Rp"], P=P, E=E)
    q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    s = _scales(rng, T, H // G, fmt)
    w = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    recv, recv_s, ri, rw = oracle.dispatch_partitioned(q, idx, play, w, x_scales=s)
    Rp, m = b["Rp"], E // P
    exp = np.zeros((Rp, H), np.uint8)
    exp_s = np.zeros((Rp, H // G), s.dtype)
    exp_i = np.full((Rp, K), -1, np.int64)
    exp_w = np.zeros((Rp, K), np.float32)
    for t in range(T):
        for qq in range(P):
            r = ts[t, qq]
            if r < 0:
                continue
            exp[r], exp_s[r] = q[t], s[t]
            for k in range(K):
                e = idx[t, k]
                if e >= 0 and e // m == qq:
                    exp_i[r, k] = e - qq * m
                    exp_w[r, k] = w[t, k]
    np.testing.assert_array_equal(recv, exp)
    np.testing.assert_array_equal(recv_s.view(np.uint8), exp_s.view(np.uint8))
    np.testing.assert_array_equal(ri, exp_i)
    np.testing.assert_array_equal(rw, exp_w)
