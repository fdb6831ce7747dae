"""Pins for the oracle's non-expanded partition layout, its dispatch and
combine, and the two-level ("reduced") combine on the expanded layout."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_torch(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("T,K,E,P,G", [(2, 2, 4, 2, 1), (3, 2, 4, 4, 2), (2, 1, 6, 3, 3), (3, 1, 4, 2, 2)])
def test_partition_layout_brute_force(T, K, E, P, G):
    for flat in itertools.product(range(-1, E), repeat=T * K):
        idx = [list(flat[t * K:(t + 1) * K]) for t in range(T)]
        b = brute.partition_layout(idx, E, P, G)
        o = oracle.partition_layout(np.array(idx, np.int64), E, P, G)
        assert o.Rp == b["Rp"]
        np.testing.assert_array_equal(o.part_offset, b["part_offset"])
        np.testing.assert_array_equal(o.token_slot, np.array(b["token_slot"]).reshape(T, P))
        np.testing.assert_array_equal(o.tok_per_part, b["tok_per_part"])
        np.testing.assert_array_equal(o.tok_per_group, b["tok_per_group"])
        np.testing.assert_array_equal(o.part_src, [t for q in range(P) for t in b["members"][q]])


def test_partition_layout_rust_page_examples():
    """The Rust EP=2 page's per-rank pair lists, reduced to the tokens each
    rank receives (each token once, in order)."""
    with open(os.path.join(GOLDEN, "ep_dispatch_rs_examples.json")) as f:
        gold = json.load(f)
    for ex in gold["examples"]:
        T, K = ex["num_tokens"], ex["top_k"]
        idx = np.array(ex["indices"], np.int64).reshape(T, K)
        o = oracle.partition_layout(idx, 512, 2)
        local = 0 if ex["local_start"] == 0 else 1
        for side, q in (("local", local), ("remote", 1 - local)):
            key = side + "_token_indices"
            if key in ex["printed"]:
                expect = sorted(set(ex["printed"][key]))
                got = [t for t in range(T) if o.token_slot[t, q] >= 0]
                assert got == expect, (ex["name"], side)
                rows = [o.token_slot[t, q] for t in got]
                assert rows == list(range(o.part_offset[q], o.part_offset[q + 1]))


def test_partition_layout_invariants_skewed():
    w = ep_inputs.make_workload("skewed", T=4096, with_x=False)
    o = oracle.partition_layout(w.topk_idx, 256, 32, 8)
    e = oracle.get_layout(w.topk_idx, 256, 128, 32)
    np.testing.assert_array_equal(o.in_part, e.in_part)
    np.testing.assert_array_equal(o.tok_per_part, e.tok_per_part)
    slots = o.token_slot[o.token_slot >= 0]
    assert len(np.unique(slots)) == slots.size == o.Rp == o.in_part.sum()
    for q in range(32):
        col = o.token_slot[:, q]
        rows = col[col >= 0]
        assert (np.diff(rows) == 1).all()                      # tokens in ascending order
    groups = o.in_part.reshape(4096, 4, 8).any(axis=2).sum(axis=0)
    np.testing.assert_array_equal(o.tok_per_group, groups)


def test_dispatch_partitioned_rows_and_metadata():
    w = ep_inputs.make_workload("skewed", T=300, H=64, drop_p=0.0)
    w.topk_idx[5, 2] = -1
    pl = oracle.partition_layout(w.topk_idx, 256, 32)
    recv, _, ridx, rw = oracle.dispatch_partitioned(w.x, w.topk_idx, pl, w.topk_weights)
    m = 8
    for t in range(300):
        for q in range(32):
            row = pl.token_slot[t, q]
            if row < 0:
                continue
            np.testing.assert_array_equal(recv[row], w.x[t])
            for k in range(8):
                e = w.topk_idx[t, k]
                if e >= 0 and e // m == q:
                    assert ridx[row, k] == e - q * m and rw[row, k] == w.topk_weights[t, k]
                else:
                    assert ridx[row, k] == -1 and rw[row, k] == 0


def test_combine_partitioned_identities():
    """Plain sum over the partitions a token reaches: with rows equal to the
    token, the result is x times the number of those partitions; matches exact
    rationals; bias only is bf16(bias0 + bias1)."""
    w = ep_inputs.make_workload("skewed", T=200, H=128)
    pl = oracle.partition_layout(w.topk_idx, 256, 32)
    recv, _, _, _ = oracle.dispatch_partitioned(w.x, w.topk_idx, pl)
    f64 = oracle.combine_partitioned_f64(recv, pl.token_slot)
    npart = pl.in_part.sum(axis=1).astype(np.float64)
    np.testing.assert_allclose(f64, oracle.bf16_to_float(w.x).astype(np.float64) * npart[:, None],
                               rtol=1e-15)
    rng = ep_inputs.make_rng(3)
    y = ep_inputs.bf16_normal(rng, (pl.Rp, 128))
    b0 = ep_inputs.bf16_normal(rng, (200, 128))
    exact = brute.combine_exact(oracle.bf16_to_float(y).tolist(), pl.token_slot.tolist(), None,
                                oracle.bf16_to_float(b0).tolist())
    ex = np.array([[float(v) for v in row] for row in exact])
    np.testing.assert_allclose(oracle.combine_partitioned_f64(y, pl.token_slot, b0), ex, rtol=1e-15,
                               atol=1e-15)
    f32 = oracle.bf16_to_float(oracle.combine_partitioned_f32(y, pl.token_slot, b0))
    assert np.all(np.abs(f32 - ex) <= 2.0 ** -8 * np.abs(ex) + 1e-5 * (np.abs(ex) + 10))
    # equals the expanded combine with unit weights on the same rows when each
    # partition holds exactly one pair of the token
    idx = np.array([[0, 9, 17], [31, 8, 16]], np.int64)      # E=32, P=4: pairs in distinct partitions
    pl2 = oracle.partition_layout(idx, 32, 4)
    y2 = ep_inputs.bf16_normal(rng, (pl2.Rp, 16))
    dst = np.full((2, 3), -1, np.int32)
    for t in range(2):
        for k in range(3):
            dst[t, k] = pl2.token_slot[t, idx[t, k] // 8]
    order = np.argsort(idx // 8, axis=1, kind="stable")          # q ascending
    dst_sorted = np.take_along_axis(dst, order, axis=1)
    np.testing.assert_array_equal(oracle.combine_partitioned_f32(y2, pl2.token_slot),
                                  oracle.combine_f32(y2, dst_sorted))


def test_reduced_combine_special_cases():
    rng = ep_inputs.make_rng(4)
    # one partition, no bias: the same fp32 order as the plain combine, one
    # extra bf16 rounding that is idempotent
    w = ep_inputs.make_workload("prefill", T=200, H=64, E=32, K=4, A=2)
    lay = oracle.get_layout(w.topk_idx, 32, 2)
    y = ep_inputs.bf16_normal(rng, (lay.R, 64))
    for b16 in (False, True):
        np.testing.assert_array_equal(
            oracle.combine_reduced_f32(y, w.topk_idx, lay.dst, 32, 1, w.topk_weights,
                                       bf16_partials=b16),
            oracle.combine_f32(y, lay.dst, w.topk_weights))
    # every pair in its own partition: the fp32 product per pair (bf16 of it
    # with bf16 partials), then fp32 adds in partition order (numpy float32 +
    # torch bf16 cast)
    idx = np.stack([rng.permutation(8)[:4] for _ in range(50)]).astype(np.int64)
    wt = rng.standard_normal((50, 4)).astype(np.float32)
    lay = oracle.get_layout(idx, 8, 1)
    y = ep_inputs.bf16_normal(rng, (lay.R, 32))
    yf = oracle.bf16_to_float(y)
    for b16 in (False, True):
        got = oracle.combine_reduced_f32(y, idx, lay.dst, 8, 8, wt, bf16_partials=b16)
        expect = np.zeros((50, 32), np.uint16)
        for t in range(50):
            acc = np.zeros(32, np.float32)
            for k in np.argsort(idx[t], kind="stable"):
                prod = (wt[t, k] * yf[lay.dst[t, k]]).astype(np.float32)
                if b16:
                    prod = oracle.bf16_to_float(_bf16_torch(prod))
                acc = (acc + prod).astype(np.float32)
            expect[t] = _bf16_torch(acc)
        np.testing.assert_array_equal(got, expect)


def test_reduced_combine_within_tolerance_of_float64():
    w = ep_inputs.make_workload("skewed", T=256, H=256)
    lay = oracle.get_layout(w.topk_idx, 256, 128, 32)
    rng = ep_inputs.make_rng(5)
    y = ep_inputs.bf16_normal(rng, (lay.R, 256))
    b0 = ep_inputs.bf16_normal(rng, (256, 256))
    red = oracle.bf16_to_float(oracle.combine_reduced_f32(y, w.topk_idx, lay.dst, 256, 32,
                                                          w.topk_weights, b0)).astype(np.float64)
    f64 = oracle.combine_f64(y, lay.dst, w.topk_weights, b0)
    assert np.all(np.abs(red - f64) <= 1e-2 + 1e-2 * np.abs(f64))


@pytest.mark.parametrize("weighted", [False, True])
def test_reduced_combine_error_bound(weighted):
    """With bf16 partials the error against the exact sum is at most
    2^-9 of each partial's magnitude plus 2^-9 of the result (and fp32
    rounding far below that): |out - exact| <= 2^-8 (|exact| + S) with
    S = sum_k |w y|.  Unit weights over 8 pairs exceed a flat 1e-2 bound.
    The default fp32 partials stay within rtol = atol = 1e-2."""
    w = ep_inputs.make_workload("skewed", seed=3, T=256, K=8, E=256, A=128, drop_p=0.05,
                                with_x=False)
    lay = oracle.get_layout(w.topk_idx, 256, 128, 32)
    y = ep_inputs.make_y(w.rng, lay.R, 512)
    wt = w.topk_weights if weighted else None
    red = oracle.bf16_to_float(oracle.combine_reduced_f32(y, w.topk_idx, lay.dst, 256, 32, wt,
                                                          bf16_partials=True))
    f64 = oracle.combine_f64(y, lay.dst, wt)
    f32p = oracle.bf16_to_float(oracle.combine_reduced_f32(y, w.topk_idx, lay.dst, 256, 32, wt))
    assert np.all(np.abs(f32p.astype(np.float64) - f64) <= 1e-2 + 1e-2 * np.abs(f64))
    S = oracle.combine_f64(y & np.uint16(0x7FFF), lay.dst, None if wt is None else np.abs(wt))
    err = np.abs(red.astype(np.float64) - f64)
    assert np.all(err <= 2.0 ** -8 * (np.abs(f64) + S) + 1e-6)
    # the bf16 partials do show: some element differs from the one-level combine
    one = oracle.bf16_to_float(oracle.combine_f32(y, lay.dst, wt))
    assert np.any(one != red)
