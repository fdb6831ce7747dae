"""Pins for the oracle's layout step (counts, padded offsets, slots, partitions).

The oracle is checked against things other than itself: a separately written
pure-Python brute force over every tiny routing, a library special case
(numpy's stable argsort), the worked examples printed on the Rust EP=2 page,
the invariants the method fixes, and a closed-form statistic.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import ep_inputs
import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_invariants(idx, lay, E, A, C=0, P=1):
    idx = np.asarray(idx)
    T, K = idx.shape
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    count = lay.count.astype(np.int64)
    # total pairs = T*K minus the -1 entries
    assert count.sum() == valid.sum() == T * K - (flat == -1).sum() - ((flat < -1) | (flat >= E)).sum()
    np.testing.assert_array_equal(count, np.bincount(flat[valid], minlength=E))
    off = lay.offset.astype(np.int64)
    if C == 0:
        padded = np.diff(off)
        assert (padded % A == 0).all()
        assert ((padded - count >= 0) & (padded - count < A)).all()
        assert ((padded == 0) == (count == 0)).all()
        if A == 1:
            np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(count)]))
    else:
        np.testing.assert_array_equal(off, np.arange(E + 1) * C)
    dst = lay.dst.ravel().astype(np.int64)
    kept = dst >= 0
    # every kept slot lies in its expert's segment, below offset + count
    e_of = flat[kept]
    assert ((dst[kept] >= off[e_of]) & (dst[kept] < off[e_of] + np.minimum(count[e_of], C or 1 << 40))).all()
    # injective, and src_of_slot o dst = identity
    assert len(np.unique(dst[kept])) == kept.sum()
    src = lay.src_of_slot.astype(np.int64)
    np.testing.assert_array_equal(src[dst[kept]], np.nonzero(kept)[0])
    # image of dst plus padding slots = [0, R), disjoint
    pad = np.nonzero(src < 0)[0]
    assert len(pad) + kept.sum() == lay.R
    assert np.intersect1d(pad, dst[kept]).size == 0
    # partitions
    m = E // P
    part = np.zeros((T, P), np.uint8)
    for t in range(T):
        for e in idx[t]:
            if 0 <= e < E:
                part[t, e // m] = 1
    np.testing.assert_array_equal(lay.in_part, part)
    np.testing.assert_array_equal(lay.tok_per_part, part.sum(axis=0))
    np.testing.assert_array_equal(lay.pairs_per_part, count.reshape(P, m).sum(axis=1))


def _routings(T, K, E):
    ids = list(range(-1, E))
    for flat in itertools.product(ids, repeat=T * K):
        yield [list(flat[t * K:(t + 1) * K]) for t in range(T)]


@pytest.mark.parametrize("T,K,E", [(1, 1, 3), (2, 1, 4), (1, 2, 4), (2, 2, 3), (3, 2, 2), (3, 1, 4)])
def test_brute_force_exhaustive(T, K, E):
    """Every routing with T <= 3, K <= 2, E <= 4 (-1 and duplicates allowed),
    several alignments and partitionings: oracle == brute force."""
    parts = [p for p in (1, 2) if E % p == 0]
    n = 0
    for idx in _routings(T, K, E):
        arr = np.array(idx, dtype=np.int64)
        for A in (1, 2, 3):
            for P in parts:
                b = brute.layout(idx, E, A, P)
                o = oracle.get_layout(arr, E, A, P)
                assert o.R == b["R"] and o.status == b["status"]
                np.testing.assert_array_equal(o.count, b["count"])
                np.testing.assert_array_equal(o.offset, b["offset"])
                np.testing.assert_array_equal(o.dst, np.array(b["dst"]).reshape(T, K))
                np.testing.assert_array_equal(o.src_of_slot, b["src_of_slot"])
                np.testing.assert_array_equal(o.in_part, np.array(b["in_part"]).reshape(T, P))
                np.testing.assert_array_equal(o.tok_per_part, b["tok_per_part"])
                np.testing.assert_array_equal(o.pairs_per_part, b["pairs_per_part"])
                n += 1
    assert n > 0


@pytest.mark.parametrize("C", [1, 2])
def test_brute_force_fixed_capacity(C):
    E, T, K = 3, 3, 2
    for idx in _routings(T, K, E):
        arr = np.array(idx, dtype=np.int64)
        b = brute.layout(idx, E, 1, 1, C)
        o = oracle.get_layout(arr, E, 1, 1, C)
        assert o.R == b["R"] == E * C and o.status == b["status"]
        np.testing.assert_array_equal(o.dst, np.array(b["dst"]).reshape(T, K))
        np.testing.assert_array_equal(o.src_of_slot, b["src_of_slot"])


@pytest.mark.parametrize("T,K,E,A,C", [(2, 2, 3, 2, 0), (3, 1, 4, 3, 0), (2, 2, 3, 1, 2)])
def test_brute_force_receive_rows_cap(T, K, E, A, C):
    """Every routing, with the caller's receive rows below, at and above the
    rows the layout needs: src_of_slot keeps exactly the slots under the cap,
    dst keeps every slot, and the overflow bit is set iff R > cap."""
    n_over = 0
    for idx in _routings(T, K, E):
        arr = np.array(idx, dtype=np.int64)
        R = brute.layout(idx, E, A, 1, C)["R"]
        for cap in sorted({0, 1, max(R - 1, 0), R, R + 3}):
            if C and cap < E * C:
                continue    # a fixed-capacity layout needs all E*C rows (argument error)
            b = brute.layout(idx, E, A, 1, C, rows_cap=cap)
            o = oracle.get_layout(arr, E, A, 1, C, rows_cap=cap)
            assert o.R == b["R"] == R and o.status == b["status"]
            assert bool(o.status & oracle.RECV_OVERFLOW) == (R > cap)
            n_over += R > cap
            np.testing.assert_array_equal(o.dst, np.array(b["dst"]).reshape(T, K))
            np.testing.assert_array_equal(o.src_of_slot, b["src_of_slot"])
            assert len(o.src_of_slot) == min(R, cap)
    assert n_over > 0 or C


def test_bad_expert_ids_flagged_and_ignored():
    idx = np.array([[0, 5], [-2, 1], [1, -1]], np.int64)
    o = oracle.get_layout(idx, 4, 1)
    assert o.status & oracle.BAD_EXPERT
    np.testing.assert_array_equal(o.count, [1, 2, 0, 0])
    np.testing.assert_array_equal(o.dst, [[0, -1], [-1, 1], [2, -1]])


def test_stable_argsort_special_case():
    """A=1: the slot order is numpy's stable argsort of the valid pairs by
    expert id (a library routine)."""
    w = ep_inputs.make_workload("prefill", T=512, H=8, with_x=False)
    flat = w.topk_idx.ravel()
    valid = np.nonzero(flat >= 0)[0]
    order = valid[np.argsort(flat[valid], kind="stable")]
    o = oracle.get_layout(w.topk_idx, w.num_experts, 1)
    dst = o.dst.ravel()
    np.testing.assert_array_equal(dst[order], np.arange(len(order)))
    # with A = 128: slot = offset[e] + position of the pair inside e's run
    o128 = oracle.get_layout(w.topk_idx, w.num_experts, 128)
    e_sorted = flat[order]
    first = np.searchsorted(e_sorted, e_sorted, side="left")
    expect = o128.offset[e_sorted] + (np.arange(len(order)) - first)
    np.testing.assert_array_equal(o128.dst.ravel()[order], expect)


@pytest.mark.parametrize("name", list(ep_inputs.WORKLOADS))
def test_invariants_all_workloads(name):
    w = ep_inputs.make_workload(name, with_x=False)
    o = oracle.get_layout(w.topk_idx, w.num_experts, w.expert_alignment, w.num_partitions,
                          w.capacity)
    assert o.status == 0
    _check_invariants(w.topk_idx, o, w.num_experts, w.expert_alignment, w.capacity,
                      w.num_partitions)
    assert o.R <= w.worst_case_recv_rows()


def test_prefill_workload_shape():
    """The prefill workload's seed-0 statistics (a drift check of the generator)."""
    w = ep_inputs.make_workload("prefill", with_x=False)
    o = oracle.get_layout(w.topk_idx, 256, 128)
    frac_drop = (w.topk_idx == -1).mean()
    assert 0.015 < frac_drop < 0.025
    assert 120 < (o.count == 0).sum() < 180
    assert 35000 < o.R < 48000


def test_rust_page_examples():
    """The worked examples printed on the Rust EP=2 routing page: E = 512,
    partitions [0,256) and [256,512); each partition's pairs in (t, k) order."""
    with open(os.path.join(GOLDEN, "ep_dispatch_rs_examples.json")) as f:
        gold = json.load(f)
    for ex in gold["examples"]:
        T, K = ex["num_tokens"], ex["top_k"]
        idx = np.array(ex["indices"], np.int64).reshape(T, K)
        wts = np.array(ex["weights"], np.float32).reshape(T, K)
        o = oracle.get_layout(idx, 512, 1, 2)
        local = 0 if ex["local_start"] == 0 else 1
        lists = {}
        for side, q in (("local", local), ("remote", 1 - local)):
            lo, hi = o.offset[q * 256], o.offset[(q + 1) * 256]
            flat = np.nonzero((o.dst.ravel() >= lo) & (o.dst.ravel() < hi))[0]
            flat.sort()
            lists[side + "_count"] = len(flat)
            lists[side + "_token_indices"] = (flat // K).tolist()
            lists[side + "_expert_ids"] = idx.ravel()[flat].tolist()
            lists[side + "_weights"] = wts.ravel()[flat].tolist()
            assert o.pairs_per_part[q] == len(flat)
        lists["total_count"] = lists["local_count"] + lists["remote_count"]
        for key, val in ex["printed"].items():
            if key.endswith("weights"):
                np.testing.assert_allclose(lists[key], val, rtol=1e-7)
            else:
                assert lists[key] == val, (ex["name"], key)
        d = ex.get("derived")
        if d:
            np.testing.assert_array_equal(o.in_part, d["is_token_in_partition"])
            np.testing.assert_array_equal(o.tok_per_part, d["num_tokens_per_partition"])
            o1 = oracle.get_layout(idx, 512, 1, 1)
            np.testing.assert_array_equal(o1.dst, d["dst_A1"])
            np.testing.assert_array_equal(o1.src_of_slot, d["src_of_slot_A1"])
            _, _, rw = oracle.dispatch(np.zeros((T, 8), np.uint16), o1, wts)
            np.testing.assert_allclose(rw, d["recv_weights_A1"], rtol=1e-7)
            o4 = oracle.get_layout(idx, 512, 4, 1)
            np.testing.assert_array_equal(o4.dst, d["dst_A4"])
            assert o4.R == d["R_A4"]


def test_partition_hit_rate_closed_form():
    """Uniform distinct top-8 of 256 experts, 32 partitions of 8: a token hits a
    given partition with probability 1 - C(248,8)/C(256,8) (hypergeometric)."""
    w = ep_inputs.make_workload("decode", T=16384, H=8, with_x=False)
    o = oracle.get_layout(w.topk_idx, 256, 1, 32)
    p = 1 - math.comb(248, 8) / math.comb(256, 8)
    est = o.in_part.mean()
    sd = math.sqrt(p * (1 - p) / (16384 * 32))
    assert abs(est - p) < 6 * sd + 2e-3
    assert abs(o.in_part.sum(axis=1).mean() - 32 * p) < 0.05


def test_empty_and_all_dropped():
    o = oracle.get_layout(np.zeros((0, 4), np.int64), 8, 128)
    assert o.R == 0 and o.count.sum() == 0
    o = oracle.get_layout(np.full((5, 3), -1, np.int64), 8, 4, 2)
    assert o.R == 0 and (o.dst == -1).all() and o.in_part.sum() == 0


def test_invalid_arguments():
    idx = np.zeros((2, 2), np.int64)
    with pytest.raises(ValueError):
        oracle.get_layout(idx, 6, 1, 4)          # E % P != 0
    with pytest.raises(ValueError):
        oracle.get_layout(idx, 6, 0)             # A < 1
    with pytest.raises(ValueError):
        oracle.get_layout(idx, 6, 4, 1, 6)       # C % A != 0
