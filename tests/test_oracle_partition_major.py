"""Pins for the oracle's partition-major layout: one receive segment per
partition (partitions standing for the ranks of "DeepEP test target API
reference" sec. 3.1), holding the pairs of its experts in (t, k) order,
padded to expert_alignment or given C rows with a fixed capacity.

* The Rust EP=2 page ("spark_model/layers/ep_dispatch.rs") prints, for each
  rank, its list of (token, expert, weight) entries in token-major then k
  order: with E = 512 split into two partitions those lists are exactly the
  rows of the two segments, in slot order.
* Every routing of up to four pairs over four experts, against a sort by
  (partition, flat index) written here.
* Special cases: P = E is the expert-major layout; P = 1 with A = 1 gives
  each kept pair the number of kept pairs before it.
* Invariants on the skewed workload."""
import itertools
import json
import os

import numpy as np
import pytest

import ep_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_rust_page_lists_are_the_partition_segments():
    with open(os.path.join(GOLDEN, "ep_dispatch_rs_examples.json")) as f:
        gold = json.load(f)
    for ex in gold["examples"]:
        T, K = ex["num_tokens"], ex["top_k"]
        idx = np.array(ex["indices"], np.int64).reshape(T, K)
        wts = np.array(ex["weights"], np.float32).ravel()
        o = oracle.get_layout(idx, 512, 1, 2, partition_major=True)
        assert o.count.shape == (2,) and o.offset.shape == (3,)
        local = 0 if ex["local_start"] == 0 else 1
        got = {}
        for side, q in (("local", local), ("remote", 1 - local)):
            rows = o.src_of_slot[o.offset[q]:o.offset[q + 1]]   # slot order, A = 1: no padding
            got[side + "_count"] = int(o.count[q])
            got[side + "_token_indices"] = (rows // K).tolist()
            got[side + "_expert_ids"] = idx.ravel()[rows].tolist()
            got[side + "_weights"] = wts[rows].tolist()
        got["total_count"] = got["local_count"] + got["remote_count"]
        for key, val in ex["printed"].items():
            if key.endswith("weights"):
                np.testing.assert_allclose(got[key], val, rtol=1e-7)
            else:
                assert got[key] == val, (ex["name"], key)


def _sorted_layout(idx, E, A, P, C):
    """The partition-major layout by sorting: kept pairs ordered by
    (partition, flat index); a segment's rows are its pairs then padding."""
    T, K = idx.shape
    m = E // P
    flat = idx.ravel()
    keep = [p for p in range(T * K) if 0 <= flat[p] < E]
    order = sorted(keep, key=lambda p: (flat[p] // m, p))
    count = [sum(1 for p in keep if flat[p] // m == q) for q in range(P)]
    if C > 0:
        offset = [q * C for q in range(P + 1)]
    else:
        offset = [0]
        for q in range(P):
            offset.append(offset[-1] + -(-count[q] // A) * A)
    dst = [-1] * (T * K)
    rank = [0] * P
    for p in order:
        q = flat[p] // m
        if C == 0 or rank[q] < C:
            dst[p] = offset[q] + rank[q]
        rank[q] += 1
    return count, offset, dst


def test_all_small_routings_against_a_sort():
    E = 4
    n = 0
    for T, K in ((1, 1), (1, 2), (2, 1), (2, 2), (1, 3), (3, 1), (4, 1)):
        for ids in itertools.product(range(-1, E), repeat=T * K):
            idx = np.array(ids, np.int64).reshape(T, K)
            for P, A, C in ((1, 1, 0), (2, 1, 0), (4, 1, 0), (2, 3, 0), (1, 2, 0), (2, 1, 1),
                            (2, 2, 2), (4, 1, 1)):
                count, offset, dst = _sorted_layout(idx, E, A, P, C)
                o = oracle.get_layout(idx, E, A, P, C, partition_major=True)
                assert o.count.tolist() == count, (ids, P, A, C)
                assert o.offset.tolist() == offset, (ids, P, A, C)
                assert o.dst.ravel().tolist() == dst, (ids, P, A, C)
                src = [-1] * offset[-1]
                for p, s in enumerate(dst):
                    if s >= 0:
                        src[s] = p
                assert o.src_of_slot.tolist() == src, (ids, P, A, C)
                over = C > 0 and max(count) > C
                assert bool(o.status & oracle.CAPACITY) == over
                n += 1
    assert n > 5000


def test_one_partition_per_expert_is_the_expert_major_layout():
    rng = ep_inputs.make_rng(41)
    idx, _ = ep_inputs.routing_uniform(rng, 300, 16, 4)
    idx[rng.random(idx.shape) < 0.1] = -1
    for A, C in ((1, 0), (8, 0), (4, 64)):
        a = oracle.get_layout(idx, 16, A, 16, C, partition_major=True)
        b = oracle.get_layout(idx, 16, A, 16, C)
        for key in ("count", "offset", "dst", "src_of_slot", "in_part", "tok_per_part"):
            np.testing.assert_array_equal(a[key], b[key])
        assert a.status == b.status


def test_one_partition_gives_the_rank_among_kept_pairs():
    rng = ep_inputs.make_rng(42)
    idx, _ = ep_inputs.routing_uniform(rng, 200, 64, 6)
    idx[rng.random(idx.shape) < 0.2] = -1
    o = oracle.get_layout(idx, 64, 1, 1, partition_major=True)
    keep = (idx.ravel() >= 0)
    expect = np.where(keep, np.cumsum(keep) - 1, -1)
    np.testing.assert_array_equal(o.dst.ravel(), expect)
    assert o.R == keep.sum() and o.count.tolist() == [keep.sum()]


def test_skewed_workload_invariants():
    w = ep_inputs.make_workload("skewed")
    E, A, P = w.num_experts, w.expert_alignment, w.num_partitions
    o = oracle.get_layout(w.topk_idx, E, A, P, partition_major=True)
    e = oracle.get_layout(w.topk_idx, E, A, P)
    m = E // P
    np.testing.assert_array_equal(o.count, e.pairs_per_part)
    np.testing.assert_array_equal(o.count, e.count.reshape(P, m).sum(1))
    np.testing.assert_array_equal(o.in_part, e.in_part)
    np.testing.assert_array_equal(o.tok_per_part, e.tok_per_part)
    assert np.all(np.diff(o.offset) % A == 0)
    assert np.all(np.diff(o.offset) - o.count < A) and np.all(np.diff(o.offset) >= o.count)
    flat = w.topk_idx.ravel()
    for q in range(P):
        rows = o.src_of_slot[o.offset[q]:o.offset[q] + o.count[q]]
        assert np.all(np.diff(rows) > 0)                  # (t, k) order
        assert np.all(flat[rows] // m == q)               # only this partition's pairs
        assert np.all(o.src_of_slot[o.offset[q] + o.count[q]:o.offset[q + 1]] == -1)


@pytest.mark.parametrize("bad", [-2, 512, 10**9])
def test_bad_ids_are_flagged_and_dropped(bad):
    idx = np.array([[3, bad], [300, 7]], np.int64)
    o = oracle.get_layout(idx, 512, 1, 2, partition_major=True)
    assert o.status & oracle.BAD_EXPERT
    assert o.dst.tolist() == [[0, -1], [2, 1]]
