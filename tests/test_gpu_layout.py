"""GPU parity of ep_get_layout against the oracle: bit-exact counts,
offsets, slot map, inverse map, partitions and status bits."""
import itertools

import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu


def _compare(ep, idx, E, A=1, P=1, C=0, rows=None, stats=None):
    announce("layout", idx.shape, E, A, P, C, rows)
    lay = ep.ep_get_layout(to_dev(idx), E, A, P, C, max_recv_rows=rows,
                           cumulative_expert_stats=stats)
    ref = oracle.get_layout(idx, E, A, P, C, rows_cap=lay.max_recv_rows)
    torch.cuda.synchronize()
    assert int(lay.status.item()) == ref.status
    np.testing.assert_array_equal(lay.num_tokens_per_expert.cpu().numpy(), ref.count)
    np.testing.assert_array_equal(lay.expert_offset.cpu().numpy(), ref.offset)
    np.testing.assert_array_equal(lay.dst_slot.cpu().numpy(), ref.dst)
    n = min(ref.R, lay.max_recv_rows)
    np.testing.assert_array_equal(lay.src_of_slot[:n].cpu().numpy(), ref.src_of_slot[:n])
    np.testing.assert_array_equal(lay.is_token_in_partition.cpu().numpy(), ref.in_part)
    np.testing.assert_array_equal(lay.num_tokens_per_partition.cpu().numpy(), ref.tok_per_part)
    return lay, ref


@pytest.mark.parametrize("name", list(ep_inputs.WORKLOADS))
def test_layout_workloads_full_size(gpu, name):
    w = ep_inputs.make_workload(name, with_x=False)
    _compare(gpu, w.topk_idx, w.num_experts, w.expert_alignment, w.num_partitions, w.capacity)


@pytest.mark.parametrize("T,K,E,A,P,drop", [
    (1000, 6, 64, 3, 4, 0.1),      # several tiles, ragged tail
    (1, 1, 1, 1, 1, 0.0),
    (3, 8, 256, 128, 32, 0.3),
    (777, 8, 4096, 2, 64, 0.02),   # largest E; 64-bit partition masks
    # tile rows of 513..1024 column quads: one partial per column in the slots
    # kernel's column sums, with threads past the first span holding none
    (150, 8, 2048, 4, 1, 0.1),     # 513 quads
    (600, 8, 3000, 1, 8, 0.05),    # 753 quads
    (300, 4, 4080, 1, 4, 0.0),     # 1,022 quads
    (700, 8, 1500, 2, 4, 0.05),    # 377 quads: two partials per column
    (513, 4, 256, 16, 128, 0.05),  # more than 64 partitions
    (2049, 1, 7, 5, 7, 0.0),       # K = 1, odd E
    (300, 64, 512, 1, 2, 0.5),     # K = 64: a token fills a whole wave chunk
    (40, 200, 1024, 7, 8, 0.2),    # K > 64
    (9, 256, 4096, 3, 64, 0.1),    # largest K with the largest E
    (1, 256, 512, 1, 8, 0.0),      # largest K in one workgroup (256 pairs)
    (32, 8, 512, 1, 4, 0.05),      # 256 pairs, the largest one-workgroup batch
    (33, 8, 512, 1, 4, 0.05),      # 264 pairs: the two-kernel path again
    (9000, 8, 256, 16, 32, 0.05),  # 141 tiles: the tile rows scanned once, ragged tail
    (20000, 4, 64, 1, 8, 0.1),     # 157 tiles, few experts
    (200000, 8, 256, 128, 32, 0.02),  # 1,563 tiles: runs of 7 tiles per scan thread
    (300000, 8, 256, 1, 8, 0.02),  # 2,344 tiles: past the scan's 2,048, reduced per tile
])
def test_layout_shapes(gpu, T, K, E, A, P, drop):
    rng = ep_inputs.make_rng(T * 7 + K)
    idx, _ = ep_inputs.routing_uniform(rng, T, E, K)
    idx[rng.random((T, K)) < drop] = -1
    _compare(gpu, idx, E, A, P)


def test_layout_duplicates_and_hot_expert(gpu):
    """Duplicate ids inside a token and one expert taking most pairs."""
    rng = ep_inputs.make_rng(5)
    idx = rng.integers(0, 32, size=(3000, 8)).astype(np.int64)
    idx[rng.random((3000, 8)) < 0.7] = 3
    _compare(gpu, idx, 32, 128, 4)


def test_layout_brute_force_tiny_all_routings(gpu):
    """Every routing of 2 tokens x 2 slots over 3 experts (with -1)."""
    for flat in itertools.product(range(-1, 3), repeat=4):
        idx = np.array(flat, np.int64).reshape(2, 2)
        for A in (1, 2):
            _compare(gpu, idx, 3, A, 1)


def test_layout_fixed_capacity_and_overflow(gpu):
    w = ep_inputs.make_workload("decode", with_x=False)
    _compare(gpu, w.topk_idx, 256, 1, 1, 128)
    # capacity 4 is too small for some experts: pairs past it are dropped
    _, ref = _compare(gpu, w.topk_idx, 256, 1, 1, 4)
    assert ref.status & oracle.CAPACITY
    _compare(gpu, w.topk_idx, 256, 2, 1, 8)


def test_layout_bad_expert_ids(gpu):
    idx = np.array([[0, 5, 9], [-2, 1, -1], [1, 300, 2]], np.int64)
    lay, ref = _compare(gpu, idx, 8, 2, 2)
    assert ref.status & oracle.BAD_EXPERT
    with pytest.raises(ValueError):
        lay.check()


def test_layout_recv_overflow_flag(gpu):
    w = ep_inputs.make_workload("prefill", T=256, with_x=False)
    _, ref = _compare(gpu, w.topk_idx, 256, 128, 1, 0, rows=1000)
    assert ref.status & oracle.RECV_OVERFLOW


def test_layout_empty_and_all_dropped(gpu):
    _compare(gpu, np.zeros((0, 8), np.int64), 256, 128, 32)
    _compare(gpu, np.full((100, 4), -1, np.int64), 16, 8, 2)
    _compare(gpu, np.zeros((0, 2), np.int64), 4, 1, 1, 3)


def test_layout_cumulative_stats_accumulate(gpu):
    w = ep_inputs.make_workload("prefill", T=512, with_x=False)
    stats = torch.full((256,), 5, dtype=torch.int32, device="cuda:0")
    _, ref = _compare(gpu, w.topk_idx, 256, 128, stats=stats)
    _compare(gpu, w.topk_idx, 256, 128, stats=stats)
    np.testing.assert_array_equal(stats.cpu().numpy(), 5 + 2 * ref.count)


def test_layout_deterministic_and_reusable(gpu):
    w = ep_inputs.make_workload("skewed", T=8192, with_x=False)
    idx = to_dev(w.topk_idx)
    a = gpu.ep_get_layout(idx, 256, 128, 32)
    d0 = a.dst_slot.clone()
    gpu.ep_get_layout(idx, 256, 128, 32, layout=a)
    assert torch.equal(d0, a.dst_slot)
