"""GPU parity of the partition-major layout (one receive segment per
partition, its pairs in (t, k) order): ep_get_layout and
ep_dispatch_with_layout against the oracle bit for bit, and dispatch,
combine and the two-level combine over it."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_bits, bf16_to_dev, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check(lay, ref):
    torch.cuda.synchronize()
    assert int(lay.status.item()) == ref.status
    np.testing.assert_array_equal(lay.num_tokens_per_expert.cpu().numpy(), ref.count)
    np.testing.assert_array_equal(lay.expert_offset.cpu().numpy(), ref.offset)
    np.testing.assert_array_equal(lay.dst_slot.cpu().numpy(), ref.dst)
    n = min(ref.R, lay.max_recv_rows)
    np.testing.assert_array_equal(lay.src_of_slot[:n].cpu().numpy(), ref.src_of_slot[:n])
    np.testing.assert_array_equal(lay.is_token_in_partition.cpu().numpy(), ref.in_part)
    np.testing.assert_array_equal(lay.num_tokens_per_partition.cpu().numpy(), ref.tok_per_part)


@pytest.mark.parametrize("T,K,E,A,P,C,drop", [
    (4096, 8, 256, 128, 32, 0, 0.02),   # prefill shape, 32 partitions
    (1000, 6, 64, 3, 4, 0, 0.1),        # ragged tile tail
    (32, 8, 512, 1, 4, 0, 0.05),        # 256 pairs: one-workgroup layout
    (33, 8, 512, 1, 4, 0, 0.05),        # 264 pairs: the two kernels
    (9000, 8, 256, 16, 8, 0, 0.05),     # more than 96 tiles: the column scan
    (777, 8, 4096, 2, 64, 0, 0.02),     # largest E, 64 partitions
    (500, 4, 1024, 1, 1024, 0, 0.0),    # one expert per partition: the expert-major layout
    (300, 4, 64, 4, 8, 96, 0.1),        # fixed capacity, some partitions over it
    (0, 8, 256, 1, 8, 0, 0.0),
])
def test_partition_major_layout_both_paths(gpu, T, K, E, A, P, C, drop):
    announce("partition-major layout", T, K, E, A, P, C)
    rng = ep_inputs.make_rng(T * 3 + P)
    idx, wts = ep_inputs.routing_uniform(rng, T, E, K)
    idx[rng.random((T, K)) < drop] = -1
    lay = gpu.ep_get_layout(to_dev(idx), E, A, P, C, partition_major=True)
    assert lay.num_segments == P and lay.num_tokens_per_expert.numel() == P
    ref = oracle.get_layout(idx, E, A, P, C, rows_cap=lay.max_recv_rows, partition_major=True)
    _check(lay, ref)
    H = 64
    xb = ep_inputs.bf16_normal(rng, (T, H))
    lay2, recv, _, rw = gpu.ep_dispatch_with_layout(bf16_to_dev(xb), to_dev(idx), E, A, to_dev(wts),
                                                    P, C, zero_padding=True, partition_major=True)
    _check(lay2, ref)
    exp, _, exp_w = oracle.dispatch(xb, ref, wts, zero_padding=True)
    R = min(ref.R, lay2.max_recv_rows)
    np.testing.assert_array_equal(bf16_bits(recv[:R]), exp[:R])
    np.testing.assert_array_equal(rw[:R].cpu().numpy(), exp_w[:R])


def test_partition_major_prefill_rows_and_combines(gpu):
    """The prefill workload with 32 partitions in partition-major order: every
    receive row, the combine bitwise against the oracle, and the two-level
    combine equal bit for bit to the one over the expert-major layout."""
    w = ep_inputs.make_workload("prefill")
    T, H, E, K, A, P = w.num_tokens, w.hidden, w.num_experts, w.num_topk, w.expert_alignment, 32
    idx, wts = to_dev(w.topk_idx), to_dev(w.topk_weights)
    x = bf16_to_dev(w.x)
    announce("partition-major prefill")
    lay, recv, _, _ = gpu.ep_dispatch_with_layout(x, idx, E, A, wts, P, partition_major=True)
    ref = oracle.get_layout(w.topk_idx, E, A, P, rows_cap=lay.max_recv_rows, partition_major=True)
    _check(lay, ref)
    src = torch.from_numpy(ref.src_of_slot.astype(np.int64)).to(DEV)
    used = src >= 0
    assert torch.equal(recv[:ref.R][used].view(torch.int16), x.view(torch.int16)[src[used] // K])
    y = ep_inputs.make_y(w.rng, ref.R, H)
    yd = bf16_to_dev(y)
    out, _ = gpu.ep_combine(yd, lay, wts)
    np.testing.assert_array_equal(bf16_bits(out), oracle.combine_f32(y, ref.dst, w.topk_weights))
    red = gpu.ep_combine_reduced(yd, lay, idx, wts)
    np.testing.assert_array_equal(bf16_bits(red),
                                  oracle.combine_reduced_f32(y, w.topk_idx, ref.dst, E, P,
                                                             w.topk_weights))
    # the same rows moved into the expert-major layout give the same bits
    lay_e = gpu.ep_get_layout(idx, E, A, P)
    ref_e = oracle.get_layout(w.topk_idx, E, A, P)
    y_e = np.zeros((lay_e.max_recv_rows, H), np.uint16)
    kept = ref.dst.ravel() >= 0
    y_e[ref_e.dst.ravel()[kept]] = y[ref.dst.ravel()[kept]]
    red_e = gpu.ep_combine_reduced(bf16_to_dev(y_e), lay_e, idx, wts)
    assert torch.equal(red.view(torch.int16), red_e.view(torch.int16))
    assert lay.check() == 0
