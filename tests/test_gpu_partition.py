"""GPU parity of the non-expanded partition layout (token_slot,
partition_offset, num_tokens_per_group), ep_dispatch_partitioned,
ep_combine_partitioned and the two-level ep_combine_reduced against the
oracle: bit-exact for the layout, the rows and the metadata; bitwise equal to
the ordered-fp32 oracle for the combines, and within rtol = atol = 1e-2 of the
float64 reference (the reduced combine with fp32 partials too; with bf16
partials, within the bound they allow, 2^-8 of the result plus the
partials' magnitudes)."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_bits, bf16_to_dev, fp8_bits, fp8_to_dev, to_dev

pytestmark = pytest.mark.gpu

RTOL = ATOL = 1e-2

# (workload, T, K, E, P, G): skewed 8-rank / 4-node shape, uniform prefill,
# one expert per partition, a single partition, ragged tiles, tiny
LAYOUT_CASES = [
    ("skewed", 4096, 8, 256, 32, 8),
    ("prefill", 4096, 8, 256, 8, 0),
    ("prefill", 1025, 6, 64, 64, 16),
    ("prefill", 777, 4, 32, 1, 0),
    ("skewed", 300, 8, 256, 16, 4),
    ("skewed", 12000, 8, 256, 32, 8),   # 188 tiles: the tile rows scanned once
    ("tiny", 3, 2, 4, 2, 1),
    ("prefill", 1, 1, 8, 8, 2),
]


def _routing(name, T, K, E, seed=0):
    w = ep_inputs.make_workload(name, seed=seed, T=T, K=K, E=E, with_x=False,
                                **({} if name == "tiny" else {"A": 1}))
    return w


def _layouts(gpu, idx, E, P, G, A=1):
    lay = gpu.ep_get_layout(to_dev(idx), E, A, num_partitions=P, partition_layout=True,
                            partitions_per_group=G)
    ref = oracle.partition_layout(idx, E, P, G or P)
    return lay, ref


@pytest.mark.parametrize("name,T,K,E,P,G", LAYOUT_CASES)
def test_partition_layout_parity(gpu, name, T, K, E, P, G):
    announce("partition_layout", name, T, K, E, P, G)
    w = _routing(name, T, K, E)
    lay, ref = _layouts(gpu, w.topk_idx, E, P, G)
    torch.cuda.synchronize()
    assert lay.check() == 0
    np.testing.assert_array_equal(lay.is_token_in_partition.cpu().numpy(), ref.in_part)
    np.testing.assert_array_equal(lay.num_tokens_per_partition.cpu().numpy(), ref.tok_per_part)
    np.testing.assert_array_equal(lay.partition_offset.cpu().numpy(), ref.part_offset)
    np.testing.assert_array_equal(lay.token_slot.cpu().numpy(), ref.token_slot)
    np.testing.assert_array_equal(lay.num_tokens_per_group.cpu().numpy(), ref.tok_per_group)
    assert lay.num_partition_rows() == ref.Rp
    np.testing.assert_array_equal(lay.partition_src.cpu().numpy()[:ref.Rp], ref.part_src)
    # the expanded layout beside it is unchanged
    exp = oracle.get_layout(w.topk_idx, E, 1, P)
    np.testing.assert_array_equal(lay.dst_slot.cpu().numpy(), exp.dst)


def test_partition_layout_empty_and_dropped(gpu):
    announce("partition_layout empty")
    idx = np.zeros((0, 4), np.int64)
    lay, ref = _layouts(gpu, idx, 32, 4, 2)
    np.testing.assert_array_equal(lay.partition_offset.cpu().numpy(), np.zeros(5, np.int32))
    np.testing.assert_array_equal(lay.num_tokens_per_group.cpu().numpy(), np.zeros(2, np.int32))
    idx = np.full((70, 3), -1, np.int64)
    idx[::7, 1] = 5
    lay, ref = _layouts(gpu, idx, 32, 4, 2)
    np.testing.assert_array_equal(lay.token_slot.cpu().numpy(), ref.token_slot)
    np.testing.assert_array_equal(lay.partition_offset.cpu().numpy(), ref.part_offset)


def test_partition_layout_with_capacity(gpu):
    """The non-expanded layout counts every routed pair, also those a fixed
    capacity drops from the expanded layout."""
    announce("partition_layout capacity")
    w = _routing("skewed", 2048, 8, 256)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), 256, 1, num_partitions=32, capacity=64,
                            partition_layout=True)
    ref = oracle.partition_layout(w.topk_idx, 256, 32)
    np.testing.assert_array_equal(lay.token_slot.cpu().numpy(), ref.token_slot)


@pytest.mark.parametrize("mode", ["bf16", "fp8", "cast"])
@pytest.mark.parametrize("name,T,K,E,P,H", [
    ("skewed", 1000, 8, 256, 32, 7168), ("prefill", 333, 6, 64, 64, 1024),
    ("prefill", 129, 4, 32, 4, 2048), ("tiny", 3, 2, 4, 2, 128),
    ("prefill", 70, 100, 512, 16, 256),     # K > 64: metadata in two passes
    ("prefill", 70, 30, 512, 16, 256),      # K % 4 != 0: metadata by single stores
])
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("row_order", [True, False])
def test_dispatch_partitioned_parity(gpu, mode, name, T, K, E, P, H, weighted, row_order):
    announce("dispatch_partitioned", mode, name, T, K, E, P, H, weighted, row_order)
    w = ep_inputs.make_workload(name, seed=1, T=T, K=K, E=E, H=H,
                                **({} if name == "tiny" else {"A": 1}))
    lay, ref = _layouts(gpu, w.topk_idx, E, P, 0)
    if not row_order:
        lay.partition_src = None    # metadata written by the token waves instead
    wt = w.topk_weights if weighted else None
    wt_d = to_dev(wt) if weighted else None
    idx_d = to_dev(w.topk_idx)
    G = 128
    if mode == "bf16":
        out = gpu.ep_dispatch_partitioned(bf16_to_dev(w.x), lay, idx_d, wt_d)
        rx, rs, ri, rw = oracle.dispatch_partitioned(w.x, w.topk_idx, ref, wt)
        got = bf16_bits(out[0])[:ref.Rp]
    else:
        codes, scales = oracle.cast_fp8(w.x, G)
        if mode == "fp8":
            out = gpu.ep_dispatch_partitioned((fp8_to_dev(codes), to_dev(scales)), lay, idx_d, wt_d)
        else:
            out = gpu.ep_dispatch_partitioned(bf16_to_dev(w.x), lay, idx_d, wt_d, recv_fp8=True,
                                              scale_group=G)
        rx, rs, ri, rw = oracle.dispatch_partitioned(codes, w.topk_idx, ref, wt, x_scales=scales)
        got = fp8_bits(out[0])[:ref.Rp]
        np.testing.assert_array_equal(out[1].cpu().numpy()[:ref.Rp], rs)
    np.testing.assert_array_equal(got, rx)
    np.testing.assert_array_equal(out[2].cpu().numpy()[:ref.Rp], ri)
    if weighted:
        np.testing.assert_array_equal(out[3].cpu().numpy()[:ref.Rp], rw)
    assert lay.check() == 0


def _check_part(out_bits, y, slot, b0, b1):
    f64 = oracle.combine_partitioned_f64(y, slot, b0, b1)
    got = oracle.bf16_to_float(out_bits).astype(np.float64)
    assert np.all(np.abs(got - f64) <= ATOL + RTOL * np.abs(f64))
    np.testing.assert_array_equal(out_bits, oracle.combine_partitioned_f32(y, slot, b0, b1))


@pytest.mark.parametrize("name,T,K,E,P,H", [
    ("skewed", 4096, 8, 256, 32, 7168), ("prefill", 1025, 6, 64, 64, 1000),
    ("prefill", 65, 4, 32, 1, 256), ("tiny", 3, 2, 4, 2, 8),
])
@pytest.mark.parametrize("bias", [0, 1, 2])
def test_combine_partitioned_parity(gpu, name, T, K, E, P, H, bias):
    announce("combine_partitioned", name, T, K, E, P, H, bias)
    w = _routing(name, T, K, E, seed=2)
    lay, ref = _layouts(gpu, w.topk_idx, E, P, 0)
    y = ep_inputs.make_y(w.rng, ref.Rp, H)
    b = [ep_inputs.bf16_normal(w.rng, (T, H)) for _ in range(bias)]
    out = gpu.ep_combine_partitioned(bf16_to_dev(y) if ref.Rp else
                                     torch.empty((0, H), dtype=torch.bfloat16, device="cuda:0"),
                                     lay, bias=tuple(bf16_to_dev(bb) for bb in b) if b else None)
    _check_part(bf16_bits(out), y, ref.token_slot, *(b + [None] * (2 - len(b))))


def test_partitioned_round_trip(gpu):
    """combine_partitioned(dispatch_partitioned(x)) = x times the number of
    partitions the token reaches (exact in fp32, then one bf16 rounding)."""
    announce("partitioned round trip")
    w = ep_inputs.make_workload("skewed", T=2000, H=4096)
    lay, ref = _layouts(gpu, w.topk_idx, 256, 32, 8)
    recv, _, _, _ = gpu.ep_dispatch_partitioned(bf16_to_dev(w.x), lay, to_dev(w.topk_idx))
    out = gpu.ep_combine_partitioned(recv, lay)
    n = torch.from_numpy(ref.in_part.sum(axis=1).astype(np.float32))[:, None]
    x = torch.from_numpy(w.x.view(np.int16)).view(torch.bfloat16).float()
    expect = (x * n).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits(out), expect)


@pytest.mark.parametrize("name,T,K,E,P,A,H", [
    ("skewed", 4096, 8, 256, 32, 128, 7168), ("prefill", 1000, 8, 256, 8, 128, 2048),
    ("prefill", 333, 6, 64, 64, 4, 1000), ("prefill", 257, 64, 512, 16, 1, 512),
    ("prefill", 129, 4, 32, 1, 1, 256), ("tiny", 3, 2, 4, 2, 1, 8),
])
@pytest.mark.parametrize("bias", [0, 2])
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("b16", [False, True])
def test_combine_reduced_parity(gpu, name, T, K, E, P, A, H, bias, weighted, b16):
    announce("combine_reduced", name, T, K, E, P, A, H, bias, weighted, b16)
    w = ep_inputs.make_workload(name, seed=3, T=T, K=K, E=E, with_x=False,
                                **({} if name == "tiny" else {"A": A, "drop_p": 0.05}))
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), E, A, num_partitions=P)
    exp = oracle.get_layout(w.topk_idx, E, A, P)
    y = ep_inputs.make_y(w.rng, exp.R, H)
    b = [ep_inputs.bf16_normal(w.rng, (T, H)) for _ in range(bias)]
    wt = w.topk_weights if weighted else None
    out = gpu.ep_combine_reduced(bf16_to_dev(y), lay, to_dev(w.topk_idx),
                                 to_dev(wt) if weighted else None,
                                 bias=tuple(bf16_to_dev(bb) for bb in b) if b else None,
                                 bf16_partials=b16)
    bb = b + [None] * (2 - len(b))
    got = bf16_bits(out)
    np.testing.assert_array_equal(
        got, oracle.combine_reduced_f32(y, w.topk_idx, exp.dst, E, P, wt, *bb, bf16_partials=b16))
    f64 = oracle.combine_f64(y, exp.dst, wt, *bb)
    g = oracle.bf16_to_float(got).astype(np.float64)
    if not b16:
        # fp32 partials: the stated tolerance against float64
        assert np.all(np.abs(g - f64) <= 1e-2 + 1e-2 * np.abs(f64))
        return
    # bf16 partials: each partial is rounded to bf16 (relative error 2^-9 of
    # the partial) and so is the result: |got - exact| <= 2^-8 (|exact| + S),
    # S = sum of |w y| + |bias| bounding the sum of the partials' magnitudes.
    absy = y & np.uint16(0x7FFF)                          # |y|: sign bit cleared
    absb = [None if v is None else v & np.uint16(0x7FFF) for v in bb]
    S = oracle.combine_f64(absy, exp.dst, None if wt is None else np.abs(wt), *absb)
    assert np.all(np.abs(g - f64) <= 2.0 ** -8 * (np.abs(f64) + S) + 1e-6)


def test_combine_reduced_with_capacity_drops(gpu):
    """Pairs a fixed capacity dropped (dst_slot = -1) contribute nothing."""
    announce("combine_reduced capacity")
    T, K, E, P, C, H = 1500, 8, 64, 8, 128, 512
    w = ep_inputs.make_workload("skewed", seed=4, T=T, K=K, E=E, with_x=False)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), E, 1, num_partitions=P, capacity=C)
    exp = oracle.get_layout(w.topk_idx, E, 1, P, C)
    assert (exp.dst < 0).sum() > (w.topk_idx < 0).sum()      # some pairs were dropped
    y = ep_inputs.make_y(w.rng, E * C, H)
    out = gpu.ep_combine_reduced(bf16_to_dev(y), lay, to_dev(w.topk_idx), to_dev(w.topk_weights))
    np.testing.assert_array_equal(
        bf16_bits(out), oracle.combine_reduced_f32(y, w.topk_idx, exp.dst, E, P, w.topk_weights))


def test_partition_major_order_and_reduced_combine(gpu):
    """The partition-major receive order (partition, t, k) is the expanded
    layout of topk_idx // (E/P) over P "experts", one per partition; the
    reduced combine over it (routing given as those partition ids) equals, bit
    for bit, the reduced combine over the expert-major layout holding the same
    rows (its partial sums fold each partition's pairs in k order either way)."""
    announce("partition-major order")
    T, K, E, P, H = 1500, 8, 256, 32, 1024
    w = ep_inputs.make_workload("skewed", seed=6, T=T, K=K, E=E, with_x=False)
    m = E // P
    idx_q = np.where(w.topk_idx >= 0, w.topk_idx // m, -1)
    lay_e = gpu.ep_get_layout(to_dev(w.topk_idx), E, 1, num_partitions=P)
    lay_q = gpu.ep_get_layout(to_dev(idx_q), P, 1, num_partitions=P)
    ref_q = oracle.get_layout(idx_q, P, 1)
    dst_q = lay_q.dst_slot.cpu().numpy()
    np.testing.assert_array_equal(dst_q, ref_q.dst)
    # slots in (partition, t, k) order
    pairs = [(idx_q[t, k], t, k) for t in range(T) for k in range(K) if idx_q[t, k] >= 0]
    order = sorted(pairs)
    np.testing.assert_array_equal([dst_q[t, k] for _, t, k in order], np.arange(len(order)))
    # the same expert outputs in both receive orders
    rng = ep_inputs.make_rng(7)
    vals = ep_inputs.bf16_normal(rng, (T * K, H))           # one row per (t, k)
    dst_e = lay_e.dst_slot.cpu().numpy()
    y_e = np.zeros((lay_e.num_recv_rows(), H), np.uint16)
    y_q = np.zeros((lay_q.num_recv_rows(), H), np.uint16)
    for t in range(T):
        for k in range(K):
            if dst_e[t, k] >= 0:
                y_e[dst_e[t, k]] = vals[t * K + k]
                y_q[dst_q[t, k]] = vals[t * K + k]
    out_e = gpu.ep_combine_reduced(bf16_to_dev(y_e), lay_e, to_dev(w.topk_idx), to_dev(w.topk_weights))
    out_q = gpu.ep_combine_reduced(bf16_to_dev(y_q), lay_q, to_dev(idx_q), to_dev(w.topk_weights))
    np.testing.assert_array_equal(bf16_bits(out_e), bf16_bits(out_q))
    np.testing.assert_array_equal(
        bf16_bits(out_q), oracle.combine_reduced_f32(y_q, w.topk_idx, dst_q, E, P, w.topk_weights))


def test_partition_offsets_many_partitions(gpu):
    """Past 64 partitions the layout still gives the partition offsets and the
    group counts (no token_slot): E = 4096 experts, P = 1024, G = 1 and 8."""
    announce("partition offsets P=1024")
    w = ep_inputs.make_workload("prefill", seed=8, T=300, K=8, E=4096, A=1, with_x=False)
    for G in (1, 8):
        lay = gpu.ep_get_layout(to_dev(w.topk_idx), 4096, 1, num_partitions=1024,
                                partition_layout=True, partitions_per_group=G)
        assert lay.token_slot is None
        ref = oracle.partition_layout(w.topk_idx, 4096, 1024, G)
        np.testing.assert_array_equal(lay.partition_offset.cpu().numpy(), ref.part_offset)
        np.testing.assert_array_equal(lay.num_tokens_per_group.cpu().numpy(), ref.tok_per_group)
        np.testing.assert_array_equal(lay.num_tokens_per_partition.cpu().numpy(), ref.tok_per_part)
        np.testing.assert_array_equal(lay.is_token_in_partition.cpu().numpy(), ref.in_part)
        exp = oracle.get_layout(w.topk_idx, 4096, 1, 1024)
        np.testing.assert_array_equal(lay.dst_slot.cpu().numpy(), exp.dst)
