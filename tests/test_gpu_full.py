"""Full-size workloads in the launch configuration the benchmark times:
layout compared in full, rows and combine outputs compared on sampled
tokens the oracle computes one by one."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_bits, bf16_to_dev, fp8_bits, to_dev

pytestmark = pytest.mark.gpu


def _sample(T, n=256, seed=1):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=min(n, T), replace=False)]))


def _tiled_y(rng, rows, H, block=8192):
    base = ep_inputs.make_y(rng, min(block, rows), H)
    reps = -(-rows // base.shape[0])
    return np.tile(base, (reps, 1))[:rows]


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_full_bf16_dispatch_combine(gpu, name):
    w = ep_inputs.make_workload(name)
    T, H, E = w.num_tokens, w.hidden, w.num_experts
    announce("full", name, "layout")
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), E, w.expert_alignment, w.num_partitions)
    ref = oracle.get_layout(w.topk_idx, E, w.expert_alignment, w.num_partitions)
    np.testing.assert_array_equal(lay.dst_slot.cpu().numpy(), ref.dst)
    announce("full", name, "dispatch")
    recv, _, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights))
    toks = _sample(T)
    for t in toks:
        slots = ref.dst[t][ref.dst[t] >= 0]
        got = bf16_bits(recv[torch.from_numpy(slots.astype(np.int64)).to(recv.device)])
        np.testing.assert_array_equal(got, np.broadcast_to(w.x[t], got.shape))
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy()[ref.src_of_slot >= 0],
                                  w.topk_weights.ravel()[ref.src_of_slot[ref.src_of_slot >= 0]])
    del recv
    announce("full", name, "combine")
    y = _tiled_y(w.rng, ref.R, H)
    out, _ = gpu.ep_combine(bf16_to_dev(y), lay, to_dev(w.topk_weights))
    got = bf16_bits(out)[toks]
    np.testing.assert_array_equal(got, oracle.combine_f32(y, ref.dst, w.topk_weights, tokens=toks))
    f64 = oracle.combine_f64(y, ref.dst, w.topk_weights, tokens=toks)
    g = oracle.bf16_to_float(got).astype(np.float64)
    assert np.all(np.abs(g - f64) <= 1e-2 + 1e-2 * np.abs(f64))
    assert lay.check() == 0


def test_full_fp8_fused_dispatch(gpu):
    w = ep_inputs.make_workload("fp8")
    announce("full fp8")
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), 256, 128)
    ref = oracle.get_layout(w.topk_idx, 256, 128)
    recv, rs, _ = gpu.ep_dispatch(bf16_to_dev(w.x), lay, recv_fp8=True, scale_group=128)
    toks = _sample(w.num_tokens)
    q, s = oracle.cast_fp8(w.x[toks], 128)
    for i, t in enumerate(toks):
        slots = torch.from_numpy(ref.dst[t][ref.dst[t] >= 0].astype(np.int64)).to(recv.device)
        got_q = fp8_bits(recv[slots])
        np.testing.assert_array_equal(got_q, np.broadcast_to(q[i], got_q.shape))
        got_s = rs[slots].cpu().numpy()
        np.testing.assert_array_equal(got_s.view(np.uint32), np.broadcast_to(s[i], got_s.shape).view(np.uint32))
    announce("full fp8 cast")
    q_all, s_all = gpu.ep_cast_fp8(bf16_to_dev(w.x), 128)
    np.testing.assert_array_equal(fp8_bits(q_all)[toks], q)
    np.testing.assert_array_equal(s_all.cpu().numpy()[toks], s)


def test_full_decode_zero_padding(gpu):
    w = ep_inputs.make_workload("decode")
    announce("full decode")
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), 256, 1, 1, 128)
    ref = oracle.get_layout(w.topk_idx, 256, 1, 1, 128)
    recv = torch.empty((lay.max_recv_rows, w.hidden), dtype=torch.bfloat16, device="cuda:0")
    recv.view(torch.int16).fill_(0x7777)
    recv, _, _ = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights), zero_padding=True,
                                 out=(recv, None, None))
    exp, _, _ = oracle.dispatch(w.x, ref, w.topk_weights, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv), exp)
    y = ep_inputs.make_y(w.rng, ref.R, w.hidden)
    out, _ = gpu.ep_combine(bf16_to_dev(y), lay, to_dev(w.topk_weights))
    np.testing.assert_array_equal(bf16_bits(out), oracle.combine_f32(y, ref.dst, w.topk_weights))


def test_full_skewed_partitioned_legs(gpu):
    """The skewed workload's partition layout (compared in full), its
    dispatch (rows on sampled tokens, per-row routing metadata in full) and
    combine, and the two-level combine on the expanded layout, in the calls
    the benchmark times."""
    w = ep_inputs.make_workload("skewed")
    T, H, E, K, P, A = (w.num_tokens, w.hidden, w.num_experts, w.num_topk, w.num_partitions,
                        w.expert_alignment)
    idx = to_dev(w.topk_idx)
    wts = to_dev(w.topk_weights)
    announce("full skewed partition layout")
    pl = gpu.ep_get_layout(idx, E, A, P, w.capacity, partition_layout=True)
    ref = oracle.partition_layout(w.topk_idx, E, P)
    np.testing.assert_array_equal(pl.token_slot.cpu().numpy(), ref.token_slot)
    np.testing.assert_array_equal(pl.partition_offset.cpu().numpy(), ref.part_offset)
    np.testing.assert_array_equal(pl.partition_src[:ref.Rp].cpu().numpy(), ref.part_src)
    assert pl.num_partition_rows() == ref.Rp
    announce("full skewed dispatch_partitioned")
    recv, _, ri, rw = gpu.ep_dispatch_partitioned(bf16_to_dev(w.x), pl, idx, wts,
                                                  num_recv_rows=ref.Rp)
    toks = _sample(T)
    for t in toks:
        slots = ref.token_slot[t][ref.token_slot[t] >= 0]
        got = bf16_bits(recv[torch.from_numpy(slots.astype(np.int64)).to(recv.device)])
        np.testing.assert_array_equal(got, np.broadcast_to(w.x[t], got.shape))
    # metadata from the oracle with one-channel rows (the row bytes are checked above)
    _, _, ri_ref, rw_ref = oracle.dispatch_partitioned(np.zeros((T, 1), np.uint16), w.topk_idx,
                                                       ref, w.topk_weights)
    np.testing.assert_array_equal(ri.cpu().numpy(), ri_ref)
    np.testing.assert_array_equal(rw.cpu().numpy(), rw_ref)
    del recv, ri, rw
    announce("full skewed combine_partitioned")
    y = _tiled_y(w.rng, ref.Rp, H)
    out = gpu.ep_combine_partitioned(bf16_to_dev(y), pl)
    np.testing.assert_array_equal(bf16_bits(out)[toks],
                                  oracle.combine_partitioned_f32(y, ref.token_slot, tokens=toks))
    del y, out
    announce("full skewed combine_reduced")
    lay = gpu.ep_get_layout(idx, E, A, P)
    exp = oracle.get_layout(w.topk_idx, E, A, P)
    y = _tiled_y(w.rng, exp.R, H)
    out = gpu.ep_combine_reduced(bf16_to_dev(y), lay, idx, wts)
    np.testing.assert_array_equal(
        bf16_bits(out)[toks],
        oracle.combine_reduced_f32(y, w.topk_idx, exp.dst, E, P, w.topk_weights, tokens=toks))
    assert pl.check() == 0 and lay.check() == 0
