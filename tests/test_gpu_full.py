"""Full-size workloads in the launch configuration the benchmark times,
compared in full: the layout against the oracle; every receive row on the
device against x gathered by the oracle's inverse slot map (and padding rows
and rows past R against their sentinel); every combine output against the
oracle's ordered fp32 combine bit for bit and against its float64 reference
within rtol = atol = 1e-2."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_bits, bf16_to_dev, fp8_bits, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL16 = 0x7777
SENTINEL8 = 0x5A


def _tiled_y(rng, rows, H, block=8192):
    base = ep_inputs.make_y(rng, min(block, max(rows, 1)), H)
    reps = -(-rows // base.shape[0])
    return np.tile(base, (reps, 1))[:rows]


def _rows_equal_gather(recv_raw, x_raw, src, K, R, sentinel):
    """recv_raw[r] == x_raw[src[r] // K] for every used row r < R, the
    sentinel on padding rows and on every row past R (device compare)."""
    s = torch.from_numpy(np.asarray(src[:R], np.int64)).to(DEV)
    used = s >= 0
    assert torch.equal(recv_raw[:R][used], x_raw[s[used] // K])
    assert bool((recv_raw[:R][~used] == sentinel).all())
    assert bool((recv_raw[R:] == sentinel).all())


def _combine_all(got_bits, y, dst, w, tol=1e-2):
    np.testing.assert_array_equal(got_bits, oracle.combine_f32(y, dst, w))
    f64 = oracle.combine_f64(y, dst, w)
    g = oracle.bf16_to_float(got_bits).astype(np.float64)
    assert np.all(np.abs(g - f64) <= tol + tol * np.abs(f64))


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_full_bf16_dispatch_combine(gpu, name):
    w = ep_inputs.make_workload(name)
    T, H, E, K = w.num_tokens, w.hidden, w.num_experts, w.num_topk
    announce("full", name, "layout")
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), E, w.expert_alignment, w.num_partitions)
    ref = oracle.get_layout(w.topk_idx, E, w.expert_alignment, w.num_partitions)
    np.testing.assert_array_equal(lay.dst_slot.cpu().numpy(), ref.dst)
    np.testing.assert_array_equal(lay.src_of_slot[:ref.R].cpu().numpy(), ref.src_of_slot)
    np.testing.assert_array_equal(lay.expert_offset.cpu().numpy(), ref.offset)
    announce("full", name, "dispatch")
    x = bf16_to_dev(w.x)
    recv = torch.empty((lay.max_recv_rows, H), dtype=torch.int16, device=DEV).fill_(SENTINEL16)
    rw = torch.full((lay.max_recv_rows,), -9.0, device=DEV)
    gpu.ep_dispatch(x, lay, to_dev(w.topk_weights), out=(recv.view(torch.bfloat16), None, rw))
    _rows_equal_gather(recv, x.view(torch.int16), ref.src_of_slot, K, ref.R, SENTINEL16)
    _, _, exp_w = oracle.dispatch(np.zeros((T, 1), np.uint16), ref, w.topk_weights)
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)
    assert bool((rw[ref.R:] == -9.0).all())
    del recv, rw, x
    announce("full", name, "combine")
    y = _tiled_y(w.rng, ref.R, H)
    out, _ = gpu.ep_combine(bf16_to_dev(y), lay, to_dev(w.topk_weights))
    _combine_all(bf16_bits(out), y, ref.dst, w.topk_weights)
    assert lay.check() == 0


def test_full_fp8_dispatches_and_cast(gpu):
    """The fp8 workload: the standalone cast of every token, the fused cast +
    dispatch and the fp8 copy dispatch, every receive row and scale row."""
    w = ep_inputs.make_workload("fp8")
    T, H, K = w.num_tokens, w.hidden, w.num_topk
    G = w.fp8_group
    announce("full fp8 cast")
    x = bf16_to_dev(w.x)
    q_ref, s_ref = oracle.cast_fp8(w.x, G)
    q_all, s_all = gpu.ep_cast_fp8(x, G)
    np.testing.assert_array_equal(fp8_bits(q_all), q_ref)
    np.testing.assert_array_equal(s_all.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), 256, 128)
    ref = oracle.get_layout(w.topk_idx, 256, 128)
    q_dev = torch.from_numpy(q_ref).to(DEV)
    s_dev = torch.from_numpy(s_ref).to(DEV)
    for fused in (True, False):
        announce("full fp8 dispatch", "fused" if fused else "copy")
        recv = torch.empty((lay.max_recv_rows, H), dtype=torch.uint8, device=DEV).fill_(SENTINEL8)
        rs = torch.full((lay.max_recv_rows, H // G), -3.0, device=DEV)
        src = x if fused else (q_all, s_all)
        gpu.ep_dispatch(src, lay, recv_fp8=fused, scale_group=G,
                        out=(recv.view(torch.float8_e4m3fn), rs, None))
        _rows_equal_gather(recv, q_dev, ref.src_of_slot, K, ref.R, SENTINEL8)
        s = torch.from_numpy(ref.src_of_slot.astype(np.int64)).to(DEV)
        used = s >= 0
        assert torch.equal(rs[:ref.R][used].view(torch.int32), s_dev[s[used] // K].view(torch.int32))
        assert bool((rs[:ref.R][~used] == -3.0).all()) and bool((rs[ref.R:] == -3.0).all())
        del recv, rs


def test_full_decode_zero_padding(gpu):
    w = ep_inputs.make_workload("decode")
    announce("full decode")
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), 256, 1, 1, 128)
    ref = oracle.get_layout(w.topk_idx, 256, 1, 1, 128)
    recv = torch.empty((lay.max_recv_rows, w.hidden), dtype=torch.bfloat16, device=DEV)
    recv.view(torch.int16).fill_(SENTINEL16)
    recv, _, _ = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights), zero_padding=True,
                                 out=(recv, None, None))
    exp, _, _ = oracle.dispatch(w.x, ref, w.topk_weights, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv), exp)
    y = ep_inputs.make_y(w.rng, ref.R, w.hidden)
    out, _ = gpu.ep_combine(bf16_to_dev(y), lay, to_dev(w.topk_weights))
    _combine_all(bf16_bits(out), y, ref.dst, w.topk_weights)


def test_full_skewed_partitioned_legs(gpu):
    """The skewed workload's partition layout, its dispatch (every row and
    the per-row routing metadata) and combine, and the two-level combine on
    the expanded layout, in the calls the benchmark times, all in full."""
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
    x = bf16_to_dev(w.x)
    recv = torch.empty((ref.Rp + 16, H), dtype=torch.int16, device=DEV).fill_(SENTINEL16)
    ri = torch.empty((ref.Rp, K), dtype=torch.int64, device=DEV)
    rw = torch.empty((ref.Rp, K), dtype=torch.float32, device=DEV)
    gpu.ep_dispatch_partitioned(x, pl, idx, wts, num_recv_rows=ref.Rp,
                                out=(recv.view(torch.bfloat16), None, ri, rw))
    # row r holds token part_src[r]: gather with K = 1
    _rows_equal_gather(recv, x.view(torch.int16), ref.part_src, 1, ref.Rp, SENTINEL16)
    # metadata from the oracle with one-channel rows (the row bytes are checked above)
    _, _, ri_ref, rw_ref = oracle.dispatch_partitioned(np.zeros((T, 1), np.uint16), w.topk_idx,
                                                       ref, w.topk_weights)
    np.testing.assert_array_equal(ri.cpu().numpy(), ri_ref)
    np.testing.assert_array_equal(rw.cpu().numpy(), rw_ref)
    del recv, ri, rw, x
    announce("full skewed combine_partitioned")
    y = _tiled_y(w.rng, ref.Rp, H)
    out = gpu.ep_combine_partitioned(bf16_to_dev(y), pl)
    got = bf16_bits(out)
    np.testing.assert_array_equal(got, oracle.combine_partitioned_f32(y, ref.token_slot))
    f64 = oracle.combine_partitioned_f64(y, ref.token_slot)
    assert np.all(np.abs(oracle.bf16_to_float(got).astype(np.float64) - f64) <= 1e-2 + 1e-2 * np.abs(f64))
    del y, out, f64
    announce("full skewed combine_reduced")
    lay = gpu.ep_get_layout(idx, E, A, P)
    exp = oracle.get_layout(w.topk_idx, E, A, P)
    y = _tiled_y(w.rng, exp.R, H)
    out = gpu.ep_combine_reduced(bf16_to_dev(y), lay, idx, wts)
    got = bf16_bits(out)
    np.testing.assert_array_equal(
        got, oracle.combine_reduced_f32(y, w.topk_idx, exp.dst, E, P, w.topk_weights))
    f64 = oracle.combine_f64(y, exp.dst, w.topk_weights)
    assert np.all(np.abs(oracle.bf16_to_float(got).astype(np.float64) - f64) <= 1e-2 + 1e-2 * np.abs(f64))
    assert pl.check() == 0 and lay.check() == 0
