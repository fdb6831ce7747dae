"""GPU parity of ep_dispatch_with_layout: one call that derives the layout
and dispatches, with the slots found by the dispatch kernels.  Every output
(layout buffers, status, cumulative stats, receive rows, scales, weights,
padding) must equal both the oracle and the two calls ep_get_layout +
ep_dispatch, over sentinel-filled buffers."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_to_dev, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bufs(rows, H, fp8, G, weights):
    if fp8:
        rx = torch.empty((rows, H), dtype=torch.uint8, device=DEV).fill_(0x5A).view(torch.float8_e4m3fn)
        rs = torch.full((rows, H // G), -3.0, dtype=torch.float32, device=DEV)
    else:
        rx = torch.empty((rows, H), dtype=torch.int16, device=DEV).fill_(0x7777).view(torch.bfloat16)
        rs = None
    rw = torch.full((rows,), -9.0, dtype=torch.float32, device=DEV) if weights else None
    return rx, rs, rw


def _raw(t):
    return None if t is None else t.contiguous().view(torch.uint8) if t.dtype == torch.float8_e4m3fn \
        else t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t


def _layout_equal(a, b, n_src=None):
    """Every layout buffer equal; src_of_slot on its first n_src entries
    (None: the whole buffer, for buffers filled with a sentinel first)."""
    for name in ("num_tokens_per_expert", "expert_offset", "num_tokens_per_partition",
                 "is_token_in_partition", "dst_slot", "status"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.equal(a.src_of_slot[:n_src], b.src_of_slot[:n_src]), "src_of_slot"


def _run(ep, idx_np, w_np, x, E, A=1, P=1, C=0, rows=None, recv_fp8=False, G=128,
         zero_padding=False, stats=False):
    """Both paths over sentinel-filled buffers; returns (fused layout, fused
    outputs, oracle layout)."""
    T, K = idx_np.shape
    H = x.shape[1] if not isinstance(x, tuple) else x[0].shape[1]
    fp8 = recv_fp8 or isinstance(x, tuple)
    announce("dispatch_with_layout", T, K, E, A, P, C, rows, H, fp8, zero_padding)
    idx = to_dev(idx_np)
    w = to_dev(w_np) if w_np is not None else None
    st_a = torch.full((E,), 3, dtype=torch.int32, device=DEV) if stats else None
    st_b = st_a.clone() if stats else None
    lay_a = ep.ep_get_layout(idx, E, A, P, C, max_recv_rows=rows)
    lay_a.src_of_slot.fill_(-77)
    lay_a = ep.ep_get_layout(idx, E, A, P, C, max_recv_rows=rows, cumulative_expert_stats=st_a,
                             layout=lay_a)
    nrows = lay_a.max_recv_rows
    out_a = _bufs(nrows, H, fp8, G, w is not None)
    ep.ep_dispatch(x, lay_a, w, recv_fp8=recv_fp8, scale_group=G, zero_padding=zero_padding,
                   out=out_a)
    # the fused call writes into a layout whose buffers hold garbage first
    lay_b = ep.Layout(lay_a.params, idx.device)
    for t in (lay_b.num_tokens_per_expert, lay_b.expert_offset, lay_b.dst_slot,
              lay_b.num_tokens_per_partition):
        t.fill_(-55)
    lay_b.src_of_slot.fill_(-77)
    lay_b.is_token_in_partition.fill_(9)
    out_b = _bufs(nrows, H, fp8, G, w is not None)
    res = ep.ep_dispatch_with_layout(x, idx, E, A, w, P, C, max_recv_rows=rows,
                                     cumulative_expert_stats=st_b, layout=lay_b,
                                     recv_fp8=recv_fp8, scale_group=G,
                                     zero_padding=zero_padding, out=out_b)
    assert res[0] is lay_b
    torch.cuda.synchronize()
    _layout_equal(lay_a, lay_b)
    for i, (ta, tb) in enumerate(zip(out_a, out_b)):
        if ta is not None:
            assert torch.equal(_raw(ta), _raw(tb)), f"output {i}"
    if stats:
        assert torch.equal(st_a, st_b)
    ref = oracle.get_layout(idx_np, E, A, P, C, rows_cap=nrows)
    assert int(lay_b.status.item()) == ref.status
    np.testing.assert_array_equal(lay_b.dst_slot.cpu().numpy(), ref.dst)
    np.testing.assert_array_equal(lay_b.expert_offset.cpu().numpy(), ref.offset)
    n = min(ref.R, nrows)
    np.testing.assert_array_equal(lay_b.src_of_slot[:n].cpu().numpy(), ref.src_of_slot[:n])
    assert bool((lay_b.src_of_slot[n:] == -77).all())
    return lay_b, out_b, ref


def _check_rows_on_device(recv, x, ref, K, zero_padding=False, sentinel=0x7777):
    """recv rows against x gathered by the oracle's src_of_slot, on the device:
    every used row, every padding row (zeros, or the untouched sentinel) and
    every row past R."""
    R = min(ref.R, recv.shape[0])
    src = torch.from_numpy(ref.src_of_slot[:R].astype(np.int64)).to(DEV)
    used = src >= 0
    r16 = recv.view(torch.int16)
    x16 = x.view(torch.int16)
    assert torch.equal(r16[:R][used], x16[src[used] // K])
    pad = r16[:R][~used]
    assert bool((pad == (0 if zero_padding else sentinel)).all())
    assert bool((r16[R:] == sentinel).all())


def _prefill_like(T, seed=0):
    rng = ep_inputs.make_rng(seed)
    idx, w = ep_inputs.routing_prefill(rng, T, 256, 8)
    return idx, w


def test_with_layout_prefill_full_size(gpu):
    """The benchmark's workload in its launch configuration: every receive
    row compared on the device, the layout in full."""
    w = ep_inputs.make_workload("prefill")
    x = bf16_to_dev(w.x)
    lay, (recv, _, rw), ref = _run(gpu, w.topk_idx, w.topk_weights, x, 256, 128)
    _check_rows_on_device(recv, x, ref, 8)
    exp_w = np.zeros(ref.R, np.float32)
    used = ref.src_of_slot >= 0
    exp_w[used] = w.topk_weights.ravel()[ref.src_of_slot[used]]
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)
    assert lay.check() == 0


def test_with_layout_skewed_full_size(gpu):
    """T = 32,768 with Zipf routing: many count tiles and the resident
    grid's stride loop over several token groups per wave."""
    w = ep_inputs.make_workload("skewed")
    x = bf16_to_dev(w.x)
    lay, (recv, _, _), ref = _run(gpu, w.topk_idx, w.topk_weights, x, 256, 128)
    _check_rows_on_device(recv, x, ref, 8)


@pytest.mark.parametrize("T,K,E,A,H,drop", [
    (64, 2, 8, 1, 256, 0.0),       # one workgroup for the whole layout
    (1000, 6, 64, 3, 1000, 0.1),   # ragged tile tail, H not a multiple of 64 vectors
    (2049, 1, 7, 5, 16, 0.0),      # K = 1, one vector per row
    (300, 64, 512, 1, 64, 0.5),    # a token fills a wave's pair chunk
    (40, 100, 1024, 7, 128, 0.2),  # K > 64: two passes of 64 destinations
    (33, 8, 512, 1, 7168, 0.05),   # 264 pairs: just past the one-workgroup batch
    (9000, 8, 256, 16, 2048, 0.05),  # many tiles, ragged tail
    (5, 3, 4, 2, 8, 0.0),
    (150, 8, 2048, 4, 256, 0.1),   # E > 1024: 4-wave count workgroups, slots still derived
    (2000, 8, 2048, 1, 128, 0.0),  # tile rows beyond the row kernels' LDS: two-kernel layout
    (16387, 4, 64, 2, 256, 0.05),  # token queue, XCD ranges of unequal length
])
def test_with_layout_shapes(gpu, T, K, E, A, H, drop):
    rng = ep_inputs.make_rng(T * 13 + K)
    idx, wt = ep_inputs.routing_uniform(rng, T, E, K)
    idx[rng.random((T, K)) < drop] = -1
    xb = ep_inputs.bf16_normal(rng, (T, H))
    x = bf16_to_dev(xb)
    lay, (recv, _, rw), ref = _run(gpu, idx, wt, x, E, A)
    exp, _, exp_w = oracle.dispatch(xb, ref, wt)
    got = recv[:ref.R].view(torch.int16).cpu().numpy().view(np.uint16)
    used = ref.src_of_slot >= 0
    np.testing.assert_array_equal(got[used], exp[used])
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)


@pytest.mark.parametrize("fmt", ["fp32", "pow2", "ue8m0"])
def test_with_layout_fused_cast(gpu, fmt):
    idx, wt = _prefill_like(700, seed=3)
    rng = ep_inputs.make_rng(4)
    xb = ep_inputs.bf16_normal(rng, (700, 1024))
    x = bf16_to_dev(xb)
    announce("with_layout fused cast", fmt)
    lay_a = gpu.ep_get_layout(to_dev(idx), 256, 128)
    a = gpu.ep_dispatch(x, lay_a, to_dev(wt), recv_fp8=True, scale_group=128, scale_fmt=fmt)
    lay_b, *b = gpu.ep_dispatch_with_layout(x, to_dev(idx), 256, 128, to_dev(wt), recv_fp8=True,
                                            scale_group=128, scale_fmt=fmt)
    R = lay_a.num_recv_rows()
    _layout_equal(lay_a, lay_b, min(R, lay_a.max_recv_rows))
    ref = oracle.get_layout(idx, 256, 128)
    used = torch.from_numpy(ref.src_of_slot >= 0).to(DEV)
    assert torch.equal(a[0][:R].view(torch.uint8)[used], b[0][:R].view(torch.uint8)[used])
    assert torch.equal(a[1][:R][used], b[1][:R][used])
    assert torch.equal(a[2][:R], b[2][:R])
    # and the codes against the oracle's cast of each row's token
    if fmt == "fp32":
        q, s = oracle.cast_fp8(xb, 128)
    else:
        q, s32, e8 = oracle.cast_fp8_pow2(xb, 128, ue8m0=fmt == "ue8m0")
        s = e8 if fmt == "ue8m0" else s32
    src = ref.src_of_slot
    t_of = src[src >= 0] // 8
    np.testing.assert_array_equal(b[0][:R].view(torch.uint8).cpu().numpy()[src >= 0], q[t_of])
    np.testing.assert_array_equal(b[1][:R].cpu().numpy()[src >= 0], s[t_of])


def test_with_layout_fp8_copy_and_zero_padding(gpu):
    idx, wt = _prefill_like(500, seed=5)
    rng = ep_inputs.make_rng(6)
    xb = ep_inputs.bf16_normal(rng, (500, 2048))
    q, s = oracle.cast_fp8(xb, 128)
    x8 = (torch.from_numpy(q).to(DEV).view(torch.float8_e4m3fn), to_dev(s))
    _, (recv, rs, _), ref = _run(gpu, idx, wt, x8, 256, 128, G=128, zero_padding=True)
    exp, exp_s, _ = oracle.dispatch(q, ref, wt, x_scales=s, zero_padding=True)
    np.testing.assert_array_equal(recv[:ref.R].view(torch.uint8).cpu().numpy(), exp)
    np.testing.assert_array_equal(rs[:ref.R].cpu().numpy(), exp_s)


@pytest.mark.parametrize("zero_padding", [False, True])
def test_with_layout_fp8_copy_token_queue(gpu, zero_padding):
    """fp8 rows with fp32 scales at T >= 16,384: the queue kernel's fp8 copy
    (scale rows held in registers), padding workgroups appended to it."""
    T, H, G = 16400, 512, 128
    idx, wt = _prefill_like(T, seed=31)
    xb = ep_inputs.bf16_normal(ep_inputs.make_rng(32), (T, H))
    q, s = oracle.cast_fp8(xb, G)
    x8 = (torch.from_numpy(q).to(DEV).view(torch.float8_e4m3fn), to_dev(s))
    _, (recv, rs, rw), ref = _run(gpu, idx, wt, x8, 256, 128, G=G, zero_padding=zero_padding)
    exp, exp_s, exp_w = oracle.dispatch(q, ref, wt, x_scales=s, zero_padding=zero_padding)
    used = ref.src_of_slot >= 0
    rows = slice(None) if zero_padding else used
    np.testing.assert_array_equal(recv[:ref.R].view(torch.uint8).cpu().numpy()[rows], exp[rows])
    np.testing.assert_array_equal(rs[:ref.R].cpu().numpy()[rows], exp_s[rows])
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)


def test_with_layout_token_queue_fixed_capacity(gpu):
    """The queue kernel with a fixed capacity: pairs past C dropped (status
    bit), every expert's unused rows visited by the padding workgroups."""
    T, K, E, C, H = 16500, 2, 64, 512, 64
    rng = ep_inputs.make_rng(33)
    idx, wt = ep_inputs.routing_uniform(rng, T, E, K)
    xb = ep_inputs.bf16_normal(rng, (T, H))
    _, (recv, _, rw), ref = _run(gpu, idx, wt, bf16_to_dev(xb), E, 1, 1, C, zero_padding=True)
    assert ref.status & oracle.CAPACITY
    exp, _, exp_w = oracle.dispatch(xb, ref, wt, zero_padding=True)
    np.testing.assert_array_equal(recv.view(torch.int16).cpu().numpy().view(np.uint16), exp)
    np.testing.assert_array_equal(rw.cpu().numpy(), exp_w)


def test_with_layout_decode_fixed_capacity(gpu):
    """Fixed capacity with zero padding, mostly padding: the region is zero
    filled first; src_of_slot's padding comes from the padding workgroups."""
    w = ep_inputs.make_workload("decode")
    x = bf16_to_dev(w.x)
    _, (recv, _, rw), ref = _run(gpu, w.topk_idx, w.topk_weights, x, 256, 1, 1, 128,
                                 zero_padding=True)
    exp, _, exp_w = oracle.dispatch(w.x, ref, w.topk_weights, zero_padding=True)
    np.testing.assert_array_equal(recv.view(torch.int16).cpu().numpy().view(np.uint16), exp)
    np.testing.assert_array_equal(rw.cpu().numpy(), exp_w)


def test_with_layout_status_cases(gpu):
    rng = ep_inputs.make_rng(11)
    x = bf16_to_dev(ep_inputs.bf16_normal(rng, (3, 64)))
    # bad ids: ignored and reported
    idx = np.array([[0, 5, 9], [-2, 1, -1], [1, 300, 2]], np.int64)
    lay, _, ref = _run(gpu, idx, None, x, 8, 2, 2)
    assert ref.status & oracle.BAD_EXPERT
    # capacity overflow: pairs past C dropped
    w = ep_inputs.make_workload("decode")
    xd = bf16_to_dev(w.x)
    _, _, ref = _run(gpu, w.topk_idx, w.topk_weights, xd, 256, 1, 1, 4)
    assert ref.status & oracle.CAPACITY
    # receive rows past the allocated buffer
    w = ep_inputs.make_workload("prefill", T=256)
    _, _, ref = _run(gpu, w.topk_idx, w.topk_weights, bf16_to_dev(w.x), 256, 128, rows=1000)
    assert ref.status & oracle.RECV_OVERFLOW


def test_with_layout_empty_and_all_dropped(gpu):
    x0 = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    _run(gpu, np.zeros((0, 8), np.int64), None, x0, 256, 128)
    _run(gpu, np.zeros((0, 2), np.int64), None, x0, 4, 1, 1, 3)
    rng = ep_inputs.make_rng(12)
    x = bf16_to_dev(ep_inputs.bf16_normal(rng, (400, 64)))
    _run(gpu, np.full((400, 4), -1, np.int64), np.ones((400, 4), np.float32), x, 16, 8)


def test_with_layout_cumulative_stats(gpu):
    idx, wt = _prefill_like(512, seed=13)
    x = bf16_to_dev(ep_inputs.bf16_normal(ep_inputs.make_rng(14), (512, 128)))
    _run(gpu, idx, wt, x, 256, 128, stats=True)


def test_with_layout_reuse_and_interleave(gpu):
    """Calls alternate between the fused path and the two-call path on one
    layout and workspace; each matches the oracle."""
    x = bf16_to_dev(ep_inputs.bf16_normal(ep_inputs.make_rng(15), (3000, 256)))
    lay = None
    for i in range(4):
        idx, wt = _prefill_like(3000, seed=20 + i)
        announce("reuse", i)
        if i % 2 == 0:
            lay, recv, _, _ = gpu.ep_dispatch_with_layout(x, to_dev(idx), 256, 128, to_dev(wt),
                                                          layout=lay)
        else:
            lay = gpu.ep_get_layout(to_dev(idx), 256, 128, layout=lay)
            recv, _, _ = gpu.ep_dispatch(x, lay, to_dev(wt))
        ref = oracle.get_layout(idx, 256, 128, rows_cap=lay.max_recv_rows)
        np.testing.assert_array_equal(lay.dst_slot.cpu().numpy(), ref.dst)
        np.testing.assert_array_equal(lay.src_of_slot[:ref.R].cpu().numpy(), ref.src_of_slot)
        assert lay.check() == 0
