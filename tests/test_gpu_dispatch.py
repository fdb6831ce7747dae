"""GPU parity of ep_dispatch (bf16 rows, fp8 rows, fused cast, zero padding,
fixed capacity) and ep_cast_fp8 against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_bits, bf16_to_dev, fp8_bits, fp8_to_dev, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A


def _setup(gpu, w, A=None, C=None, P=None):
    A = w.expert_alignment if A is None else A
    C = w.capacity if C is None else C
    P = w.num_partitions if P is None else P
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), w.num_experts, A, P, C)
    ref = oracle.get_layout(w.topk_idx, w.num_experts, A, P, C, rows_cap=lay.max_recv_rows)
    return lay, ref


@pytest.mark.parametrize("T,H,E,K,A,zero", [
    (64, 256, 8, 2, 1, False),
    (1000, 7168, 256, 8, 128, False),
    (1000, 7168, 256, 8, 128, True),
    (333, 1000, 32, 4, 3, True),     # ragged row: 125 vectors
    (129, 8, 16, 3, 4, True),        # one vector per row
    (65, 16384, 64, 2, 2, True),     # row wider than one wave chunk
    (50, 2056, 128, 8, 1, False),
    (90, 1024, 1024, 100, 1, True),  # K > 64: destinations in two 64-lane passes
])
def test_dispatch_bf16(gpu, T, H, E, K, A, zero):
    announce("dispatch bf16", T, H, E, K, A, zero)
    w = ep_inputs.make_workload("prefill", T=T, H=H, E=E, K=K, A=A, drop_p=0.05)
    lay, ref = _setup(gpu, w)
    rows = lay.max_recv_rows
    recv = torch.full((rows, H), 0, dtype=torch.bfloat16, device="cuda:0")
    recv.view(torch.int16).fill_(SENTINEL)
    recv, _, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights),
                                  zero_padding=zero, out=(recv, None, None))
    init = np.full((ref.R, H), SENTINEL, np.uint16)
    exp, _, exp_w = oracle.dispatch(w.x, ref, w.topk_weights, zero_padding=zero, recv_init=init)
    got = bf16_bits(recv[:ref.R])
    np.testing.assert_array_equal(got, exp)
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)
    assert (bf16_bits(recv[ref.R:]) == SENTINEL).all()    # rows past R untouched
    assert lay.check() == 0


def test_dispatch_unweighted_recv_weights_are_one(gpu):
    w = ep_inputs.make_workload("prefill", T=200, H=64, A=4)
    lay, ref = _setup(gpu, w)
    rw = torch.full((lay.max_recv_rows,), 7.0, dtype=torch.float32, device="cuda:0")
    recv, _, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, None, out=(None, None, rw))
    exp_recv, _, exp_w = oracle.dispatch(w.x, ref, None)
    used = ref.src_of_slot >= 0
    np.testing.assert_array_equal(bf16_bits(recv[:ref.R])[used], exp_recv[used])
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)
    assert set(np.unique(exp_w)) <= {0.0, 1.0}


def test_dispatch_fixed_capacity_decode_full(gpu):
    w = ep_inputs.make_workload("decode")
    lay, ref = _setup(gpu, w)
    recv = torch.empty((lay.max_recv_rows, w.hidden), dtype=torch.bfloat16, device="cuda:0")
    recv.view(torch.int16).fill_(SENTINEL)
    recv, _, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights), zero_padding=True,
                                  out=(recv, None, None))
    exp, _, exp_w = oracle.dispatch(w.x, ref, w.topk_weights, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv), exp)
    np.testing.assert_array_equal(rw.cpu().numpy(), exp_w)


@pytest.mark.parametrize("mode", ["bf16", "fp8", "fused"])
@pytest.mark.parametrize("short", [False, True])
def test_dispatch_capacity_mostly_padding(gpu, mode, short):
    """Fixed capacity with at most one row in eight used (the region is
    zero-filled first, then the token rows written): every byte of rows,
    scale rows and weights against the oracle over sentinel-filled buffers,
    with the full buffer and with one shorter than E*C."""
    announce("dispatch capacity mostly padding", mode, short)
    w = ep_inputs.make_workload("decode", T=37, H=1040, E=64, K=4, C=32)
    lay, ref = _setup(gpu, w)
    rows = lay.max_recv_rows // 2 if short else lay.max_recv_rows
    H, G = w.hidden, 16
    rw = torch.full((rows,), 7.0, dtype=torch.float32, device="cuda:0")
    if mode == "bf16":
        recv = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda:0")
        recv.view(torch.int16).fill_(SENTINEL)
        recv, _, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights),
                                      num_recv_rows=rows, zero_padding=True, out=(recv, None, rw))
        exp, _, exp_w = oracle.dispatch(w.x, ref, w.topk_weights, zero_padding=True)
        np.testing.assert_array_equal(bf16_bits(recv), exp[:rows])
    else:
        q_ref, s_ref = oracle.cast_fp8(w.x, G)
        recv = torch.empty((rows, H), dtype=torch.float8_e4m3fn, device="cuda:0")
        recv.view(torch.uint8).fill_(0x5A)
        rs = torch.full((rows, H // G), 3.0, dtype=torch.float32, device="cuda:0")
        src = (bf16_to_dev(w.x) if mode == "fused"
               else (fp8_to_dev(q_ref), to_dev(s_ref)))
        recv, rs, rw = gpu.ep_dispatch(src, lay, to_dev(w.topk_weights), recv_fp8=mode == "fused",
                                       scale_group=G, num_recv_rows=rows, zero_padding=True,
                                       out=(recv, rs, rw))
        exp, exp_s, exp_w = oracle.dispatch(q_ref, ref, w.topk_weights, x_scales=s_ref,
                                            zero_padding=True)
        np.testing.assert_array_equal(fp8_bits(recv), exp[:rows])
        np.testing.assert_array_equal(rs.cpu().numpy().view(np.uint32),
                                      exp_s[:rows].view(np.uint32))
    np.testing.assert_array_equal(rw.cpu().numpy(), exp_w[:rows])
    status = int(lay.status.item())
    assert bool(status & oracle.RECV_OVERFLOW) == (short and (ref.dst >= rows).any())


def test_dispatch_capacity_no_tokens(gpu):
    """T = 0 with a fixed capacity and zero padding: every row is padding."""
    lay = gpu.ep_get_layout(torch.zeros((0, 8), dtype=torch.int64, device="cuda:0"), 16, 1, 1, 8)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    recv = torch.empty((lay.max_recv_rows, 64), dtype=torch.bfloat16, device="cuda:0")
    recv.view(torch.int16).fill_(SENTINEL)
    recv, _, _ = gpu.ep_dispatch(x, lay, None, zero_padding=True, out=(recv, None, None))
    assert (bf16_bits(recv) == 0).all()


def test_dispatch_capacity_overflow_drops_pairs(gpu):
    w = ep_inputs.make_workload("decode", H=128)
    lay, ref = _setup(gpu, w, C=4)
    recv, _, _ = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights), zero_padding=True)
    exp, _, _ = oracle.dispatch(w.x, ref, w.topk_weights, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv), exp)
    with pytest.raises(RuntimeError):
        lay.check()


def test_dispatch_recv_rows_bound(gpu):
    """Receive buffers shorter than R: rows past them are skipped and flagged."""
    w = ep_inputs.make_workload("prefill", T=300, H=64, A=8)
    lay, ref = _setup(gpu, w)
    n = ref.R // 2
    recv, _, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights), num_recv_rows=n,
                                  zero_padding=True)
    assert recv.shape[0] == n
    exp, _, exp_w = oracle.dispatch(w.x, ref, w.topk_weights, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv), exp[:n])
    np.testing.assert_array_equal(rw.cpu().numpy(), exp_w[:n])
    assert int(lay.status.item()) & oracle.RECV_OVERFLOW


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_dispatch_fp8_copy_recv_rows_bound(gpu, fmt):
    """fp8 copy into a receive buffer shorter than R, over sentinel scales:
    rows and scale rows past it untouched and flagged, every other byte as the
    oracle's (padding zeroed)."""
    announce("dispatch fp8 copy recv rows bound", fmt)
    w = ep_inputs.make_workload("fp8", T=300, H=1024, A=8, drop_p=0.05)
    lay, ref = _setup(gpu, w)
    n = ref.R // 2 + 3
    if fmt == "fp32":
        q_ref, s_ref = oracle.cast_fp8(w.x, 128)
        rs = torch.full((n, 8), 3.0, dtype=torch.float32, device="cuda:0")
        xs = to_dev(s_ref)
    else:
        q_ref, _, s_ref = oracle.cast_fp8_pow2(w.x, 128, ue8m0=True)
        rs = torch.full((n, 8), 7, dtype=torch.uint8, device="cuda:0")
        xs = torch.from_numpy(np.ascontiguousarray(s_ref)).to("cuda:0")
    recv = torch.empty((n, 1024), dtype=torch.float8_e4m3fn, device="cuda:0")
    recv.view(torch.uint8).fill_(0x5A)
    recv, rs, rw = gpu.ep_dispatch((fp8_to_dev(q_ref), xs), lay, to_dev(w.topk_weights),
                                   num_recv_rows=n, zero_padding=True, out=(recv, rs, None))
    exp, exp_s, exp_w = oracle.dispatch(q_ref, ref, w.topk_weights, x_scales=s_ref,
                                        zero_padding=True)
    np.testing.assert_array_equal(fp8_bits(recv), exp[:n])
    got_s = rs.cpu().numpy()
    np.testing.assert_array_equal(got_s.view(np.uint8), np.ascontiguousarray(exp_s[:n]).view(np.uint8))
    np.testing.assert_array_equal(rw.cpu().numpy(), exp_w[:n])
    assert int(lay.status.item()) & oracle.RECV_OVERFLOW


@pytest.mark.parametrize("G", [128, 16, 64, 512, "H"])
@pytest.mark.parametrize("fused", [False, True])
def test_dispatch_fp8(gpu, G, fused):
    T, H = 700, 7168 if G != "H" else 2048
    G = H if G == "H" else G
    announce("dispatch fp8", G, fused)
    w = ep_inputs.make_workload("fp8", T=T, H=H, drop_p=0.03)
    lay, ref = _setup(gpu, w)
    q_ref, s_ref = oracle.cast_fp8(w.x, G)
    if fused:
        recv, rs, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights),
                                       recv_fp8=True, scale_group=G, zero_padding=True)
    else:
        recv, rs, rw = gpu.ep_dispatch((fp8_to_dev(q_ref), to_dev(s_ref)), lay,
                                       to_dev(w.topk_weights), zero_padding=True)
    exp, exp_s, exp_w = oracle.dispatch(q_ref, ref, w.topk_weights, x_scales=s_ref,
                                        zero_padding=True)
    np.testing.assert_array_equal(fp8_bits(recv[:ref.R]), exp)
    np.testing.assert_array_equal(rs[:ref.R].cpu().numpy().view(np.uint32), exp_s.view(np.uint32))
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)


@pytest.mark.parametrize("G", [16, 32, 64, 128, 256, 512, "H"])
def test_cast_fp8_groups(gpu, G):
    H = 7168 if G != "H" else 4096
    G = H if G == "H" else G
    x = ep_inputs.bf16_normal(ep_inputs.make_rng(G), (257, H))
    x[3, :G] = 0                              # floor
    x[4, 7] = 0x7F7F                          # huge value in a group
    x[5, :G] = 0x8001                         # negative subnormals only
    x[6, 1::2] = 0x0001
    announce("cast", G)
    q, s = gpu.ep_cast_fp8(bf16_to_dev(x), G)
    rq, rs = oracle.cast_fp8(x, G)
    np.testing.assert_array_equal(fp8_bits(q), rq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_cast_fp8_every_bf16_pattern(gpu):
    """All finite bf16 patterns, each in groups whose amax is set by one of
    several leading values, so every pattern is cast under many scales.  The
    leads 448 and 0.875 give the exact scales 1 and 2^-9: there the quotients
    are the bf16 values themselves (times 2^9), which include every e4m3 code,
    every rounding midpoint (ties) and their bf16 neighbours."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7F80) != 0x7F80]
    mags = np.abs(oracle.bf16_to_float(finite))
    rows = []
    for lead in (0x7F7F, 0x4380, 0x43E0, 0x3F80, 0x3F60, 0x3400, 0x0080):
        lead_v = abs(float(oracle.bf16_to_float(np.array([lead], np.uint16))[0]))
        vals = finite[mags <= lead_v]
        pad = (-len(vals)) % 127
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 127)
        rows.append(np.concatenate([np.full((len(vals), 1), lead, np.uint16), vals], axis=1))
    groups = np.concatenate(rows)
    groups = np.concatenate([groups, np.zeros(((-len(groups)) % 8, 128), np.uint16)])
    x = groups.reshape(-1, 128 * 8)
    q, s = gpu.ep_cast_fp8(bf16_to_dev(x), 128)
    rq, rs = oracle.cast_fp8(x, 128)
    np.testing.assert_array_equal(fp8_bits(q), rq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_fused_equals_cast_then_dispatch_on_gpu(gpu):
    w = ep_inputs.make_workload("fp8", T=513)
    lay, ref = _setup(gpu, w)
    x = bf16_to_dev(w.x)
    q, s = gpu.ep_cast_fp8(x, 128)
    a, a_s, _ = gpu.ep_dispatch((q, s), lay, zero_padding=True)
    b, b_s, _ = gpu.ep_dispatch(x, lay, recv_fp8=True, zero_padding=True)
    R = ref.R
    assert torch.equal(a[:R].view(torch.uint8), b[:R].view(torch.uint8))
    assert torch.equal(a_s[:R], b_s[:R])


def test_dispatch_reused_layout(gpu):
    """A layout (handle) reused for a second dispatch with new rows."""
    w = ep_inputs.make_workload("prefill", T=400, H=512)
    lay, ref = _setup(gpu, w)
    x2 = ep_inputs.bf16_normal(w.rng, (400, 512))
    gpu.ep_dispatch(bf16_to_dev(w.x), lay)
    recv, _, _ = gpu.ep_dispatch(bf16_to_dev(x2), lay, zero_padding=True)
    exp, _, _ = oracle.dispatch(x2, ref, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv[:ref.R]), exp)


def test_dispatch_empty(gpu):
    lay = gpu.ep_get_layout(torch.zeros((0, 8), dtype=torch.int64, device="cuda:0"), 256, 128)
    recv, _, _ = gpu.ep_dispatch(torch.zeros((0, 7168), dtype=torch.bfloat16, device="cuda:0"),
                                 lay, zero_padding=True)
    torch.cuda.synchronize()
    assert lay.num_recv_rows() == 0


def test_widest_rows(gpu):
    """Rows of EP_MAX_HIDDEN channels (2 MiB in bf16): many waves per row in
    every kernel.  bf16 dispatch with zero padding (two calls and one call),
    the fused cast, the fp8 copy with its 8,192 scales per row, the
    standalone cast and the combine, all bit-exact."""
    from combine_ep_get_layout_amd import _abi
    H = _abi.EP_MAX_HIDDEN
    T, E, K, A, G = 5, 4, 2, 2, 128
    announce("widest rows", T, H)
    rng = ep_inputs.make_rng(77)
    idx, wts = ep_inputs.routing_uniform(rng, T, E, K)
    idx[1, 1] = -1
    x = ep_inputs.bf16_normal(rng, (T, H))
    xd = bf16_to_dev(x)
    lay = gpu.ep_get_layout(to_dev(idx), E, A)
    ref = oracle.get_layout(idx, E, A, rows_cap=lay.max_recv_rows)
    recv, _, rw = gpu.ep_dispatch(xd, lay, to_dev(wts), zero_padding=True)
    exp, _, exp_w = oracle.dispatch(x, ref, wts, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv[:ref.R]), exp)
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)
    _, recv1, _, _ = gpu.ep_dispatch_with_layout(xd, to_dev(idx), E, A, to_dev(wts),
                                                 zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv1[:ref.R]), exp)
    q_ref, s_ref = oracle.cast_fp8(x, G)
    q, s = gpu.ep_cast_fp8(xd, G)
    np.testing.assert_array_equal(fp8_bits(q), q_ref)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    exp8, exp_s, _ = oracle.dispatch(q_ref, ref, wts, x_scales=s_ref, zero_padding=True)
    for fused in (True, False):
        src = xd if fused else (fp8_to_dev(q_ref), to_dev(s_ref))
        r8, rs, _ = gpu.ep_dispatch(src, lay, to_dev(wts), recv_fp8=fused, scale_group=G,
                                    zero_padding=True)
        np.testing.assert_array_equal(fp8_bits(r8[:ref.R]), exp8)
        np.testing.assert_array_equal(rs[:ref.R].cpu().numpy().view(np.uint32),
                                      exp_s.view(np.uint32))
    y = ep_inputs.make_y(rng, ref.R, H)
    out, _ = gpu.ep_combine(bf16_to_dev(y), lay, to_dev(wts))
    np.testing.assert_array_equal(bf16_bits(out), oracle.combine_f32(y, ref.dst, wts))
    assert lay.check() == 0


@pytest.mark.parametrize("T,H,E,K,A", [
    (4096, 7168, 256, 8, 128),   # the prefill shape, the kernel instance the bench times
    (333, 1000, 32, 4, 3),       # ragged row
])
def test_probe_dispatch_stores(gpu, T, H, E, K, A):
    """The stores-only measurement aid writes the pattern into exactly the
    rows that hold a pair (the oracle's src_of_slot) and nothing else."""
    announce("probe stores", T, H, E, K, A)
    w = ep_inputs.make_workload("prefill", T=T, H=H, E=E, K=K, A=A, drop_p=0.02)
    lay, ref = _setup(gpu, w)
    rows = lay.max_recv_rows
    recv = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda:0")
    recv.view(torch.int16).fill_(SENTINEL)
    gpu.ep_probe_dispatch_stores(recv, lay, pattern=0x3F80BF80)
    torch.cuda.synchronize()
    used = torch.from_numpy(ref.src_of_slot >= 0).to("cuda:0")
    words = recv[:ref.R].view(torch.int32)
    assert bool((words[used] == 0x3F80BF80).all())
    assert bool((recv[:ref.R][~used].view(torch.int16) == SENTINEL).all())
    assert bool((recv[ref.R:].view(torch.int16) == SENTINEL).all())
    assert lay.check() == 0
