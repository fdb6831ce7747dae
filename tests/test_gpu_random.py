"""Seeded random shapes through the whole path: layout, bf16 dispatch,
combine and the two-level combine, the non-expanded layout with its dispatch
and combine, and (where the shape allows fp8 rows) the cast, the fp8 copy and
the fused cast dispatch, each compared in full with the oracle bit for bit.  The
shapes are drawn once from a fixed seed, so every run checks the same cases."""
import os

import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_bits, bf16_to_dev, fp8_bits, fp8_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _cases(n=int(os.environ.get("EP_RANDOM_CASES", "48")), seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 5, 8, 16, 33, 64, 128, 256, 300]))
        K = int(rng.integers(1, min(E, 12) + 1))
        T = int(rng.choice([0, 1, 2, 31, 64, 257, 700, 1500]))
        A = int(rng.choice([1, 2, 3, 8, 128]))
        divs = [p for p in range(1, E + 1) if E % p == 0 and p <= 64]
        P = int(rng.choice(divs))
        C = 0 if rng.random() < 0.7 else A * int(rng.integers(1, 5))
        H = int(rng.choice([16, 64, 256, 1040, 2048]))
        drop = float(rng.choice([0.0, 0.1, 0.5]))
        out.append((i, T, K, E, A, P, C, H, drop))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"c{c[0]}")
def test_random_shape_whole_path(gpu, case):
    i, T, K, E, A, P, C, H, drop = case
    announce("random", case)
    rng = ep_inputs.make_rng(1000 + i)
    idx, wts = ep_inputs.routing_uniform(rng, T, E, K)
    idx[rng.random((T, K)) < drop] = -1
    x = ep_inputs.bf16_normal(rng, (T, H))
    lay = gpu.ep_get_layout(to_dev(idx), E, A, P, C)
    ref = oracle.get_layout(idx, E, A, P, C, rows_cap=lay.max_recv_rows)
    torch.cuda.synchronize()
    assert int(lay.status.item()) == ref.status
    np.testing.assert_array_equal(lay.num_tokens_per_expert.cpu().numpy(), ref.count)
    np.testing.assert_array_equal(lay.expert_offset.cpu().numpy(), ref.offset)
    np.testing.assert_array_equal(lay.dst_slot.cpu().numpy(), ref.dst)
    np.testing.assert_array_equal(lay.is_token_in_partition.cpu().numpy(), ref.in_part)
    np.testing.assert_array_equal(lay.num_tokens_per_partition.cpu().numpy(), ref.tok_per_part)
    R = min(ref.R, lay.max_recv_rows)
    np.testing.assert_array_equal(lay.src_of_slot[:R].cpu().numpy(), ref.src_of_slot[:R])
    if ref.status:                      # capacity overflow: drops are checked above
        return

    wd = to_dev(wts)
    recv, _, rw = gpu.ep_dispatch(bf16_to_dev(x), lay, wd, zero_padding=True)
    exp, _, exp_w = oracle.dispatch(x, ref, wts, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv[:R]), exp[:R])
    np.testing.assert_array_equal(rw[:R].cpu().numpy(), exp_w[:R])

    y = ep_inputs.make_y(rng, max(lay.max_recv_rows, 1), H)
    out, _ = gpu.ep_combine(bf16_to_dev(y), lay, wd)
    np.testing.assert_array_equal(bf16_bits(out), oracle.combine_f32(y, ref.dst, wts))
    out_r = gpu.ep_combine_reduced(bf16_to_dev(y), lay, to_dev(idx), wd)
    np.testing.assert_array_equal(bf16_bits(out_r),
                                  oracle.combine_reduced_f32(y, idx, ref.dst, E, P, wts))

    # the non-expanded layout, its dispatch and combine
    pl = gpu.ep_get_layout(to_dev(idx), E, A, P, C, partition_layout=True)
    pref = oracle.partition_layout(idx, E, P)
    np.testing.assert_array_equal(pl.token_slot.cpu().numpy(), pref.token_slot)
    np.testing.assert_array_equal(pl.partition_offset.cpu().numpy(), pref.part_offset)
    np.testing.assert_array_equal(pl.partition_src[:pref.Rp].cpu().numpy(), pref.part_src)
    px, _, pi, pw = gpu.ep_dispatch_partitioned(bf16_to_dev(x), pl, to_dev(idx), wd)
    ex, _, ei, ew = oracle.dispatch_partitioned(x, idx, pref, wts)
    np.testing.assert_array_equal(bf16_bits(px[:pref.Rp]), ex)
    np.testing.assert_array_equal(pi[:pref.Rp].cpu().numpy(), ei)
    np.testing.assert_array_equal(pw[:pref.Rp].cpu().numpy(), ew)
    yp = ep_inputs.make_y(rng, max(pref.Rp, 1), H)
    outp = gpu.ep_combine_partitioned(bf16_to_dev(yp), pl)
    np.testing.assert_array_equal(bf16_bits(outp),
                                  oracle.combine_partitioned_f32(yp, pref.token_slot))

    G = 16 if H % 16 == 0 else None
    if G is None or T == 0:
        return
    G = min(128, H) if H % 128 == 0 else 16
    q, s = oracle.cast_fp8(x, G)
    gq, gs = gpu.ep_cast_fp8(bf16_to_dev(x), G)
    np.testing.assert_array_equal(fp8_bits(gq), q)
    np.testing.assert_array_equal(gs.cpu().numpy().view(np.uint32), s.view(np.uint32))
    exp8, exp_s, _ = oracle.dispatch(q, ref, wts, x_scales=s, zero_padding=True)
    for src in ((fp8_to_dev(q), to_dev(s)), bf16_to_dev(x)):
        fused = not isinstance(src, tuple)
        r8, rs, _ = gpu.ep_dispatch(src, lay, wd, recv_fp8=fused, scale_group=G,
                                    zero_padding=True)
        np.testing.assert_array_equal(fp8_bits(r8[:R]), exp8[:R])
        np.testing.assert_array_equal(rs[:R].cpu().numpy().view(np.uint32),
                                      exp_s[:R].view(np.uint32))
    assert lay.check() == 0


def _layout_cases(n=int(os.environ.get("EP_RANDOM_LAYOUT_CASES", "32")), seed=20261204):
    """Layout-heavy shapes over the whole expert range: E log-uniform in
    [1, 4096] (so the tile rows take every width the column sums and the row
    kernels' LDS see), T up to 20,000, K up to 16, P up to 1,024."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(np.clip(np.round(np.exp(rng.uniform(0, np.log(4096)))), 1, 4096))
        K = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.choice([0, 1, 100, 257, 1000, 3000, 9000, 20000]))
        A = int(rng.choice([1, 2, 4, 16, 128]))
        divs = [p for p in range(1, min(E, 1024) + 1) if E % p == 0]
        P = int(rng.choice(divs))
        C = 0 if rng.random() < 0.75 else A * int(rng.integers(1, 9))
        drop = float(rng.choice([0.0, 0.05, 0.5]))
        out.append((i, T, K, E, A, P, C, drop))
    return out


@pytest.mark.parametrize("case", _layout_cases(), ids=lambda c: f"l{c[0]}")
def test_random_layout_both_paths(gpu, case):
    """ep_get_layout and ep_dispatch_with_layout against the oracle: every
    layout buffer, and the one-call path's receive rows (H = 16)."""
    i, T, K, E, A, P, C, drop = case
    announce("random layout", case)
    rng = ep_inputs.make_rng(5000 + i)
    idx, wts = ep_inputs.routing_uniform(rng, T, E, K)
    idx[rng.random((T, K)) < drop] = -1
    H = 16
    x = ep_inputs.bf16_normal(rng, (T, H))
    lay = gpu.ep_get_layout(to_dev(idx), E, A, P, C)
    ref = oracle.get_layout(idx, E, A, P, C, rows_cap=lay.max_recv_rows)
    R = min(ref.R, lay.max_recv_rows)

    def check(l):
        torch.cuda.synchronize()
        assert int(l.status.item()) == ref.status
        np.testing.assert_array_equal(l.num_tokens_per_expert.cpu().numpy(), ref.count)
        np.testing.assert_array_equal(l.expert_offset.cpu().numpy(), ref.offset)
        np.testing.assert_array_equal(l.dst_slot.cpu().numpy(), ref.dst)
        np.testing.assert_array_equal(l.is_token_in_partition.cpu().numpy(), ref.in_part)
        np.testing.assert_array_equal(l.num_tokens_per_partition.cpu().numpy(), ref.tok_per_part)
        np.testing.assert_array_equal(l.src_of_slot[:R].cpu().numpy(), ref.src_of_slot[:R])

    check(lay)
    lay2, recv, _, rw = gpu.ep_dispatch_with_layout(bf16_to_dev(x), to_dev(idx), E, A,
                                                    to_dev(wts), P, C, zero_padding=True)
    check(lay2)
    exp, _, exp_w = oracle.dispatch(x, ref, wts, zero_padding=True)
    np.testing.assert_array_equal(bf16_bits(recv[:R]), exp[:R])
    np.testing.assert_array_equal(rw[:R].cpu().numpy(), exp_w[:R])


def _logfmt_cases(n=int(os.environ.get("EP_RANDOM_LOGFMT_CASES", "24")), seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([4, 16, 33, 64, 256]))
        K = int(rng.integers(1, min(E, 10) + 1))
        T = int(rng.choice([1, 17, 128, 500, 1500]))
        A = int(rng.choice([1, 4, 128]))
        C = 0 if rng.random() < 0.6 else A * int(rng.integers(1, 6))
        H = 128 * int(rng.choice([1, 2, 7, 8, 9, 56, 72]))
        drop = float(rng.choice([0.0, 0.1, 0.5]))
        bias = int(rng.integers(0, 3))
        weighted = bool(rng.random() < 0.7)
        out.append((i, T, K, E, A, C, H, drop, bias, weighted))
    return out


@pytest.mark.parametrize("case", _logfmt_cases(), ids=lambda c: f"l{c[0]}")
def test_random_logfmt_payload(gpu, case):
    """The 10-bit logarithmic payload on random layouts: the encoder given the
    layout (dense or sparse launch by the pair count) writes exactly the rows
    that hold a pair, byte for byte as the oracle packs them, and the combine
    over the payload equals the oracle's combine of the decoded rows."""
    i, T, K, E, A, C, H, drop, bias, weighted = case
    announce("random logfmt", case)
    rng = ep_inputs.make_rng(3000 + i)
    idx, wts = ep_inputs.routing_uniform(rng, T, E, K)
    idx[rng.random((T, K)) < drop] = -1
    lay = gpu.ep_get_layout(to_dev(idx), E, A, 1, C)
    ref = oracle.get_layout(idx, E, A, 1, C, rows_cap=lay.max_recv_rows)
    R = min(ref.R, lay.max_recv_rows)
    y = ep_inputs.make_y_wide(rng, R, H)
    b = [ep_inputs.bf16_normal(rng, (T, H)) for _ in range(bias)]
    wt = wts if weighted else None
    used_bytes = H + H // 4 + 2 * (H // 128)
    pay = torch.full((R, gpu.logfmt_row_bytes(H)), 0x5A, dtype=torch.uint8, device="cuda:0")
    gpu.ep_logfmt_encode(bf16_to_dev(y), out=pay, layout=lay)
    got = pay.cpu().numpy()
    used = ref.src_of_slot[:R] >= 0
    assert np.all(got[~used] == 0x5A) and np.all(got[:, used_bytes:] == 0x5A)
    # the oracle encodes the rows that hold a pair; the others decode to 0
    # here and no pair reads them
    cu, ru = oracle.logfmt_encode(y[used])
    np.testing.assert_array_equal(got[used, :used_bytes], oracle.logfmt_pack(cu, ru)[:, :used_bytes])
    codes = np.zeros((R, H), np.uint16)
    refs = np.zeros((R, H // 128), np.uint16)
    codes[used], refs[used] = cu, ru
    out, _ = gpu.ep_combine_logfmt(pay, H, lay, to_dev(wt) if weighted else None,
                                   bias=tuple(bf16_to_dev(bb) for bb in b) if b else None)
    dst = np.where(ref.dst < R, ref.dst, -1).astype(np.int32)
    want = oracle.combine_logfmt_f32(codes, refs, dst, wt, *(b + [None] * (2 - len(b))))
    gotb = bf16_bits(out)
    gn, wn = (gotb & 0x7FFF) > 0x7F80, (want & 0x7FFF) > 0x7F80
    np.testing.assert_array_equal(gn, wn)
    np.testing.assert_array_equal(np.where(gn, 0, gotb), np.where(wn, 0, want))
