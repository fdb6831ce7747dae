"""GPU parity of the 10-bit logarithmic combine payload ("DeepEP test target
API reference" sec. 3.4, use_logfmt): ep_logfmt_encode byte for byte against
the oracle's codes packed in the documented layout, ep_logfmt_decode and
ep_combine_logfmt bit for bit against the oracle, and the combine over the
payload equal to ep_combine over the decoded rows."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_bits, bf16_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _used(H):
    return H + H // 4 + 2 * (H // 128)


def _same_bits_or_both_nan(got, want):
    gn = (got & 0x7FFF) > 0x7F80
    wn = (want & 0x7FFF) > 0x7F80
    np.testing.assert_array_equal(gn, wn)
    np.testing.assert_array_equal(np.where(gn, 0, got), np.where(wn, 0, want))


def _check_codec(gpu, y):
    rows, H = y.shape
    pay = gpu.ep_logfmt_encode(bf16_to_dev(y))
    assert pay.shape == (rows, gpu.logfmt_row_bytes(H)) and pay.dtype == torch.uint8
    codes, refs = oracle.logfmt_encode(y)
    want = oracle.logfmt_pack(codes, refs)
    got = pay.cpu().numpy()
    np.testing.assert_array_equal(got[:, :_used(H)], want[:, :_used(H)])
    dec = gpu.ep_logfmt_decode(pay, H)
    np.testing.assert_array_equal(bf16_bits(dec), oracle.logfmt_decode(codes, refs))
    return pay


@pytest.mark.parametrize("rows,H,seed", [
    (1, 128, 0), (37, 256, 1), (300, 7168, 2), (1000, 1152, 3), (5, 2048, 4), (64, 9216, 5),
    (3, 128 * 127, 6),
])
def test_encode_decode_parity(gpu, rows, H, seed):
    announce("logfmt codec", rows, H, seed)
    y = ep_inputs.make_y_wide(ep_inputs.make_rng(seed), rows, H)
    _check_codec(gpu, y)


def test_every_pattern_alone_and_under_maxima(gpu):
    """All 65536 bf16 patterns, each alone in a group, then each beside a
    power-of-two maximum of 2^k (k = 0, 100, -110) and beside the largest
    finite bf16 value."""
    announce("logfmt exhaustive")
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rows = np.zeros((65536, 128), np.uint16)
    rows[:, 0] = allp
    _check_codec(gpu, rows)
    for top in (0x3F80, 0x7180, 0x0880, 0x7F7F):
        rows = np.zeros((65536, 128), np.uint16)
        rows[:, 5] = top
        rows[:, 77] = allp
        _check_codec(gpu, rows)


@pytest.mark.parametrize("T,E,C", [
    (300, 32, 0),      # aligned layout: padding rows skipped, one wave per row
    (300, 32, 64),     # fixed capacity, most rows used: one wave per row
    (100, 64, 64),     # 400 pairs in 4,096 rows: the sparse launch
    (50, 256, 128),    # decode-like region (3% of 32,768 rows used): sparse
    (10, 33, 8),       # sparse, 264 rows: a ragged last block of 64 rows
])
def test_encode_skips_rows_without_a_pair(gpu, T, E, C):
    """With the layout, rows that hold no pair (alignment padding, or the
    unused rows of a fixed-capacity region) keep their bytes, and no row's
    tail past the payload is written; the combine over it equals the one over
    the fully encoded rows."""
    H, K, A = 1152, 4, 8
    announce("logfmt encode with the layout", T, E, C)
    w = ep_inputs.make_workload("prefill", seed=21 + T + C, T=T, H=H, E=E, K=K, A=A, drop_p=0.05,
                                with_x=False)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), E, A, 1, C)
    ref = oracle.get_layout(w.topk_idx, E, A, 1, C)
    y = ep_inputs.make_y_wide(w.rng, ref.R, H)
    yd = bf16_to_dev(y)
    pay = torch.full((ref.R, gpu.logfmt_row_bytes(H)), 0xAB, dtype=torch.uint8, device="cuda:0")
    gpu.ep_logfmt_encode(yd, out=pay, layout=lay)
    got = pay.cpu().numpy()
    used = ref.src_of_slot >= 0
    assert 0 < used.sum() < ref.R
    assert np.all(got[~used] == 0xAB)
    assert np.all(got[:, _used(H):] == 0xAB)
    codes, refs = oracle.logfmt_encode(y[used])
    np.testing.assert_array_equal(got[used, :_used(H)], oracle.logfmt_pack(codes, refs)[:, :_used(H)])
    wt = to_dev(w.topk_weights)
    out, _ = gpu.ep_combine_logfmt(pay, H, lay, wt)
    out_full, _ = gpu.ep_combine_logfmt(gpu.ep_logfmt_encode(yd), H, lay, wt)
    assert torch.equal(out.view(torch.int16), out_full.view(torch.int16))


def test_empty_rows(gpu):
    pay = gpu.ep_logfmt_encode(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda:0"))
    assert pay.shape == (0, 384)
    assert gpu.ep_logfmt_decode(pay, 256).shape == (0, 256)


def _layout_case(gpu, T, H, E, K, A, seed, drop=0.05):
    w = ep_inputs.make_workload("prefill", seed=seed, T=T, H=H, E=E, K=K, A=A, drop_p=drop,
                                with_x=False)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), E, A)
    ref = oracle.get_layout(w.topk_idx, E, A)
    return w, lay, ref


@pytest.mark.parametrize("T,H,E,K,A", [
    (64, 256, 8, 2, 1), (1000, 7168, 256, 8, 128), (333, 1152, 32, 4, 3), (65, 16384, 64, 2, 2),
    (77, 2048, 512, 64, 1), (20, 512, 1024, 100, 1),
])
@pytest.mark.parametrize("bias,weighted", [(0, True), (2, True), (1, False)])
def test_combine_logfmt_parity(gpu, T, H, E, K, A, bias, weighted):
    announce("combine logfmt", T, H, E, K, A, bias, weighted)
    w, lay, ref = _layout_case(gpu, T, H, E, K, A, seed=T + H)
    y = ep_inputs.make_y_wide(w.rng, ref.R, H)
    b = [ep_inputs.bf16_normal(w.rng, (T, H)) for _ in range(bias)]
    wt = w.topk_weights if weighted else None
    pay = _check_codec(gpu, y)
    out, _ = gpu.ep_combine_logfmt(pay, H, lay, to_dev(wt) if weighted else None,
                                   bias=tuple(bf16_to_dev(bb) for bb in b) if b else None)
    codes, refs = oracle.logfmt_encode(y)
    want = oracle.combine_logfmt_f32(codes, refs, ref.dst, wt, *(b + [None] * (2 - len(b))))
    _same_bits_or_both_nan(bf16_bits(out), want)
    # the same bits as ep_combine over the decoded rows
    out2, _ = gpu.ep_combine(gpu.ep_logfmt_decode(pay, H), lay, to_dev(wt) if weighted else None,
                             bias=tuple(bf16_to_dev(bb) for bb in b) if b else None)
    _same_bits_or_both_nan(bf16_bits(out), bf16_bits(out2))


def test_combine_logfmt_prefill(gpu):
    """The prefill workload (T = 4096, H = 7168, E = 256, K = 8, A = 128):
    payload rows sampled against the oracle, the combine of every token equal
    to ep_combine over the decoded rows, and sampled tokens against the
    oracle; combined_topk_weights as ep_combine's."""
    w = ep_inputs.make_workload("prefill", with_x=False)
    T, H, E, K, A = w.num_tokens, w.hidden, w.num_experts, w.num_topk, w.expert_alignment
    announce("combine logfmt prefill", T, H)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), E, A)
    ref = oracle.get_layout(w.topk_idx, E, A)
    y = ep_inputs.make_y(w.rng, ref.R, H)
    yd = bf16_to_dev(y)
    pay = gpu.ep_logfmt_encode(yd)
    rng = ep_inputs.make_rng(11)
    rows = np.sort(rng.choice(ref.R, 512, replace=False))
    codes_s, refs_s = oracle.logfmt_encode(y[rows])
    np.testing.assert_array_equal(pay[torch.from_numpy(rows).cuda()].cpu().numpy()[:, :_used(H)],
                                  oracle.logfmt_pack(codes_s, refs_s)[:, :_used(H)])
    wt = to_dev(w.topk_weights)
    rw = torch.from_numpy(rng.random(ref.R).astype(np.float32)).cuda()
    out, cw = gpu.ep_combine_logfmt(pay, H, lay, wt, recv_topk_weights=rw)
    out2, cw2 = gpu.ep_combine(gpu.ep_logfmt_decode(pay, H), lay, wt, recv_topk_weights=rw)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(cw, cw2)
    tokens = np.sort(rng.choice(T, 256, replace=False))
    codes, refs = oracle.logfmt_encode(y)
    want = oracle.combine_logfmt_f32(codes, refs, ref.dst, w.topk_weights, tokens=tokens)
    np.testing.assert_array_equal(bf16_bits(out)[tokens], want)
    # the codec's error against the exact combine: 2^-6 of each kept
    # magnitude, each flushed value under 2^-15 of its group's maximum, plus
    # the bf16 rounding of the result
    exact = oracle.combine_f64(y, ref.dst, w.topk_weights, tokens=tokens)
    got = oracle.bf16_to_float(want).astype(np.float64)
    ay = y & np.uint16(0x7FFF)
    aw = np.abs(w.topk_weights)
    mag = oracle.combine_f64(ay, ref.dst, aw, tokens=tokens)
    gmax = np.repeat(ay.reshape(ref.R, H // 128, 128).max(axis=2), 128, axis=1)
    top = oracle.combine_f64(gmax, ref.dst, aw, tokens=tokens)
    bound = 2.0 ** -6 * mag + 2.0 ** -15 * top + 2.0 ** -8 * np.abs(exact)
    assert np.all(np.abs(got - exact) <= bound * 1.0001)
    assert lay.check() == 0


def test_combine_logfmt_y_rows_bound_and_empty(gpu):
    w, lay, ref = _layout_case(gpu, 200, 128, 32, 4, 4, seed=3)
    y = ep_inputs.make_y_wide(w.rng, ref.R, 128)
    n = ref.R // 2
    pay = gpu.ep_logfmt_encode(bf16_to_dev(y[:n]))
    out, _ = gpu.ep_combine_logfmt(pay, 128, lay, to_dev(w.topk_weights))
    dst = np.where(ref.dst < n, ref.dst, -1).astype(np.int32)
    codes, refs = oracle.logfmt_encode(y[:n])
    _same_bits_or_both_nan(bf16_bits(out),
                           oracle.combine_logfmt_f32(codes, refs, dst, w.topk_weights))
    assert int(lay.status.item()) & oracle.RECV_OVERFLOW
    # no tokens
    lay0 = gpu.ep_get_layout(torch.empty((0, 4), dtype=torch.int64, device="cuda:0"), 32, 4)
    out0, _ = gpu.ep_combine_logfmt(pay, 128, lay0)
    assert out0.shape == (0, 128)


def test_combine_logfmt_marked_group_is_nan(gpu):
    """A row whose second group holds an infinity: the tokens reading it get
    NaN in exactly those 128 channels."""
    w, lay, ref = _layout_case(gpu, 64, 512, 8, 2, 1, seed=4, drop=0.0)
    y = ep_inputs.make_y(w.rng, ref.R, 512)
    y[0, 200] = 0x7F80
    pay = gpu.ep_logfmt_encode(bf16_to_dev(y))
    out, _ = gpu.ep_combine_logfmt(pay, 512, lay, to_dev(w.topk_weights))
    bits = bf16_bits(out)
    nan = (bits & 0x7FFF) > 0x7F80
    readers = np.nonzero((ref.dst == 0).any(axis=1))[0]
    assert readers.size == 1
    expect = np.zeros_like(nan)
    expect[readers[0], 128:256] = True
    np.testing.assert_array_equal(nan, expect)
