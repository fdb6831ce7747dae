"""GPU parity of ep_combine: within rtol = atol = 1e-2 of the float64
oracle (the acceptance bound), and bitwise equal to the ordered-fp32 oracle
(same accumulation order and rounding); deterministic and batch-invariant."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_bits, bf16_to_dev, to_dev

pytestmark = pytest.mark.gpu

RTOL = ATOL = 1e-2


def _check(out_bits, y, dst, w, b0, b1, tokens=None):
    f64 = oracle.combine_f64(y, dst, w, b0, b1, tokens=tokens)
    got = oracle.bf16_to_float(out_bits).astype(np.float64)
    assert np.all(np.abs(got - f64) <= ATOL + RTOL * np.abs(f64))
    f32 = oracle.combine_f32(y, dst, w, b0, b1, tokens=tokens)
    np.testing.assert_array_equal(out_bits, f32)


def _case(gpu, T, H, E, K, A, bias, weighted, seed=0, drop=0.05):
    w = ep_inputs.make_workload("prefill", seed=seed, T=T, H=H, E=E, K=K, A=A, drop_p=drop,
                                with_x=False)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), E, A)
    ref = oracle.get_layout(w.topk_idx, E, A)
    y = ep_inputs.make_y(w.rng, ref.R, H)
    b = [ep_inputs.bf16_normal(w.rng, (T, H)) for _ in range(bias)]
    return w, lay, ref, y, b


@pytest.mark.parametrize("T,H,E,K,A", [
    (64, 256, 8, 2, 1), (1000, 7168, 256, 8, 128), (333, 1000, 32, 4, 3), (129, 8, 16, 3, 4),
    (65, 16384, 64, 2, 2), (77, 2048, 512, 64, 1), (20, 512, 1024, 100, 1),
])
@pytest.mark.parametrize("bias", [0, 1, 2])
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_parity(gpu, T, H, E, K, A, bias, weighted):
    announce("combine", T, H, E, K, A, bias, weighted)
    w, lay, ref, y, b = _case(gpu, T, H, E, K, A, bias, weighted)
    wt = w.topk_weights if weighted else None
    out, _ = gpu.ep_combine(bf16_to_dev(y), lay, to_dev(wt) if weighted else None,
                            bias=tuple(bf16_to_dev(bb) for bb in b) if b else None)
    _check(bf16_bits(out), y, ref.dst, wt, *(b + [None] * (2 - len(b))))


def test_combine_of_dispatch_invariant(gpu):
    """combine(dispatch(x)) = x * sum_k w[t,k], on the GPU path end to end."""
    w = ep_inputs.make_workload("prefill", T=700, H=2048)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), 256, 128)
    wt = to_dev(w.topk_weights)
    recv, _, _ = gpu.ep_dispatch(bf16_to_dev(w.x), lay, wt)
    out, _ = gpu.ep_combine(recv, lay, wt)
    wsum = np.where(w.topk_idx >= 0, w.topk_weights.astype(np.float64), 0).sum(axis=1)
    expect = oracle.bf16_to_float(w.x).astype(np.float64) * wsum[:, None]
    got = oracle.bf16_to_float(bf16_bits(out)).astype(np.float64)
    assert np.all(np.abs(got - expect) <= 2.0 ** -8 * np.abs(expect) + 1e-30)


def test_combine_deterministic(gpu):
    w, lay, ref, y, b = _case(gpu, 2000, 7168, 256, 8, 128, 2, True)
    yd = bf16_to_dev(y)
    args = dict(topk_weights=to_dev(w.topk_weights), bias=tuple(bf16_to_dev(bb) for bb in b))
    o1, _ = gpu.ep_combine(yd, lay, **args)
    o2, _ = gpu.ep_combine(yd, lay, **args)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("n", [1, 16, 64, 257])
def test_combine_batch_invariance(gpu, n):
    """Rows of a token prefix equal the full batch's rows bit for bit, when
    each (token, expert) pair sees the same expert output."""
    T, H, E, K = 600, 1024, 64, 6
    w = ep_inputs.make_workload("prefill", T=T, H=H, E=E, K=K, A=4, with_x=False)
    full = oracle.get_layout(w.topk_idx, E, 4)
    y_full = ep_inputs.make_y(w.rng, full.R, H)
    lay_f = gpu.ep_get_layout(to_dev(w.topk_idx), E, 4)
    out_f, _ = gpu.ep_combine(bf16_to_dev(y_full), lay_f, to_dev(w.topk_weights))
    sub = oracle.get_layout(w.topk_idx[:n], E, 4)
    y_sub = np.zeros((max(sub.R, 1), H), np.uint16)
    for t in range(n):
        for k in range(K):
            if sub.dst[t, k] >= 0:
                y_sub[sub.dst[t, k]] = y_full[full.dst[t, k]]
    lay_s = gpu.ep_get_layout(to_dev(w.topk_idx[:n]), E, 4)
    out_s, _ = gpu.ep_combine(bf16_to_dev(y_sub), lay_s, to_dev(w.topk_weights[:n]))
    assert torch.equal(out_s.view(torch.int16), out_f[:n].view(torch.int16))


def test_combined_topk_weights(gpu):
    w = ep_inputs.make_workload("prefill", T=300, H=64, A=8)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), 256, 8)
    ref = oracle.get_layout(w.topk_idx, 256, 8)
    _, _, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights))
    y = bf16_to_dev(ep_inputs.make_y(w.rng, lay.max_recv_rows, 64))
    _, cw = gpu.ep_combine(y, lay, to_dev(w.topk_weights), recv_topk_weights=rw)
    _, _, ref_rw = oracle.dispatch(w.x, ref, w.topk_weights)
    np.testing.assert_array_equal(cw.cpu().numpy(), oracle.combined_weights(ref_rw, ref.dst))


def test_combine_bias_only_and_empty(gpu):
    T, H = 50, 256
    rng = ep_inputs.make_rng(9)
    idx = np.full((T, 4), -1, np.int64)
    b0 = ep_inputs.bf16_normal(rng, (T, H))
    b1 = ep_inputs.bf16_normal(rng, (T, H))
    lay = gpu.ep_get_layout(to_dev(idx), 16, 4)
    y = torch.zeros((1, H), dtype=torch.bfloat16, device="cuda:0")
    out, _ = gpu.ep_combine(y, lay, None, bias=(bf16_to_dev(b0), bf16_to_dev(b1)))
    np.testing.assert_array_equal(bf16_bits(out), oracle.combine_f32(np.zeros((1, H), np.uint16),
                                                                     np.full((T, 4), -1, np.int32),
                                                                     None, b0, b1))
    lay0 = gpu.ep_get_layout(torch.zeros((0, 4), dtype=torch.int64, device="cuda:0"), 16, 4)
    out0, _ = gpu.ep_combine(y, lay0, None)
    assert out0.shape == (0, H)


def test_combine_y_rows_bound(gpu):
    w, lay, ref, y, b = _case(gpu, 200, 128, 32, 4, 4, 0, True)
    n = ref.R // 2
    out, _ = gpu.ep_combine(bf16_to_dev(y[:n]), lay, to_dev(w.topk_weights))
    dst = np.where(ref.dst < n, ref.dst, -1).astype(np.int32)
    np.testing.assert_array_equal(bf16_bits(out), oracle.combine_f32(y[:n], dst, w.topk_weights))
    assert int(lay.status.item()) & oracle.RECV_OVERFLOW
