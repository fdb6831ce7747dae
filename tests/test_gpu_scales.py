"""GPU parity of the power-of-two ("round_scale") and UE8M0 scale formats:
ep_cast_fp8, the fused-cast dispatch and the fp8 copy dispatch (UE8M0 scale
bytes travel with the rows), against the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle
from gpu_util import announce, bf16_to_dev, fp8_bits, fp8_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _x(seed, T, H, G):
    x = ep_inputs.bf16_normal(ep_inputs.make_rng(seed), (T, H))
    x[3, :G] = 0                              # floor 1e-4
    x[4, 7] = 0x7F7F                          # largest finite bf16
    x[5, :G] = 0x8001                         # negative subnormals only
    x[6, 1::2] = 0x0001
    x[7, :G] = 0x4260                         # amax 56 = 448/8: already a power of two
    return x


@pytest.mark.parametrize("fmt", ["pow2", "ue8m0"])
@pytest.mark.parametrize("G", [16, 128, 512, "H"])
def test_cast_scale_formats(gpu, fmt, G):
    H = 7168 if G != "H" else 4096
    G = H if G == "H" else G
    announce("cast", fmt, G)
    x = _x(G, 257, H, G)
    q, s = gpu.ep_cast_fp8(bf16_to_dev(x), G, scale_fmt=fmt)
    rq, rs, re8 = oracle.cast_fp8_pow2(x, G, ue8m0=fmt == "ue8m0")
    np.testing.assert_array_equal(fp8_bits(q), rq)
    if fmt == "ue8m0":
        assert s.dtype == torch.uint8
        np.testing.assert_array_equal(s.cpu().numpy(), re8)
    else:
        np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("fmt", ["pow2", "ue8m0"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("G", [128, 32, "H"])
def test_dispatch_scale_formats(gpu, fmt, fused, G):
    T, H = 700, 7168 if G != "H" else 2048
    G = H if G == "H" else G
    announce("dispatch", fmt, fused, G)
    w = ep_inputs.make_workload("fp8", T=T, H=H, drop_p=0.03)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), w.num_experts, w.expert_alignment)
    ref = oracle.get_layout(w.topk_idx, w.num_experts, w.expert_alignment,
                            rows_cap=lay.max_recv_rows)
    q_ref, s_ref, e8_ref = oracle.cast_fp8_pow2(w.x, G, ue8m0=fmt == "ue8m0")
    scales_ref = e8_ref if fmt == "ue8m0" else s_ref
    if fused:
        recv, rs, rw = gpu.ep_dispatch(bf16_to_dev(w.x), lay, to_dev(w.topk_weights),
                                       recv_fp8=True, scale_group=G, zero_padding=True,
                                       scale_fmt=fmt)
    else:
        recv, rs, rw = gpu.ep_dispatch((fp8_to_dev(q_ref), to_dev(scales_ref)), lay,
                                       to_dev(w.topk_weights), zero_padding=True, scale_fmt=fmt)
    exp, exp_s, exp_w = oracle.dispatch(q_ref, ref, w.topk_weights, x_scales=scales_ref,
                                        zero_padding=True)
    np.testing.assert_array_equal(fp8_bits(recv[:ref.R]), exp)
    got_s = rs[:ref.R].cpu().numpy()
    np.testing.assert_array_equal(got_s.view(np.uint8), exp_s.view(np.uint8))
    np.testing.assert_array_equal(rw[:ref.R].cpu().numpy(), exp_w)
    assert lay.check() == 0


def test_partitioned_dispatch_ue8m0(gpu):
    announce("partitioned ue8m0")
    w = ep_inputs.make_workload("skewed", T=500, H=2048)
    lay = gpu.ep_get_layout(to_dev(w.topk_idx), 256, 1, num_partitions=32, partition_layout=True)
    pl = oracle.partition_layout(w.topk_idx, 256, 32)
    q_ref, _, e8 = oracle.cast_fp8_pow2(w.x, 128, ue8m0=True)
    out = gpu.ep_dispatch_partitioned(bf16_to_dev(w.x), lay, to_dev(w.topk_idx), recv_fp8=True,
                                      scale_fmt="ue8m0")
    rx, rs, ri, _ = oracle.dispatch_partitioned(q_ref, w.topk_idx, pl, x_scales=e8)
    np.testing.assert_array_equal(fp8_bits(out[0])[:pl.Rp], rx)
    np.testing.assert_array_equal(out[1].cpu().numpy()[:pl.Rp], rs)
    np.testing.assert_array_equal(out[2].cpu().numpy()[:pl.Rp], ri)


def test_ue8m0_decodes_to_pow2_scales(gpu):
    """The UE8M0 bytes decode (2^(b-127)) to the fp32 power-of-two scales,
    and the codes of the two formats are the same."""
    x = bf16_to_dev(_x(9, 300, 1024, 128))
    q1, s1 = gpu.ep_cast_fp8(x, 128, scale_fmt="pow2")
    q2, s2 = gpu.ep_cast_fp8(x, 128, scale_fmt="ue8m0")
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8))
    dec = torch.ldexp(torch.ones_like(s1), s2.to(torch.int32) - 127)
    assert torch.equal(dec, s1)
