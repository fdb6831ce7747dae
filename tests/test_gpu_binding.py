"""The binding refuses buffers the kernels would misread or overrun (wrong
dtype, width or row count) before anything is launched."""
import numpy as np
import pytest
import torch

import ep_inputs
from gpu_util import announce, bf16_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _setup(gpu, partition=False):
    w = ep_inputs.make_workload("prefill", T=64, H=256, E=16, K=4, A=4)
    idx = to_dev(w.topk_idx)
    lay = gpu.ep_get_layout(idx, 16, 4, 2, partition_layout=partition)
    return w, idx, lay


def test_dispatch_rejects_bad_buffers(gpu):
    announce("binding checks: dispatch")
    w, idx, lay = _setup(gpu)
    x, wts = bf16_to_dev(w.x), to_dev(w.topk_weights)
    rows, dev = lay.max_recv_rows, "cuda:0"
    bad = [
        dict(out=(torch.empty((rows, 256), dtype=torch.uint8, device=dev), None, None)),
        dict(out=(torch.empty((rows - 1, 256), dtype=torch.bfloat16, device=dev), None, None)),
        dict(out=(torch.empty((rows, 128), dtype=torch.bfloat16, device=dev), None, None)),
        dict(out=(None, None, torch.empty(rows - 1, dtype=torch.float32, device=dev))),
        dict(out=(None, None, torch.empty(rows, dtype=torch.float64, device=dev))),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            gpu.ep_dispatch(x, lay, wts, **kw)
    with pytest.raises(ValueError):
        gpu.ep_dispatch(x, lay, wts.double())
    with pytest.raises(ValueError):
        gpu.ep_dispatch(x, lay, wts[:, :2].contiguous())
    with pytest.raises(ValueError):     # fp32 scales for a UE8M0 dispatch
        gpu.ep_dispatch(x, lay, wts, recv_fp8=True, scale_fmt="ue8m0",
                        out=(None, torch.empty((rows, 2), dtype=torch.float32, device=dev), None))
    with pytest.raises(ValueError):     # scale rows of the wrong width
        gpu.ep_dispatch(x, lay, wts, recv_fp8=True,
                        out=(None, torch.empty((rows, 4), dtype=torch.float32, device=dev), None))
    q, s = gpu.ep_cast_fp8(x, 128)
    with pytest.raises(ValueError):     # scales not [T, H / G]
        gpu.ep_dispatch((q, s[:32].contiguous()), lay, wts)
    recv, _, rw = gpu.ep_dispatch(x, lay, wts)    # the good call still works
    torch.cuda.synchronize()
    assert lay.check() == 0


def test_combine_and_cast_reject_bad_buffers(gpu):
    announce("binding checks: combine, cast")
    w, idx, lay = _setup(gpu)
    x, wts = bf16_to_dev(w.x), to_dev(w.topk_weights)
    dev = "cuda:0"
    y = torch.zeros((lay.max_recv_rows, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        gpu.ep_combine(y, lay, wts, out=torch.empty((63, 256), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        gpu.ep_combine(y, lay, wts, out=torch.empty((64, 256), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        gpu.ep_combine(y, lay, wts.double())
    with pytest.raises(ValueError):
        gpu.ep_combine(y, lay, wts, recv_topk_weights=torch.ones(3, device=dev))
    with pytest.raises(ValueError):
        gpu.ep_combine_reduced(y, lay, idx.int(), wts)
    with pytest.raises(ValueError):
        gpu.ep_cast_fp8(x, 128, out=(torch.empty((64, 256), dtype=torch.uint8, device=dev),
                                     torch.empty((64, 1), dtype=torch.float32, device=dev)))
    with pytest.raises(ValueError):
        gpu.ep_cast_fp8(x, 128, out=(torch.empty((64, 255), dtype=torch.uint8, device=dev),
                                     torch.empty((64, 2), dtype=torch.float32, device=dev)))
    out, _ = gpu.ep_combine(y, lay, wts)
    torch.cuda.synchronize()
    assert (out.float() == 0).all()


def test_partitioned_calls_reject_bad_buffers(gpu):
    announce("binding checks: partitioned")
    w, idx, lay = _setup(gpu, partition=True)
    x, wts = bf16_to_dev(w.x), to_dev(w.topk_weights)
    dev, rows = "cuda:0", 64 * 2
    with pytest.raises(ValueError):
        gpu.ep_dispatch_partitioned(x, lay, idx.int(), wts)
    with pytest.raises(ValueError):
        gpu.ep_dispatch_partitioned(x, lay, idx, wts, out=(
            None, None, torch.empty((rows, 4), dtype=torch.int32, device=dev), None))
    with pytest.raises(ValueError):
        gpu.ep_dispatch_partitioned(x, lay, idx, wts, out=(
            None, None, None, torch.empty((rows, 3), dtype=torch.float32, device=dev)))
    recv, _, _, _ = gpu.ep_dispatch_partitioned(x, lay, idx, wts)
    with pytest.raises(ValueError):
        gpu.ep_combine_partitioned(recv, lay, out=torch.empty((64, 128), dtype=torch.bfloat16,
                                                               device=dev))
    gpu.ep_combine_partitioned(recv, lay)
    torch.cuda.synchronize()
    assert lay.check() == 0
