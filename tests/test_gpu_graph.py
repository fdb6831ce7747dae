"""The path under HIP graph capture: layout (which then takes its two-kernel
form), dispatch and combine captured once and replayed with new inputs, with
eager work and synchronisation between replays; every replay must equal the
eager (cooperative single-launch layout) results bit for bit."""
import numpy as np
import pytest
import torch

import ep_inputs
from gpu_util import announce, bf16_to_dev, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu):
    T, H, E, K, A = 1000, 1024, 256, 8, 128
    rows = gpu.worst_case_recv_rows(T, K, E, A)
    dev = "cuda:0"
    s_idx = torch.empty((T, K), dtype=torch.int64, device=dev)
    s_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    s_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    s_y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    recv = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    rw = torch.empty(rows, dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def fill(seed):
        w = ep_inputs.make_workload("prefill", seed=seed, T=T, H=H)
        s_idx.copy_(to_dev(w.topk_idx))
        s_w.copy_(to_dev(w.topk_weights))
        s_x.copy_(bf16_to_dev(w.x))
        s_y.copy_(bf16_to_dev(ep_inputs.make_y(w.rng, rows, H)))

    fill(0)
    lay = gpu.ep_get_layout(s_idx, E, A)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        gpu.ep_get_layout(s_idx, E, A, layout=lay)     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu.ep_get_layout(s_idx, E, A, layout=lay)
        gpu.ep_dispatch(s_x, lay, s_w, out=(recv, None, rw), zero_padding=True)
        gpu.ep_combine(s_y, lay, s_w, out=out)
    for seed in (1, 2, 3, 4):
        announce("graph replay", seed)
        fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [lay.dst_slot.clone(), lay.expert_offset.clone(), recv.clone(), rw.clone(), out.clone()]
        # eager reference on the same inputs (cooperative layout path)
        lay_e = gpu.ep_get_layout(s_idx, E, A)
        recv_e, _, rw_e = gpu.ep_dispatch(s_x, lay_e, s_w, zero_padding=True)
        out_e, _ = gpu.ep_combine(s_y, lay_e, s_w)
        torch.cuda.synchronize()
        R = int(lay_e.expert_offset[-1].item())
        assert torch.equal(got[0], lay_e.dst_slot)
        assert torch.equal(got[1], lay_e.expert_offset)
        assert torch.equal(got[2][:R].view(torch.int16), recv_e[:R].view(torch.int16))
        assert torch.equal(got[3][:R], rw_e[:R])
        assert torch.equal(got[4].view(torch.int16), out_e.view(torch.int16))
