"""The path under HIP graph capture: layout, dispatch and combine captured
once and replayed with new inputs, with eager work and synchronisation
between replays; every replay must equal the eager results bit for bit.
Covers the two-kernel and the one-workgroup layout, the streaming dispatch,
the zero fill of a mostly-padding fixed-capacity region, the fused fp8
cast, and the 10-bit logarithmic payload (encode of the rows holding a pair,
then the combine over it)."""
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
    pay = torch.empty((rows, gpu.logfmt_row_bytes(H)), dtype=torch.uint8, device=dev)
    out_l = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

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
        gpu.ep_logfmt_encode(s_y, out=pay, layout=lay)
        gpu.ep_combine_logfmt(pay, H, lay, s_w, out=out_l)
    for seed in (1, 2, 3, 4):
        announce("graph replay", seed)
        fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [lay.dst_slot.clone(), lay.expert_offset.clone(), recv.clone(), rw.clone(), out.clone(),
               out_l.clone()]
        # eager reference on the same inputs
        lay_e = gpu.ep_get_layout(s_idx, E, A)
        recv_e, _, rw_e = gpu.ep_dispatch(s_x, lay_e, s_w, zero_padding=True)
        out_e, _ = gpu.ep_combine(s_y, lay_e, s_w)
        out_le, _ = gpu.ep_combine_logfmt(gpu.ep_logfmt_encode(s_y), H, lay_e, s_w)
        torch.cuda.synchronize()
        R = int(lay_e.expert_offset[-1].item())
        assert torch.equal(got[0], lay_e.dst_slot)
        assert torch.equal(got[1], lay_e.expert_offset)
        assert torch.equal(got[2][:R].view(torch.int16), recv_e[:R].view(torch.int16))
        assert torch.equal(got[3][:R], rw_e[:R])
        assert torch.equal(got[4].view(torch.int16), out_e.view(torch.int16))
        assert torch.equal(got[5].view(torch.int16), out_le.view(torch.int16))


def test_graph_capacity_fill_small_batch_and_fp8(gpu):
    """A decode-like fixed-capacity dispatch with zero padding (zero fill, then
    the token rows), a 20-token batch (one-workgroup layout) with a fused fp8
    dispatch, and their combines, in one graph."""
    dev = "cuda:0"
    Td, Hd, Ed, Kd, Cd = 100, 512, 64, 4, 64      # T*K*8 <= E*C: the zero-fill path
    Tt, Ht, Et, Kt = 20, 256, 16, 4               # 80 pairs: the one-workgroup layout
    rows_d = Ed * Cd
    rows_t = gpu.worst_case_recv_rows(Tt, Kt, Et, 1)
    st = {n: torch.empty(shape, dtype=dt, device=dev) for n, shape, dt in (
        ("idx_d", (Td, Kd), torch.int64), ("w_d", (Td, Kd), torch.float32),
        ("x_d", (Td, Hd), torch.bfloat16), ("y_d", (rows_d, Hd), torch.bfloat16),
        ("idx_t", (Tt, Kt), torch.int64), ("w_t", (Tt, Kt), torch.float32),
        ("x_t", (Tt, Ht), torch.bfloat16), ("y_t", (rows_t, Ht), torch.bfloat16))}
    recv_d = torch.empty((rows_d, Hd), dtype=torch.bfloat16, device=dev)
    rw_d = torch.empty(rows_d, dtype=torch.float32, device=dev)
    out_d = torch.empty((Td, Hd), dtype=torch.bfloat16, device=dev)
    recv_t = torch.empty((rows_t, Ht), dtype=torch.float8_e4m3fn, device=dev)
    rs_t = torch.empty((rows_t, Ht // 128), dtype=torch.float32, device=dev)
    out_t = torch.empty((Tt, Ht), dtype=torch.bfloat16, device=dev)

    def fill(seed):
        wd = ep_inputs.make_workload("decode", seed=seed, T=Td, H=Hd, E=Ed, K=Kd, C=Cd)
        wt = ep_inputs.make_workload("tiny", seed=seed, T=Tt, H=Ht, E=Et, K=Kt)
        for n, v in (("idx_d", wd.topk_idx), ("w_d", wd.topk_weights), ("idx_t", wt.topk_idx),
                     ("w_t", wt.topk_weights)):
            st[n].copy_(to_dev(v))
        st["x_d"].copy_(bf16_to_dev(wd.x))
        st["x_t"].copy_(bf16_to_dev(wt.x))
        st["y_d"].copy_(bf16_to_dev(ep_inputs.make_y(wd.rng, rows_d, Hd)))
        st["y_t"].copy_(bf16_to_dev(ep_inputs.make_y(wt.rng, rows_t, Ht)))

    def run(lay_d, lay_t, eager):
        gpu.ep_get_layout(st["idx_d"], Ed, 1, 1, Cd, layout=lay_d)
        gpu.ep_get_layout(st["idx_t"], Et, 1, layout=lay_t)
        if eager:
            r = gpu.ep_dispatch(st["x_d"], lay_d, st["w_d"], zero_padding=True)
            q = gpu.ep_dispatch(st["x_t"], lay_t, st["w_t"], recv_fp8=True)
            o_d, _ = gpu.ep_combine(st["y_d"], lay_d, st["w_d"])
            o_t, _ = gpu.ep_combine(st["y_t"], lay_t, st["w_t"])
            return r[0], r[2], q[0], q[1], o_d, o_t
        gpu.ep_dispatch(st["x_d"], lay_d, st["w_d"], zero_padding=True, out=(recv_d, None, rw_d))
        gpu.ep_dispatch(st["x_t"], lay_t, st["w_t"], recv_fp8=True, out=(recv_t, rs_t, None))
        gpu.ep_combine(st["y_d"], lay_d, st["w_d"], out=out_d)
        gpu.ep_combine(st["y_t"], lay_t, st["w_t"], out=out_t)

    fill(0)
    lay_d = gpu.ep_get_layout(st["idx_d"], Ed, 1, 1, Cd)
    lay_t = gpu.ep_get_layout(st["idx_t"], Et, 1)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        run(lay_d, lay_t, False)                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(lay_d, lay_t, False)
    for seed in (1, 2, 3):
        announce("graph replay (capacity fill, small batch, fp8)", seed)
        fill(seed)
        recv_d.view(torch.int16).fill_(0x5A5A)   # the fill must rewrite every padding row
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [recv_d.clone(), rw_d.clone(), recv_t.clone(), rs_t.clone(), out_d.clone(),
               out_t.clone(), lay_t.dst_slot.clone()]
        le_d = gpu.ep_get_layout(st["idx_d"], Ed, 1, 1, Cd)
        le_t = gpu.ep_get_layout(st["idx_t"], Et, 1)
        exp = run(le_d, le_t, True)
        torch.cuda.synchronize()
        R_t = int(le_t.expert_offset[-1].item())
        assert torch.equal(got[0].view(torch.int16), exp[0].view(torch.int16))
        assert torch.equal(got[1], exp[1])
        assert torch.equal(got[2][:R_t].view(torch.uint8), exp[2][:R_t].view(torch.uint8))
        assert torch.equal(got[3][:R_t], exp[3][:R_t])
        assert torch.equal(got[4].view(torch.int16), exp[4].view(torch.int16))
        assert torch.equal(got[5].view(torch.int16), exp[5].view(torch.int16))
        assert torch.equal(got[6], le_t.dst_slot)


@pytest.mark.parametrize("T,H", [(2000, 1024), (17000, 64)])
def test_graph_one_call_and_noalloc_layout(gpu, T, H):
    """ep_dispatch_with_layout + ep_combine (the benchmark's step: count kernel,
    row kernel deriving the slots; at T >= 16,384 the token queue), and
    ep_get_layout_noalloc + ep_dispatch, captured once and replayed with new
    inputs; every replay equals the eager two-call path bit for bit."""
    E, K, A = 256, 8, 128
    dev = "cuda:0"
    rows = gpu.worst_case_recv_rows(T, K, E, A)
    s_idx = torch.empty((T, K), dtype=torch.int64, device=dev)
    s_w = torch.empty((T, K), dtype=torch.float32, device=dev)
    s_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    s_y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    recv = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    rw = torch.empty(rows, dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    recv2 = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    out2 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def fill(seed):
        w = ep_inputs.make_workload("prefill", seed=seed, T=T, H=H)
        s_idx.copy_(to_dev(w.topk_idx))
        s_w.copy_(to_dev(w.topk_weights))
        s_x.copy_(bf16_to_dev(w.x))
        s_y.copy_(bf16_to_dev(ep_inputs.make_y(w.rng, rows, H)))

    fill(0)
    lay = gpu.ep_get_layout(s_idx, E, A)
    lay2 = gpu.ep_get_layout(s_idx, E, A)

    def step():
        gpu.ep_dispatch_with_layout(s_x, s_idx, E, A, s_w, layout=lay, out=(recv, None, rw))
        gpu.ep_combine(s_y, lay, s_w, out=out)
        gpu.ep_get_layout_noalloc(s_idx, lay2)
        gpu.ep_dispatch(s_x, lay2, s_w, out=(recv2, None, None))
        gpu.ep_combine(s_y, lay2, s_w, out=out2)

    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for seed in (1, 2, 3):
        announce("graph replay (one call, no-alloc layout)", T, H, seed)
        fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        lay_e = gpu.ep_get_layout(s_idx, E, A)
        recv_e, _, rw_e = gpu.ep_dispatch(s_x, lay_e, s_w)
        out_e, _ = gpu.ep_combine(s_y, lay_e, s_w)
        torch.cuda.synchronize()
        R = lay_e.num_recv_rows()
        for l in (lay, lay2):
            assert torch.equal(l.dst_slot, lay_e.dst_slot)
            assert torch.equal(l.expert_offset, lay_e.expert_offset)
            assert torch.equal(l.src_of_slot[:R], lay_e.src_of_slot[:R])
            assert int(l.status.item()) == 0
        used = lay_e.src_of_slot[:R] >= 0        # padding rows are left as they were
        for r in (recv, recv2):
            assert torch.equal(r[:R][used].view(torch.int16), recv_e[:R][used].view(torch.int16))
        assert torch.equal(rw[:R], rw_e[:R])
        for o in (out, out2):
            assert torch.equal(o.view(torch.int16), out_e.view(torch.int16))
