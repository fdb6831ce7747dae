"""Benchmark: MoE dispatch + combine on one MI355X.

One step = the whole hot path over one batch: ep_dispatch_with_layout
(routing count, padded scan and slot map, bf16 row scatter, in one call)
-> ep_combine (weighted reduction back to the tokens), on the prefill
workload: 4096
tokens x hidden 7168 bf16, 256 experts, top-8 from unbalanced gate scores,
~2% of slots -1, expert_alignment 128.  Inputs are resident in HBM before
the timed region.

Prints one JSON line.  `value` is dispatch+combine throughput in GB/s of
algorithmic bytes (what the method must move: each token row read once,
every valid (token, expert) row written once, and the reverse for combine,
plus the routing tables); `tokens_per_s` is the same step counted in tokens.
The headline region runs the K steps back to back between two events on
the launch stream.  Per-kernel durations come from HIP events on the same
stream around K back-to-back launches of each operation (an event record
between launches would leave a few microseconds of idle GPU time);
`roofline` reports the longer of the two row kernels (the dispatch rows are
timed on a reused layout, where the call is that one kernel) against
MI355X's 8 TB/s HBM peak.  `kernels` also times the low-latency combine's
10-bit logarithmic payload (use_logfmt): `logfmt_encode` of the N receive
rows that hold a pair (padding rows skipped) and `combine_logfmt`, the
combine that reads that payload (N payload rows of H + H/4 + H/64 bytes
instead of 2H); the decode workload of `other_workloads` times both too.  `cold_cache` times each
operation after a 768 MiB flush, `torch_reference` PyTorch's own
index_copy_ / index_select over the same routed slots, and `cpu_baseline`
the CPU oracle on the same whole batch, on one thread and on the host's
threads.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(T, H, K, N, R, elem=2):
    """Bytes the method must move (per call)."""
    layout = T * K * 8 + T * K * 4 + R * 4                 # idx read, dst + src_of_slot written
    rows = T * H * elem + N * H * elem + T * K * 4 + T * K * 4 + R * 4   # x, rows, dst, w, recv_w
    combine = N * H * elem + T * K * 8 + T * H * elem      # y rows, dst + w, out
    return layout, rows, combine


def kernel_source_hash():
    """Hash of the device sources (every csrc file but the host-only C-ABI
    layer) with comments and whitespace removed: profiles/traffic.json is used
    only while it matches, so any change to the code voids it and a change to
    the comments does not."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "combine_ep_get_layout_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f == "ep_api.hip":
            continue
        with open(os.path.join(d, f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(f.encode() + " ".join(src.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM bytes per launch measured by rocprofv3 PMC runs (profiles/), if they
    were taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        data = json.load(f)
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    return data.get("kernels", {}).get(name)


def partitioned_legs(ep, torch, dev, w, idx, wts, x, y, lay, out_c, per_op):
    """The non-expanded partition layout, its dispatch and combine, and the
    two-level combine on the expanded layout (algorithmic bytes per op:
    rows moved plus the per-row metadata each kernel reads or writes)."""
    T, H, E, K, P = w.num_tokens, w.hidden, w.num_experts, w.num_topk, w.num_partitions
    A, C = w.expert_alignment, w.capacity
    pl = ep.ep_get_layout(idx, E, A, P, C, partition_layout=True)
    Rp = pl.num_partition_rows()
    N = int((w.topk_idx >= 0).sum())
    res = {"Rp": Rp}
    res["layout_partitioned"] = per_op(
        lambda: ep.ep_get_layout(idx, E, A, P, C, layout=pl, partition_layout=True),
        T * K * 8 + T * K * 4 + T * P + T * P * 4 + R_of(pl) * 4, T)
    recv = torch.empty((Rp, H), dtype=torch.bfloat16, device=dev)
    ri = torch.empty((Rp, K), dtype=torch.int64, device=dev)
    rw = torch.empty((Rp, K), dtype=torch.float32, device=dev)
    meta = T * P * 4 + T * K * 12
    res["dispatch_partitioned"] = per_op(
        lambda: ep.ep_dispatch_partitioned(x, pl, idx, wts, num_recv_rows=Rp,
                                           out=(recv, None, ri, rw)),
        T * H * 2 + Rp * H * 2 + Rp * K * 12 + meta, T)
    res["combine_partitioned"] = per_op(
        lambda: ep.ep_combine_partitioned(recv, pl, out=out_c), Rp * H * 2 + T * H * 2 + T * P * 4, T)
    res["combine_reduced"] = per_op(
        lambda: ep.ep_combine_reduced(y, lay, idx, wts, out=out_c),
        N * H * 2 + T * H * 2 + T * K * 16, T)
    assert pl.check() == 0
    del recv, ri, rw
    return res


def R_of(lay):
    return int(lay.expert_offset[-1].item())


def other_workloads(ep, torch, dev, steps, cold_iters=0):
    """Per-operation timings for the fp8, decode, skewed and tiny workloads
    (K back-to-back launches between two events; algorithmic bytes per op).
    With cold_iters > 0 each operation is also timed alone that many times
    after a 768 MiB write that evicts L2 and the memory-side cache (median in
    cold_us): back to back, an operation whose buffers fit that 256 MB cache
    finds them there."""
    import ep_inputs

    flush = torch.empty(768 << 20, dtype=torch.uint8, device=dev) if cold_iters > 0 else None

    def per_op(fn, nbytes, T):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        r = {"us": round(ms * 1e3, 2), "tokens_per_s": round(T / (ms * 1e-3), 1)}
        if nbytes:
            r["GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            r["hbm_frac"] = round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        if flush is not None:
            pairs = []
            for _ in range(cold_iters):
                flush.fill_(1)
                c0 = torch.cuda.Event(enable_timing=True)
                c1 = torch.cuda.Event(enable_timing=True)
                c0.record()
                fn()
                c1.record()
                pairs.append((c0, c1))
            torch.cuda.synchronize()
            cus = float(np.median([a.elapsed_time(b) * 1e3 for a, b in pairs]))
            r["cold_us"] = round(cus, 2)
            if nbytes:
                r["cold_GBps"] = round(nbytes / (cus * 1e-6) / 1e9, 1)
                r["cold_hbm_frac"] = round(nbytes / (cus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        return r

    out = {}
    for name in ("fp8", "decode", "skewed", "tiny"):
        w = ep_inputs.make_workload(name)
        T, H, E, K, A = w.num_tokens, w.hidden, w.num_experts, w.num_topk, w.expert_alignment
        idx = torch.from_numpy(w.topk_idx).to(dev)
        wts = torch.from_numpy(w.topk_weights).to(dev)
        x = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
        lay = ep.ep_get_layout(idx, E, A, w.num_partitions, w.capacity)
        rows = lay.max_recv_rows
        R = lay.num_recv_rows()
        N = int((w.topk_idx >= 0).sum())
        y = torch.randn((rows, H), device=dev).to(torch.bfloat16)
        res = {"T": T, "H": H, "E": E, "K": K, "A": A, "P": w.num_partitions,
               "C": w.capacity, "N": N, "R": R}
        lb, rb, cb = algorithmic_bytes(T, H, K, N, R)
        res["layout"] = per_op(lambda: ep.ep_get_layout(idx, E, A, w.num_partitions, w.capacity,
                                                        layout=lay), lb, T)
        out_c = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        if name == "fp8":
            G = w.fp8_group
            q, sc = ep.ep_cast_fp8(x, G)
            recv8 = torch.empty((rows, H), dtype=torch.float8_e4m3fn, device=dev)
            rs = torch.empty((rows, H // G), dtype=torch.float32, device=dev)
            rw = torch.empty(rows, dtype=torch.float32, device=dev)
            srow = H // G * 4
            res["cast_fp8"] = per_op(lambda: ep.ep_cast_fp8(x, G, out=(q, sc)),
                                     T * H * 2 + T * H + T * srow, T)
            res["dispatch_fp8"] = per_op(lambda: ep.ep_dispatch((q, sc), lay, wts, out=(recv8, rs, rw)),
                                         T * (H + srow) + N * (H + srow) + T * K * 8 + R * 4, T)
            res["dispatch_fused_cast"] = per_op(
                lambda: ep.ep_dispatch(x, lay, wts, recv_fp8=True, out=(recv8, rs, rw)),
                T * H * 2 + N * (H + srow) + T * K * 8 + R * 4, T)
            res["dispatch_fused_cast_with_layout"] = per_op(
                lambda: ep.ep_dispatch_with_layout(x, idx, E, A, wts, w.num_partitions, w.capacity,
                                                   layout=lay, recv_fp8=True, out=(recv8, rs, rw)),
                lb + T * H * 2 + N * (H + srow) + T * K * 8 + R * 4, T)
        else:
            recv = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
            rw = torch.empty(rows, dtype=torch.float32, device=dev)
            zero = w.zero_padding
            nb = rb + ((R - N) * H * 2 if zero else 0)
            res["dispatch"] = per_op(lambda: ep.ep_dispatch(x, lay, wts, zero_padding=zero,
                                                            out=(recv, None, rw)), nb, T)
            res["dispatch_with_layout"] = per_op(
                lambda: ep.ep_dispatch_with_layout(x, idx, E, A, wts, w.num_partitions, w.capacity,
                                                   layout=lay, zero_padding=zero,
                                                   out=(recv, None, rw)), lb + nb, T)
            if zero:
                res["dispatch"]["valid_row_GBps"] = round(rb / (res["dispatch"]["us"] * 1e-6) / 1e9, 1)
            del recv
        res["combine"] = per_op(lambda: ep.ep_combine(y, lay, wts, out=out_c), cb, T)
        if name == "decode":
            # the low-latency combine's 10-bit payload: only the N rows of the
            # capacity region that hold a pair are encoded
            prow = H + H // 4 + 2 * (H // 128)
            y_r = y[:R]
            pay = ep.ep_logfmt_encode(y_r, layout=lay)
            res["logfmt_encode"] = per_op(lambda: ep.ep_logfmt_encode(y_r, out=pay, layout=lay),
                                          N * (H * 2 + prow), T)
            res["combine_logfmt"] = per_op(lambda: ep.ep_combine_logfmt(pay, H, lay, wts, out=out_c),
                                           N * prow + T * K * 8 + T * H * 2, T)
            del pay, y_r
        assert lay.check() == 0
        if w.num_partitions > 1:
            res.update(partitioned_legs(ep, torch, dev, w, idx, wts, x, y, lay, out_c, per_op))
        out[name] = res
        del y, x, lay
        torch.cuda.empty_cache()
    return out


def row_placement(ep, torch, dev, steps, iters):
    """The same dispatch kernel moving the same kind of bytes, with only the
    placement of the receive rows changed: the prefill routing (top-8 of 256
    experts: ~256 receive segments written at once), and a routing that sends
    every token's k-th pair to expert 32k (8 segments, each written in
    address order, one front per segment).  Also the sequential write of the
    same receive buffer by torch's fill kernel.  For each routing,
    `stores_only` runs the same kernel with every token row replaced by a
    register pattern (no token row read): the cost of the scatter's writes
    alone.  Back to back and cold."""
    import ep_inputs
    w = ep_inputs.make_workload("prefill")
    T, H, E, K, A = w.num_tokens, w.hidden, w.num_experts, w.num_topk, w.expert_alignment
    x = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
    wts = torch.from_numpy(w.topk_weights).to(dev)
    fronts = np.tile(np.arange(K, dtype=np.int64) * (E // K), (T, 1))
    out = {}
    recv = None
    for name, idx_np in (("prefill_routing", w.topk_idx), ("eight_fronts", fronts)):
        idx = torch.from_numpy(idx_np).to(dev)
        lay = ep.ep_get_layout(idx, E, A)
        R = lay.num_recv_rows()
        N = int((idx_np >= 0).sum())
        if recv is None or recv.shape[0] < lay.max_recv_rows:
            recv = torch.empty((lay.max_recv_rows, H), dtype=torch.bfloat16, device=dev)
        rw = torch.empty(lay.max_recv_rows, dtype=torch.float32, device=dev)
        nbytes = algorithmic_bytes(T, H, K, N, R)[1]
        fn = lambda: ep.ep_dispatch(x, lay, wts, out=(recv, None, rw))
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        cold = cold_per_op(torch, dev, iters, {name: fn})[name]
        out[name] = {"N": N, "R": R, "bytes": nbytes, "us": round(us, 2),
                     "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "cold_us": cold["median_us"],
                     "cold_GBps": round(nbytes / (cold["median_us"] * 1e-6) / 1e9, 1)}
        # the same kernel's stores alone: every row a register pattern, no
        # token row read (ep_probe_dispatch_stores); N rows of H bf16 written
        probe = lambda: ep.ep_probe_dispatch_stores(recv, lay)
        probe()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            probe()
        e1.record()
        torch.cuda.synchronize()
        sus = e0.elapsed_time(e1) / steps * 1e3
        scold = cold_per_op(torch, dev, iters, {"stores": probe})["stores"]
        sb = N * H * 2
        out[name]["stores_only"] = {"bytes": sb, "us": round(sus, 2),
                                    "GBps": round(sb / (sus * 1e-6) / 1e9, 1),
                                    "cold_us": scold["median_us"],
                                    "cold_GBps": round(sb / (scold["median_us"] * 1e-6) / 1e9, 1)}
        assert lay.check() == 0
        del lay, rw
    fill = recv[:T * K]
    cold = cold_per_op(torch, dev, iters, {"fill": lambda: fill.fill_(1.0)})["fill"]
    nb = fill.numel() * 2
    out["sequential_write"] = {"bytes": nb, "cold_us": cold["median_us"],
                               "cold_GBps": round(nb / (cold["median_us"] * 1e-6) / 1e9, 1)}
    del recv, fill, x
    torch.cuda.empty_cache()
    return out


def cold_per_op(torch, dev, iters, ops):
    """Each operation timed alone, `iters` times, after a 768 MiB write that
    evicts L2 and the memory-side cache; the flush is outside the event pair.
    Returns median / p10 / p90 in microseconds."""
    flush = torch.empty(768 << 20, dtype=torch.uint8, device=dev)
    out = {}
    for name, fn in ops.items():
        fn()
        pairs = []
        for _ in range(iters):
            flush.fill_(1)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
        out[name] = {"median_us": round(float(np.median(us)), 2),
                     "p10_us": round(float(np.percentile(us, 10)), 2),
                     "p90_us": round(float(np.percentile(us, 90)), 2)}
    del flush
    torch.cuda.empty_cache()
    return out


def torch_reference(torch, dev, iters, lay, x, K, N):
    """PyTorch's own row moves at the same routed slots, cold (768 MiB flush
    before each, median of `iters`): index_copy_ of the N pre-expanded
    token rows into their slots (the scatter; the rows are expanded outside
    the timed region), and index_select of x by each used slot's token in
    slot order (the gather form of the same permutation)."""
    R = lay.num_recv_rows()
    src = lay.src_of_slot[:R].long()
    used = torch.nonzero(src >= 0).squeeze(1)
    tok = src[used] // K
    rows = x.index_select(0, tok)                  # [N, H], outside the timed region
    recv = torch.empty((R, x.shape[1]), dtype=x.dtype, device=dev)
    gath = torch.empty_like(rows)
    ops = {"index_copy_scatter": lambda: recv.index_copy_(0, used, rows),
           "index_select_gather": lambda: torch.index_select(x, 0, tok, out=gath)}
    res = cold_per_op(torch, dev, iters, ops)
    H = x.shape[1]
    moved = {"index_copy_scatter": 2 * N * H * 2, "index_select_gather": 2 * N * H * 2}
    for k, v in res.items():
        v["bytes_moved"] = moved[k]
        v["GBps_moved"] = round(moved[k] / (v["median_us"] * 1e-6) / 1e9, 1)
    assert torch.equal(recv.index_select(0, used), gath)
    del recv, gath, rows
    return res


def _host_threads():
    """Threads for the all-cores oracle leg: the CPUs this process may run on,
    at most the OMP_NUM_THREADS share (16 if unset)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, int(os.environ.get("OMP_NUM_THREADS", "16") or 16)))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, runs=7):
    """The oracle, as it stands, on the whole prefill batch: layout, bf16
    dispatch and ordered fp32 combine (the same step the GPU line times).
    Timed once on one thread and once with the rows and the combine split
    into token ranges over the host's threads (ctypes releases the GIL, so
    the oracle's own C loops run side by side); the layout stays one call,
    since it fixes the slot order.  Median of `runs` passes each."""
    import concurrent.futures

    import ep_inputs
    import oracle

    T, H, E, K, A = w.num_tokens, w.hidden, w.num_experts, w.num_topk, w.expert_alignment
    idx, wt, x = w.topk_idx, w.topk_weights, w.x
    lay = oracle.get_layout(idx, E, A)
    y = ep_inputs.make_y(ep_inputs.make_rng(2), lay.R, H)
    recv = np.empty((lay.R, H), np.uint16)
    recv_w = np.empty(lay.R, np.float32)
    N = int((idx >= 0).sum())
    lb, rb, cb = algorithmic_bytes(T, H, K, N, lay.R)
    nbytes = lb + rb + cb

    def one_pass(nt, pool):
        t0 = time.perf_counter()
        lay_p = oracle.get_layout(idx, E, A)
        bounds = np.linspace(0, T, nt + 1).astype(int)
        ranges = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        if pool is None:
            oracle.dispatch_tokens(x, lay_p, wt, recv, recv_w, 0, T)
            oracle.combine_f32(y, lay_p.dst, wt)
        else:
            list(pool.map(lambda r: oracle.dispatch_tokens(x, lay_p, wt, recv, recv_w, *r), ranges))
            list(pool.map(lambda r: oracle.combine_f32(y, lay_p.dst, wt, tokens=np.arange(*r)),
                          ranges))
        return time.perf_counter() - t0

    nt = _host_threads()
    one = statistics.median(one_pass(1, None) for _ in range(runs))
    with concurrent.futures.ThreadPoolExecutor(nt) as pool:
        one_pass(nt, pool)
        many = statistics.median(one_pass(nt, pool) for _ in range(runs))
    try:
        n_aff = len(os.sched_getaffinity(0))
    except AttributeError:
        n_aff = None
    return {"value": round(nbytes / many / 1e9, 3), "unit": "GB/s", "cores": nt, "kind": "oracle",
            "sample": f"the whole prefill batch ({T} tokens: layout + bf16 dispatch + ordered "
                      f"fp32 combine, {nbytes / 1e6:.1f} MB of algorithmic bytes), median of "
                      f"{runs} passes; rows and combine split into {nt} token ranges on {nt} "
                      f"threads, layout one call",
            "ms_per_step": round(many * 1e3, 1), "tokens_per_s": round(T / many, 1),
            "one_core": {"value": round(nbytes / one / 1e9, 3), "unit": "GB/s", "cores": 1,
                         "ms_per_step": round(one * 1e3, 1), "tokens_per_s": round(T / one, 1)},
            "nproc": os.cpu_count(), "affinity": n_aff, "cpu_model": _cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the per-operation timings after a cache flush")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before timing, run one plain device copy of MIB MiB (a known-size "
                         "reference for HBM byte counters under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark measures one GPU's share only; --gpus {args.gpus} is not "
              "supported (no collectives, no sharding).", file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_ep_get_layout_amd as ep
    import ep_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = ep_inputs.make_workload(args.workload)
    T, H, E, K, A = w.num_tokens, w.hidden, w.num_experts, w.num_topk, w.expert_alignment
    idx = torch.from_numpy(w.topk_idx).to(dev)
    wts = torch.from_numpy(w.topk_weights).to(dev)
    x = torch.from_numpy(w.x.view(np.int16)).to(dev).view(torch.bfloat16)
    lay = ep.ep_get_layout(idx, E, A, w.num_partitions, w.capacity)
    rows = lay.max_recv_rows
    R = lay.num_recv_rows()
    N = int((w.topk_idx >= 0).sum())
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    y = torch.randn((rows, H), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    recv = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    recv_w = torch.empty(rows, dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def fused_dispatch():
        ep.ep_dispatch_with_layout(x, idx, E, A, wts, w.num_partitions, w.capacity, layout=lay,
                                   out=(recv, None, recv_w))

    def step():
        fused_dispatch()
        ep.ep_combine(y, lay, wts, out=out)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src_c = torch.ones(n, dtype=torch.uint8, device=dev)
        dst_c = torch.empty(n, dtype=torch.uint8, device=dev)
        evict = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        evict.fill_(0)          # push src out of L2 and the memory-side cache
        torch.cuda.synchronize()
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c, evict
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record()
    for i in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_begin.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    # per-operation pass: each operation launched K times back to back between two
    # events on the launch stream (no event between launches, so no idle gaps)
    def per_op(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # the same pass over a layout derived once before the timed region
    # (dispatch rows + combine back to back, the layout handle reused)
    reused_ms = per_op(lambda: (ep.ep_dispatch(x, lay, wts, out=(recv, None, recv_w)),
                                ep.ep_combine(y, lay, wts, out=out)))
    lay_ms = per_op(lambda: ep.ep_get_layout(idx, E, A, w.num_partitions, w.capacity, layout=lay))
    fus_ms = per_op(fused_dispatch)
    dis_ms = per_op(lambda: ep.ep_dispatch(x, lay, wts, out=(recv, None, recv_w)))
    com_ms = per_op(lambda: ep.ep_combine(y, lay, wts, out=out))
    # the low-latency combine's 10-bit logarithmic payload: encode the N
    # receive rows that hold a pair (padding rows skipped by the layout's
    # src_of_slot), then the combine that reads the payload
    y_used = y[:R]
    pay = ep.ep_logfmt_encode(y_used, layout=lay)
    enc_ms = per_op(lambda: ep.ep_logfmt_encode(y_used, out=pay, layout=lay))
    lcm_ms = per_op(lambda: ep.ep_combine_logfmt(pay, H, lay, wts, out=out))
    assert lay.check() == 0
    cold = None
    if not args.no_cold:
        cold = cold_per_op(torch, dev, args.steps, {
            "layout": lambda: ep.ep_get_layout(idx, E, A, w.num_partitions, w.capacity, layout=lay),
            "dispatch_reused_layout": lambda: ep.ep_dispatch(x, lay, wts, out=(recv, None, recv_w)),
            "dispatch_fresh_layout": fused_dispatch,
            "dispatch_fresh_layout_two_calls": lambda: (
                ep.ep_get_layout(idx, E, A, w.num_partitions, w.capacity, layout=lay),
                ep.ep_dispatch(x, lay, wts, out=(recv, None, recv_w))),
            "combine": lambda: ep.ep_combine(y, lay, wts, out=out),
            "logfmt_encode": lambda: ep.ep_logfmt_encode(y_used, out=pay, layout=lay),
            "combine_logfmt": lambda: ep.ep_combine_logfmt(pay, H, lay, wts, out=out),
        })
    reference = None if args.no_cold else torch_reference(torch, dev, args.steps, lay, x, K, N)

    lb, rb, cb = algorithmic_bytes(T, H, K, N, R)
    total = lb + rb + cb
    value = total / (ms_step * 1e-3) / 1e9
    kern = {
        "layout": {"ms": lay_ms, "bytes": lb, "GBps": lb / (lay_ms * 1e-3) / 1e9},
        "dispatch_with_layout": {"ms": fus_ms, "bytes": lb + rb,
                                 "GBps": (lb + rb) / (fus_ms * 1e-3) / 1e9},
        "dispatch_rows": {"ms": dis_ms, "bytes": rb, "GBps": rb / (dis_ms * 1e-3) / 1e9},
        "combine": {"ms": com_ms, "bytes": cb, "GBps": cb / (com_ms * 1e-3) / 1e9},
    }
    pay_row = H + H // 4 + 2 * (H // 128)      # payload bytes per row, tail excluded
    enc_b = N * H * 2 + N * pay_row
    lcm_b = N * pay_row + T * K * 8 + T * H * 2
    kern["logfmt_encode"] = {"ms": enc_ms, "bytes": enc_b, "GBps": enc_b / (enc_ms * 1e-3) / 1e9}
    kern["combine_logfmt"] = {"ms": lcm_ms, "bytes": lcm_b, "GBps": lcm_b / (lcm_ms * 1e-3) / 1e9}
    for k, v in kern.items():   # each operation as a fraction of the HBM roofline, and tokens/s
        v["hbm_frac"] = v["GBps"] / HBM_PEAK_GBS
        v["tokens_per_s"] = T / (v["ms"] * 1e-3)
        v["traffic"] = load_traffic(k)   # HBM bytes per launch from the PMC runs, or None
    dom = "dispatch_rows" if dis_ms >= com_ms else "combine"
    ach = kern[dom]["GBps"]
    tr = load_traffic(dom)
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": tr, "kernel": dom}
    res = {
        "metric": "dispatch+combine GB/s and tokens/s on 1 MI355X; % of HBM roofline",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: T={T} H={H} E={E} top-{K} A={A} "
                               f"P={w.num_partitions} N={N} R={R}",
                   "tokens": T, "hidden": H, "experts": E, "topk": K, "alignment": A},
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "step_reused_layout": {
            "what": "ep_dispatch (bf16 rows) + ep_combine back to back on a layout derived "
                    "before the timed region; not the headline (which derives the layout "
                    "in every step)",
            "ms": round(reused_ms, 5), "bytes": rb + cb,
            "GBps": round((rb + cb) / (reused_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round((rb + cb) / (reused_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(T / (reused_ms * 1e-3), 1)},
        "roofline": roof,
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kern.items()},
        "wall_s_timed": round(wall, 4),
    }
    if cold is not None:
        lb_, rb_, cb_ = algorithmic_bytes(T, H, K, N, R)
        nbytes = {"layout": lb_, "dispatch_reused_layout": rb_, "dispatch_fresh_layout": lb_ + rb_,
                  "dispatch_fresh_layout_two_calls": lb_ + rb_, "combine": cb_,
                  "logfmt_encode": enc_b, "combine_logfmt": lcm_b}
        for k, v in cold.items():
            v["GBps_median"] = round(nbytes[k] / (v["median_us"] * 1e-6) / 1e9, 1)
            v["hbm_frac_median"] = round(v["GBps_median"] / HBM_PEAK_GBS, 4)
        res["cold_cache"] = cold
    if reference is not None:
        res["torch_reference"] = reference
    if not args.no_other_workloads:
        del recv, y, y_used, pay
        torch.cuda.empty_cache()
        res["other_workloads"] = other_workloads(ep, torch, dev, args.steps,
                                                 0 if args.no_cold else min(args.steps, 20))
        if not args.no_cold:
            res["row_placement"] = row_placement(ep, torch, dev, args.steps, min(args.steps, 20))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
