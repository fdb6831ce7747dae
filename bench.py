"""Benchmark: MoE dispatch + combine on one MI355X.

One step = the whole hot path over one batch: ep_get_layout (routing count,
padded scan, slot map) -> ep_dispatch (bf16 row scatter) -> ep_combine
(weighted reduction back to the tokens), on the prefill workload: 4096
tokens x hidden 7168 bf16, 256 experts, top-8 from unbalanced gate scores,
~2% of slots -1, expert_alignment 128.  Inputs are resident in HBM before
the timed region.

Prints one JSON line.  `value` is dispatch+combine throughput in GB/s of
algorithmic bytes (what the method must move: each token row read once,
every valid (token, expert) row written once, and the reverse for combine,
plus the routing tables); `tokens_per_s` is the same step counted in tokens.
The headline region runs the K steps back to back between two events on
the launch stream.  Per-kernel durations come from a second pass over the
same K steps with HIP events recorded on the launch stream between the
calls (each event record leaves a few microseconds of idle GPU time, so they
stay out of the headline region); `roofline` reports the longer of the two
row kernels against MI355X's 8 TB/s HBM peak.  `cpu_baseline` times the CPU
oracle (single thread) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
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
    h = hashlib.sha256()
    d = os.path.join(ROOT, "combine_ep_get_layout_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
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


def cpu_baseline(w, budget_s=12.0):
    """The oracle, as it stands, on a token prefix of the same workload."""
    import oracle
    T_s = 512
    idx = w.topk_idx[:T_s]
    wt = w.topk_weights[:T_s]
    x = w.x[:T_s]
    lay = oracle.get_layout(idx, w.num_experts, w.expert_alignment)
    import ep_inputs
    y = ep_inputs.make_y(ep_inputs.make_rng(2), lay.R, w.hidden)
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or len(times) < 2:
        t0 = time.perf_counter()
        lay = oracle.get_layout(idx, w.num_experts, w.expert_alignment)
        oracle.dispatch(x, lay, wt)
        oracle.combine_f32(y, lay.dst, wt)
        times.append(time.perf_counter() - t0)
        if len(times) >= 20:
            break
    N = int((idx >= 0).sum())
    lb, rb, cb = algorithmic_bytes(T_s, w.hidden, w.num_topk, N, lay.R)
    med = statistics.median(times)
    return {"value": round((lb + rb + cb) / med / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"first {T_s} of {w.num_tokens} prefill tokens (layout + bf16 dispatch + "
                      f"fp32 ordered combine), median of {len(times)} runs, "
                      f"{med * 1e3:.1f} ms per run, tokens/s {T_s / med:.1f}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU's share only; --gpus {args.gpus} is not "
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

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ep.ep_get_layout(idx, E, A, w.num_partitions, w.capacity, layout=lay)
        if ev is not None:
            ev[1].record()
        ep.ep_dispatch(x, lay, wts, out=(recv, None, recv_w))
        if ev is not None:
            ev[2].record()
        ep.ep_combine(y, lay, wts, out=out)
        if ev is not None:
            ev[3].record()

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
    # per-kernel pass: the same steps with events between the calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    lay_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    dis_ms = statistics.mean(e[1].elapsed_time(e[2]) for e in evs)
    com_ms = statistics.mean(e[2].elapsed_time(e[3]) for e in evs)
    assert lay.check() == 0

    lb, rb, cb = algorithmic_bytes(T, H, K, N, R)
    total = lb + rb + cb
    value = total / (ms_step * 1e-3) / 1e9
    kern = {
        "layout": {"ms": lay_ms, "bytes": lb, "GBps": lb / (lay_ms * 1e-3) / 1e9},
        "dispatch_rows": {"ms": dis_ms, "bytes": rb, "GBps": rb / (dis_ms * 1e-3) / 1e9},
        "combine": {"ms": com_ms, "bytes": cb, "GBps": cb / (com_ms * 1e-3) / 1e9},
    }
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
        "roofline": roof,
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kern.items()},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
