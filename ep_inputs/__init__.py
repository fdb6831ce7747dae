"""Seeded synthetic inputs for MoE expert-parallel dispatch / combine.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws random inputs: routing (``topk_idx`` with -1 for
"no expert", ``topk_weights``), token rows ``x`` and expert outputs ``y``.  It
holds none of the method's arithmetic (no counting, no layout, no casting,
no reduction); bf16 values are produced by rounding fp32 normals with torch's
CPU cast, which is input generation, not the method.

Every generator takes a ``numpy.random.Generator`` (PCG64) so that callers
draw routing first, then ``x``, then ``y`` from one seeded stream.

Workloads (shapes and distributions of the DeepEP v2 test page's dispatch /
combine problem, "DeepEP test target API reference", sections 2.1-2.2 and the
routing generator of section 4.3, restated as explicit distributions):

=========  =====  =====  ===  ==  ====================================  =====
name       T      H      E    K   routing                               A
=========  =====  =====  ===  ==  ====================================  =====
tiny       64     256    8    2   uniform distinct, no -1               1
prefill    4096   7168   256  8   N(0,1)+bias N(0,sd 2), top-8, 2% -1   128
fp8        4096   7168   256  8   as prefill; x cast per 128-channel    128
decode     128    7168   256  8   uniform distinct; capacity 128, zero  1
skewed     32768  7168   256  8   Zipf(1.2) popularity; 32 partitions   128
=========  =====  =====  ===  ==  ====================================  =====
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "make_rng", "bf16_normal", "routing_uniform", "routing_prefill",
    "routing_zipf", "softmax_weights", "make_workload", "make_y", "WORKLOADS",
    "worst_case_recv_rows", "make_y_wide",
]


def make_rng(seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_normal(rng: np.random.Generator, shape, chunk_rows: int = 8192) -> np.ndarray:
    """N(0,1) fp32 draws rounded to bf16; returned as uint16 bit patterns."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    if out.size == 0:
        return out
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = _f32_to_bf16_bits(
            rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32))
    return out


def softmax_weights(logits: np.ndarray) -> np.ndarray:
    """Row softmax in float64, stored as fp32 routing weights."""
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def routing_uniform(rng, T, E, K):
    """K distinct experts per token, uniformly at random (random order);
    weights = softmax of K N(0,1) logits."""
    if K > E:
        raise ValueError("K > E")
    keys = rng.random((T, E))
    idx = np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int64)
    w = softmax_weights(rng.standard_normal((T, K)))
    return idx, w


def routing_prefill(rng, T, E, K, bias_sd=2.0, drop_p=0.02):
    """Unbalanced gate: scores = N(0,1) + per-expert bias N(0, sd=bias_sd);
    top-K by score (descending, ties to the lower id); weights = softmax of
    the K selected scores; each slot independently dropped to -1 with
    probability drop_p; surviving weights renormalised to sum to one (a fully
    dropped token keeps all-zero weights)."""
    bias = rng.normal(0.0, bias_sd, size=E)
    scores = rng.standard_normal((T, E)) + bias[None, :]
    order = np.argsort(-scores, axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(scores, order, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    drop = rng.random((T, K)) < drop_p
    idx = order.astype(np.int64)
    idx[drop] = -1
    w = np.where(drop, 0.0, w)
    s = w.sum(axis=1, keepdims=True)
    w = np.divide(w, s, out=np.zeros_like(w), where=s > 0)
    return idx, w.astype(np.float32)


def routing_zipf(rng, T, E, K, s=1.2):
    """Expert r-1 has popularity proportional to r**-s (r = 1..E); K distinct
    experts per token are drawn without replacement in proportion to it
    (Gumbel-top-K on log popularity); weights = softmax of K N(0,1) logits."""
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    idx = np.empty((T, K), dtype=np.int64)
    step = 4096
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        g = rng.gumbel(size=(t1 - t0, E))
        idx[t0:t1] = np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :K]
    w = softmax_weights(rng.standard_normal((T, K)))
    return idx, w


@dataclasses.dataclass
class Workload:
    name: str
    num_tokens: int
    hidden: int
    num_experts: int
    num_topk: int
    expert_alignment: int
    num_partitions: int
    capacity: int            # 0 = compact padded layout, >0 = fixed per-expert capacity
    zero_padding: bool
    fp8: bool                # x is cast to e4m3 per (token, group) before dispatch
    fp8_group: int
    topk_idx: np.ndarray     # int64 [T, K], -1 = no expert
    topk_weights: np.ndarray  # float32 [T, K]
    x: Optional[np.ndarray]  # uint16 bf16 bits [T, H]
    rng: np.random.Generator  # continues after x: draw y from it

    def worst_case_recv_rows(self) -> int:
        return worst_case_recv_rows(self.num_tokens, self.num_topk, self.num_experts,
                                    self.expert_alignment, self.capacity)


def worst_case_recv_rows(T, K, E, A, capacity=0):
    """Receive rows that always suffice: E*C in fixed-capacity mode, else every
    pair plus A-1 padding rows for each expert that can be non-empty."""
    if capacity > 0:
        return E * capacity
    return T * K + min(E, T * K) * (A - 1)


WORKLOADS = {
    #          T      H     E    K  A    P   C    zero   fp8    routing
    "tiny":    (64,   256,  8,   2, 1,   1,  0,   False, False, "uniform"),
    "prefill": (4096, 7168, 256, 8, 128, 1,  0,   False, False, "prefill"),
    "fp8":     (4096, 7168, 256, 8, 128, 1,  0,   False, True,  "prefill"),
    "decode":  (128,  7168, 256, 8, 1,   1,  128, True,  False, "uniform"),
    "skewed":  (32768, 7168, 256, 8, 128, 32, 0,  False, False, "zipf"),
}


def make_workload(name: str, seed: int = 0, with_x: bool = True, **over) -> Workload:
    """Build one named workload (overrides: T, H, E, K, A, P, C, zero, routing)."""
    T, H, E, K, A, P, C, zero, fp8, routing = WORKLOADS[name]
    T = over.pop("T", T)
    H = over.pop("H", H)
    E = over.pop("E", E)
    K = over.pop("K", K)
    A = over.pop("A", A)
    P = over.pop("P", P)
    C = over.pop("C", C)
    zero = over.pop("zero", zero)
    routing = over.pop("routing", routing)
    drop_p = over.pop("drop_p", 0.02)
    if over:
        raise TypeError(f"unknown overrides {sorted(over)}")
    rng = make_rng(seed)
    if routing == "uniform":
        idx, w = routing_uniform(rng, T, E, K)
    elif routing == "prefill":
        idx, w = routing_prefill(rng, T, E, K, drop_p=drop_p)
    elif routing == "zipf":
        idx, w = routing_zipf(rng, T, E, K)
    else:
        raise ValueError(routing)
    x = bf16_normal(rng, (T, H)) if with_x else None
    return Workload(name, T, H, E, K, A, P, C, bool(zero), fp8, 128, idx, w, x, rng)


def make_y(rng: np.random.Generator, rows: int, hidden: int) -> np.ndarray:
    """Expert outputs for combine: bf16 N(0,1), uint16 bits [rows, hidden]."""
    return bf16_normal(rng, (rows, hidden))


def make_y_wide(rng: np.random.Generator, rows: int, hidden: int, specials: bool = True) -> np.ndarray:
    """Expert outputs with a wide dynamic range, for the logarithmic payload:
    per 128-channel group a scale 2^U(-60, 60), per element a spread of
    2^N(0, 5) and a random sign; about 3% exact zeros (both signs), 1% bf16
    subnormals, a few magnitudes at the top of the bf16 range, and with
    ``specials`` about 1% of groups holding an infinity or a NaN.  uint16
    bits [rows, hidden]; hidden a multiple of 128."""
    shape = (int(rows), int(hidden))
    if rows == 0:
        return np.empty(shape, np.uint16)
    G = hidden // 128
    scale = rng.uniform(-60.0, 60.0, (rows, G, 1))
    spread = rng.normal(0.0, 5.0, (rows, G, 128))
    sign = np.where(rng.random((rows, G, 128)) < 0.5, -1.0, 1.0)
    v = (sign * np.exp2(scale + spread)).astype(np.float32).reshape(shape)
    out = _f32_to_bf16_bits(v)
    u = rng.random(shape)
    out[u < 0.03] = np.where(rng.random(shape) < 0.5, 0x0000, 0x8000)[u < 0.03]
    sub = (u >= 0.03) & (u < 0.04)
    out[sub] = rng.integers(1, 128, shape, dtype=np.uint16)[sub] | \
        np.where(rng.random(shape) < 0.5, 0, 0x8000).astype(np.uint16)[sub]
    top = (u >= 0.04) & (u < 0.0405)
    out[top] = rng.integers(0x7F70, 0x7F80, shape, dtype=np.uint16)[top]
    if specials:
        grp = rng.random((rows, G)) < 0.01
        r, g = np.nonzero(grp)
        c = g * 128 + rng.integers(0, 128, r.size)
        out[r, c] = rng.choice(np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1], np.uint16), r.size)
    return out
