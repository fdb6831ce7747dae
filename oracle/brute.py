"""Pure-Python brute force for tiny routing inputs (TEST INFRASTRUCTURE ONLY).

Written separately from ep_oracle.c, by a different route, so that the two
pin each other: here the receive layout is obtained by listing every valid
(token, k) pair, sorting the list by (expert, flat index t*K+k), and placing
expert e's segment after the padded segments of all lower experts; the C
oracle instead walks the pairs once with one cursor per expert.

Definitions followed: "DeepEP test target API reference", sec. 2.1 (topk_idx
with -1, expert_alignment), sec. 3.1 (num_tokens_per_expert, is_token_in_rank
per destination), sec. 4.2 (align); "spark_model/layers/ep_dispatch.rs"
(partition of pairs by owning expert range, token-major then k order).
"""
from __future__ import annotations


def align(x: int, a: int) -> int:
    return -(-x // a) * a


def layout(idx, E, A=1, P=1, C=0, rows_cap=None):
    """idx: list of T lists of K ints.  Returns a dict with the same keys as
    the C oracle (count, offset, dst, src_of_slot, in_part, tok_per_part,
    pairs_per_part, R, status).  rows_cap: receive rows the caller holds
    (None: as many as the layout needs); src_of_slot keeps only the slots
    below it, dst keeps every slot, and status bit 4 reports R > rows_cap."""
    T = len(idx)
    K = len(idx[0]) if T else 0
    status = 0
    pairs = []
    for t in range(T):
        for k in range(K):
            e = idx[t][k]
            if e == -1:
                continue
            if not (0 <= e < E):
                status |= 1
                continue
            pairs.append((e, t * K + k))
    count = [sum(1 for (e2, _) in pairs if e2 == e) for e in range(E)]
    if C:
        offset = [e * C for e in range(E + 1)]
        if any(c > C for c in count):
            status |= 2
    else:
        offset = [sum(align(count[j], A) for j in range(e)) for e in range(E + 1)]
    R = offset[E]
    if rows_cap is not None and R > rows_cap:
        status |= 4
    dst = [[-1] * K for _ in range(T)]
    src = [-1] * R
    for e in range(E):
        mine = sorted(p for (e2, p) in pairs if e2 == e)
        for j, p in enumerate(mine):
            if C and j >= C:
                continue
            slot = offset[e] + j
            dst[p // K][p % K] = slot
            src[slot] = p
    m = E // P
    in_part = [[0] * P for _ in range(T)]
    for t in range(T):
        for k in range(K):
            e = idx[t][k]
            if 0 <= e < E:
                in_part[t][e // m] = 1
    tok_per_part = [sum(in_part[t][q] for t in range(T)) for q in range(P)]
    pairs_per_part = [sum(count[e] for e in range(q * m, (q + 1) * m)) for q in range(P)]
    if rows_cap is not None:
        src = src[:rows_cap]
    return dict(count=count, offset=offset, dst=dst, src_of_slot=src, in_part=in_part,
                tok_per_part=tok_per_part, pairs_per_part=pairs_per_part, R=R, status=status)


def combine_exact(y_rows, dst, w=None, bias0=None, bias1=None):
    """Exact rational combine of small float inputs (fractions.Fraction):
    out[t][c] = bias0 + bias1 + sum over valid k of w[t][k] * y[dst[t][k]][c]."""
    from fractions import Fraction
    T = len(dst)
    H = len(y_rows[0]) if y_rows else (len(bias0[0]) if bias0 else 0)
    out = []
    for t in range(T):
        row = []
        for c in range(H):
            acc = Fraction(0)
            for b in (bias0, bias1):
                if b is not None:
                    acc += Fraction(float(b[t][c]))
            for k, s in enumerate(dst[t]):
                if s < 0:
                    continue
                wk = Fraction(float(w[t][k])) if w is not None else Fraction(1)
                acc += wk * Fraction(float(y_rows[s][c]))
            row.append(acc)
        out.append(row)
    return out


def partition_layout(idx, E, P, G=None):
    """Per-rank receive lists: partition q receives, once each and in token
    order, every token with at least one expert in [q*m, (q+1)*m)."""
    G = P if G is None else G
    m = E // P
    T = len(idx)
    members = [sorted({t for t in range(T) for e in idx[t] if 0 <= e < E and e // m == q})
               for q in range(P)]
    offset = [0]
    for q in range(P):
        offset.append(offset[-1] + len(members[q]))
    token_slot = [[-1] * P for _ in range(T)]
    for q in range(P):
        for j, t in enumerate(members[q]):
            token_slot[t][q] = offset[q] + j
    groups = [len({t for q in range(n * G, (n + 1) * G) for t in members[q]}) for n in range(P // G)]
    return dict(members=members, part_offset=offset, token_slot=token_slot,
                tok_per_part=[len(mm) for mm in members], tok_per_group=groups, Rp=offset[-1])
