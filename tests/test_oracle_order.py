"""Bitwise pins of the oracle's ordered fp32 reductions.

The combine ("DeepEP test target API reference", sec. 2.2 weighted combine
with bias; sec. 3.2 the plain sum; sec. 4.1 refs: an ordered accumulation
instead of scatter_add) is read as: acc = 0; acc += bias0; acc += bias1;
then acc = fmaf(w[t,k], y[dst[t,k]], acc) for k ascending over kept pairs;
out = bf16 round to nearest even.  The partitioned combine adds rows for
partitions in ascending order; the two-level combine folds each partition's
pairs (k ascending, fmaf from 0) and adds the partials (fp32, or rounded to
bf16 first on request) in ascending partition order after the biases.

Each step is simulated here with exact rational arithmetic and one
round-to-nearest-even to float32 per operation (an independent fmaf), the
final bf16 rounding by torch's CPU cast.  The inputs are built so that large
terms cancel exactly while small ones survive: an fp32 partial sum holding a
large term absorbs the small ones, so the order of the operations shows in
the bf16 result.  Each test also checks that another order (k descending,
biases last, float64 accumulation, partitions descending, unrounded
partials) changes the bits of several outputs, and one test builds elements
where fmaf and a separate multiply and add differ, so an oracle that did the
reduction another way would fail."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

from test_cast_division import _fma32, _rn32


def _bf16(vals):
    """float32 values -> bf16 bits (round to nearest even), torch's CPU cast."""
    t = torch.from_numpy(np.asarray(vals, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f(bits):
    return np.float32(oracle.bf16_to_float(np.array([bits], np.uint16))[0])


def _add32(a, b):
    return _rn32(Fraction(float(a)) + Fraction(float(b)))


def _mul32(a, b):
    return _rn32(Fraction(float(a)) * Fraction(float(b)))


def _small_bf16(rng, n):
    """bf16 values of magnitude 2^-6 .. 1 with random mantissas and signs."""
    m = rng.uniform(1.0, 2.0, size=n)
    e = rng.integers(-6, 0, size=n)
    s = rng.choice([-1.0, 1.0], size=n)
    return (s * m * np.exp2(e)).astype(np.float32)


def _cancelling_terms(rng, n):
    """n term values (float32, each a bf16 value) whose exact sum is small
    (a few small terms) while three of them are +a*2^16, +b*2^16 and
    -(a+b)*2^16 (a, b in 1..127, so all three are bf16): an fp32 partial sum
    that holds one or two of the big terms absorbs the small ones, so the
    order of the additions decides the result well above bf16 resolution."""
    v = _small_bf16(rng, n)
    if n >= 3:
        a, b = (int(z) for z in rng.integers(1, 128, size=2))
        pos = rng.permutation(n)[:3]
        v[pos] = np.array([a, b, -(a + b)], np.float32) * np.float32(2.0 ** 16)
    return _bf16(v)


def _case(seed, T=24, K=6, H=16, E=12, drop=0.15):
    """Routing (every token keeps at least one pair), weights that are signed
    powers of two (exact products, so every term below is exact), and y and
    biases such that each output element's terms cancel as in
    _cancelling_terms."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    dropm = rng.random((T, K)) < drop
    dropm[:, 0] = False
    idx[dropm] = -1
    lay = brute.layout(idx.tolist(), E, 1, 1)
    dst = np.array(lay["dst"], np.int32).reshape(T, K)
    w = (rng.choice([-1.0, 1.0], size=(T, K)) * np.exp2(rng.integers(-1, 2, size=(T, K)))).astype(np.float32)
    y = np.zeros((lay["R"], H), np.uint16)
    b0 = np.zeros((T, H), np.uint16)
    b1 = np.zeros((T, H), np.uint16)
    for t in range(T):
        ks = [k for k in range(K) if dst[t, k] >= 0]
        for c in range(H):
            terms = oracle.bf16_to_float(_cancelling_terms(rng, len(ks) + 2))
            b0[t, c], b1[t, c] = _bf16(terms[:2])
            for j, k in enumerate(ks):   # y = term / w, exact: w is a power of two
                y[dst[t, k], c] = _bf16([terms[2 + j] / w[t, k]])[0]
    return idx, dst, y, w, b0, b1


def _chain(terms, start=np.float32(0.0)):
    """Ordered fp32 chain: terms are ('add', v) or ('fma', w, y)."""
    acc = start
    for t in terms:
        acc = _add32(acc, t[1]) if t[0] == "add" else _fma32(t[1], t[2], acc)
    return acc


def _combine_sim(y, dst, w, b0, b1, order="spec"):
    T, K = dst.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.float32)
    for t in range(T):
        ks = [k for k in range(K) if dst[t, k] >= 0]
        if order == "k_desc":
            ks = ks[::-1]
        for c in range(H):
            biases = [("add", _f(b[t, c])) for b in (b0, b1) if b is not None]
            prods = [("fma", np.float32(w[t, k]) if w is not None else np.float32(1.0),
                      _f(y[dst[t, k], c])) for k in ks]
            if order == "f64":
                acc = sum(float(v[1]) for v in biases) + sum(float(p[1]) * float(p[2]) for p in prods)
                out[t, c] = np.float32(acc)
                continue
            if order == "mul_add":
                acc = np.float32(0.0)
                for v in biases:
                    acc = _add32(acc, v[1])
                for p in prods:
                    acc = _add32(acc, _mul32(p[1], p[2]))
                out[t, c] = acc
                continue
            terms = prods + biases if order == "bias_last" else biases + prods
            out[t, c] = _chain(terms)
    return _bf16(out.ravel()).reshape(T, H)


@pytest.mark.parametrize("seed,weighted,nb", [(0, True, 2), (1, True, 1), (2, False, 2), (3, True, 0)])
def test_combine_f32_order_is_bias0_bias1_then_k_ascending_fmaf(seed, weighted, nb):
    idx, dst, y, w, b0, b1 = _case(seed)
    w = w if weighted else None
    b0 = b0 if nb >= 1 else None
    b1 = b1 if nb >= 2 else None
    got = oracle.combine_f32(y, dst, w, b0, b1)
    spec = _combine_sim(y, dst, w, b0, b1, "spec")
    np.testing.assert_array_equal(got, spec)
    # the pin discriminates: other orders give other bits on this input
    alts = ["k_desc", "f64"] + (["bias_last"] if nb else [])
    for order in alts:
        other = _combine_sim(y, dst, w, b0, b1, order)
        assert (other != spec).sum() >= 3, order


def _partitioned_sim(y, token_slot, b0, b1, order="spec"):
    T, P = token_slot.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.float32)
    for t in range(T):
        qs = [q for q in range(P) if token_slot[t, q] >= 0]
        if order == "q_desc":
            qs = qs[::-1]
        for c in range(H):
            biases = [("add", _f(b[t, c])) for b in (b0, b1) if b is not None]
            rows = [("add", _f(y[token_slot[t, q], c])) for q in qs]
            terms = rows + biases if order == "bias_last" else biases + rows
            out[t, c] = _chain(terms)
    return _bf16(out.ravel()).reshape(T, H)


def test_combine_partitioned_f32_order():
    rng = np.random.default_rng(7)
    T, P, H, E = 30, 6, 16, 24
    idx = np.stack([rng.permutation(E)[:5] for _ in range(T)]).astype(np.int64)
    pl = brute.partition_layout(idx.tolist(), E, P)
    ts = np.array(pl["token_slot"], np.int32).reshape(T, P)
    y = np.zeros((pl["Rp"], H), np.uint16)
    b0 = np.zeros((T, H), np.uint16)
    b1 = np.zeros((T, H), np.uint16)
    for t in range(T):
        rows = [ts[t, q] for q in range(P) if ts[t, q] >= 0]
        for c in range(H):
            terms = _cancelling_terms(rng, len(rows) + 2)
            b0[t, c], b1[t, c] = terms[:2]
            for j, r in enumerate(rows):
                y[r, c] = terms[2 + j]
    got = oracle.combine_partitioned_f32(y, ts, b0, b1)
    spec = _partitioned_sim(y, ts, b0, b1)
    np.testing.assert_array_equal(got, spec)
    for order in ("q_desc", "bias_last"):
        assert (_partitioned_sim(y, ts, b0, b1, order) != spec).sum() >= 3, order


def _reduced_sim(y, idx, dst, w, E, P, b0, b1, order="spec"):
    T, K = dst.shape
    H = y.shape[1]
    m = E // P
    out = np.zeros((T, H), np.float32)
    for t in range(T):
        qs = list(range(P))[::-1] if order == "q_desc" else list(range(P))
        for c in range(H):
            acc = np.float32(0.0)
            for b in (b0, b1):
                if b is not None:
                    acc = _add32(acc, _f(b[t, c]))
            for q in qs:
                ks = [k for k in range(K) if idx[t, k] >= 0 and idx[t, k] // m == q and dst[t, k] >= 0]
                if not ks:
                    continue
                if order == "k_desc":
                    ks = ks[::-1]
                part = _chain([("fma", np.float32(w[t, k]) if w is not None else np.float32(1.0),
                                _f(y[dst[t, k], c])) for k in ks])
                if order != "no_round":
                    part = _f(_bf16([part])[0])
                acc = _add32(acc, part)
            out[t, c] = acc
    return _bf16(out.ravel()).reshape(T, H)


def _reduced_case(seed, T, E, P, parts, big2, weighted, H=16):
    """Each token's K = len(parts) pairs go to the partitions listed (distinct
    experts); weights are signed powers of two.  The terms cancel (as in
    _cancelling_terms) among the pairs of partition `parts[0]` in level one;
    with big2 the biases and the single-pair partials of level two cancel
    too, else they are all small."""
    rng = np.random.default_rng(seed)
    m = E // P
    K = len(parts)
    idx = np.zeros((T, K), np.int64)
    for t in range(T):
        used = {}
        for k, q in enumerate(parts):
            j = used.get(q, 0)
            used[q] = j + 1
            idx[t, k] = q * m + (rng.permutation(m)[j] if j == 0 else j)
    lay = brute.layout(idx.tolist(), E, 1, 1)
    dst = np.array(lay["dst"], np.int32).reshape(T, K)
    w = (rng.choice([-1.0, 1.0], size=(T, K)) * np.exp2(rng.integers(-1, 2, size=(T, K)))).astype(np.float32)
    if not weighted:
        w = np.ones((T, K), np.float32)
    y = np.zeros((lay["R"], H), np.uint16)
    b0 = np.zeros((T, H), np.uint16)
    b1 = np.zeros((T, H), np.uint16)
    first = [k for k in range(K) if parts[k] == parts[0]]
    rest = [k for k in range(K) if parts[k] != parts[0]]
    for t in range(T):
        for c in range(H):
            v1 = oracle.bf16_to_float(_cancelling_terms(rng, len(first)))
            for j, k in enumerate(first):
                y[dst[t, k], c] = _bf16([v1[j] / w[t, k]])[0]
            v2 = oracle.bf16_to_float(_cancelling_terms(rng, len(rest) + 2) if big2 else
                                      _bf16(_small_bf16(rng, len(rest) + 2)))
            b0[t, c], b1[t, c] = _bf16(v2[:2])
            for j, k in enumerate(rest):
                y[dst[t, k], c] = _bf16([v2[2 + j] / w[t, k]])[0]
    return idx, dst, y, w, b0, b1


@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("big2", [False, True])
def test_combine_reduced_f32_two_levels(weighted, big2):
    """Partition 1 holds five of the token's pairs, three large ones that
    cancel and two small ones, so the k order and the bf16 rounding of the
    partial decide the bits; the other pairs are alone in partitions 0, 2 and
    3.  With level-two terms that cancel, the partition order decides them."""
    E, P = 16, 4
    idx, dst, y, w, b0, b1 = _reduced_case(11, 24, E, P, [1, 3, 1, 0, 1, 2, 1, 1], big2, weighted)
    if not weighted:
        w = None
    # bf16 partials
    got = oracle.combine_reduced_f32(y, idx, dst, E, P, w, b0, b1, bf16_partials=True)
    spec = _reduced_sim(y, idx, dst, w, E, P, b0, b1)
    np.testing.assert_array_equal(got, spec)
    for order in ("k_desc",) + (("q_desc",) if big2 else ("no_round",)):
        assert (_reduced_sim(y, idx, dst, w, E, P, b0, b1, order) != spec).sum() >= 3, order
    # fp32 partials (the default)
    got = oracle.combine_reduced_f32(y, idx, dst, E, P, w, b0, b1)
    np.testing.assert_array_equal(got, _reduced_sim(y, idx, dst, w, E, P, b0, b1, "no_round"))


def test_combine_f32_uses_fused_multiply_add():
    """Elements built so that fmaf(w, y, acc) and acc + RN(w*y) differ: acc =
    B, then pair 0 (w, y) with an inexact fp32 product, then pair 1 (1, -B)
    and pair 2 (1, -q) with q = bf16(w*y), so the result is RN(B + w*y) - B - q
    (every step after the first fmaf is exact) and shows the product's own
    rounding.  Pairs (w, y) are drawn until 64 such elements are found."""
    rng = np.random.default_rng(21)
    B = np.float32(256.0)
    found = []
    while len(found) < 64:
        w = np.float32(rng.uniform(1.0, 2.0))
        yb = _bf16([rng.uniform(1.0, 2.0)])[0]
        yv = _f(yb)
        q = _f(_bf16([np.float32(w) * yv])[0])
        fused = _add32(_add32(_fma32(w, yv, B), -B), -q)
        split = _add32(_add32(_add32(B, _mul32(w, yv)), -B), -q)
        if _bf16([fused])[0] != _bf16([split])[0]:
            found.append((w, yb, _bf16([q])[0], _bf16([fused])[0]))
    T = len(found)
    dst = np.arange(3 * T, dtype=np.int32).reshape(T, 3)
    y = np.zeros((3 * T, 1), np.uint16)
    w = np.ones((T, 3), np.float32)
    b0 = np.full((T, 1), _bf16([B])[0], np.uint16)
    for t, (wt, yb, qb, _) in enumerate(found):
        w[t, 0] = wt
        y[3 * t, 0] = yb
        y[3 * t + 1, 0] = _bf16([-B])[0]
        y[3 * t + 2, 0] = qb ^ 0x8000
    got = oracle.combine_f32(y, dst, w, b0)
    np.testing.assert_array_equal(got[:, 0], [f[3] for f in found])
