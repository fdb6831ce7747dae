"""CPU oracle for MoE expert-parallel layout / dispatch / combine / fp8 cast / the
10-bit logarithmic combine payload.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only callers.  The GPU library never imports, links or
runs anything here, and nothing here imports the GPU package.

The arithmetic lives in ``ep_oracle.c`` (plain C loops, one function per step
of the method, each citing the passage it follows); this module compiles it
with gcc on first use and marshals numpy arrays through ctypes.  ``brute`` is a
separately written pure-Python brute force for tiny inputs that pins the C
code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BAD_EXPERT = 1
CAPACITY = 2
RECV_OVERFLOW = 4

_lib = None


def build(force: bool = False) -> str:
    """Compile ep_oracle.c into liboracle.so with gcc (plain -O2, no FMA
    contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _lib.oracle_bf16_from_float.restype = ctypes.c_uint16
        _lib.oracle_bf16_from_float.argtypes = [ctypes.c_float]
        _lib.oracle_e4m3_from_float.restype = ctypes.c_uint8
        _lib.oracle_e4m3_from_float.argtypes = [ctypes.c_float]
        _lib.oracle_e4m3_to_float.restype = ctypes.c_float
        _lib.oracle_e4m3_to_float.argtypes = [ctypes.c_uint8]
        _lib.oracle_bf16_to_float.restype = ctypes.c_float
        _lib.oracle_bf16_to_float.argtypes = [ctypes.c_uint16]
        _lib.oracle_pow2_ceil.restype = ctypes.c_float
        _lib.oracle_pow2_ceil.argtypes = [ctypes.c_float]
        _lib.oracle_ue8m0_of.restype = ctypes.c_uint8
        _lib.oracle_ue8m0_of.argtypes = [ctypes.c_float]
        _lib.oracle_ue8m0_to_float.restype = ctypes.c_float
        _lib.oracle_ue8m0_to_float.argtypes = [ctypes.c_uint8]
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i64(v):
    return ctypes.c_int64(int(v))


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class Layout(dict):
    """Plain dict of the oracle layout: count, offset, dst, src_of_slot,
    in_part, tok_per_part, pairs_per_part, R, status."""
    __getattr__ = dict.__getitem__


def get_layout(topk_idx, num_experts, expert_alignment=1, num_partitions=1,
               capacity=0, rows_cap=None, partition_major=False) -> Layout:
    """oracle_get_layout: count, offset (per receive segment: expert, or
    partition when partition_major), dst, src_of_slot, partition membership."""
    lib = _load()
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    E, A, P, C = int(num_experts), int(expert_alignment), int(num_partitions), int(capacity)
    S = P if partition_major else E
    if rows_cap is None:
        rows_cap = S * C if C > 0 else T * K + min(S, T * K) * (A - 1)
    count = np.zeros(S, np.int32)
    offset = np.zeros(S + 1, np.int32)
    dst = np.zeros(T * K, np.int32)
    src = np.full(max(int(rows_cap), 1), -1, np.int32)
    in_part = np.zeros(max(T * P, 1), np.uint8)
    tpp = np.zeros(P, np.int32)
    ppp = np.zeros(P, np.int32)
    R = ctypes.c_int64(0)
    st = ctypes.c_int32(0)
    rc = lib.oracle_get_layout(_p(idx), _i64(T), _i64(K), _i64(E), _i64(A), _i64(P), _i64(C),
                               _i64(1 if partition_major else 0), _p(count), _p(offset), _p(dst), _p(src), _i64(rows_cap),
                               _p(in_part), _p(tpp), _p(ppp), ctypes.byref(R), ctypes.byref(st))
    if rc != 0:
        raise ValueError("oracle_get_layout: invalid arguments")
    R = int(R.value)
    return Layout(count=count, offset=offset, dst=dst.reshape(T, K),
                  src_of_slot=src[:min(R, int(rows_cap))], in_part=in_part[:T * P].reshape(T, P),
                  tok_per_part=tpp, pairs_per_part=ppp, R=R, status=int(st.value))


def dispatch(x_rows, layout: Layout, topk_weights=None, x_scales=None, zero_padding=False,
             recv_init=None, scales_init=None):
    """recv[dst[t,k]] = x[t] byte for byte.  x_rows is [T, H] of any dtype
    (bf16 bits as uint16, fp8 codes as uint8); x_scales [T, H/G] (float32, or
    uint8 UE8M0 bytes) or None.  Returns (recv [R, ...], recv_scales or None, recv_w [R]).  Padding
    rows keep recv_init's content (zeros by default) unless zero_padding."""
    lib = _load()
    x = np.ascontiguousarray(x_rows)
    T = x.shape[0]
    K = layout.dst.shape[1] if T else 1
    R = layout.R
    row_bytes = x[0].nbytes if T else x.itemsize * int(np.prod(x.shape[1:]))
    recv = (np.zeros((R,) + x.shape[1:], x.dtype) if recv_init is None
            else np.array(recv_init, dtype=x.dtype, copy=True))
    xs = None if x_scales is None else np.ascontiguousarray(x_scales)   # f32 or UE8M0 bytes
    recv_s = None
    srow = 0
    if xs is not None:
        srow = xs.shape[1] * xs.itemsize
        recv_s = (np.zeros((R, xs.shape[1]), xs.dtype) if scales_init is None
                  else np.array(scales_init, dtype=xs.dtype, copy=True))
    recv_w = np.zeros(R, np.float32)
    w = _c(topk_weights, np.float32)
    lib.oracle_dispatch(_p(x), _i64(row_bytes), _p(xs), _i64(srow), _p(w), _i64(T), _i64(K),
                        _p(np.ascontiguousarray(layout.dst, np.int32)),
                        _p(np.ascontiguousarray(layout.src_of_slot, np.int32)), _i64(R),
                        ctypes.c_int(1 if zero_padding else 0), _p(recv), _p(recv_s), _p(recv_w))
    return recv, recv_s, recv_w


def dispatch_tokens(x_rows, layout: Layout, topk_weights, recv, recv_w, t0, t1):
    """oracle_dispatch over tokens [t0, t1) only, into caller-owned recv
    [R, ...] and recv_w [R] (no zero padding): lets disjoint token ranges run
    on separate threads (ctypes releases the GIL during the call)."""
    lib = _load()
    x = np.ascontiguousarray(x_rows)
    K = layout.dst.shape[1]
    row_bytes = x[0].nbytes
    dst = np.ascontiguousarray(layout.dst, np.int32)
    w = _c(topk_weights, np.float32)
    src = np.ascontiguousarray(layout.src_of_slot, np.int32)
    lib.oracle_dispatch(ctypes.c_void_p(x.ctypes.data + t0 * row_bytes), _i64(row_bytes), None,
                        _i64(0), None if w is None else ctypes.c_void_p(w.ctypes.data + t0 * K * 4),
                        _i64(t1 - t0), _i64(K), ctypes.c_void_p(dst.ctypes.data + t0 * K * 4),
                        _p(src), _i64(min(layout.R, len(src))), ctypes.c_int(0), _p(recv), None,
                        _p(recv_w))


def cast_fp8(x_bits, group=128):
    """Per (token, group) e4m3 cast.  Returns (codes uint8 [T,H], scales f32 [T,H/G])."""
    lib = _load()
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    q = np.zeros((T, H), np.uint8)
    s = np.zeros((T, H // group), np.float32)
    rc = lib.oracle_cast_fp8(_p(x), _i64(T), _i64(H), _i64(group), _p(q), _p(s))
    if rc != 0:
        raise ValueError("oracle_cast_fp8: invalid arguments")
    return q, s


def cast_fp8_pow2(x_bits, group=128, ue8m0=False):
    """Per (token, group) e4m3 cast with the scale rounded up to a power of
    two.  Returns (codes uint8 [T,H], scales f32 [T,H/G], UE8M0 bytes uint8
    [T,H/G] or None)."""
    lib = _load()
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    q = np.zeros((T, H), np.uint8)
    s = np.zeros((T, H // group), np.float32)
    e8 = np.zeros((T, H // group), np.uint8) if ue8m0 else None
    rc = lib.oracle_cast_fp8_pow2(_p(x), _i64(T), _i64(H), _i64(group),
                                  ctypes.c_int(2 if ue8m0 else 1), _p(q), _p(s), _p(e8))
    if rc != 0:
        raise ValueError("oracle_cast_fp8_pow2: invalid arguments")
    return q, s, e8


def pow2_ceil(v):
    lib = _load()
    return np.array([lib.oracle_pow2_ceil(ctypes.c_float(float(a))) for a in np.ravel(v)],
                    np.float32)


def ue8m0_of(v):
    lib = _load()
    return np.array([lib.oracle_ue8m0_of(ctypes.c_float(float(a))) for a in np.ravel(v)],
                    np.uint8)


def ue8m0_to_float(b):
    lib = _load()
    return np.array([lib.oracle_ue8m0_to_float(ctypes.c_uint8(int(a))) for a in np.ravel(b)],
                    np.float32)


def cast_back(q, scales, group=128):
    lib = _load()
    q = _c(q, np.uint8)
    s = _c(scales, np.float32)
    T, H = q.shape
    out = np.zeros((T, H), np.float32)
    lib.oracle_cast_back(_p(q), _p(s), _i64(T), _i64(H), _i64(group), _p(out))
    return out


def _combine(fn, out_dtype, y, dst, topk_weights, bias0, bias1, tokens):
    y = _c(y, np.uint16)
    H = y.shape[1]
    dst = _c(dst, np.int32)
    T, K = dst.shape
    w = _c(topk_weights, np.float32)
    b0 = _c(bias0, np.uint16)
    b1 = _c(bias1, np.uint16)
    tk = _c(tokens, np.int64)
    n = T if tk is None else tk.shape[0]
    out = np.zeros((n, H), out_dtype)
    fn(_p(y), _i64(H), _p(w), _p(b0), _p(b1), _i64(T), _i64(K), _p(dst), _p(tk), _i64(n), _p(out))
    return out


def combine_f64(y, dst, topk_weights=None, bias0=None, bias1=None, tokens=None):
    """float64 reference: sum of biases + sum_k w[t,k] * y[dst[t,k]]."""
    return _combine(_load().oracle_combine_f64, np.float64, y, dst, topk_weights, bias0, bias1,
                    tokens)


def combine_f32(y, dst, topk_weights=None, bias0=None, bias1=None, tokens=None):
    """Ordered fp32 accumulation (bias0, bias1, then fmaf over k ascending),
    rounded to bf16; returns uint16 bits."""
    return _combine(_load().oracle_combine_f32, np.uint16, y, dst, topk_weights, bias0, bias1,
                    tokens)


def combined_weights(recv_w, dst):
    lib = _load()
    dst = _c(dst, np.int32)
    T, K = dst.shape
    rw = _c(recv_w, np.float32)
    out = np.zeros((T, K), np.float32)
    lib.oracle_combined_weights(_p(rw), _i64(T), _i64(K), _p(dst), _p(out))
    return out


def e4m3_from_float(v):
    v = _c(v, np.float32).ravel()
    out = np.zeros(v.shape, np.uint8)
    _load().oracle_e4m3_from_float_n(_p(v), _i64(v.size), _p(out))
    return out


def e4m3_to_float(codes):
    lib = _load()
    return np.array([lib.oracle_e4m3_to_float(int(c)) for c in np.asarray(codes).ravel()],
                    np.float32)


def bf16_from_float(v):
    v = _c(v, np.float32).ravel()
    out = np.zeros(v.shape, np.uint16)
    _load().oracle_bf16_from_float_n(_p(v), _i64(v.size), _p(out))
    return out


def div_f32(a, b):
    a = _c(a, np.float32).ravel()
    b = _c(b, np.float32).ravel()
    out = np.zeros(a.shape, np.float32)
    _load().oracle_div_f32_n(_p(a), _p(b), _i64(a.size), _p(out))
    return out


def bf16_to_float(bits):
    """bf16 bit patterns (uint16) widened to float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def partition_layout(topk_idx, num_experts, num_partitions, partitions_per_group=None):
    """Non-expanded (per-rank) receive layout.  Returns a Layout dict with
    in_part [T,P], tok_per_part [P], part_offset [P+1], token_slot [T,P],
    tok_per_group [P/G], part_src [Rp] (the token of each row), Rp."""
    lib = _load()
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    E, P = int(num_experts), int(num_partitions)
    G = P if partitions_per_group is None else int(partitions_per_group)
    in_part = np.zeros(max(T * P, 1), np.uint8)
    tpp = np.zeros(P, np.int32)
    off = np.zeros(P + 1, np.int32)
    slot = np.zeros(max(T * P, 1), np.int32)
    tpg = np.zeros(max(P // G, 1), np.int32)
    src = np.full(max(T * P, 1), -1, np.int32)
    Rp = ctypes.c_int64(0)
    rc = lib.oracle_partition_layout(_p(idx), _i64(T), _i64(K), _i64(E), _i64(P), _i64(G),
                                     _p(in_part), _p(tpp), _p(off), _p(slot), _p(tpg), _p(src),
                                     ctypes.byref(Rp))
    if rc != 0:
        raise ValueError("oracle_partition_layout: invalid arguments")
    return Layout(in_part=in_part[:T * P].reshape(T, P), tok_per_part=tpp, part_offset=off,
                  token_slot=slot[:T * P].reshape(T, P), tok_per_group=tpg[:P // G],
                  part_src=src[:int(Rp.value)], Rp=int(Rp.value), P=P, E=E)


def dispatch_partitioned(x_rows, topk_idx, play, topk_weights=None, x_scales=None,
                         recv_init=None):
    """recv[token_slot[t,q]] = x[t]; per row the local expert ids (-1 when the
    pair is elsewhere) and weights.  Returns (recv, recv_scales, recv_idx, recv_w)."""
    lib = _load()
    x = np.ascontiguousarray(x_rows)
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    Rp = play.Rp
    row_bytes = x[0].nbytes if T else x.itemsize * int(np.prod(x.shape[1:]))
    recv = (np.zeros((Rp,) + x.shape[1:], x.dtype) if recv_init is None
            else np.array(recv_init, dtype=x.dtype, copy=True))
    xs = None if x_scales is None else np.ascontiguousarray(x_scales)   # f32 or UE8M0 bytes
    recv_s, srow = None, 0
    if xs is not None:
        srow = xs.shape[1] * xs.itemsize
        recv_s = np.zeros((Rp, xs.shape[1]), xs.dtype)
    recv_idx = np.zeros((max(Rp, 1), K), np.int64)
    recv_w = np.zeros((max(Rp, 1), K), np.float32)
    w = _c(topk_weights, np.float32)
    lib.oracle_dispatch_partitioned(_p(x), _i64(row_bytes), _p(xs), _i64(srow), _p(idx), _p(w),
                                    _i64(T), _i64(K), _i64(play.E), _i64(play.P),
                                    _p(np.ascontiguousarray(play.token_slot, np.int32)), _i64(Rp),
                                    _p(recv), _p(recv_s), _p(recv_idx), _p(recv_w))
    return recv, recv_s, recv_idx[:Rp], recv_w[:Rp]


def _combine_part(fn, out_dtype, y, token_slot, bias0, bias1, tokens):
    y = _c(y, np.uint16)
    H = y.shape[1]
    ts = _c(token_slot, np.int32)
    T, P = ts.shape
    b0, b1, tk = _c(bias0, np.uint16), _c(bias1, np.uint16), _c(tokens, np.int64)
    n = T if tk is None else tk.shape[0]
    out = np.zeros((n, H), out_dtype)
    fn(_p(y), _i64(H), _p(b0), _p(b1), _i64(T), _i64(P), _p(ts), _p(tk), _i64(n), _p(out))
    return out


def combine_partitioned_f32(y, token_slot, bias0=None, bias1=None, tokens=None):
    return _combine_part(_load().oracle_combine_partitioned_f32, np.uint16, y, token_slot,
                         bias0, bias1, tokens)


def combine_partitioned_f64(y, token_slot, bias0=None, bias1=None, tokens=None):
    return _combine_part(_load().oracle_combine_partitioned_f64, np.float64, y, token_slot,
                         bias0, bias1, tokens)


def combine_reduced_f32(y, topk_idx, dst, num_experts, num_partitions, topk_weights=None,
                        bias0=None, bias1=None, tokens=None, bf16_partials=False):
    """Two-level combine: per-partition fp32 partial (rounded to bf16 with
    bf16_partials), then the partials summed over partitions in ascending
    order (with the biases first), bf16 result."""
    lib = _load()
    y = _c(y, np.uint16)
    H = y.shape[1]
    idx = _c(topk_idx, np.int64)
    dst = _c(dst, np.int32)
    T, K = dst.shape
    w, b0, b1, tk = (_c(topk_weights, np.float32), _c(bias0, np.uint16), _c(bias1, np.uint16),
                     _c(tokens, np.int64))
    n = T if tk is None else tk.shape[0]
    out = np.zeros((n, H), np.uint16)
    lib.oracle_combine_reduced_f32(_p(y), _i64(H), _p(idx), _p(w), _p(b0), _p(b1), _i64(T),
                                   _i64(K), _i64(num_experts), _i64(num_partitions), _p(dst),
                                   ctypes.c_int(1 if bf16_partials else 0), _p(tk), _i64(n),
                                   _p(out))
    return out


# --- 10-bit logarithmic combine payload ([API] sec. 3.4, use_logfmt) -------
LOGFMT_GROUP = 128
LOGFMT_POISON = 0xFFFF


def logfmt_encode(x_bits):
    """bf16 rows [rows, H] -> (codes uint16 [rows, H] holding 10-bit codes,
    refs uint16 [rows, H/128]); see the reading in ep_oracle.c."""
    x = _c(x_bits, np.uint16)
    rows, H = x.shape
    codes = np.zeros((rows, H), np.uint16)
    refs = np.zeros((rows, H // LOGFMT_GROUP), np.uint16)
    rc = _load().oracle_logfmt_encode(_p(x), _i64(rows), _i64(H), _p(codes), _p(refs))
    if rc != 0:
        raise ValueError("logfmt_encode: hidden must be a positive multiple of 128")
    return codes, refs


def logfmt_decode(codes, refs):
    """(codes, refs) -> bf16 bit patterns [rows, H] (exact); raises on a code
    or reference the encoder never writes."""
    codes = _c(codes, np.uint16)
    refs = _c(refs, np.uint16)
    rows, H = codes.shape
    out = np.zeros((rows, H), np.uint16)
    rc = _load().oracle_logfmt_decode(_p(codes), _p(refs), _i64(rows), _i64(H), _p(out))
    if rc != 0:
        raise ValueError("logfmt_decode: invalid code or reference")
    return out


def logfmt_row_bytes(hidden):
    """Bytes of one packed payload row: H code bytes, H/4 bytes of high-bit
    words, H/128 references of two bytes, padded to a multiple of 128."""
    used = hidden + hidden // 4 + 2 * (hidden // LOGFMT_GROUP)
    return (used + 127) // 128 * 128


def logfmt_pack(codes, refs):
    """Packed payload rows (uint8 [rows, logfmt_row_bytes(H)]): bytes [0, H)
    hold each code's low eight bits; then one little-endian 32-bit word per 16
    channels: channel 16v + 2p + e (p = 0..7, e = 0 or 1) puts its code's
    bit 8 at bit 7 - p + 16e and its sign bit at bit 15 - p + 16e; then the
    references as little-endian uint16; zero padding."""
    codes = np.asarray(codes, np.uint32)
    refs = np.asarray(refs, np.uint16)
    rows, H = codes.shape
    out = np.zeros((rows, logfmt_row_bytes(H)), np.uint8)
    out[:, :H] = (codes & 0xFF).astype(np.uint8)
    blocks = codes.reshape(rows, H // 16, 16)
    pos8, pos9 = _logfmt_high_bit_positions()
    words = (((blocks >> 8) & 1) << pos8).sum(axis=2, dtype=np.uint32) \
        | (((blocks >> 9) & 1) << pos9).sum(axis=2, dtype=np.uint32)
    out[:, H:H + H // 4] = words.astype("<u4").view(np.uint8).reshape(rows, H // 4)
    G = H // LOGFMT_GROUP
    out[:, H + H // 4:H + H // 4 + 2 * G] = refs.astype("<u2").view(np.uint8).reshape(rows, 2 * G)
    return out


def _logfmt_high_bit_positions():
    """Bit positions, within a channel block's word, of bit 8 and of the sign
    of the block's 16 codes (channel 2p + e: 7 - p + 16e and 15 - p + 16e)."""
    j = np.arange(16, dtype=np.uint32)
    p, e = j // 2, j % 2
    return 7 - p + 16 * e, 15 - p + 16 * e


def logfmt_unpack(payload, hidden):
    """Inverse of logfmt_pack: (codes, refs)."""
    payload = np.asarray(payload, np.uint8)
    rows, H = payload.shape[0], hidden
    lo = payload[:, :H].astype(np.uint16)
    words = np.ascontiguousarray(payload[:, H:H + H // 4]).view("<u4").reshape(rows, H // 16, 1)
    pos8, pos9 = _logfmt_high_bit_positions()
    b8 = ((words >> pos8) & 1).reshape(rows, H).astype(np.uint16)
    sg = ((words >> pos9) & 1).reshape(rows, H).astype(np.uint16)
    G = H // LOGFMT_GROUP
    refs = np.ascontiguousarray(payload[:, H + H // 4:H + H // 4 + 2 * G]).view("<u2").reshape(rows, G)
    return lo | (b8 << 8) | (sg << 9), refs.astype(np.uint16)


def combine_logfmt_f32(codes, refs, dst, topk_weights=None, bias0=None, bias1=None, tokens=None):
    """The combine over a logfmt payload: the rows decoded (exactly, to bf16),
    then the ordered fp32 combine of combine_f32."""
    return combine_f32(logfmt_decode(codes, refs), dst, topk_weights, bias0, bias1, tokens)
