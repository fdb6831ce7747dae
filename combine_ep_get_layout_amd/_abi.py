"""ctypes view of include/ep.h (libep.so).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libep.so")

EP_OK = 0
EP_ERR_INVALID_ARG = -1
EP_ERR_UNSUPPORTED = -2
EP_ERR_WORKSPACE = -3
EP_ERR_LAUNCH = -4

EP_DEV_BAD_EXPERT = 1
EP_DEV_CAPACITY = 2
EP_DEV_RECV_OVERFLOW = 4

EP_DTYPE_BF16 = 0
EP_DTYPE_FP8_E4M3 = 1
EP_DTYPE_FP8_E4M3_POW2 = 2
EP_DTYPE_FP8_E4M3_UE8M0 = 3

EP_MAX_EXPERTS = 4096
EP_MAX_PARTITIONS = 1024
EP_MAX_TOPK = 256
EP_MAX_SLOT_PARTITIONS = 64
EP_MAX_HIDDEN = 1 << 20

# Every symbol include/ep.h declares.
EXPORTS = ("ep_get_layout_workspace_bytes", "ep_worst_case_recv_rows", "ep_get_layout",
           "ep_get_layout_noalloc",
           "ep_dispatch", "ep_dispatch_with_layout", "ep_combine", "ep_dispatch_partitioned", "ep_combine_partitioned",
           "ep_combine_reduced", "ep_cast_fp8", "ep_logfmt_row_bytes", "ep_logfmt_encode",
           "ep_logfmt_decode", "ep_combine_logfmt", "ep_probe_dispatch_stores",
           "ep_status_string")


class LayoutParams(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_topk", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("expert_alignment", ctypes.c_int32),
                ("num_partitions", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("partitions_per_group", ctypes.c_int32), ("partition_major", ctypes.c_int32),
                ("max_recv_rows", ctypes.c_int64)]


class LayoutPtrs(ctypes.Structure):
    _fields_ = [("num_tokens_per_expert", ctypes.c_void_p), ("expert_offset", ctypes.c_void_p),
                ("num_tokens_per_partition", ctypes.c_void_p),
                ("is_token_in_partition", ctypes.c_void_p), ("dst_slot", ctypes.c_void_p),
                ("src_of_slot", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("partition_offset", ctypes.c_void_p), ("token_slot", ctypes.c_void_p),
                ("num_tokens_per_group", ctypes.c_void_p), ("partition_src", ctypes.c_void_p)]


_lib = None


class EpError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = _lib.ep_status_string(code).decode() if _lib is not None else str(code)
        super().__init__(f"{fn} returned {code} ({msg})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libep.so.  Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libep.so not built ({path}); run __graft_entry__.build() or "
                           "python combine_ep_get_layout_amd/build.py")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.ep_get_layout_workspace_bytes.argtypes = [P(LayoutParams)]
    lib.ep_get_layout_workspace_bytes.restype = sz
    lib.ep_worst_case_recv_rows.argtypes = [P(LayoutParams)]
    lib.ep_worst_case_recv_rows.restype = i64
    lib.ep_get_layout.argtypes = [vp, P(LayoutParams), P(LayoutPtrs), vp, vp, sz, vp]
    lib.ep_get_layout.restype = ctypes.c_int
    lib.ep_get_layout_noalloc.argtypes = [vp, P(LayoutParams), P(LayoutPtrs), vp, vp]
    lib.ep_get_layout_noalloc.restype = ctypes.c_int
    lib.ep_dispatch.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i32, i32, vp,
                                P(LayoutParams), P(LayoutPtrs), vp, vp, vp, i64, ctypes.c_int, vp]
    lib.ep_dispatch.restype = ctypes.c_int
    lib.ep_dispatch_with_layout.argtypes = [vp, P(LayoutParams), P(LayoutPtrs), vp, vp, sz,
                                            vp, ctypes.c_int, vp, ctypes.c_int, i32, i32, vp,
                                            vp, vp, vp, i64, ctypes.c_int, vp]
    lib.ep_dispatch_with_layout.restype = ctypes.c_int
    lib.ep_combine.argtypes = [vp, i32, i64, vp, vp, vp, P(LayoutParams), P(LayoutPtrs), vp, vp,
                               vp, vp]
    lib.ep_combine.restype = ctypes.c_int
    lib.ep_dispatch_partitioned.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i32, i32, vp, vp,
                                            P(LayoutParams), P(LayoutPtrs), vp, vp, vp, vp, i64,
                                            vp]
    lib.ep_dispatch_partitioned.restype = ctypes.c_int
    lib.ep_combine_partitioned.argtypes = [vp, i32, i64, vp, vp, P(LayoutParams), P(LayoutPtrs),
                                           vp, vp]
    lib.ep_combine_partitioned.restype = ctypes.c_int
    lib.ep_combine_reduced.argtypes = [vp, i32, i64, vp, vp, vp, vp, P(LayoutParams),
                                       P(LayoutPtrs), vp, ctypes.c_int, vp]
    lib.ep_combine_reduced.restype = ctypes.c_int
    lib.ep_cast_fp8.argtypes = [vp, i32, i32, i32, ctypes.c_int, vp, vp, vp]
    lib.ep_cast_fp8.restype = ctypes.c_int
    lib.ep_logfmt_row_bytes.argtypes = [i32]
    lib.ep_logfmt_row_bytes.restype = i64
    lib.ep_logfmt_encode.argtypes = [vp, i64, i32, P(LayoutParams), P(LayoutPtrs), vp, vp]
    lib.ep_logfmt_encode.restype = ctypes.c_int
    lib.ep_logfmt_decode.argtypes = [vp, i64, i32, vp, vp]
    lib.ep_logfmt_decode.restype = ctypes.c_int
    lib.ep_combine_logfmt.argtypes = [vp, i32, i64, vp, vp, vp, P(LayoutParams), P(LayoutPtrs),
                                      vp, vp, vp, vp]
    lib.ep_combine_logfmt.restype = ctypes.c_int
    lib.ep_probe_dispatch_stores.argtypes = [i32, ctypes.c_uint32, P(LayoutParams), P(LayoutPtrs),
                                             vp, i64, vp]
    lib.ep_probe_dispatch_stores.restype = ctypes.c_int
    lib.ep_status_string.argtypes = [ctypes.c_int]
    lib.ep_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != EP_OK:
        raise EpError(fn, code)
