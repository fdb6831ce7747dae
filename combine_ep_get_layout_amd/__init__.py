"""MI355X-native MoE expert-parallel layout / dispatch / combine.

Thin PyTorch binding over libep.so (include/ep.h).  PyTorch only provides
device memory and the current HIP stream; every step of the path runs in the
library's gfx950 kernels.  The functions carry the C entry points' names:

  ep_get_layout(topk_idx, num_experts, ...)        -> Layout
  ep_get_layout_noalloc(topk_idx, layout, ...)     -> layout (the library's own scratch)
  ep_dispatch(x, layout, ...)                      -> (recv_x, recv_scales, recv_topk_weights)
  ep_dispatch_with_layout(x, topk_idx, num_experts, ...)
                                                   -> (layout, recv_x, recv_scales, recv_topk_weights)
  ep_combine(y, layout, ...)                       -> (combined_x, combined_topk_weights)
  ep_cast_fp8(x, group=128)                        -> (x_fp8, scales)
  ep_dispatch_partitioned(x, layout, topk_idx, ...) -> (recv_x, recv_scales, recv_topk_idx,
                                                        recv_topk_weights)
  ep_combine_partitioned(y, layout, ...)            -> combined_x
  ep_combine_reduced(y, layout, topk_idx, ...)      -> combined_x

Semantics follow the DeepEP v2 test page ("DeepEP test target API
reference", sec. 2.1 dispatch, 2.2 combine, 3.1-3.2 the V1 layout tensors and
unweighted combine, 4.2 the per-token e4m3 cast); the layout object plays the
part of the page's handle.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple, Union

import torch

from . import _abi
from ._abi import (EP_DEV_BAD_EXPERT, EP_DEV_CAPACITY, EP_DEV_RECV_OVERFLOW, EpError,
                   LayoutParams, LayoutPtrs)

__all__ = ["load_library", "Layout", "ep_get_layout", "ep_get_layout_noalloc", "ep_dispatch",
           "ep_dispatch_with_layout",
           "ep_combine", "ep_cast_fp8", "logfmt_row_bytes", "ep_logfmt_encode",
           "ep_logfmt_decode", "ep_combine_logfmt",
           "ep_dispatch_partitioned", "ep_combine_partitioned", "ep_combine_reduced",
           "worst_case_recv_rows", "ep_probe_dispatch_stores", "EpError", "EP_DEV_BAD_EXPERT", "EP_DEV_CAPACITY",
           "EP_DEV_RECV_OVERFLOW"]


def load_library() -> ctypes.CDLL:
    return _abi.load()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    """The raw handle of the current stream of `device` (torch's current
    stream, which HIP graph capture also records into)."""
    idx = device.index if device.index is not None else torch._C._cuda_getDevice()
    return torch._C._cuda_getCurrentRawStream(idx)


def _launch(name: str, device, fn, *tensors_then_args):
    """Call entry point `fn` with `device` current (the library launches on the
    calling thread's current device), after checking that every tensor given
    before the plain arguments lives on it.  Usage:
    _launch(name, dev, fn, [tensors...], arg0, arg1, ...)."""
    tensors, args = tensors_then_args[0], tensors_then_args[1:]
    cur = torch._C._cuda_getDevice()
    idx = cur if device.index is None else device.index
    for t in tensors:
        if t is not None and t.get_device() != idx:
            raise ValueError(f"{name}: all tensors must be on cuda:{idx}, found {t.device}")
    if idx == cur:
        rc = fn(*args)
    else:
        with torch.cuda.device(idx):
            rc = fn(*args)
    _abi.check(name, rc)


def _need_cuda(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(t: Optional[torch.Tensor], name: str, dtypes, cols=None, min_rows=None, rows=None):
    """A GPU buffer the kernels will read or write: contiguous, of one of
    `dtypes`, 2-D with `cols` columns (1-D when cols is None) and `rows` rows
    exactly or at least `min_rows`.  Catches a buffer the kernels would
    overrun before anything is launched."""
    if t is None:
        return
    _need_cuda(t, name)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if cols is None:
        n = t.numel()
        if (rows is not None and n != rows) or (min_rows is not None and n < min_rows):
            raise ValueError(f"{name} has {n} elements, needs {rows if rows is not None else min_rows}")
        return
    if t.dim() != 2 or t.shape[1] != cols:
        raise ValueError(f"{name} must be [rows, {cols}], not {list(t.shape)}")
    if (rows is not None and t.shape[0] != rows) or (min_rows is not None and t.shape[0] < min_rows):
        raise ValueError(f"{name} has {t.shape[0]} rows, needs "
                         f"{rows if rows is not None else f'at least {min_rows}'}")


_F8 = (torch.float8_e4m3fn, torch.uint8)
_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_I64 = (torch.int64,)


def worst_case_recv_rows(num_tokens, num_topk, num_experts, expert_alignment=1, capacity=0,
                         num_partitions=1, partition_major=False) -> int:
    p = LayoutParams(num_tokens=num_tokens, num_topk=num_topk, num_experts=num_experts,
                     expert_alignment=expert_alignment, num_partitions=num_partitions,
                     capacity=capacity, partition_major=1 if partition_major else 0)
    return int(load_library().ep_worst_case_recv_rows(ctypes.byref(p)))


class Layout:
    """Device-resident receive layout (the dispatch "handle").

    Tensors: num_tokens_per_expert [S], expert_offset [S+1] (R at [S]), S the
    receive segments (E, or P for a partition-major layout),
    num_tokens_per_partition [P], is_token_in_partition [T, P] uint8,
    dst_slot [T, K], src_of_slot [max_recv_rows], status [1]; with the
    partition layout also partition_offset [P+1], num_tokens_per_group [P/G]
    and, for P <= 64, token_slot [T, P] and partition_src [T*P] (the token of
    each partition row) (else None).  A buffer may be replaced or dropped by
    assigning the attribute; resizing one in place is not supported (the
    calls pass each buffer's address as it was when last assigned)."""

    def __init__(self, params: LayoutParams, device, partition_layout: bool = False):
        T, K, P = params.num_tokens, params.num_topk, params.num_partitions
        S = P if params.partition_major else params.num_experts
        i32 = dict(dtype=torch.int32, device=device)
        self.params = params
        self.device = device
        self.num_tokens_per_expert = torch.empty(S, **i32)
        self.expert_offset = torch.empty(S + 1, **i32)
        self.num_tokens_per_partition = torch.empty(P, **i32)
        self.is_token_in_partition = torch.empty((T, P), dtype=torch.uint8, device=device)
        self.dst_slot = torch.empty((T, K), **i32)
        self.src_of_slot = torch.empty(max(params.max_recv_rows, 1), **i32)
        self.status = torch.zeros(1, **i32)
        self.partition_offset = self.token_slot = self.num_tokens_per_group = None
        self.partition_src = None
        if partition_layout:
            G = params.partitions_per_group or P
            self.partition_offset = torch.empty(P + 1, **i32)
            self.num_tokens_per_group = torch.empty(P // G, **i32)
            if P <= _abi.EP_MAX_SLOT_PARTITIONS:      # token_slot only up to 64 partitions
                self.token_slot = torch.empty((T, P), **i32)
                self.partition_src = torch.empty(max(T * P, 1), **i32)
        nbytes = load_library().ep_get_layout_workspace_bytes(ctypes.byref(params))
        self.workspace = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        self._ptrs = None

    @property
    def num_tokens(self):
        return self.params.num_tokens

    @property
    def num_topk(self):
        return self.params.num_topk

    @property
    def num_experts(self):
        return self.params.num_experts

    @property
    def partition_major(self) -> bool:
        return bool(self.params.partition_major)

    @property
    def num_segments(self) -> int:
        """Receive segments: experts, or partitions when partition-major."""
        return self.params.num_partitions if self.params.partition_major else self.params.num_experts

    @property
    def max_recv_rows(self) -> int:
        return int(self.params.max_recv_rows)

    @property
    def num_partitions(self):
        return self.params.num_partitions

    _BUFFERS = frozenset(("num_tokens_per_expert", "expert_offset", "num_tokens_per_partition",
                          "is_token_in_partition", "dst_slot", "src_of_slot", "status",
                          "partition_offset", "token_slot", "num_tokens_per_group",
                          "partition_src"))

    def __setattr__(self, name, value):
        object.__setattr__(self, name, value)
        if name in Layout._BUFFERS:
            # a replaced (or dropped) buffer: the pointer struct must not keep
            # the old address, whose memory torch may hand out again
            object.__setattr__(self, "_ptrs", None)

    def ptrs(self) -> LayoutPtrs:
        """The buffers' device pointers as the C struct, built on first use
        after any buffer attribute was (re)assigned."""
        if self._ptrs is None:
            opt = [None if t is None else t.data_ptr()
                   for t in (self.partition_offset, self.token_slot, self.num_tokens_per_group,
                             self.partition_src)]
            self._ptrs = LayoutPtrs(self.num_tokens_per_expert.data_ptr(),
                                    self.expert_offset.data_ptr(),
                                    self.num_tokens_per_partition.data_ptr(),
                                    self.is_token_in_partition.data_ptr(), self.dst_slot.data_ptr(),
                                    self.src_of_slot.data_ptr(), self.status.data_ptr(), *opt)
        return self._ptrs

    def num_partition_rows(self) -> int:
        """Rp, rows of the non-expanded partition layout (synchronises)."""
        if self.partition_offset is None:
            raise ValueError("layout was built without the partition layout")
        return int(self.partition_offset[-1].item())

    def num_recv_rows(self) -> int:
        """R, the receive rows in use (synchronises: the page's do_cpu_sync)."""
        return int(self.expert_offset[-1].item())

    def check(self) -> int:
        """Synchronise and raise on device status bits; returns the bits."""
        st = int(self.status.item())
        if st & EP_DEV_BAD_EXPERT:
            raise ValueError("topk_idx holds an expert id outside [-1, num_experts)")
        if st & EP_DEV_CAPACITY:
            raise RuntimeError("an expert received more pairs than the fixed capacity")
        if st & EP_DEV_RECV_OVERFLOW:
            raise RuntimeError("receive rows exceed the allocated buffer")
        return st


def ep_get_layout(topk_idx: torch.Tensor, num_experts: int, expert_alignment: int = 1,
                  num_partitions: int = 1, capacity: int = 0,
                  max_recv_rows: Optional[int] = None,
                  cumulative_expert_stats: Optional[torch.Tensor] = None,
                  layout: Optional[Layout] = None, partition_layout: bool = False,
                  partitions_per_group: int = 0, partition_major: bool = False) -> Layout:
    """Derive the receive layout from topk_idx (int64 [T, K], -1 = none).
    capacity > 0 selects the fixed-capacity ("expand") layout.
    partition_layout=True also derives the non-expanded per-partition layout
    (token_slot etc., P <= 64); partitions_per_group sets G for
    num_tokens_per_group (0: one group).  partition_major=True groups the
    receive rows by partition instead of expert (pairs in (t, k) order inside
    each partition's segment; the per-expert tables then hold one entry per
    partition).  A `layout` of the same shape may be passed in to be
    rewritten in place."""
    lib = load_library()
    layout, params = _prepare_layout(topk_idx, num_experts, expert_alignment, num_partitions,
                                     capacity, max_recv_rows, cumulative_expert_stats, layout,
                                     partition_layout, partitions_per_group, partition_major)
    ptrs = layout.ptrs()
    _launch("ep_get_layout", topk_idx.device, lib.ep_get_layout,
            [cumulative_expert_stats, layout.workspace, layout.status],
            _ptr(topk_idx), ctypes.byref(params), ctypes.byref(ptrs),
            _ptr(cumulative_expert_stats), _ptr(layout.workspace),
            layout.workspace.numel(), _stream(topk_idx.device))
    return layout


def ep_get_layout_noalloc(topk_idx: torch.Tensor, layout: Layout,
                          cumulative_expert_stats: Optional[torch.Tensor] = None) -> Layout:
    """ep_get_layout into an existing `layout` (same shapes) with no
    workspace: the library's static per-GPU scratch is used instead (calls
    that overlap on one GPU race).  Allocates nothing."""
    lib = load_library()
    p = layout.params
    layout, params = _prepare_layout(topk_idx, p.num_experts, p.expert_alignment,
                                     p.num_partitions, p.capacity, p.max_recv_rows,
                                     cumulative_expert_stats, layout,
                                     layout.partition_offset is not None,
                                     p.partitions_per_group, bool(p.partition_major))
    ptrs = layout.ptrs()
    _launch("ep_get_layout_noalloc", topk_idx.device, lib.ep_get_layout_noalloc,
            [cumulative_expert_stats, layout.status],
            _ptr(topk_idx), ctypes.byref(params), ctypes.byref(ptrs),
            _ptr(cumulative_expert_stats), _stream(topk_idx.device))
    return layout


def _prepare_layout(topk_idx, num_experts, expert_alignment, num_partitions, capacity,
                    max_recv_rows, cumulative_expert_stats, layout, partition_layout,
                    partitions_per_group, partition_major=False):
    """(layout, params) for a layout call: a new Layout, or `layout` checked
    against these shapes."""
    _need_cuda(topk_idx, "topk_idx")
    if topk_idx.dtype != torch.int64 or topk_idx.dim() != 2:
        raise ValueError("topk_idx must be int64 [T, K]")
    T, K = topk_idx.shape
    pm = 1 if partition_major else 0
    if max_recv_rows is None:
        max_recv_rows = worst_case_recv_rows(T, K, num_experts, expert_alignment, capacity,
                                             num_partitions, partition_major)
    params = LayoutParams(num_tokens=T, num_topk=K, num_experts=num_experts,
                          expert_alignment=expert_alignment, num_partitions=num_partitions,
                          capacity=capacity, partitions_per_group=partitions_per_group,
                          partition_major=pm, max_recv_rows=int(max_recv_rows))
    if layout is None:
        layout = Layout(params, topk_idx.device, partition_layout)
    elif ((layout.params.num_tokens, layout.params.num_topk, layout.params.num_experts,
           layout.params.num_partitions, layout.params.max_recv_rows,
           layout.params.partitions_per_group or num_partitions, layout.params.partition_major)
          != (T, K, num_experts, num_partitions, int(max_recv_rows),
              partitions_per_group or num_partitions, pm)
          or (layout.partition_offset is not None) != partition_layout):
        raise ValueError("layout buffers do not match these shapes")
    else:
        layout.params = params
    if cumulative_expert_stats is not None:
        _need_cuda(cumulative_expert_stats, "cumulative_expert_stats")
        S = num_partitions if partition_major else num_experts
        if cumulative_expert_stats.dtype != torch.int32 or cumulative_expert_stats.numel() != S:
            raise ValueError("cumulative_expert_stats must be int32 [receive segments]")
    return layout, params


def _is_fp8(t: torch.Tensor) -> bool:
    return t.dtype in (torch.float8_e4m3fn, torch.uint8)


# Scale formats of the fp8 rows: fp32 amax/448, fp32 rounded up to a power of
# two, or that power of two as one UE8M0 byte (biased exponent).
_FP8_DTYPES = {"fp32": _abi.EP_DTYPE_FP8_E4M3, "pow2": _abi.EP_DTYPE_FP8_E4M3_POW2,
               "ue8m0": _abi.EP_DTYPE_FP8_E4M3_UE8M0}


def _fp8_dtype(scale_fmt: str) -> int:
    if scale_fmt not in _FP8_DTYPES:
        raise ValueError(f"scale_fmt must be one of {sorted(_FP8_DTYPES)}")
    return _FP8_DTYPES[scale_fmt]


def _scale_dtype(scale_fmt: str):
    return torch.uint8 if scale_fmt == "ue8m0" else torch.float32


def ep_dispatch(x: Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]], layout: Layout,
                topk_weights: Optional[torch.Tensor] = None, recv_fp8: bool = False,
                scale_group: int = 128, zero_padding: bool = False,
                num_recv_rows: Optional[int] = None,
                out: Optional[Sequence[Optional[torch.Tensor]]] = None,
                scale_fmt: str = "fp32"):
    """Permute token rows into the receive buffer.

    x: bf16 [T, H], or (fp8 codes [T, H], scales [T, H/G]: float32, or uint8
    UE8M0 bytes).  With bf16 x and recv_fp8=True the rows are cast to e4m3 on
    the fly with scales in `scale_fmt` ("fp32", "pow2" or "ue8m0").  Returns
    (recv_x, recv_scales or None, recv_topk_weights or None); recv buffers
    have num_recv_rows rows (default: the layout's max_recv_rows)."""
    lib = load_library()
    x, x_scales, scale_group, x_dtype, recv_dtype, scale_fmt = _x_and_dtypes(
        x, recv_fp8, scale_group, scale_fmt)
    bufs = _dispatch_buffers(x, layout, topk_weights, recv_dtype, scale_group, scale_fmt,
                             num_recv_rows, out)
    recv_x, recv_s, recv_w, rows = bufs
    params = layout.params
    ptrs = layout.ptrs()
    _launch("ep_dispatch", x.device, lib.ep_dispatch,
            [x_scales, topk_weights, recv_x, recv_s, recv_w, layout.status],
            _ptr(x), x_dtype, _ptr(x_scales), recv_dtype, x.shape[1], scale_group,
            _ptr(topk_weights), ctypes.byref(params), ctypes.byref(ptrs),
            _ptr(recv_x), _ptr(recv_s), _ptr(recv_w), rows,
            1 if zero_padding else 0, _stream(x.device))
    return recv_x, recv_s, recv_w


def ep_dispatch_with_layout(x: Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]],
                            topk_idx: torch.Tensor, num_experts: int, expert_alignment: int = 1,
                            topk_weights: Optional[torch.Tensor] = None, num_partitions: int = 1,
                            capacity: int = 0, max_recv_rows: Optional[int] = None,
                            cumulative_expert_stats: Optional[torch.Tensor] = None,
                            layout: Optional[Layout] = None, recv_fp8: bool = False,
                            scale_group: int = 128, zero_padding: bool = False,
                            num_recv_rows: Optional[int] = None,
                            out: Optional[Sequence[Optional[torch.Tensor]]] = None,
                            scale_fmt: str = "fp32", partition_major: bool = False):
    """ep_get_layout followed by ep_dispatch in one call (the layout's slots
    are derived by the dispatch kernels).  Arguments as the two calls; returns
    (layout, recv_x, recv_scales or None, recv_topk_weights or None), bit for
    bit what the two calls return."""
    lib = load_library()
    layout, params = _prepare_layout(topk_idx, num_experts, expert_alignment, num_partitions,
                                     capacity, max_recv_rows, cumulative_expert_stats, layout,
                                     False, 0, partition_major)
    x, x_scales, scale_group, x_dtype, recv_dtype, scale_fmt = _x_and_dtypes(
        x, recv_fp8, scale_group, scale_fmt)
    recv_x, recv_s, recv_w, rows = _dispatch_buffers(x, layout, topk_weights, recv_dtype,
                                                     scale_group, scale_fmt, num_recv_rows, out)
    ptrs = layout.ptrs()
    _launch("ep_dispatch_with_layout", x.device, lib.ep_dispatch_with_layout,
            [topk_idx, cumulative_expert_stats, layout.workspace, layout.status, x_scales,
             topk_weights, recv_x, recv_s, recv_w],
            _ptr(topk_idx), ctypes.byref(params), ctypes.byref(ptrs),
            _ptr(cumulative_expert_stats), _ptr(layout.workspace), layout.workspace.numel(),
            _ptr(x), x_dtype, _ptr(x_scales), recv_dtype, x.shape[1], scale_group,
            _ptr(topk_weights), _ptr(recv_x), _ptr(recv_s), _ptr(recv_w), rows,
            1 if zero_padding else 0, _stream(x.device))
    return layout, recv_x, recv_s, recv_w


def _dispatch_buffers(x, layout, topk_weights, recv_dtype, scale_group, scale_fmt,
                      num_recv_rows, out):
    """(recv_x, recv_scales, recv_topk_weights, rows) of a dispatch: the
    buffers given in `out`, checked, or new ones."""
    T, H = x.shape
    if T != layout.num_tokens:
        raise ValueError("x rows != layout tokens")
    rows = layout.max_recv_rows if num_recv_rows is None else int(num_recv_rows)
    dev = x.device
    recv_x = recv_s = recv_w = None
    if out is not None:
        recv_x, recv_s, recv_w = (list(out) + [None, None, None])[:3]
    fp8_out = recv_dtype != _abi.EP_DTYPE_BF16
    if recv_x is None:
        recv_x = torch.empty((rows, H), dtype=torch.float8_e4m3fn if fp8_out else torch.bfloat16,
                             device=dev)
    if fp8_out and recv_s is None:
        recv_s = torch.empty((rows, H // scale_group), dtype=_scale_dtype(scale_fmt), device=dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", _F32, layout.num_topk, rows=T)
        if recv_w is None:
            recv_w = torch.empty(rows, dtype=torch.float32, device=dev)
    _check(recv_x, "recv_x", _F8 if fp8_out else _BF16, H, min_rows=rows)
    if fp8_out:
        _check(recv_s, "recv_scales", (_scale_dtype(scale_fmt),), H // scale_group, min_rows=rows)
    _check(recv_w, "recv_topk_weights", _F32, min_rows=rows)
    return recv_x, recv_s, recv_w, rows


def ep_combine(y: torch.Tensor, layout: Layout, topk_weights: Optional[torch.Tensor] = None,
               bias: Union[None, torch.Tensor, Tuple[torch.Tensor, torch.Tensor]] = None,
               recv_topk_weights: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None):
    """Reduce expert outputs y (bf16 [rows, H], the receive layout) back to the
    tokens: out[t] = bias0 + bias1 + sum_k w[t,k] * y[dst_slot[t,k]] (fp32,
    k ascending, bf16 round to nearest even).  Returns (combined_x,
    combined_topk_weights or None)."""
    lib = load_library()
    _need_cuda(y, "y")
    if y.dtype != torch.bfloat16:
        raise ValueError("y must be bf16")
    rows, H = y.shape
    T, K = layout.num_tokens, layout.num_topk
    b0 = b1 = None
    if isinstance(bias, (tuple, list)):
        b0, b1 = (list(bias) + [None, None])[:2]
    elif bias is not None:
        b0 = bias
    for name, b in (("bias0", b0), ("bias1", b1)):
        if b is not None:
            _need_cuda(b, name)
            if b.dtype != torch.bfloat16 or tuple(b.shape) != (T, H):
                raise ValueError(f"{name} must be bf16 [T, H]")
    _check(topk_weights, "topk_weights", _F32, K, rows=T)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check(out, "out", _BF16, H, rows=T)
    cw = None
    if recv_topk_weights is not None:
        _check(recv_topk_weights, "recv_topk_weights", _F32, min_rows=rows)
        cw = torch.empty((T, K), dtype=torch.float32, device=y.device)
    params = layout.params
    ptrs = layout.ptrs()
    _launch("ep_combine", y.device, lib.ep_combine,
            [topk_weights, b0, b1, recv_topk_weights, out, layout.status],
            _ptr(y), H, rows, _ptr(topk_weights), _ptr(b0), _ptr(b1),
            ctypes.byref(params), ctypes.byref(ptrs), _ptr(recv_topk_weights),
            _ptr(cw), _ptr(out), _stream(y.device))
    return out, cw


def ep_probe_dispatch_stores(recv_x: torch.Tensor, layout: Layout, pattern: int = 0x3F803F80):
    """A measurement aid, not a step of the method: the bf16 dispatch's row
    stores (same kernel, grid and order) with every token row replaced by the
    32-bit `pattern`, so that no token row is read.  Writes
    recv_x[dst_slot[t, k]] for every kept pair; returns recv_x."""
    lib = load_library()
    _need_cuda(recv_x, "recv_x")
    if recv_x.dtype != torch.bfloat16 or recv_x.dim() != 2:
        raise ValueError("recv_x must be bf16 [rows, H]")
    _check(recv_x, "recv_x", _BF16, recv_x.shape[1])
    params = layout.params
    ptrs = layout.ptrs()
    _launch("ep_probe_dispatch_stores", recv_x.device, lib.ep_probe_dispatch_stores,
            [recv_x, layout.status], recv_x.shape[1], int(pattern) & 0xFFFFFFFF,
            ctypes.byref(params), ctypes.byref(ptrs), _ptr(recv_x), recv_x.shape[0],
            _stream(recv_x.device))
    return recv_x


def logfmt_row_bytes(hidden: int) -> int:
    """Bytes of one row of the 10-bit logarithmic payload (hidden a positive
    multiple of 128)."""
    n = int(load_library().ep_logfmt_row_bytes(int(hidden)))
    if n < 0:
        raise ValueError("hidden must be a positive multiple of 128")
    return n


_U8 = (torch.uint8,)


def ep_logfmt_encode(y: torch.Tensor, out: Optional[torch.Tensor] = None,
                     layout: Optional[Layout] = None) -> torch.Tensor:
    """bf16 rows [rows, H] -> 10-bit logarithmic payload, uint8
    [rows, logfmt_row_bytes(H)] (the use_logfmt format of the low-latency
    combine; layout and rounding in include/ep.h).  With `layout` (the
    receive layout the rows belong to) only rows that hold a pair are
    encoded; the others are left as they are (a combine never reads them)."""
    lib = load_library()
    _need_cuda(y, "y")
    if y.dtype != torch.bfloat16 or y.dim() != 2:
        raise ValueError("y must be bf16 [rows, H]")
    rows, H = y.shape
    rb = logfmt_row_bytes(H)
    if out is None:
        out = torch.empty((rows, rb), dtype=torch.uint8, device=y.device)
    _check(out, "out", _U8, rb, rows=rows)
    if layout is None:
        _launch("ep_logfmt_encode", y.device, lib.ep_logfmt_encode, [out],
                _ptr(y), rows, H, None, None, _ptr(out), _stream(y.device))
        return out
    if rows > layout.max_recv_rows:
        raise ValueError("y has more rows than the layout's max_recv_rows")
    params = layout.params
    ptrs = layout.ptrs()
    _launch("ep_logfmt_encode", y.device, lib.ep_logfmt_encode, [out, layout.src_of_slot],
            _ptr(y), rows, H, ctypes.byref(params), ctypes.byref(ptrs), _ptr(out),
            _stream(y.device))
    return out


def ep_logfmt_decode(payload: torch.Tensor, hidden: int,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """10-bit logarithmic payload -> bf16 rows [rows, hidden] (exact)."""
    lib = load_library()
    rb = logfmt_row_bytes(hidden)
    _check(payload, "payload", _U8, rb)
    rows = payload.shape[0]
    if out is None:
        out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=payload.device)
    _check(out, "out", _BF16, hidden, rows=rows)
    _launch("ep_logfmt_decode", payload.device, lib.ep_logfmt_decode, [out],
            _ptr(payload), rows, hidden, _ptr(out), _stream(payload.device))
    return out


def ep_combine_logfmt(payload: torch.Tensor, hidden: int, layout: Layout,
                      topk_weights: Optional[torch.Tensor] = None,
                      bias: Union[None, torch.Tensor, Tuple[torch.Tensor, torch.Tensor]] = None,
                      recv_topk_weights: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None):
    """ep_combine over payload rows from ep_logfmt_encode (uint8
    [rows, logfmt_row_bytes(hidden)]): bit for bit the combine of the decoded
    rows.  Returns (combined_x, combined_topk_weights or None)."""
    lib = load_library()
    rb = logfmt_row_bytes(hidden)
    _check(payload, "payload", _U8, rb)
    rows, H = payload.shape[0], hidden
    T, K = layout.num_tokens, layout.num_topk
    b0 = b1 = None
    if isinstance(bias, (tuple, list)):
        b0, b1 = (list(bias) + [None, None])[:2]
    elif bias is not None:
        b0 = bias
    for name, b in (("bias0", b0), ("bias1", b1)):
        if b is not None:
            _need_cuda(b, name)
            if b.dtype != torch.bfloat16 or tuple(b.shape) != (T, H):
                raise ValueError(f"{name} must be bf16 [T, H]")
    _check(topk_weights, "topk_weights", _F32, K, rows=T)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=payload.device)
    _check(out, "out", _BF16, H, rows=T)
    cw = None
    if recv_topk_weights is not None:
        _check(recv_topk_weights, "recv_topk_weights", _F32, min_rows=rows)
        cw = torch.empty((T, K), dtype=torch.float32, device=payload.device)
    params = layout.params
    ptrs = layout.ptrs()
    _launch("ep_combine_logfmt", payload.device, lib.ep_combine_logfmt,
            [topk_weights, b0, b1, recv_topk_weights, out, layout.status],
            _ptr(payload), H, rows, _ptr(topk_weights), _ptr(b0), _ptr(b1),
            ctypes.byref(params), ctypes.byref(ptrs), _ptr(recv_topk_weights),
            _ptr(cw), _ptr(out), _stream(payload.device))
    return out, cw


def ep_cast_fp8(x: torch.Tensor, group: int = 128,
                out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None, scale_fmt: str = "fp32"):
    """Per (token, group of `group` channels) cast of bf16 rows to e4m3.
    Returns (codes float8_e4m3fn [T, H], scales [T, H/group]): float32 for
    scale_fmt "fp32" (amax/448) and "pow2" (rounded up to a power of two),
    uint8 biased exponents for "ue8m0"."""
    lib = load_library()
    _need_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    out_dtype = _fp8_dtype(scale_fmt)
    T, H = x.shape
    if out is None:
        q = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=x.device)
        s = torch.empty((T, H // group), dtype=_scale_dtype(scale_fmt), device=x.device)
    else:
        q, s = out
    _check(q, "x_fp8", _F8, H, rows=T)
    _check(s, "scales", (_scale_dtype(scale_fmt),), H // group, rows=T)
    _launch("ep_cast_fp8", x.device, lib.ep_cast_fp8, [q, s],
            _ptr(x), T, H, group, out_dtype, _ptr(q), _ptr(s), _stream(x.device))
    return q, s


def _x_and_dtypes(x, recv_fp8, scale_group, scale_fmt="fp32"):
    """(x, x_scales, G, x_dtype, recv_dtype, scale_fmt) for a dispatch call;
    fp8 input with uint8 scales is UE8M0."""
    x_scales = None
    if isinstance(x, (tuple, list)):
        x, x_scales = x
    _need_cuda(x, "x")
    H = x.shape[1]
    if _is_fp8(x):
        if x_scales is None:
            raise ValueError("fp8 x needs its scales")
        _need_cuda(x_scales, "x_scales")
        if x_scales.dtype == torch.uint8:
            scale_fmt = "ue8m0"
        elif x_scales.dtype != torch.float32:
            raise ValueError("fp8 scales must be float32 or uint8 (UE8M0)")
        elif scale_fmt == "ue8m0":
            scale_fmt = "fp32"
        d = _fp8_dtype(scale_fmt)
        if x_scales.dim() != 2 or x_scales.shape[0] != x.shape[0] or x_scales.shape[1] < 1 \
                or H % x_scales.shape[1] != 0:
            raise ValueError("x_scales must be [T, H / group]")
        return x, x_scales, H // x_scales.shape[1], d, d, scale_fmt
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16 or fp8")
    recv = _fp8_dtype(scale_fmt) if recv_fp8 else _abi.EP_DTYPE_BF16
    return x, None, scale_group, _abi.EP_DTYPE_BF16, recv, scale_fmt


def ep_dispatch_partitioned(x: Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]],
                            layout: Layout, topk_idx: torch.Tensor,
                            topk_weights: Optional[torch.Tensor] = None, recv_fp8: bool = False,
                            scale_group: int = 128, num_recv_rows: Optional[int] = None,
                            out: Optional[Sequence[Optional[torch.Tensor]]] = None,
                            scale_fmt: str = "fp32"):
    """Non-expanded dispatch: token t's row goes once to every partition q
    that owns one of its experts, at layout.token_slot[t, q].  Returns
    (recv_x, recv_scales or None, recv_topk_idx int64 [rows, K] with the
    partition-local expert id or -1, recv_topk_weights float32 [rows, K] or
    None).  rows defaults to T*P, the worst case; `out` may supply the four
    buffers (None entries are allocated)."""
    lib = load_library()
    if layout.token_slot is None:
        raise ValueError("the partitioned dispatch needs token_slot: partition_layout=True, P <= 64")
    x, x_scales, scale_group, x_dtype, recv_dtype, scale_fmt = _x_and_dtypes(
        x, recv_fp8, scale_group, scale_fmt)
    T, H = x.shape
    K = layout.num_topk
    if T != layout.num_tokens:
        raise ValueError("x rows != layout tokens")
    _check(topk_idx, "topk_idx", _I64, K, rows=T)
    rows = T * layout.num_partitions if num_recv_rows is None else int(num_recv_rows)
    dev = x.device
    fp8_out = recv_dtype != _abi.EP_DTYPE_BF16
    recv_x = recv_s = recv_i = recv_w = None
    if out is not None:
        recv_x, recv_s, recv_i, recv_w = (list(out) + [None] * 4)[:4]
    if recv_x is None:
        recv_x = torch.empty((rows, H), dtype=torch.float8_e4m3fn if fp8_out else torch.bfloat16,
                             device=dev)
    if fp8_out and recv_s is None:
        recv_s = torch.empty((rows, H // scale_group), dtype=_scale_dtype(scale_fmt), device=dev)
    if recv_i is None:
        recv_i = torch.empty((rows, K), dtype=torch.int64, device=dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", _F32, K, rows=T)
        if recv_w is None:
            recv_w = torch.empty((rows, K), dtype=torch.float32, device=dev)
    else:
        recv_w = None
    _check(recv_x, "recv_x", _F8 if fp8_out else _BF16, H, min_rows=rows)
    if fp8_out:
        _check(recv_s, "recv_scales", (_scale_dtype(scale_fmt),), H // scale_group, min_rows=rows)
    _check(recv_i, "recv_topk_idx", _I64, K, min_rows=rows)
    _check(recv_w, "recv_topk_weights", _F32, K, min_rows=rows)
    params = layout.params
    ptrs = layout.ptrs()
    _launch("ep_dispatch_partitioned", dev, lib.ep_dispatch_partitioned,
            [x_scales, topk_idx, topk_weights, recv_x, recv_s, recv_i, recv_w, layout.status],
            _ptr(x), x_dtype, _ptr(x_scales), recv_dtype, H, scale_group,
            _ptr(topk_idx), _ptr(topk_weights), ctypes.byref(params),
            ctypes.byref(ptrs), _ptr(recv_x), _ptr(recv_s), _ptr(recv_i),
            _ptr(recv_w), rows, _stream(dev))
    return recv_x, recv_s, recv_i, recv_w


def _biases(bias, T, H):
    b0 = b1 = None
    if isinstance(bias, (tuple, list)):
        b0, b1 = (list(bias) + [None, None])[:2]
    elif bias is not None:
        b0 = bias
    for name, b in (("bias0", b0), ("bias1", b1)):
        if b is not None:
            _need_cuda(b, name)
            if b.dtype != torch.bfloat16 or tuple(b.shape) != (T, H):
                raise ValueError(f"{name} must be bf16 [T, H]")
    return b0, b1


def ep_combine_partitioned(y: torch.Tensor, layout: Layout,
                           bias: Union[None, torch.Tensor, Tuple[torch.Tensor, torch.Tensor]] = None,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Plain sum of the partitions' rows back to the tokens (fp32, partition
    order, bias first, bf16 round to nearest even)."""
    lib = load_library()
    if layout.token_slot is None:
        raise ValueError("the partitioned combine needs token_slot: partition_layout=True, P <= 64")
    _need_cuda(y, "y")
    if y.dtype != torch.bfloat16:
        raise ValueError("y must be bf16")
    rows, H = y.shape
    T = layout.num_tokens
    b0, b1 = _biases(bias, T, H)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check(out, "out", _BF16, H, rows=T)
    params = layout.params
    ptrs = layout.ptrs()
    _launch("ep_combine_partitioned", y.device, lib.ep_combine_partitioned,
            [b0, b1, out, layout.status],
            _ptr(y), H, rows, _ptr(b0), _ptr(b1), ctypes.byref(params),
            ctypes.byref(ptrs), _ptr(out), _stream(y.device))
    return out


def ep_combine_reduced(y: torch.Tensor, layout: Layout, topk_idx: torch.Tensor,
                       topk_weights: Optional[torch.Tensor] = None,
                       bias: Union[None, torch.Tensor, Tuple[torch.Tensor, torch.Tensor]] = None,
                       out: Optional[torch.Tensor] = None,
                       bf16_partials: bool = False) -> torch.Tensor:
    """Two-level combine on the expanded layout: each partition's weighted
    pairs summed in fp32 (rounded to bf16 with bf16_partials), then the
    partials (and bias) summed in fp32 in partition order and rounded to bf16."""
    lib = load_library()
    _need_cuda(y, "y")
    if y.dtype != torch.bfloat16:
        raise ValueError("y must be bf16")
    rows, H = y.shape
    T, K = layout.num_tokens, layout.num_topk
    _check(topk_idx, "topk_idx", _I64, K, rows=T)
    b0, b1 = _biases(bias, T, H)
    _check(topk_weights, "topk_weights", _F32, K, rows=T)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check(out, "out", _BF16, H, rows=T)
    params = layout.params
    ptrs = layout.ptrs()
    _launch("ep_combine_reduced", y.device, lib.ep_combine_reduced,
            [topk_idx, topk_weights, b0, b1, out, layout.status],
            _ptr(y), H, rows, _ptr(topk_idx), _ptr(topk_weights), _ptr(b0),
            _ptr(b1), ctypes.byref(params), ctypes.byref(ptrs), _ptr(out),
            1 if bf16_partials else 0, _stream(y.device))
    return out
