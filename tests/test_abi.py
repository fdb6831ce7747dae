"""The C-ABI library loads, exports every symbol include/ep.h declares, and
rejects bad arguments on the host before any GPU work (no compute calls)."""
import ctypes
import os
import re

import pytest

from combine_ep_get_layout_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ep.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_\w+)\s*\(", src)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(_abi.EXPORTS)


def test_library_exports_every_symbol():
    lib = _abi.load()
    for name in _declared():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def _params(T=16, K=2, E=8, A=1, P=1, C=0, rows=None, G=0, PM=0):
    p = _abi.LayoutParams(T, K, E, A, P, C, G, PM)
    p.max_recv_rows = rows if rows is not None else _abi.load().ep_worst_case_recv_rows(ctypes.byref(p))
    return p


def test_worst_case_rows():
    lib = _abi.load()
    assert lib.ep_worst_case_recv_rows(ctypes.byref(_params(4096, 8, 256, 128))) == 32768 + 256 * 127
    assert lib.ep_worst_case_recv_rows(ctypes.byref(_params(2, 2, 256, 128))) == 4 + 4 * 127
    assert lib.ep_worst_case_recv_rows(ctypes.byref(_params(128, 8, 256, 1, C=128))) == 32768
    # partition-major: one segment per partition
    assert lib.ep_worst_case_recv_rows(ctypes.byref(_params(4096, 8, 256, 128, P=32, PM=1))) \
        == 32768 + 32 * 127
    assert lib.ep_worst_case_recv_rows(ctypes.byref(_params(128, 8, 256, 1, P=8, C=128, PM=1))) \
        == 8 * 128


def test_workspace_bytes():
    lib = _abi.load()
    n = lib.ep_get_layout_workspace_bytes(ctypes.byref(_params(4096, 8, 256, 128)))
    assert n > 0 and n % 256 == 0
    assert lib.ep_get_layout_workspace_bytes(ctypes.byref(_params(E=6, P=4))) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(E=6, P=4), _abi.EP_ERR_INVALID_ARG),        # E % P != 0
    (dict(A=0), _abi.EP_ERR_INVALID_ARG),             # A < 1
    (dict(K=0), _abi.EP_ERR_INVALID_ARG),
    (dict(T=-1), _abi.EP_ERR_INVALID_ARG),
    (dict(C=6, A=4), _abi.EP_ERR_INVALID_ARG),        # C % A != 0
    (dict(C=4, rows=10), _abi.EP_ERR_INVALID_ARG),    # E*C > max_recv_rows
    (dict(E=8192, P=1), _abi.EP_ERR_UNSUPPORTED),
    (dict(K=300, E=512), _abi.EP_ERR_UNSUPPORTED),
    (dict(E=8, P=4, G=3), _abi.EP_ERR_INVALID_ARG),   # P % G != 0
    (dict(E=8, P=4, G=-1), _abi.EP_ERR_INVALID_ARG),
    (dict(PM=2), _abi.EP_ERR_INVALID_ARG),            # partition_major not 0 or 1
    (dict(E=8, P=2, C=4, rows=7, PM=1), _abi.EP_ERR_INVALID_ARG),   # P*C > max_recv_rows
])
def test_get_layout_rejects_bad_params_before_launch(kw, code):
    lib = _abi.load()
    p = _params(**kw)
    lay = _abi.LayoutPtrs(*([8] * 7))       # never dereferenced: rejected first
    rc = lib.ep_get_layout(ctypes.c_void_p(16), ctypes.byref(p), ctypes.byref(lay), None,
                           ctypes.c_void_p(256), 1 << 20, None)
    assert rc == code


def test_get_layout_noalloc_rejects_layouts_beyond_its_scratch():
    """More than the static scratch holds (8 MiB) is refused on the host,
    before any GPU call (so this runs without a GPU)."""
    lib = _abi.load()
    p = _params(T=2_000_000, K=8, E=256, A=1)
    assert lib.ep_get_layout_workspace_bytes(ctypes.byref(p)) > 8 << 20
    lay = _abi.LayoutPtrs(*([16] * 7))
    assert lib.ep_get_layout_noalloc(ctypes.c_void_p(16), ctypes.byref(p), ctypes.byref(lay), None,
                                     None) == _abi.EP_ERR_WORKSPACE
    assert lib.ep_get_layout_noalloc(ctypes.c_void_p(16), ctypes.byref(_params(E=6, P=4)),
                                     ctypes.byref(lay), None, None) == _abi.EP_ERR_INVALID_ARG


def test_get_layout_rejects_null_buffers_and_small_workspace():
    lib = _abi.load()
    p = _params()
    lay = _abi.LayoutPtrs(16, 16, 16, 16, 16, 16, None)   # status missing
    assert lib.ep_get_layout(ctypes.c_void_p(16), ctypes.byref(p), ctypes.byref(lay), None,
                             ctypes.c_void_p(256), 1 << 20, None) == _abi.EP_ERR_INVALID_ARG
    lay = _abi.LayoutPtrs(*([16] * 7))
    assert lib.ep_get_layout(None, ctypes.byref(p), ctypes.byref(lay), None,
                             ctypes.c_void_p(256), 1 << 20, None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_get_layout(ctypes.c_void_p(16), ctypes.byref(p), ctypes.byref(lay), None,
                             ctypes.c_void_p(256), 16, None) == _abi.EP_ERR_WORKSPACE
    assert lib.ep_get_layout(ctypes.c_void_p(16), ctypes.byref(p), ctypes.byref(lay), None,
                             ctypes.c_void_p(260), 1 << 20, None) == _abi.EP_ERR_WORKSPACE


def test_dispatch_rejects_bad_arguments():
    lib = _abi.load()
    p = _params(T=4, K=2, E=8)
    lay = _abi.LayoutPtrs(*([16] * 7))
    bf, f8 = _abi.EP_DTYPE_BF16, _abi.EP_DTYPE_FP8_E4M3

    def call(x=16, xd=bf, xs=None, rd=bf, H=64, G=128, rs=None, rows=8):
        return lib.ep_dispatch(ctypes.c_void_p(x), xd, xs, rd, H, G, None, ctypes.byref(p),
                               ctypes.byref(lay), ctypes.c_void_p(16), rs, None, rows, 0, None)
    assert call(H=60) == _abi.EP_ERR_INVALID_ARG              # hidden % 8
    assert call(x=24) == _abi.EP_ERR_INVALID_ARG              # x misaligned
    assert call(xd=f8, rd=bf) == _abi.EP_ERR_INVALID_ARG      # fp8 -> bf16 is not a mode
    assert call(rd=f8, H=128, G=128) == _abi.EP_ERR_INVALID_ARG   # fp8 recv without scales
    assert call(rd=f8, H=120, G=8, rs=16) == _abi.EP_ERR_INVALID_ARG   # hidden % 16
    assert call(rd=f8, H=192, G=96, rs=16) == _abi.EP_ERR_UNSUPPORTED  # group not a power of 2
    assert call(rd=f8, H=128, G=1024, rs=16) == _abi.EP_ERR_UNSUPPORTED
    assert call(xd=f8, rd=f8, H=128, rs=16) == _abi.EP_ERR_INVALID_ARG  # fp8 x without scales
    ue, p2 = _abi.EP_DTYPE_FP8_E4M3_UE8M0, _abi.EP_DTYPE_FP8_E4M3_POW2
    assert call(xd=ue, rd=f8, H=128, rs=16) == _abi.EP_ERR_INVALID_ARG  # copy changes scale format
    assert call(xd=p2, rd=ue, H=128, rs=16) == _abi.EP_ERR_INVALID_ARG
    assert call(xd=f8, rd=bf) == _abi.EP_ERR_INVALID_ARG
    assert call(rd=7, H=128, rs=16) == _abi.EP_ERR_INVALID_ARG           # unknown dtype
    assert call(rows=-1) == _abi.EP_ERR_INVALID_ARG
    # float scale rows must be 4-byte aligned
    assert call(rd=f8, H=128, rs=18) == _abi.EP_ERR_INVALID_ARG
    assert call(xd=f8, rd=f8, H=128, xs=ctypes.c_void_p(18), rs=16) == _abi.EP_ERR_INVALID_ARG


def test_combine_and_cast_reject_bad_arguments():
    lib = _abi.load()
    p = _params(T=4, K=2, E=8)
    lay = _abi.LayoutPtrs(*([16] * 7))
    assert lib.ep_combine(ctypes.c_void_p(16), 12, 8, None, None, None, ctypes.byref(p),
                          ctypes.byref(lay), None, None, ctypes.c_void_p(16), None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_combine(ctypes.c_void_p(16), 64, 8, None, ctypes.c_void_p(8), None,
                          ctypes.byref(p), ctypes.byref(lay), None, None, ctypes.c_void_p(16),
                          None) == _abi.EP_ERR_INVALID_ARG       # misaligned bias
    assert lib.ep_combine(ctypes.c_void_p(16), 64, 8, None, None, None, ctypes.byref(p),
                          ctypes.byref(lay), None, ctypes.c_void_p(16), ctypes.c_void_p(16),
                          None) == _abi.EP_ERR_INVALID_ARG       # combined weights need recv weights
    f8 = _abi.EP_DTYPE_FP8_E4M3
    assert lib.ep_cast_fp8(ctypes.c_void_p(16), 4, 100, 128, f8, ctypes.c_void_p(16),
                           ctypes.c_void_p(16), None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_cast_fp8(ctypes.c_void_p(16), 4, 384, 96, f8, ctypes.c_void_p(16),
                           ctypes.c_void_p(16), None) == _abi.EP_ERR_UNSUPPORTED
    assert lib.ep_cast_fp8(ctypes.c_void_p(16), 4, 128, 128, _abi.EP_DTYPE_BF16,
                           ctypes.c_void_p(16), ctypes.c_void_p(16), None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_cast_fp8(ctypes.c_void_p(16), 0, 128, 128, f8, None, None, None) == _abi.EP_OK
    assert lib.ep_cast_fp8(ctypes.c_void_p(16), 4, 128, 128, f8, ctypes.c_void_p(16),
                           ctypes.c_void_p(18), None) == _abi.EP_ERR_INVALID_ARG   # float scales


def test_probe_dispatch_stores_rejects_bad_arguments():
    lib = _abi.load()
    p = _params(T=4, K=2, E=8)
    lay = _abi.LayoutPtrs(*([16] * 7))
    f = lib.ep_probe_dispatch_stores
    assert f(12, 0, ctypes.byref(p), ctypes.byref(lay), ctypes.c_void_p(16), 8, None) \
        == _abi.EP_ERR_INVALID_ARG                               # hidden % 8 != 0
    assert f(_abi.EP_MAX_HIDDEN + 8, 0, ctypes.byref(p), ctypes.byref(lay), ctypes.c_void_p(16), 8,
             None) == _abi.EP_ERR_UNSUPPORTED
    assert f(64, 0, ctypes.byref(p), ctypes.byref(lay), ctypes.c_void_p(8), 8, None) \
        == _abi.EP_ERR_INVALID_ARG                               # misaligned rows
    assert f(64, 0, ctypes.byref(p), None, ctypes.c_void_p(16), 8, None) == _abi.EP_ERR_INVALID_ARG
    assert f(64, 0, ctypes.byref(p), ctypes.byref(lay), ctypes.c_void_p(16), -1, None) \
        == _abi.EP_ERR_INVALID_ARG
    assert f(64, 0, ctypes.byref(_params(E=6, P=4)), ctypes.byref(lay), ctypes.c_void_p(16), 8,
             None) == _abi.EP_ERR_INVALID_ARG                    # the layout params are checked


def test_logfmt_calls_reject_bad_arguments():
    lib = _abi.load()
    assert lib.ep_logfmt_row_bytes(7168) == 9088 and lib.ep_logfmt_row_bytes(128) == 256
    for h in (0, -128, 64, 200, 1000):
        assert lib.ep_logfmt_row_bytes(h) == _abi.EP_ERR_INVALID_ARG
    v16, v8 = ctypes.c_void_p(16), ctypes.c_void_p(8)
    enc = lambda x, n, h, p, s: lib.ep_logfmt_encode(x, n, h, None, None, p, s)
    for fn in (enc, lib.ep_logfmt_decode):
        assert fn(v16, 4, 192, v16, None) == _abi.EP_ERR_INVALID_ARG      # hidden % 128
        assert fn(v16, -1, 128, v16, None) == _abi.EP_ERR_INVALID_ARG
        assert fn(v8, 4, 128, v16, None) == _abi.EP_ERR_INVALID_ARG       # misaligned
        assert fn(v16, 4, 128, None, None) == _abi.EP_ERR_INVALID_ARG
        assert fn(None, 0, 128, None, None) == _abi.EP_OK                 # nothing to do
    p = _params(T=4, K=2, E=8)
    lay = _abi.LayoutPtrs(*([16] * 7))
    assert lib.ep_logfmt_encode(v16, 4, 128, ctypes.byref(p), None, v16,
                                None) == _abi.EP_ERR_INVALID_ARG     # params without layout
    assert lib.ep_logfmt_encode(v16, 4, 128, None, ctypes.byref(lay), v16,
                                None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_logfmt_encode(v16, p.max_recv_rows + 1, 128, ctypes.byref(p),
                                ctypes.byref(lay), v16, None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_combine_logfmt(v16, 64, 8, None, None, None, ctypes.byref(p), ctypes.byref(lay),
                                 None, None, v16, None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_combine_logfmt(v16, 128, 8, None, v8, None, ctypes.byref(p), ctypes.byref(lay),
                                 None, None, v16, None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_combine_logfmt(v16, 128, 8, None, None, None, ctypes.byref(p),
                                 ctypes.byref(lay), None, v16, v16,
                                 None) == _abi.EP_ERR_INVALID_ARG
    assert lib.ep_combine_logfmt(v8, 128, 8, None, None, None, ctypes.byref(p), ctypes.byref(lay),
                                 None, None, v16, None) == _abi.EP_ERR_INVALID_ARG


def test_partition_layout_limits():
    lib = _abi.load()
    p = _params(T=4, K=2, E=128, P=128)
    lay = _abi.LayoutPtrs(*([16] * 8), 16, None)           # token_slot with P > 64
    assert lib.ep_get_layout(ctypes.c_void_p(16), ctypes.byref(p), ctypes.byref(lay), None,
                             ctypes.c_void_p(256), 1 << 20, None) == _abi.EP_ERR_UNSUPPORTED


def test_partitioned_calls_reject_bad_arguments():
    lib = _abi.load()
    bf = _abi.EP_DTYPE_BF16
    p = _params(T=4, K=2, E=8, P=4)
    no_slots = _abi.LayoutPtrs(*([16] * 7))
    lay = _abi.LayoutPtrs(*([16] * 10))

    def disp(layout, H=64, idx=16, ri=16):
        return lib.ep_dispatch_partitioned(ctypes.c_void_p(16), bf, None, bf, H, 128,
                                           ctypes.c_void_p(idx) if idx else None, None,
                                           ctypes.byref(p), ctypes.byref(layout),
                                           ctypes.c_void_p(16), None,
                                           ctypes.c_void_p(ri) if ri else None, None, 16, None)
    assert disp(no_slots) == _abi.EP_ERR_INVALID_ARG           # no token_slot
    assert disp(lay, H=60) == _abi.EP_ERR_INVALID_ARG
    assert disp(lay, idx=0) == _abi.EP_ERR_INVALID_ARG         # recv_topk_idx needs topk_idx
    assert lib.ep_combine_partitioned(ctypes.c_void_p(16), 64, 16, None, None, ctypes.byref(p),
                                      ctypes.byref(no_slots), ctypes.c_void_p(16),
                                      None) == _abi.EP_ERR_INVALID_ARG
    big = _params(T=4, K=2, E=128, P=128)
    assert lib.ep_combine_partitioned(ctypes.c_void_p(16), 64, 16, None, None, ctypes.byref(big),
                                      ctypes.byref(lay), ctypes.c_void_p(16),
                                      None) == _abi.EP_ERR_UNSUPPORTED
    assert lib.ep_combine_reduced(ctypes.c_void_p(16), 64, 16, None, None, None, None,
                                  ctypes.byref(p), ctypes.byref(lay), ctypes.c_void_p(16),
                                  0, None) == _abi.EP_ERR_INVALID_ARG   # no topk_idx
    k100 = _params(T=4, K=100, E=128, P=4)
    assert lib.ep_combine_reduced(ctypes.c_void_p(16), 64, 16, ctypes.c_void_p(16), None, None,
                                  None, ctypes.byref(k100), ctypes.byref(lay),
                                  ctypes.c_void_p(16), 0, None) == _abi.EP_ERR_UNSUPPORTED


def test_status_strings():
    lib = _abi.load()
    for code in (0, -1, -2, -3, -4, 7):
        assert lib.ep_status_string(code)


def test_layout_pointer_struct_follows_buffer_changes():
    """The binding keeps each layout's pointer struct between calls; replacing
    or dropping a buffer must rebuild it, or a call would pass the freed
    buffer's address (whose memory torch may already have handed out)."""
    import torch
    import combine_ep_get_layout_amd as ep
    p = _abi.LayoutParams(num_tokens=4, num_topk=2, num_experts=8, expert_alignment=1,
                          num_partitions=2, max_recv_rows=8)
    lay = ep.Layout(p, torch.device("cpu"), partition_layout=True)
    first = lay.ptrs()
    assert lay.ptrs() is first and first.partition_src == lay.partition_src.data_ptr()
    lay.partition_src = None
    second = lay.ptrs()
    assert second is not first and not second.partition_src
    lay.dst_slot = torch.empty((4, 2), dtype=torch.int32)
    assert lay.ptrs().dst_slot == lay.dst_slot.data_ptr()
