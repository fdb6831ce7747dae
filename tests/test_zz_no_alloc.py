"""ep_get_layout_noalloc (the layout on the library's static per-GPU
scratch, for callers that cannot allocate) against ep_get_layout with its
own workspace: every layout buffer bit for bit, on two calls in a row, the
second with a smaller batch, called through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import ep_inputs
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("num_tokens_per_expert", "expert_offset", "num_tokens_per_partition",
         "is_token_in_partition", "dst_slot", "status")


def _noalloc_through_abi(ep, lay, idx, stats):
    from combine_ep_get_layout_amd import _abi
    lib = _abi.load()
    ptrs = lay.ptrs()
    rc = lib.ep_get_layout_noalloc(ctypes.c_void_p(idx.data_ptr()), ctypes.byref(lay.params),
                                   ctypes.byref(ptrs),
                                   None if stats is None else ctypes.c_void_p(stats.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == _abi.EP_OK


@pytest.mark.parametrize("first,second", [(("prefill", 4096, 128, 1), ("prefill", 1000, 16, 4)),
                                          (("skewed", 8192, 128, 32), ("tiny", 64, 1, 1))])
def test_noalloc_layout_matches_workspace_layout(gpu, first, second):
    for name, T, A, P in (first, second):
        announce("noalloc", name, T, A, P)
        w = ep_inputs.make_workload(name, T=T, with_x=False)
        E = w.num_experts
        idx = to_dev(w.topk_idx)
        st_ref = torch.full((E,), 7, dtype=torch.int32, device="cuda:0")
        st_new = st_ref.clone()
        ref = gpu.ep_get_layout(idx, E, A, P, cumulative_expert_stats=st_ref)
        new = gpu.Layout(ref.params, idx.device)
        for t in (new.num_tokens_per_expert, new.expert_offset, new.dst_slot, new.status):
            t.fill_(-5)
        new.src_of_slot.copy_(ref.src_of_slot)    # entries past R are not written by either
        new.src_of_slot[:ref.num_recv_rows()].fill_(-5)
        _noalloc_through_abi(gpu, new, idx, st_new)
        torch.cuda.synchronize()
        for n in NAMES:
            assert torch.equal(getattr(ref, n), getattr(new, n)), n
        assert torch.equal(ref.src_of_slot, new.src_of_slot)
        assert torch.equal(st_ref, st_new)
        assert new.check() == 0
