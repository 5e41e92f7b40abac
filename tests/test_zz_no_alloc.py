"""The allocation-free layout entry point (scratch in the library's static
per-GPU array) against the entry point that takes a workspace: same bits on
two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents), and a clear error past the scratch's size."""
import ctypes

import numpy as np
import pytest
import torch

import combine_router_softmax_amd as moe
from combine_router_softmax_amd import LayoutDesc
from oracle import COMPACT, PADDED, dispatch_layout, route_topk, worst_case_rows
from synth import get_config, make_routing_inputs
from util import flush, i64

pytestmark = pytest.mark.gpu

KEYS = ("counts", "expert_off", "row_of", "row_token", "status")


def _case(name, seed, layout):
    cfg = get_config(name)
    d = make_routing_inputs(cfg, seed)
    idx, _ = route_topk(d["logits"], cfg.top_k)
    off = d["src_offsets"]
    N = len(idx)
    cap = worst_case_rows(N, cfg.top_k, cfg.n_local) if layout == COMPACT else int(np.diff(off).max())
    return cfg, idx, off, cap


@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_noalloc_layout_matches_workspace_entry_point(layout):
    for name, seed in (("dsv3_prefill_ep8", 0), ("tiny", 3)):  # the second call is much smaller
        cfg, idx_np, off_np, cap = _case(name, seed, layout)
        flush(f"noalloc layout {name} layout={layout} tokens={len(idx_np)}")
        idx = torch.from_numpy(idx_np.astype(np.int32)).cuda()
        off = torch.from_numpy(off_np.astype(np.int32)).cuda()
        ref = moe.moe_dispatch_layout(idx, off, cfg.n_experts, cfg.expert_lo, cfg.n_local, layout, cap)
        # outputs pre-filled with junk: every word the call owns must be written
        out = {k: torch.full_like(ref[k], -7) for k in KEYS}
        got = moe.moe_dispatch_layout_noalloc(idx, off, cfg.n_experts, cfg.expert_lo, cfg.n_local, layout, cap,
                                              out=out)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), k
        lay = dispatch_layout(idx_np, off_np, cfg.expert_lo, cfg.n_local, layout, cap)
        np.testing.assert_array_equal(i64(got["row_of"]), lay["row_of"])
        np.testing.assert_array_equal(i64(got["counts"]).reshape(cfg.n_local, -1), lay["counts"])


def test_noalloc_layout_rejects_work_beyond_its_scratch():
    # 1024 local experts x (1 + 2^20 / 64) tiles of counts: far past the fixed
    # scratch; refused on the host, nothing enqueued
    d = LayoutDesc(1 << 20, 2, 2048, 1, 0, 1024, COMPACT, 1 << 21)
    fake = ctypes.c_void_p(0x100000)
    st = moe.lib().moe_dispatch_layout_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None)
    assert st == 2  # MOE_ERR_UNSUPPORTED
