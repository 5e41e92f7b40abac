"""The down projection's weighted scatter (moe_scatter_t) and moe_combine_multi.

A token with exactly one row on this GPU and no shared-expert row has that
row as its whole combine (lehuy.net, "Decoding high-performance EP kernels",
section Combine); the GEMM epilogue writes it straight into the output. The
pair (scatter + moe_combine_multi) must give the same bits as the plain path
(y rows + moe_combine), through every MFMA kernel family, both layouts and
every place of the shared expert, and the GEMM must write exactly the
single-row tokens and leave their y rows alone.
"""
import numpy as np
import pytest
import torch

import combine_router_softmax_amd as moe
from combine_router_softmax_amd import COMPACT, PADDED
from combine_router_softmax_amd.layer import MoEShare
from synth import get_config, make_inputs

pytestmark = pytest.mark.gpu

SENT = -7.0  # sentinel: a value no output of these layers takes


def _shares(cfg, d, layout, policy=None, w8a8=False):
    off = d["src_offsets"]
    N, B0 = int(off[-1]), int(off[1])
    cap = None if layout == COMPACT else int(np.diff(off).max())
    kw = dict(n_tokens=N, hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
              n_src=cfg.n_src, expert_lo=cfg.expert_lo, n_local=cfg.n_local, act_dtype=torch.bfloat16,
              layout=layout, capacity=cap, self_range=(0, B0), policy=policy, w8a8=w8a8)
    on = MoEShare(scatter=True, **kw)
    on.set_weights(d["routed"], d["shared"])
    off_ = MoEShare(scatter=False, **kw)
    off_.share_weights_from(on)
    return on, off_


def _step(share, d, mode=None):
    logits = torch.from_numpy(d["logits"]).cuda()
    offs = torch.from_numpy(d["src_offsets"]).cuda()
    x = d["x"].cuda()
    out = torch.full_like(x, SENT)
    share.step(logits, offs, x, out, shared_mode=mode)
    torch.cuda.synchronize()
    return out


def _single_row_tokens(share):
    """Routed rows whose token has exactly one kept entry and no shared row,
    and those tokens (host arrays)."""
    K = share.K
    row_of = share.lay["row_of"].cpu().numpy().reshape(-1, K)
    n_rows = max(share.R, 1)
    kept = (row_of >= 0) & (row_of < n_rows)
    lo, hi = share._self_range()
    t = np.arange(row_of.shape[0])
    single = (kept.sum(axis=1) == 1) & ~((t >= lo) & (t < hi))
    rows = row_of[single][kept[single]]
    return rows, np.nonzero(single)[0]


KERNELS = {  # workload, GEMM policy, W8A8
    "bf16_stream_k": ("dsv3_decode_ep8", moe.GEMM_STREAM_K, False),
    "bf16_wide": ("dsv3_decode_ep8", moe.GEMM_WIDE, False),
    "fp8_w8a16": ("kimi_k2_ep8", None, False),
    "w8a8": ("kimi_k2_ep8", None, True),
}


# Hidden 1024, 8 ranks x 96 tokens, 64 experts (8 local), top-8: tiles split by
# stream-K and K-split boundaries (so the fix-up kernels' epilogues scatter too),
# gathered rows, the shared expert in the launch or on a second stream.
@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("mode", ["fused", "stream"])
def test_scatter_gives_the_combine_bits(kernel, layout, mode):
    name, policy, w8a8 = KERNELS[kernel]
    over = dict(hidden=1024, inter=512, n_experts=64, n_local=8, tokens_per_src=96)
    if w8a8:
        over["weight"] = "fp8_e4m3"
    cfg = get_config(name, **over)
    d = make_inputs(cfg, 11)
    on, off = _shares(cfg, d, layout, policy, w8a8)
    got = _step(on, d, mode)
    ref = _step(off, d, mode)
    rows, toks = _single_row_tokens(on)
    assert len(toks) > 20, "the case must hold single-row tokens"
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_scatter_writes_single_row_tokens_only():
    cfg = get_config("dsv3_decode_ep8", hidden=1024, inter=512, n_experts=64, n_local=8, tokens_per_src=96)
    d = make_inputs(cfg, 5)
    on, off = _shares(cfg, d, COMPACT, moe.GEMM_STREAM_K)
    ref = _step(off, d, "fused")
    ye_ref = off.ye[: off.R].clone()
    # every y row starts as a sentinel; after the scatter run the single-row
    # tokens' y rows must still hold it, every other routed row must not
    on.ye.fill_(SENT)
    logits = torch.from_numpy(d["logits"]).cuda()
    offs = torch.from_numpy(d["src_offsets"]).cuda()
    x = d["x"].cuda()
    out = torch.full_like(x, SENT)
    on.route(logits)
    on.layout_step(offs)
    on.gemm(moe.GG_UP, x, src=x)  # the shared expert in the same launches, as in ref
    on.gemm(moe.GG_DOWN, x, src=x, out=out)
    torch.cuda.synchronize()
    rows, toks = _single_row_tokens(on)
    assert len(toks) > 20
    ye = on.ye[: on.R].float().cpu().numpy()
    assert np.all(ye[rows] == SENT), "the scatter must not write the y rows of single-row tokens"
    row_of = on.lay["row_of"].cpu().numpy().reshape(-1, on.K)
    used = row_of[(row_of >= 0) & (row_of < on.R)]
    others = np.setdiff1d(used, rows)
    assert np.all(ye[others][:, 0] != SENT)
    # the GEMM wrote exactly the single-row tokens' output rows, with the
    # combine's value for them: round(w * y), y the plain path's bf16 row
    o = out.float().cpu().numpy()
    written = np.nonzero(o[:, 0] != SENT)[0]
    np.testing.assert_array_equal(written, toks)
    w = on.topk_w.cpu().numpy().reshape(-1, on.K)
    for t in toks[:: max(1, len(toks) // 16)]:
        k = int(np.nonzero((row_of[t] >= 0) & (row_of[t] < on.R))[0][0])
        yr = ye_ref[int(row_of[t, k])].float()
        exp = (torch.tensor(w[t, k], dtype=torch.float32) * yr.cpu()).to(torch.bfloat16)
        assert torch.equal(out[t].cpu().view(torch.int16), exp.view(torch.int16))
    # and the remaining tokens through moe_combine_multi give the plain path's bits
    on.combine(out, multi=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


# Full-size shares, in the launch configuration bench.py times: the decode
# share with two experts per GPU (the case with the most single-row tokens)
# and the fp8 share.
@pytest.mark.parametrize("name", ["dsv3_decode_ep128", "kimi_k2_ep8"])
def test_scatter_full_size_bits(name):
    cfg = get_config(name)
    d = make_inputs(cfg, 0)
    on, off = _shares(cfg, d, COMPACT)
    got = _step(on, d)
    ref = _step(off, d)
    _, toks = _single_row_tokens(on)
    assert len(toks) > 100
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
