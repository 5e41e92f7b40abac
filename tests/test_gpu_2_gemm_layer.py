"""GPU parity: grouped SwiGLU GEMM, combine and the whole layer step.

Tolerances (relative L2 against the float64 oracle on exactly upcast inputs):
1e-5 with fp32 activations and weights, 2e-2 with bf16, 5e-2 with fp8 e4m3
weights. Full-size configs compare sampled rows/tokens the oracle computes one
by one, plus exact integer results and properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import combine_router_softmax_amd as moe
from combine_router_softmax_amd.layer import MoEShare
from oracle import (COMPACT, PADDED, combine, dispatch, dispatch_layout, group_rows, grouped_ffn, moe_layer,
                    route_topk, swiglu_ffn, worst_case_rows)
from synth import get_config, make_expert_weights, make_inputs, make_routing_inputs, tiny_config
from util import f64, flush, i64, rel_l2, unblock16, weights_f64

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8_e4m3": 5e-2}


class _Lazy:
    """Item g -> NumPy array (float64 values, or uint8 codes) of a stacked weight tensor."""

    def __init__(self, t, codes=False):
        self.t, self.codes = t, codes

    def __getitem__(self, g):
        return self.t[g].cpu().numpy() if self.codes else f64(self.t[g])

    def __len__(self):
        return self.t.shape[0]


def _oracle_weights(wd):
    fp8 = wd.get("s13") is not None
    return (_Lazy(wd["w13"], fp8), _Lazy(wd["w2"], fp8),
            None if not fp8 else wd["s13"].numpy(), None if not fp8 else wd["s2"].numpy())


def _dev_weights(wd):
    return {k: v.cuda() for k, v in wd.items() if k in ("w13", "w2", "s13", "s2") and v is not None}


# --------------------------------------------------------------------------- grouped GEMM
def _gemm_case(cfg, m_per_group, layout, seed=0, S=3, C=None, policy=moe.GEMM_AUTO):
    """Random rows grouped as given; returns GPU y and oracle y on occupied rows."""
    rng = np.random.default_rng(seed)
    G = len(m_per_group)
    H, I = cfg.hidden, cfg.inter
    wd = make_expert_weights(cfg, seed, experts=range(G))
    if layout == COMPACT:
        off = np.concatenate([[0], np.cumsum(m_per_group)]).astype(np.int32)
        R = int(off[-1]) + 5
        lay = {"layout": COMPACT, "expert_off": off, "rows": R}
        counts = None
    else:
        counts = np.zeros((G, S), dtype=np.int64)
        for g, m in enumerate(m_per_group):
            cuts = np.sort(rng.integers(0, m + 1, size=S - 1))
            counts[g] = np.diff(np.concatenate([[0], cuts, [m]]))
        if C is None:
            C = int(counts.max()) + 2
        R = G * S * C
        lay = {"layout": PADDED, "counts": counts, "n_src": S, "capacity": C, "rows": R,
               "expert_off": np.arange(G + 1) * S * C}
    act = torch.float32 if cfg.act == "f32" else torch.bfloat16
    a = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(act)
    y = torch.full((R, H), 3.0, dtype=act, device="cuda")
    kw = dict(layout=layout, y=y, policy=policy)
    if layout == COMPACT:
        kw["group_off"] = torch.from_numpy(lay["expert_off"].astype(np.int32)).cuda()
    else:
        kw["counts"] = torch.from_numpy(counts.astype(np.int32)).cuda()
        kw.update(n_src=S, capacity=C)
    dw = _dev_weights(wd)
    moe.moe_grouped_gemm(a.cuda(), dw["w13"], dw["w2"], s13=dw.get("s13"), s2=dw.get("s2"), **kw)
    ref = grouped_ffn(f64(a), lay, *_oracle_weights(wd))
    occ = np.zeros(R, dtype=bool)
    for g in range(G):
        occ[group_rows(lay, g)] = True
    got = f64(y)
    assert np.all(got[~occ] == 3.0), "unoccupied rows must not be written"
    return got[occ], ref[occ], (a, dw, kw)


@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_gemm_f32_tiny_shapes(layout):
    cfg = tiny_config()
    got, ref, _ = _gemm_case(cfg, [0, 1, 31, 33, 70, 5], layout)
    assert rel_l2(got, ref) <= TOL["f32"]


# bf16 stream-K tiles are 64 rows x two N blocks; hidden 384 gives an odd
# number (3) of down-projection N blocks, whose last tile holds one block.
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("ms", [[0, 1, 31, 32, 33, 127, 128, 129, 300], [5], [0, 0, 7]])
@pytest.mark.parametrize("hidden", [512, 384])
def test_gemm_bf16_ragged(layout, ms, hidden):
    cfg = get_config("dsv3_decode_ep8", hidden=hidden, inter=256)
    got, ref, _ = _gemm_case(cfg, ms, layout, seed=len(ms))
    if len(ref):
        assert rel_l2(got, ref) <= TOL["bf16"]


# The 256 x 256 wide-tile kernel (bf16 weights, hidden % 256 == 0): forced for
# every group, and in AUTO mode beside the stream-K kernel. Sizes span ragged
# wide tiles (1..8 active 32-row blocks), several row tiles per group, and
# groups below the AUTO row threshold.
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("ms", [[127, 128, 255, 256, 257, 0, 31, 700], [1000], [129, 2, 160, 224, 96, 520]])
def test_gemm_wide_tiles(layout, ms):
    cfg = get_config("dsv3_prefill_ep8", hidden=1024, inter=512)
    got, ref, (a, dw, kw) = _gemm_case(cfg, ms, layout, seed=sum(ms) % 97, policy=moe.GEMM_WIDE)
    # bf16 operands are exact, sums are fp32; h and y are each rounded once to
    # bf16 (relative error <= 2^-9 each), far inside the bf16 bound
    assert rel_l2(got, ref) <= 8e-3
    # packed weights give the same bits as row-major ones
    y_wide = kw["y"].clone()
    p13, p2 = moe.moe_pack_weights(dw["w13"], dw["w2"], 1024, 512)
    kw["y"].fill_(3.0)
    moe.moe_grouped_gemm(a.cuda(), p13, p2, w_format=moe.W_PACKED, **kw)
    assert torch.equal(kw["y"].view(torch.int16), y_wide.view(torch.int16))
    # the stream-K kernel computes the same products (fp32 sums in another order)
    kw["y"].fill_(3.0)
    kw["policy"] = moe.GEMM_STREAM_K
    moe.moe_grouped_gemm(a.cuda(), dw["w13"], dw["w2"], **kw)
    assert rel_l2(f64(kw["y"]), f64(y_wide)) <= 4e-3


# Routed rows in the 16-row blocked layout give the same bits as row-major
# rows, through both kernels (the layout only changes addresses).
@pytest.mark.parametrize("policy", [moe.GEMM_WIDE, moe.GEMM_STREAM_K])
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_gemm_blocked_rows_match_row_major(layout, policy):
    cfg = get_config("dsv3_prefill_ep8", hidden=1024, inter=512)
    ms = [129, 0, 300, 17, 260]
    got, ref, (a, dw, kw) = _gemm_case(cfg, ms, layout, seed=11, policy=policy)
    y_rm = kw["y"].clone()
    R = a.shape[0]
    R16 = moe.blocked_rows(R)
    ab = torch.zeros((R16, 1024), dtype=torch.bfloat16)
    ab[:R] = a
    blk = ab.reshape(R16 // 16, 16, 1024 // 32, 32).permute(0, 2, 1, 3).contiguous().reshape(R16, 1024)
    assert torch.equal(unblock16(blk, R), a)
    kw["y"].fill_(3.0)
    moe.moe_grouped_gemm(blk.cuda(), dw["w13"], dw["w2"], a_layout=moe.ACT_BLOCKED16, rows=R, **kw)
    assert torch.equal(kw["y"].view(torch.int16), y_rm.view(torch.int16))
    assert rel_l2(got, ref) <= 8e-3


# fp8 tiles are 96 rows x two N blocks: the sizes span 1..3 active row blocks,
# groups of two row tiles (129 = 96 + 33), and (hidden 384) an odd number of
# down-projection N blocks, whose last tile holds one block.
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("hidden,inter", [(512, 384), (384, 256)])
def test_gemm_fp8_ragged(layout, hidden, inter):
    cfg = get_config("kimi_k2_ep8", hidden=hidden, inter=inter)
    got, ref, _ = _gemm_case(cfg, [3, 0, 64, 129, 40, 96, 97], layout, seed=9)
    assert rel_l2(got, ref) <= TOL["fp8_e4m3"]
    # the fp8 path must be far better than the bound: it decodes codes exactly
    assert rel_l2(got, ref) <= 1e-2


# A policy that asks for the wide-tile kernel where it cannot run (fp8
# weights) leaves every group to the stream-K kernel: the same bits as AUTO.
# (Regression: the schedule once gave such groups to the absent wide kernel,
# and nothing was computed.)
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_gemm_fp8_policy_wide_runs_stream_k(layout):
    cfg = get_config("kimi_k2_ep8", hidden=512, inter=256)
    got, ref, (a, dw, kw) = _gemm_case(cfg, [300, 0, 129, 1000], layout, seed=21, policy=moe.GEMM_WIDE)
    assert rel_l2(got, ref) <= 1e-2
    y_wide = kw["y"].clone()
    kw["y"].fill_(3.0)
    moe.moe_grouped_gemm(a.cuda(), dw["w13"], dw["w2"], s13=dw["s13"], s2=dw["s2"], **dict(kw, policy=moe.GEMM_AUTO))
    assert torch.equal(kw["y"].view(torch.int16), y_wide.view(torch.int16))


# Blocked activation rows through the fp8 kernel give the same bits as row-major rows.
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_gemm_fp8_blocked_rows_match_row_major(layout):
    cfg = get_config("kimi_k2_ep8", hidden=1024, inter=256)
    got, ref, (a, dw, kw) = _gemm_case(cfg, [70, 0, 200, 5, 96], layout, seed=12)
    assert rel_l2(got, ref) <= 1e-2
    y_rm = kw["y"].clone()
    R = a.shape[0]
    R16 = moe.blocked_rows(R)
    ab = torch.zeros((R16, 1024), dtype=torch.bfloat16)
    ab[:R] = a
    blk = ab.reshape(R16 // 16, 16, 1024 // 32, 32).permute(0, 2, 1, 3).contiguous().reshape(R16, 1024)
    kw["y"].fill_(3.0)
    moe.moe_grouped_gemm(blk.cuda(), dw["w13"], dw["w2"], s13=dw["s13"], s2=dw["s2"], a_layout=moe.ACT_BLOCKED16,
                         rows=R, **kw)
    assert torch.equal(kw["y"].view(torch.int16), y_rm.view(torch.int16))


def test_gemm_stages_match_full_and_are_deterministic():
    cfg = get_config("dsv3_decode_ep8", hidden=512, inter=256)
    got, ref, (a, dw, kw) = _gemm_case(cfg, [40, 3, 200], COMPACT, seed=4)
    y_full = kw["y"].clone()
    desc = moe.gemm_desc(3, 512, 256, torch.bfloat16, torch.bfloat16, COMPACT, 1, 0, a.shape[0])
    ws = torch.zeros(moe.moe_grouped_gemm_workspace(desc), dtype=torch.uint8, device="cuda")
    kw2 = dict(kw)
    kw2["y"] = torch.zeros_like(y_full)
    moe.moe_grouped_gemm(a.cuda(), dw["w13"], dw["w2"], stage=moe.GG_UP, ws=ws, **{k: v for k, v in kw2.items()})
    moe.moe_grouped_gemm(a.cuda(), dw["w13"], dw["w2"], stage=moe.GG_DOWN, ws=ws, **{k: v for k, v in kw2.items()})
    occ = slice(0, 243)
    assert torch.equal(kw2["y"][occ], y_full[occ])


# --------------------------------------------------------------------------- whole layer (small)
def _share_from_inputs(d, layout, cap=None):
    cfg = d["cfg"]
    off = d["src_offsets"]
    N = int(off[-1])
    act = torch.float32 if cfg.act == "f32" else torch.bfloat16
    if cap is None and layout == PADDED:
        cap = int(np.diff(off).max())
    share = MoEShare(n_tokens=N, hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                     n_src=cfg.n_src, expert_lo=cfg.expert_lo, n_local=cfg.n_local, act_dtype=act, layout=layout,
                     capacity=cap, self_range=(0, int(off[1])))
    share.set_weights(d["routed"], d["shared"])
    return share


def _run(share, d, sentinel=-9.0):
    logits = torch.from_numpy(d["logits"]).cuda()
    off = torch.from_numpy(d["src_offsets"]).cuda()
    x = d["x"].cuda()
    out = torch.full_like(x, sentinel)
    share.step(logits, off, x, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("seed", range(16))
def test_layer_tiny(seed, layout, shared):
    cfg = tiny_config(shared=shared)
    d = make_inputs(cfg, seed)
    share = _share_from_inputs(d, layout)
    out = _run(share, d)
    w13, w2, _, _ = _oracle_weights(d["routed"])
    sh = None
    if shared:
        sw = d["shared"]
        sh = (_Lazy(sw["w13"]), _Lazy(sw["w2"]), None, None)
    off = d["src_offsets"]
    ref = moe_layer(f64(d["x"]), d["logits"], off, cfg.top_k, 0, cfg.n_local, w13, w2, shared=sh,
                    self_range=(0, int(off[1])), layout=layout, capacity=share.capacity,
                    out_init=np.full(tuple(d["x"].shape), -9.0))
    got = f64(out)
    np.testing.assert_array_equal(i64(share.topk_idx), ref["topk_idx"])
    np.testing.assert_array_equal(i64(share.lay["row_of"]), ref["layout"]["row_of"])
    touched = ref["out"] != -9.0
    assert np.all(got[~touched] == -9.0)
    assert rel_l2(got[touched], ref["out"][touched]) <= TOL["f32"]


# The up projection reads its rows straight from the tokens (a_rows = the
# layout's row_token) instead of a dispatched copy: the same arithmetic, so the
# same bits as through moe_dispatch, for the bf16 stream-K, fp8 and wide-tile
# kernels, both layouts, groups of several row tiles, an empty source and a
# shared expert in the launch.
@pytest.mark.parametrize("wname", ["bf16", "fp8", "bf16_wide"])
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_gemm_gather_matches_dispatched(wname, layout):
    wide = wname == "bf16_wide"
    cfg = get_config("kimi_k2_ep8" if wname == "fp8" else "dsv3_decode_ep8", hidden=512 if wide else 384, inter=256)
    pol = moe.GEMM_WIDE if wide else moe.GEMM_STREAM_K
    rng = np.random.default_rng(21)
    E, L, K = 32, 12, 4
    off = np.array([0, 60, 60, 200, 300], dtype=np.int32)  # source 1 is empty
    S, N, H = len(off) - 1, int(off[-1]), cfg.hidden
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(N)]).astype(np.int32)
    hot = np.arange(N) < 150  # expert 0 holds 150 rows: several row tiles
    idx[hot] = np.stack([np.concatenate([[0], 1 + rng.choice(E - 1, K - 1, replace=False)]) for _ in range(150)])
    cap = N * K if layout == COMPACT else int(np.diff(off).max())
    lay = moe.moe_dispatch_layout(torch.from_numpy(idx).cuda(), torch.from_numpy(off).cuda(), E, 0, L, layout, cap)
    R = lay["rows"]
    x = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    xe = moe.moe_dispatch(x, lay["row_of"], K, R)
    wd = make_expert_weights(cfg, 5, experts=range(L))
    dw = _dev_weights(wd)
    sw = _dev_weights(make_expert_weights(cfg, 6, shared=True))
    kw = dict(group_off=lay["expert_off"], counts=lay["counts"], s13=dw.get("s13"), s2=dw.get("s2"), layout=layout,
              n_src=S, capacity=cap, rows=R)
    outs = []
    for a, extra in ((xe, dict(policy=pol)), (x, dict(policy=pol, a_rows=lay["row_token"]))):
        y = torch.full((R, H), 3.0, dtype=torch.bfloat16, device="cuda")
        ys = torch.zeros((60, H), dtype=torch.bfloat16, device="cuda")
        shared = {"a": x[:60], "w13": sw["w13"], "w2": sw["w2"], "y": ys, "s13": sw.get("s13"), "s2": sw.get("s2")}
        moe.moe_grouped_gemm(a, dw["w13"], dw["w2"], y=y, shared=shared, **kw, **extra)
        outs.append((y, ys))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
    # the oracle's own layout and dispatch (the GPU layout is the same: it is exact)
    lo = dispatch_layout(idx, off, 0, L, layout, cap)
    np.testing.assert_array_equal(lay["row_of"].cpu().numpy().reshape(-1), np.asarray(lo["row_of"]).reshape(-1))
    rows = np.concatenate([group_rows(lo, g) for g in range(L)])
    assert len(rows) == int(np.sum(lo["counts"])) and int(np.sum(lo["counts"][0])) >= 150
    ref = grouped_ffn(dispatch(f64(x), lo["row_of"], K, lo["rows"]), lo, *_oracle_weights(wd))
    assert rel_l2(f64(outs[1][0])[rows], ref[rows]) <= (1e-2 if wname == "fp8" else TOL["bf16"])


def test_layer_identity_property_bf16():
    # combine(dispatch(x)) with identity experts: out = (sum of local weights) * x.
    cfg = get_config("dsv3_decode_ep8")
    d = make_routing_inputs(cfg, 1)
    from synth import make_x
    x = make_x(cfg, 1, d["src_offsets"]).cuda()
    logits = torch.from_numpy(d["logits"]).cuda()
    off = torch.from_numpy(d["src_offsets"]).cuda()
    N = x.shape[0]
    idx, w = moe.moe_route_topk(logits, 8)
    lay = moe.moe_dispatch_layout(idx, off, 256, 0, 32, COMPACT, N * 8)
    xe = moe.moe_dispatch(x, lay["row_of"], 8, lay["rows"])
    out = torch.zeros_like(x)
    moe.moe_combine(xe, lay["row_of"], w, out)
    ridx, rw = route_topk(d["logits"], 8)
    local = (ridx < 32)
    ref = (rw * local).sum(axis=1)[:, None] * f64(x)
    assert rel_l2(f64(out), ref) <= 4e-3  # one bf16 rounding of each output


# Many tokens take the combine's throughput shape (four pieces per thread, two
# kept rows per round trip): tokens keeping 0..8 local rows exercise every
# number of round trips, plus the shared rows of the self range; rows with
# nothing to add keep their previous contents.
def test_combine_many_tokens_all_kept_counts():
    rng = np.random.default_rng(31)
    N, K, H = 20000, 8, 264  # 33 pieces per row: a ragged last piece group
    R = N * K
    keep = rng.random((N, K)) < rng.random((N, 1))  # per-token keep rate: kept counts spread over 0..8
    row_of = np.where(keep, rng.permutation(R).reshape(N, K), -1).astype(np.int32)
    w = rng.random((N, K)).astype(np.float32)
    ye = torch.randn(R, H).to(torch.bfloat16)
    lo, hi = 1000, 3000
    sy = torch.randn(hi - lo, H).to(torch.bfloat16)
    out = torch.full((N, H), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(ye.cuda(), torch.from_numpy(row_of).cuda(), torch.from_numpy(w).cuda(), out, sy.cuda(), lo, hi)
    sample = np.sort(rng.choice(N, 3000, replace=False))
    ref = combine(f64(ye), row_of.reshape(-1), w, K, np.full((N, H), 7.0), f64(sy), lo, hi, tokens=sample)
    got = f64(out)
    assert rel_l2(got[sample], ref[sample]) <= 4e-3  # one bf16 rounding of each output
    untouched = np.array([t for t in sample if not keep[t].any() and not lo <= t < hi])
    assert len(untouched) > 0 and (got[untouched] == 7.0).all()
    assert {int(c) for c in keep[sample].sum(axis=1)} >= set(range(K + 1))


# Rows for at most half the (token, entry) pairs (few local experts, as at
# the EP128 decode share): the combine takes strided batches of tokens and
# combines only the touched ones. Every touched token against the oracle,
# untouched rows keep their contents; rows of 8704 bf16 values take two
# chunks; K = 2, 8, 16; fewer and more than 1024 tokens (the two piece shapes).
@pytest.mark.parametrize("N,K,H", [(8192, 8, 7168), (5000, 16, 8704), (3000, 2, 264), (700, 8, 264)])
def test_combine_few_rows_many_tokens(N, K, H):
    rng = np.random.default_rng(N + K)
    R = N * K // 4
    keep = rng.random((N, K)) < 0.03
    row_of = np.full((N, K), -1, dtype=np.int32)
    row_of[keep] = rng.permutation(R)[: int(keep.sum())]
    w = rng.random((N, K)).astype(np.float32)
    ye = torch.randn(R, H).to(torch.bfloat16)
    lo, hi = 40, 200
    sy = torch.randn(hi - lo, H).to(torch.bfloat16)
    out = torch.full((N, H), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(ye.cuda(), torch.from_numpy(row_of).cuda(), torch.from_numpy(w).cuda(), out, sy.cuda(), lo, hi)
    touched = keep.any(axis=1) | ((np.arange(N) >= lo) & (np.arange(N) < hi))
    tok = np.nonzero(touched)[0]
    ref = combine(f64(ye), row_of.reshape(-1), w, K, np.full((N, H), 7.0), f64(sy), lo, hi, tokens=tok)
    got = f64(out)
    assert rel_l2(got[tok], ref[tok]) <= 4e-3  # one bf16 rounding of each output
    assert (got[~touched] == 7.0).all()
    assert 0 < len(tok) < N // 2


# No routed rows at all (no token picked a local expert): only the self
# range's shared rows are written, whichever form the combine takes.
@pytest.mark.parametrize("N", [700, 4000])
def test_combine_no_rows_shared_only(N):
    K, H = 8, 264
    row_of = np.full((N, K), -1, dtype=np.int32)
    w = np.random.default_rng(3).random((N, K)).astype(np.float32)
    lo, hi = 10, 50
    sy = torch.randn(hi - lo, H).to(torch.bfloat16)
    out = torch.full((N, H), 7.0, dtype=torch.bfloat16, device="cuda")
    ye = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(ye, torch.from_numpy(row_of).cuda(), torch.from_numpy(w).cuda(), out, sy.cuda(), lo, hi)
    got = out.cpu()
    assert torch.equal(got[lo:hi].view(torch.int16), sy.view(torch.int16))
    assert (got[:lo] == 7.0).all() and (got[hi:] == 7.0).all()


# --------------------------------------------------------------------------- whole layer (full size)
FULL = ["dsv3_decode_ep8", "dsv3_decode_ep128", "kimi_k2_ep8", "dsv3_prefill_ep8"]


@pytest.fixture(scope="module", params=FULL)
def full_case(request):
    cfg = get_config(request.param)
    flush(f"generate {cfg.name}")
    d = make_inputs(cfg, 0)
    yield cfg, d
    torch.cuda.empty_cache()


def _shared_oracle_weights(sw):
    fp8 = sw.get("s13") is not None
    return (_Lazy(sw["w13"], fp8), _Lazy(sw["w2"], fp8), None if not fp8 else sw["s13"].numpy(),
            None if not fp8 else sw["s2"].numpy())


def _assert_rows_close(got, ref, tol, what, row_tol=None):
    """Relative L2 over all compared rows (<= tol), and over each row on its
    own (<= row_tol, default tol): a single wrong row must fail even among
    thousands of right ones."""
    row_tol = tol if row_tol is None else row_tol
    err = rel_l2(got, ref)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    worst = int(np.argmax(num / den))
    flush(f"  {what}: {len(ref)} rows, rel-L2 {err:.3e}, worst row {worst} rel {num[worst] / den[worst]:.3e}")
    assert err <= tol, f"{what}: rel-L2 {err:.3e} > {tol}"
    assert num[worst] / den[worst] <= row_tol, f"{what}: row {worst} rel {num[worst] / den[worst]:.3e} > {row_tol}"


def _split_experts(m, ntn):
    """Local experts that hold wide tiles split along K: the wide kernel takes
    whole tiles in rounds of 256 and splits the last (tiles % 256), which are
    the last tiles of the schedule (the shared expert first, then the routed
    experts in index order, 256-row tiles, ntn weight tiles per row tile)."""
    tiles = [(int(mm) + 255) // 256 * ntn for mm in m]
    total = sum(tiles) + ntn * 16  # + the shared expert's 4096 rows
    rem = total % 256
    out, acc = [], 0
    for g in reversed(range(len(m))):
        if acc >= rem:
            break
        if tiles[g]:
            out.append(g)
        acc += tiles[g]
    return out


def test_layer_full_size(full_case):
    """Whole layer at the full configuration, compact and padded layouts.

    Exact integer results; the two layouts and two runs give the same bits.
    Decode-sized shares (every touched token affordable on the CPU): every
    touched output row against the oracle's whole layer. The prefill share
    (32,768 tokens): every row of the GPU's own 4096 tokens end to end, and
    every expert-output row of the hottest local expert, of the experts whose
    wide tiles are split along K, and of the shared expert."""
    cfg, d = full_case
    flush(f"layer {cfg.name}")
    off = d["src_offsets"]
    N, B0 = int(off[-1]), int(off[1])
    tol = TOL[cfg.weight]
    outs = {}
    keep = {}
    for layout in (COMPACT, PADDED):
        share = _share_from_inputs(d, layout)
        out = _run(share, d)
        if layout == COMPACT:
            ridx, rw = route_topk(d["logits"], cfg.top_k)
            np.testing.assert_array_equal(i64(share.topk_idx), ridx)
            assert rel_l2(f64(share.topk_w), rw) <= 1e-5
            lay = dispatch_layout(ridx, off, cfg.expert_lo, cfg.n_local, COMPACT, share.capacity)
            np.testing.assert_array_equal(i64(share.lay["row_of"]), lay["row_of"])
            np.testing.assert_array_equal(i64(share.lay["counts"]).reshape(cfg.n_local, -1), lay["counts"])
            np.testing.assert_array_equal(i64(share.lay["expert_off"]), lay["expert_off"])
            assert int(share.lay["status"].item()) == 0
            keep["lay"] = lay
            keep["ye"] = share.ye[: int(lay["expert_off"][-1])].cpu()
            keep["ys"] = share.ys[:B0].cpu()
        outs[layout] = out
        # determinism: a second step gives the same bits
        out2 = _run(share, d)
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
        del share
        torch.cuda.empty_cache()
    # the two layouts compute every row the same way
    assert torch.equal(outs[COMPACT].view(torch.int16), outs[PADDED].view(torch.int16))

    w13, w2, s13, s2 = _oracle_weights(d["routed"])
    sh = _shared_oracle_weights(d["shared"])
    got_all = f64(outs[COMPACT])
    if N * cfg.n_local <= 4096 * 48:
        # every token, end to end
        flush(f"  oracle layer over {N} tokens")
        ref = moe_layer(f64(d["x"]), d["logits"], off, cfg.top_k, cfg.expert_lo, cfg.n_local, w13, w2, s13, s2,
                        shared=sh, self_range=(0, B0), out_init=np.full(tuple(d["x"].shape), -9.0))
        touched = ref["out"][:, 0] != -9.0
        assert np.all(got_all[~touched] == -9.0)
        assert touched[:B0].all()
        _assert_rows_close(got_all[touched], ref["out"][touched], tol, f"{cfg.name} touched rows")
        return

    # prefill share: the GPU's own tokens end to end ...
    flush(f"  oracle layer over the {B0} own tokens")
    ref = moe_layer(f64(d["x"][:B0]), d["logits"][:B0], [0, B0], cfg.top_k, cfg.expert_lo, cfg.n_local, w13, w2,
                    s13, s2, shared=sh, self_range=(0, B0), out_init=np.full((B0, cfg.hidden), -9.0))
    _assert_rows_close(got_all[:B0], ref["out"], tol, f"{cfg.name} own tokens")
    # ... and whole experts' output rows of the routed GEMM
    lay = keep["lay"]
    m = lay["counts"].sum(axis=1)
    ye = f64(keep["ye"])
    experts = {int(np.argmax(m))} | set(_split_experts(m, 16)) | set(_split_experts(m, 28))
    for g in sorted(experts):
        rows = group_rows(lay, g)
        a13, a2 = weights_f64(d["routed"], g)
        flush(f"  oracle expert {g}: {len(rows)} rows")
        ref_g = swiglu_ffn(f64(d["x"])[lay["row_token"][rows]], a13, a2)
        _assert_rows_close(ye[rows], ref_g, tol, f"{cfg.name} expert {g}")
    a13, a2 = weights_f64(d["shared"], 0)
    _assert_rows_close(f64(keep["ys"]), swiglu_ffn(f64(d["x"][:B0]), a13, a2), tol, f"{cfg.name} shared expert")


# A mid-sized whole layer through each MFMA kernel (bf16 stream-K, bf16 wide
# tiles forced, fp8 stream-K), every touched output row against the oracle.
# Hidden 1024, 8 ranks x 96 tokens, 64 experts (8 local), top-8, intermediate
# 512: several tiles per expert, stream-K ranges cut inside tiles (fixups),
# gathered rows, a shared expert in the launch.
@pytest.mark.parametrize("kernel", ["bf16_stream_k", "bf16_wide", "fp8"])
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_layer_mid_size_every_row(kernel, layout):
    name = "kimi_k2_ep8" if kernel == "fp8" else "dsv3_decode_ep8"
    cfg = get_config(name, hidden=1024, inter=512, n_experts=64, n_local=8, tokens_per_src=96)
    d = make_inputs(cfg, 7)
    off = d["src_offsets"]
    N, B0 = int(off[-1]), int(off[1])
    cap = None if layout == COMPACT else int(np.diff(off).max())
    share = MoEShare(n_tokens=N, hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                     n_src=cfg.n_src, expert_lo=0, n_local=cfg.n_local, act_dtype=torch.bfloat16, layout=layout,
                     capacity=cap, self_range=(0, B0),
                     policy=moe.GEMM_WIDE if kernel == "bf16_wide" else moe.GEMM_STREAM_K)
    share.set_weights(d["routed"], d["shared"])
    out = _run(share, d)
    w13, w2, s13, s2 = _oracle_weights(d["routed"])
    ref = moe_layer(f64(d["x"]), d["logits"], off, cfg.top_k, 0, cfg.n_local, w13, w2, s13, s2,
                    shared=_shared_oracle_weights(d["shared"]), self_range=(0, B0), layout=layout,
                    capacity=share.capacity, out_init=np.full(tuple(d["x"].shape), -9.0))
    np.testing.assert_array_equal(i64(share.lay["row_of"]), ref["layout"]["row_of"])
    got = f64(out)
    touched = ref["out"][:, 0] != -9.0
    assert np.all(got[~touched] == -9.0)
    assert touched.sum() > B0
    # bf16 operands are exact, sums fp32; h and y (and fp8 weights, once) are
    # rounded to bf16: far inside the relative-L2 bounds of TOL, which hold per row
    _assert_rows_close(got[touched], ref["out"][touched], 1e-2, f"mid {kernel} layout={layout}",
                       row_tol=TOL[cfg.weight])


@pytest.mark.parametrize("name", ["dsv3_decode_ep8", "kimi_k2_ep8"])
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_fused_shared_expert_matches_separate_calls(name, layout):
    # the shared expert inside the routed launches matches calls of its own, on
    # the same or on a second stream (up to
    # the fp32 order of stream-K partial sums, which depends on the launch's tile
    # count) and the oracle
    cfg = get_config(name, hidden=1024, inter=512, n_experts=64, n_local=8, tokens_per_src=96)
    d = make_inputs(cfg, 2)
    share = _share_from_inputs(d, layout)
    logits = torch.from_numpy(d["logits"]).cuda()
    off = torch.from_numpy(d["src_offsets"]).cuda()
    x = d["x"].cuda()
    outs = {}
    for mode in ("fused", "serial", "stream"):  # in the routed launches, own calls, own calls on a second stream
        o = torch.full_like(x, -9.0)
        share.step(logits, off, x, o, shared_mode=mode)
        torch.cuda.synchronize()
        outs[mode] = (o, share.ys.clone())
    o1, ys1 = outs["fused"]
    for mode in ("serial", "stream"):
        assert rel_l2(f64(ys1), f64(outs[mode][1])) <= 2e-3
        assert rel_l2(f64(o1), f64(outs[mode][0])) <= 2e-3
    # the shared expert's own calls give the same bits on either stream
    assert torch.equal(outs["serial"][0].view(torch.int16), outs["stream"][0].view(torch.int16))
    sw = d["shared"]
    fp8 = sw.get("s13") is not None
    B0 = int(d["src_offsets"][1])
    ref = swiglu_ffn(f64(d["x"][:B0]), *(weights_f64(sw, 0)))
    assert rel_l2(f64(ys1[:B0]), ref) <= TOL[cfg.weight]


def test_shared_expert_only_call():
    cfg = get_config("dsv3_decode_ep8", hidden=512, inter=256)
    sw = make_expert_weights(cfg, 3, shared=True)
    a = torch.randn(77, 512, dtype=torch.bfloat16, device="cuda")
    y = torch.full((77, 512), 5.0, dtype=torch.bfloat16, device="cuda")
    dummy = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    w13, w2 = sw["w13"].cuda(), sw["w2"].cuda()
    moe.moe_grouped_gemm(dummy, w13[:0], w2[:0], group_off=torch.zeros(1, dtype=torch.int32, device="cuda"),
                         shared={"a": a, "w13": w13, "w2": w2, "y": y})
    ref = swiglu_ffn(f64(a), *(weights_f64(sw, 0)))
    assert rel_l2(f64(y), ref) <= TOL["bf16"]


@pytest.mark.parametrize("wname", ["bf16", "fp8"])
@pytest.mark.parametrize("hidden", [1024, 640])  # 640: an odd number of down-projection N blocks
def test_pack_weights_is_a_permutation_and_gemm_matches(wname, hidden):
    cfg = get_config("dsv3_decode_ep8" if wname == "bf16" else "kimi_k2_ep8", hidden=hidden, inter=512)
    G = 5
    wd = make_expert_weights(cfg, 1, experts=range(G))
    w13, w2 = wd["w13"].cuda(), wd["w2"].cuda()
    p13, p2 = moe.moe_pack_weights(w13, w2, cfg.hidden, cfg.inter)
    torch.cuda.synchronize()
    for a, b in ((w13, p13), (w2, p2)):
        ab = a.view(torch.uint8).reshape(-1).cpu().numpy()
        bb = b.view(torch.uint8).reshape(-1).cpu().numpy()
        assert not np.array_equal(ab, bb)
        np.testing.assert_array_equal(np.sort(ab), np.sort(bb))
    # same arithmetic from either layout: bit-identical outputs, with a shared expert in the launch
    rng = np.random.default_rng(3)
    ms = [40, 0, 129, 7, 64]
    off = torch.tensor(np.concatenate([[0], np.cumsum(ms)]), dtype=torch.int32, device="cuda")
    R = int(off[-1])
    x = torch.from_numpy(rng.standard_normal((R, cfg.hidden)).astype(np.float32)).to(torch.bfloat16).cuda()
    xs = torch.from_numpy(rng.standard_normal((50, cfg.hidden)).astype(np.float32)).to(torch.bfloat16).cuda()
    sw = make_expert_weights(cfg, 2, shared=True)
    s13, s2 = sw["w13"].cuda(), sw["w2"].cuda()
    ps13, ps2 = moe.moe_pack_weights(s13, s2, cfg.hidden, cfg.inter)
    outs = []
    for fmt, (a13, a2, b13, b2) in ((moe.W_ROWMAJOR, (w13, w2, s13, s2)), (moe.W_PACKED, (p13, p2, ps13, ps2))):
        y = torch.zeros((R, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        ys = torch.zeros((50, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        sc = {} if wname == "bf16" else {"s13": wd["s13"].cuda(), "s2": wd["s2"].cuda()}
        ssc = {} if wname == "bf16" else {"s13": sw["s13"].cuda(), "s2": sw["s2"].cuda()}
        moe.moe_grouped_gemm(x, a13, a2, group_off=off, y=y, w_format=fmt,
                             shared={"a": xs, "w13": b13, "w2": b2, "y": ys, **ssc}, **sc)
        outs.append((y, ys))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
    ref = grouped_ffn(f64(x), {"layout": COMPACT, "expert_off": off.cpu().numpy(), "rows": R}, *_oracle_weights(wd))
    assert rel_l2(f64(outs[1][0]), ref) <= TOL[cfg.weight]
