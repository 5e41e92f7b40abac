"""GPU parity: routing, dispatch layout and dispatch against the CPU oracle.

Integer results (expert indices, counts, offsets, slots, dispatched rows) must
match bit for bit; routing weights within relative L2 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

import combine_router_softmax_amd as moe
from oracle import COMPACT, PADDED, dispatch, dispatch_layout, route_topk, worst_case_rows
from synth import get_config, make_routing_inputs, make_x, tiny_config
from util import f64, flush, i64, rel_l2, unblock16

pytestmark = pytest.mark.gpu

BIG = ["dsv3_decode_ep8", "dsv3_decode_ep128", "dsv3_prefill_ep8", "kimi_k2_ep8"]


def _route_check(logits_np, K, renorm=True):
    logits = torch.from_numpy(np.ascontiguousarray(logits_np)).cuda()
    idx, w = moe.moe_route_topk(logits, K, renorm)
    ridx, rw = route_topk(logits_np, K, renorm)
    np.testing.assert_array_equal(i64(idx), ridx)
    if len(rw):
        assert rel_l2(f64(w), rw) <= 1e-5
        assert np.max(np.abs(f64(w) - rw)) <= 1e-6
    return ridx


@pytest.mark.parametrize("seed", range(32))
def test_route_tiny(seed):
    cfg = tiny_config()
    _route_check(make_routing_inputs(cfg, seed)["logits"], cfg.top_k)


@pytest.mark.parametrize("name", BIG)
def test_route_full_size(name):
    cfg = get_config(name)
    flush(f"route {name}")
    _route_check(make_routing_inputs(cfg, 0)["logits"], cfg.top_k)


@pytest.mark.parametrize("E,K", [(1, 1), (16, 16), (100, 7), (64, 16), (257, 3), (1000, 8), (1024, 16)])
def test_route_shapes_and_ties(E, K):
    rng = np.random.default_rng(E * 31 + K)
    z = rng.standard_normal((333, E)).astype(np.float32)
    z[::2] = np.round(z[::2] * 2) / 2           # exact ties on half the tokens
    z[5] = 0.0                                    # a row of equal logits
    z[6, : E // 2] = -0.0                         # signed zeros compare equal
    _route_check(z, K)
    _route_check(z, K, renorm=False)


def test_route_nan_logits_give_in_range_distinct_indices():
    # NaN logits are outside the contract (no order), but the indices must stay
    # in range and distinct: 0xFFFFFFFF (memory filled with 0xFF) and other NaNs,
    # whole rows of them and mixed with finite logits
    E, K = 96, 8
    z = np.random.default_rng(3).standard_normal((6, E)).astype(np.float32)
    bits = z.view(np.uint32)
    bits[0] = 0xFFFFFFFF
    bits[1] = 0x7FC00000
    bits[2, ::3] = 0xFFFFFFFF
    bits[3, :90] = 0xFFFFFFFE
    bits[4] = 0xFFFFFFFF
    bits[4, 50] = np.float32(1.0).view(np.uint32)
    idx, _ = moe.moe_route_topk(torch.from_numpy(z).cuda(), K)
    idx = i64(idx)
    assert ((idx >= 0) & (idx < E)).all()
    assert all(len(set(r)) == K for r in idx)
    # rows with finite logits among NaNs still pick a finite maximum first
    assert idx[4, 0] == 50
    # a finite row is unaffected
    np.testing.assert_array_equal(idx[5], route_topk(z[5:6], K)[0][0])


def test_route_large_magnitude_and_empty():
    z = np.array([[1e30, -1e30, 3.0e38, -3.0e38, 1.0, 88.0, -88.0, 0.0]], dtype=np.float32)
    _route_check(np.repeat(z, 70, 0), 4)
    idx, w = moe.moe_route_topk(torch.zeros((0, 8), device="cuda"), 2)
    assert idx.shape == (0, 2)


# --------------------------------------------------------------------------- layout
def _layout_check(idx_np, off_np, E, lo, L, layout, cap):
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    off = torch.from_numpy(np.asarray(off_np, dtype=np.int32)).cuda()
    got = moe.moe_dispatch_layout(idx, off, E, lo, L, layout, cap)
    ref = dispatch_layout(idx_np, off_np, lo, L, layout, cap)
    np.testing.assert_array_equal(i64(got["counts"]).reshape(L, -1), ref["counts"])
    np.testing.assert_array_equal(i64(got["expert_off"]), ref["expert_off"])
    np.testing.assert_array_equal(i64(got["row_of"]), ref["row_of"])
    R = ref["rows"]
    assert got["rows"] == R
    np.testing.assert_array_equal(i64(got["row_token"])[:R], ref["row_token"])
    assert int(got["status"].item()) == ref["status"]
    return got, ref


@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("seed", range(32))
def test_layout_tiny(seed, layout):
    cfg = tiny_config()
    d = make_routing_inputs(cfg, seed)
    idx, _ = route_topk(d["logits"], cfg.top_k)
    N = len(idx)
    off = d["src_offsets"]
    cap = worst_case_rows(N, cfg.top_k, cfg.n_local) if layout == COMPACT else int(np.diff(off).max())
    for lo in (0, 6, 14):
        _layout_check(idx, off, cfg.n_experts, lo, cfg.n_local, layout, cap)


@pytest.mark.parametrize("name", BIG)
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_layout_full_size(name, layout):
    cfg = get_config(name)
    flush(f"layout {name} {layout}")
    d = make_routing_inputs(cfg, 0)
    idx, _ = route_topk(d["logits"], cfg.top_k)
    N = len(idx)
    off = d["src_offsets"]
    cap = worst_case_rows(N, cfg.top_k, cfg.n_local) if layout == COMPACT else int(np.diff(off).max())
    _layout_check(idx, off, cfg.n_experts, cfg.expert_lo, cfg.n_local, layout, cap)


def test_layout_zipf_identity_hot_experts():
    cfg = get_config("dsv3_prefill_ep8", zipf="identity", tokens_per_src=1024)
    d = make_routing_inputs(cfg, 0)
    idx, _ = route_topk(d["logits"], cfg.top_k)
    for layout, cap in [(COMPACT, worst_case_rows(len(idx), 8, 32)), (PADDED, 1024)]:
        _layout_check(idx, d["src_offsets"], 256, 0, 32, layout, cap)


def test_layout_overflow_and_edges():
    cfg = tiny_config()
    d = make_routing_inputs(cfg, 3)
    idx, _ = route_topk(d["logits"], cfg.top_k)
    off = d["src_offsets"]
    got, ref = _layout_check(idx, off, 16, 0, 2, PADDED, 1)
    assert ref["status"] == 1
    full = dispatch_layout(idx, off, 0, 2, COMPACT, 10 ** 4)
    M = int(full["expert_off"][-1])
    _layout_check(idx, off, 16, 0, 2, COMPACT, max(M - 5, 0))
    _layout_check(idx, off, 16, 0, 2, COMPACT, 0)
    _layout_check(idx, off, 16, 0, 2, PADDED, 0)
    # empty sources, a source larger than one 256-token tile, an empty batch
    rng = np.random.default_rng(0)
    N = 700
    z = rng.standard_normal((N, 16)).astype(np.float32)
    idx2, _ = route_topk(z, 2)
    off2 = np.array([0, 0, 300, 300, 301, 700, 700])
    for layout, cap in [(COMPACT, 1400), (PADDED, 400), (PADDED, 90)]:
        _layout_check(idx2, off2, 16, 2, 5, layout, cap)
    _layout_check(np.zeros((0, 2), np.int32), np.zeros(5, np.int64), 16, 0, 2, COMPACT, 0)
    _layout_check(np.zeros((0, 2), np.int32), np.zeros(5, np.int64), 16, 0, 2, PADDED, 3)


def test_layout_arbitrary_indices():
    # indices outside [0, E), negative, duplicated inside a token: out-of-range ones
    # are not local; duplicates are ranked in (token, k) order on both sides
    rng = np.random.default_rng(1)
    N, K = 1000, 4
    idx = rng.integers(-3, 12, size=(N, K)).astype(np.int32)
    idx[::7, 1] = idx[::7, 0]
    off = np.array([0, 250, 600, 1000])
    for layout, cap in [(COMPACT, N * K), (PADDED, 1000), (PADDED, 40)]:
        _layout_check(idx, off, 12, 3, 6, layout, cap)


@pytest.mark.parametrize("L", [1, 3, 64, 100, 256, 1024])
def test_layout_local_expert_counts(L):
    # one local expert (no index bits), non-powers of two, every expert local
    rng = np.random.default_rng(L)
    E = max(L + 7, 16)
    N, K = 900, 6
    idx = rng.integers(0, E, size=(N, K)).astype(np.int32)
    off = np.array([0, 100, 356, 357, 900])
    lo = E - L - 3
    for layout, cap in [(COMPACT, N * K), (PADDED, 300)]:
        _layout_check(idx, off, E, lo, L, layout, cap)


# --------------------------------------------------------------------------- dispatch
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("seed", range(8))
def test_dispatch_tiny_bit_exact(seed, layout):
    cfg = tiny_config()
    d = make_routing_inputs(cfg, seed)
    x = make_x(cfg, seed, d["src_offsets"])
    idx, _ = route_topk(d["logits"], cfg.top_k)
    N = len(idx)
    cap = worst_case_rows(N, 2, 2) if layout == COMPACT else int(np.diff(d["src_offsets"]).max())
    ref = dispatch_layout(idx, d["src_offsets"], 0, 2, layout, cap)
    xe_ref = dispatch(f64(x), ref["row_of"], 2, ref["rows"])
    row_of = torch.from_numpy(ref["row_of"].astype(np.int32)).cuda()
    sentinel = torch.full((ref["rows"], cfg.hidden), 7.5, device="cuda")
    xe = moe.moe_dispatch(x.cuda(), row_of, 2, ref["rows"], sentinel)
    occ = ref["row_token"] >= 0
    np.testing.assert_array_equal(f64(xe)[occ], xe_ref[occ])
    assert torch.all(xe[torch.from_numpy(~occ).cuda()] == 7.5)


@pytest.mark.parametrize("name", BIG)
def test_dispatch_full_size(name):
    cfg = get_config(name)
    flush(f"dispatch {name}")
    d = make_routing_inputs(cfg, 0)
    idx, _ = route_topk(d["logits"], cfg.top_k)
    N = len(idx)
    ref = dispatch_layout(idx, d["src_offsets"], 0, cfg.n_local, COMPACT, worst_case_rows(N, 8, cfg.n_local))
    x = make_x(cfg, 0, d["src_offsets"]).cuda()
    row_of = torch.from_numpy(ref["row_of"].astype(np.int32)).cuda()
    xe = moe.moe_dispatch(x, row_of, cfg.top_k, ref["rows"])
    M = int(ref["expert_off"][-1])
    tok = torch.from_numpy(ref["row_token"][:M]).cuda()
    # every occupied row is a bit copy of its token's row
    assert torch.equal(xe[:M].view(torch.int16), x[tok].view(torch.int16))


# the 16-row blocked layout (rows x 32-column blocks of 1 KiB)
@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("seed", range(4))
def test_dispatch_blocked_tiny_bit_exact(seed, layout):
    cfg = get_config("tiny", act="bf16")
    d = make_routing_inputs(cfg, seed)
    x = make_x(cfg, seed, d["src_offsets"]).cuda()
    idx, _ = route_topk(d["logits"], cfg.top_k)
    N = len(idx)
    cap = worst_case_rows(N, 2, 2) if layout == COMPACT else int(np.diff(d["src_offsets"]).max())
    ref = dispatch_layout(idx, d["src_offsets"], 0, 2, layout, cap)
    R = ref["rows"]
    row_of = torch.from_numpy(ref["row_of"].astype(np.int32)).cuda()
    xe = torch.full((moe.blocked_rows(R), cfg.hidden), 7.5, dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch_blocked(x, row_of, 2, R, xe)
    rows = unblock16(xe, R)
    occ = torch.from_numpy(ref["row_token"] >= 0).cuda()
    tok = torch.from_numpy(np.maximum(ref["row_token"], 0)).cuda()
    assert torch.equal(rows[occ].view(torch.int16), x[tok][occ].view(torch.int16))
    assert torch.all(rows[~occ] == 7.5)   # unused rows untouched
    # the row-major dispatch holds the same rows
    xr = moe.moe_dispatch(x, row_of, 2, R, torch.full((R, cfg.hidden), 7.5, dtype=torch.bfloat16, device="cuda"))
    assert torch.equal(rows.view(torch.int16), xr.view(torch.int16))


@pytest.mark.parametrize("name", ["dsv3_prefill_ep8", "dsv3_decode_ep128"])
def test_dispatch_blocked_full_size(name):
    cfg = get_config(name)
    flush(f"dispatch blocked {name}")
    d = make_routing_inputs(cfg, 0)
    idx, _ = route_topk(d["logits"], cfg.top_k)
    N = len(idx)
    ref = dispatch_layout(idx, d["src_offsets"], 0, cfg.n_local, COMPACT, worst_case_rows(N, 8, cfg.n_local))
    x = make_x(cfg, 0, d["src_offsets"]).cuda()
    M = int(ref["expert_off"][-1])
    row_of = torch.from_numpy(ref["row_of"].astype(np.int32)).cuda()
    xe = moe.moe_dispatch_blocked(x, row_of, cfg.top_k, ref["rows"])
    tok = torch.from_numpy(ref["row_token"][:M]).cuda()
    assert torch.equal(unblock16(xe, M).view(torch.int16), x[tok].view(torch.int16))
