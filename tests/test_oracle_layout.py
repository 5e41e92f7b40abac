"""Pins of oracle.dispatch_layout / dispatch / worst_case_rows."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import COMPACT, PADDED, STATUS_OVERFLOW, dispatch, dispatch_layout, group_rows, route_topk, worst_case_rows
from synth import get_config, make_routing_inputs


def _toy(golden_dir):
    with open(os.path.join(golden_dir, "layout_toy.json")) as f:
        return json.load(f)


def test_hand_worked_fixture(golden_dir):
    d = _toy(golden_dir)
    idx = np.array(d["topk_idx"])
    for c in d["cases"]:
        lay = dispatch_layout(idx, d["src_offsets"], c["expert_lo"], c["n_local"], c["layout"], c["capacity"])
        assert lay["counts"].tolist() == c["counts"], c["name"]
        assert lay["expert_off"].tolist() == c["expert_off"], c["name"]
        assert lay["row_of"].tolist() == c["row_of"], c["name"]
        assert lay["row_token"].tolist() == c["row_token"], c["name"]
        assert lay["status"] == c["status"], c["name"]


def _random_routing(seed, N, E, K, S):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((N, E)).astype(np.float32)
    idx, _ = route_topk(z, K)
    b = rng.multinomial(N, np.ones(S) / S)
    off = np.concatenate([[0], np.cumsum(b)])
    return idx, off


@pytest.mark.parametrize("seed", range(4))
def test_counts_sum_full_range_and_ep_split(seed):
    N, E, K, S = 97, 16, 3, 5
    idx, off = _random_routing(seed, N, E, K, S)
    full = dispatch_layout(idx, off, 0, E, COMPACT, worst_case_rows(N, K, E))
    assert full["counts"].sum() == N * K
    np.testing.assert_array_equal(full["counts"].sum(axis=0), np.diff(off) * K)
    for ep in (2, 4, 8, 16):
        L = E // ep
        tot = 0
        for r in range(ep):
            lay = dispatch_layout(idx, off, r * L, L, COMPACT, worst_case_rows(N, K, L))
            tot += lay["counts"].sum()
            assert lay["expert_off"][-1] == lay["counts"].sum()
        assert tot == N * K


@pytest.mark.parametrize("seed", range(4))
def test_compact_is_stable_bijection_matching_stable_argsort(seed):
    N, E, K, S = 120, 16, 2, 8
    idx, off = _random_routing(seed, N, E, K, S)
    lo, L = 4, 5
    lay = dispatch_layout(idx, off, lo, L, COMPACT, worst_case_rows(N, K, L))
    flat = idx.reshape(-1) - lo
    local = np.nonzero((flat >= 0) & (flat < L))[0]
    M = len(local)
    rows = lay["row_of"][local]
    assert sorted(rows.tolist()) == list(range(M))
    assert np.all(lay["row_of"][np.setdiff1d(np.arange(N * K), local)] == -1)
    # the packed order is the stable sort of the local entries by expert
    order = np.argsort(flat[local], kind="stable")
    np.testing.assert_array_equal(rows[order], np.arange(M))
    np.testing.assert_array_equal(lay["row_token"][:M], local[order] // K)
    # stability: inside one expert, rows grow with the token index
    for g in range(L):
        toks = lay["row_token"][group_rows(lay, g)]
        assert np.all(np.diff(toks) > 0)


@pytest.mark.parametrize("seed", range(4))
def test_padded_closed_form(seed):
    N, E, K, S = 90, 16, 2, 6
    idx, off = _random_routing(seed, N, E, K, S)
    lo, L = 0, 4
    C = int(np.diff(off).max())
    lay = dispatch_layout(idx, off, lo, L, PADDED, C)
    assert lay["status"] == 0
    assert lay["rows"] == L * S * C
    np.testing.assert_array_equal(lay["expert_off"], np.arange(L + 1) * S * C)
    src = np.searchsorted(off, np.arange(N), side="right") - 1
    for le in range(L):
        for s in range(S):
            ents = [t * K + k for t in range(off[s], off[s + 1]) for k in range(K) if idx[t, k] - lo == le]
            base = (le * S + s) * C
            assert lay["row_of"][ents].tolist() == list(range(base, base + len(ents)))
            assert lay["counts"][le, s] == len(ents)
            hole = lay["row_token"][base + len(ents): base + C]
            assert np.all(hole == -1)
            assert np.all(src[lay["row_token"][base: base + len(ents)]] == s)


def test_padded_overflow_drops_the_last_entries():
    N, E, K, S = 64, 8, 2, 2
    idx, off = _random_routing(11, N, E, K, S)
    full = dispatch_layout(idx, off, 0, 2, PADDED, int(np.diff(off).max()))
    C = int(full["counts"].max()) - 2
    lay = dispatch_layout(idx, off, 0, 2, PADDED, C)
    assert lay["status"] & STATUS_OVERFLOW
    kept = lay["row_of"] >= 0
    # an entry is kept iff its rank inside (expert, source) is below C
    rank = full["row_of"] - (full["row_of"] // int(np.diff(off).max())) * int(np.diff(off).max())
    np.testing.assert_array_equal(kept, (full["row_of"] >= 0) & (rank < C))
    assert np.all(lay["row_of"][kept] < 2 * S * C)


def test_compact_capacity_overflow():
    N, E, K, S = 50, 8, 2, 3
    idx, off = _random_routing(5, N, E, K, S)
    full = dispatch_layout(idx, off, 0, 4, COMPACT, worst_case_rows(N, K, 4))
    M = int(full["expert_off"][-1])
    cap = M - 7
    lay = dispatch_layout(idx, off, 0, 4, COMPACT, cap)
    assert lay["status"] & STATUS_OVERFLOW
    np.testing.assert_array_equal(lay["row_of"], np.where(full["row_of"] < cap, full["row_of"], -1))
    np.testing.assert_array_equal(lay["expert_off"], np.minimum(full["expert_off"], cap))
    assert full["status"] == 0


def test_worst_case_bound_brute_force():
    # One GPU of n_ranks hosting E/n_ranks experts; T tokens per rank; R experts per token.
    # Brute force over every R-subset: a token can land at most min(R, E/n) times here.
    for (n, T, R, E) in [(2, 3, 2, 4), (4, 2, 3, 8), (2, 2, 3, 4), (8, 1, 2, 16), (4, 1, 4, 8)]:
        L = E // n
        best = max(sum(1 for e in sub if e < L) for sub in itertools.combinations(range(E), R))
        assert best == min(R, L)
        # adversarial routing: every token picks the local experts first
        N = n * T
        logits = np.tile(-np.arange(E, dtype=np.float32), (N, 1))
        idx, _ = route_topk(logits, R)
        off = np.arange(n + 1) * T
        lay = dispatch_layout(idx, off, 0, L, COMPACT, worst_case_rows(N, R, L))
        assert lay["expert_off"][-1] == n * T * min(R, L) == worst_case_rows(N, R, L)
        # the printed bound (max instead of min) is never exceeded either
        assert lay["expert_off"][-1] <= n * T * max(R, E // n)
        pad = dispatch_layout(idx, off, 0, L, PADDED, T)
        assert pad["status"] == 0


def test_empty_sources_and_empty_batch():
    idx = np.zeros((0, 2), dtype=np.int32)
    lay = dispatch_layout(idx, [0, 0, 0], 0, 2, COMPACT, 0)
    assert lay["counts"].shape == (2, 2) and lay["counts"].sum() == 0 and lay["status"] == 0
    idx, off = _random_routing(3, 20, 8, 2, 4)
    off = np.array([0, 0, 10, 10, 20])
    lay = dispatch_layout(idx, off, 0, 4, PADDED, 10)
    assert np.all(lay["counts"][:, [0, 2]] == 0)


def test_dispatch_is_gather_of_row_token():
    rng = np.random.default_rng(9)
    N, E, K, S, H = 40, 8, 2, 4, 6
    idx, off = _random_routing(9, N, E, K, S)
    x = rng.standard_normal((N, H))
    for layout, cap in [(COMPACT, worst_case_rows(N, K, 3)), (PADDED, int(np.diff(off).max()))]:
        lay = dispatch_layout(idx, off, 1, 3, layout, cap)
        xe = dispatch(x, lay["row_of"], K, lay["rows"])
        occ = lay["row_token"] >= 0
        np.testing.assert_array_equal(xe[occ], np.take(x, lay["row_token"][occ], axis=0))
        assert np.all(np.isnan(xe[~occ]))


def test_page_arithmetic_local_experts_per_gpu():
    # 256 routed experts over EP ranks: 256/8 = 32 and 256/128 = 2 per GPU.
    assert get_config("dsv3_decode_ep8").n_local == 256 // 8 == 32
    assert get_config("dsv3_decode_ep128").n_local == 256 // 128 == 2
    assert get_config("dsv3_decode_ep128").n_src == 128
    assert get_config("kimi_k2_ep8").n_local == 384 // 8


def test_page_arithmetic_batch_one_active_experts():
    # Batch 1 with query length 2 under EP8: 2 tokens, top-8, at most 2*8 = 16
    # experts active in total, i.e. at most 2*8/8 = 2 per GPU on average.
    rng = np.random.default_rng(12)
    for _ in range(20):
        z = rng.standard_normal((2, 256)).astype(np.float32)
        idx, _ = route_topk(z, 8)
        active = 0
        for r in range(8):
            lay = dispatch_layout(idx, [0, 2], r * 32, 32, COMPACT, worst_case_rows(2, 8, 32))
            active += int(np.count_nonzero(lay["counts"].sum(axis=1)))
        assert active == len(set(idx.reshape(-1).tolist())) <= 16
        assert active / 8 <= 2


def test_page_arithmetic_large_batch_activates_all_local_experts():
    # With a large batch every one of the 32 local experts is active.
    cfg = get_config("dsv3_decode_ep8")
    d = make_routing_inputs(cfg, 0)
    idx, _ = route_topk(d["logits"], cfg.top_k)
    lay = dispatch_layout(idx, d["src_offsets"], 0, 32, COMPACT, worst_case_rows(len(idx), 8, 32))
    assert np.count_nonzero(lay["counts"].sum(axis=1)) == 32
    # mean rows per expert = N*K/E = 1024*8/256 = 32
    assert abs(lay["expert_off"][-1] / 32 - 32) < 4
