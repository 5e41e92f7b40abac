"""Pins of oracle.combine / moe_layer (composition of the whole share)."""
import numpy as np
import pytest

from oracle import COMPACT, PADDED, combine, dispatch, dispatch_layout, moe_layer, route_topk, worst_case_rows
from synth import make_inputs, tiny_config


def _tiny_f64(seed, shared=False):
    cfg = tiny_config(shared=shared)
    d = make_inputs(cfg, seed)
    x = d["x"].double().numpy()
    w13 = d["routed"]["w13"].double().numpy()
    w2 = d["routed"]["w2"].double().numpy()
    sh = None
    if shared:
        sh = (d["shared"]["w13"].double().numpy(), d["shared"]["w2"].double().numpy(), None, None)
    return cfg, d, x, w13, w2, sh


def test_hand_worked_combine():
    # 3 tokens, K = 2; rows hold known vectors; token 2 has no local entry and is
    # outside the self range, so it keeps the initial value.
    ye = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    row_of = np.array([0, 2, -1, 1, -1, -1])
    w = np.array([0.75, 0.25, 0.6, 0.4, 0.5, 0.5])
    init = np.full((3, 2), -7.0)
    ys = np.array([[0.5, 0.5]])
    out = combine(ye, row_of, w, 2, init, ys, 0, 1)
    np.testing.assert_array_equal(out[0], [0.75 * 1 + 0.25 * 100 + 0.5, 0.75 * 2 + 0.25 * 200 + 0.5])
    np.testing.assert_array_equal(out[1], [0.4 * 10, 0.4 * 20])
    np.testing.assert_array_equal(out[2], [-7.0, -7.0])


@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("seed", range(3))
def test_identity_experts_give_weighted_sum_of_x(seed, layout):
    cfg, d, x, *_ = _tiny_f64(seed)
    idx, w = route_topk(d["logits"], cfg.top_k)
    off = d["src_offsets"]
    N = len(x)
    cap = worst_case_rows(N, cfg.top_k, cfg.n_local) if layout == COMPACT else int(np.diff(off).max())
    lay = dispatch_layout(idx, off, 0, cfg.n_local, layout, cap)
    xe = dispatch(x, lay["row_of"], cfg.top_k, lay["rows"])
    out = combine(xe, lay["row_of"], w, cfg.top_k, np.zeros_like(x))
    local = (lay["row_of"].reshape(N, cfg.top_k) >= 0)
    np.testing.assert_allclose(out, (w * local).sum(axis=1)[:, None] * x, rtol=1e-14, atol=0)


def test_full_range_renormalised_identity_returns_x():
    cfg, d, x, *_ = _tiny_f64(1)
    idx, w = route_topk(d["logits"], cfg.top_k)
    lay = dispatch_layout(idx, d["src_offsets"], 0, cfg.n_experts, COMPACT, len(x) * cfg.top_k)
    xe = dispatch(x, lay["row_of"], cfg.top_k, lay["rows"])
    out = combine(xe, lay["row_of"], w, cfg.top_k, np.zeros_like(x))
    np.testing.assert_allclose(out, x, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("seed", range(3))
def test_ep_reconstruction(seed, layout):
    # Sum over the EP ranks of each rank's partial output (its own experts, plus the
    # shared expert on its own source tokens) equals the layer with every expert
    # local and the shared expert on all tokens.
    cfg, d, x, _, _, sh = _tiny_f64(seed, shared=True)
    from synth import make_expert_weights
    allw = make_expert_weights(cfg, seed, experts=range(cfg.n_experts))
    W13, W2 = allw["w13"].double().numpy(), allw["w2"].double().numpy()
    off = d["src_offsets"]
    N = len(x)
    full = moe_layer(x, d["logits"], off, cfg.top_k, 0, cfg.n_experts, W13, W2, shared=sh,
                     self_range=(0, N))["out"]
    ep = cfg.n_src
    L = cfg.n_experts // ep
    assert L == cfg.n_local
    acc = np.zeros_like(x)
    for r in range(ep):
        part = moe_layer(x, d["logits"], off, cfg.top_k, r * L, L, W13[r * L:(r + 1) * L], W2[r * L:(r + 1) * L],
                         shared=sh, self_range=(int(off[r]), int(off[r + 1])), layout=layout)
        acc += part["out"]
    np.testing.assert_allclose(acc, full, rtol=1e-12, atol=1e-14)


def test_layer_untouched_rows_keep_init():
    cfg, d, x, w13, w2, _ = _tiny_f64(2)
    init = np.full_like(x, 3.25)
    r = moe_layer(x, d["logits"], d["src_offsets"], cfg.top_k, 0, cfg.n_local, w13, w2, out_init=init)
    touched = (r["layout"]["row_of"].reshape(len(x), cfg.top_k) >= 0).any(axis=1)
    assert np.all(r["out"][~touched] == 3.25)
    assert not np.any(r["out"][touched] == 3.25)
