"""One step of the layer captured in a HIP graph: every replay gives the same
bits as an eager step on the same inputs, with new inputs copied into the
captured buffers between replays (the kernels read counts and offsets on the
device, so one graph serves every routing of the same batch shape)."""
import numpy as np
import pytest
import torch

from combine_router_softmax_amd.layer import MoEShare
from oracle import COMPACT, PADDED, moe_layer
from synth import get_config, make_inputs, make_routing_inputs, make_x, tiny_config
from util import f64, flush, rel_l2

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8_e4m3": 5e-2}


def _oracle_weights(d0):
    r, s = d0["routed"], d0["shared"]
    fp8 = r.get("s13") is not None

    def w(t):
        return t.numpy() if fp8 else t.double().numpy()
    sc = (r["s13"].numpy(), r["s2"].numpy()) if fp8 else (None, None)
    routed = (w(r["w13"]), w(r["w2"]), *sc)
    sh = None if s is None else (w(s["w13"]), w(s["w2"]),
                                 *((s["s13"].numpy(), s["s2"].numpy()) if fp8 else (None, None)))
    return routed, sh


def _oracle_check(cfg, weights, inp, got, layout, capacity):
    """The eager step (which every replay equals bit for bit) against the
    oracle: every touched row for batches up to 2048 tokens, else the GPU's
    own tokens plus 256 others."""
    lg, of, x = inp
    of = np.asarray(of, dtype=np.int64)
    N, B0 = int(of[-1]), int(of[1])
    routed, sh = weights
    if N <= 2048:
        tok = np.arange(N)
        sub_off = of
    else:
        rng = np.random.default_rng(N)
        tok = np.concatenate([np.arange(B0), np.sort(rng.choice(np.arange(B0, N), 256, replace=False))])
        sub_off, layout, capacity = [0, len(tok)], COMPACT, None
    ref = moe_layer(f64(x[torch.from_numpy(tok)]), lg[tok], sub_off, cfg.top_k, cfg.expert_lo, cfg.n_local, *routed,
                    shared=sh, self_range=(0, B0), layout=layout, capacity=capacity,
                    out_init=np.full((len(tok), cfg.hidden), -9.0))
    g = f64(got)[tok]
    touched = ref["out"][:, 0] != -9.0
    assert np.all(g[~touched] == -9.0)
    assert rel_l2(g[touched], ref["out"][touched]) <= TOL[cfg.weight]


def _inputs(cfg):
    d0 = make_inputs(cfg, 0)
    b0 = np.asarray(d0["batches"])
    # same total and same first source (its rows are the shared-expert rows),
    # other sources re-split
    b1 = np.concatenate([b0[:1], b0[1:][::-1]])
    r1 = make_routing_inputs(cfg, 1, batches=b1)
    x1 = make_x(cfg, 1, r1["src_offsets"])
    return d0, [(d0["logits"], d0["src_offsets"], d0["x"]), (r1["logits"], r1["src_offsets"], x1)]


@pytest.mark.parametrize("name,layout", [("tiny", PADDED), ("tiny", COMPACT), ("dsv3_decode_ep8", COMPACT),
                                         ("kimi_k2_ep8", COMPACT), ("dsv3_decode_ep8", PADDED),
                                         ("dsv3_decode_ep128", COMPACT)])  # wide-tile kernel, gathered rows
def test_graph_replays_match_eager(name, layout):
    cfg = tiny_config(shared=True) if name == "tiny" else get_config(name)
    flush(f"graph {cfg.name} layout={layout}")
    d0, ins = _inputs(cfg)
    off0 = d0["src_offsets"]
    N = int(off0[-1])
    cap = None
    if layout == PADDED:
        cap = int(max(np.diff(o).max() for _, o, _ in ins))
    act = torch.float32 if cfg.act == "f32" else torch.bfloat16
    share = MoEShare(n_tokens=N, hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                     n_src=cfg.n_src, expert_lo=cfg.expert_lo, n_local=cfg.n_local, act_dtype=act, layout=layout,
                     capacity=cap, self_range=(0, int(off0[1])))
    share.set_weights(d0["routed"], d0["shared"])

    L = torch.empty((N, cfg.n_experts), dtype=torch.float32, device="cuda")
    O = torch.empty(len(off0), dtype=torch.int32, device="cuda")
    X = torch.empty((N, cfg.hidden), dtype=act, device="cuda")
    out = torch.empty_like(X)

    def load(i):
        lg, of, x = ins[i]
        L.copy_(torch.from_numpy(lg))
        O.copy_(torch.from_numpy(np.asarray(of, dtype=np.int32)))
        X.copy_(x)
        out.fill_(-9.0)

    weights = _oracle_weights(d0)
    eager = []
    for i in range(2):
        load(i)
        share.step(L, O, X, out)
        torch.cuda.synchronize()
        eager.append(out.clone())
        _oracle_check(cfg, weights, ins[i], eager[i], layout, share.capacity)
    assert not torch.equal(eager[0], eager[1])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        share.step(L, O, X, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        share.step(L, O, X, out)
    torch.cuda.synchronize()

    for rep, i in enumerate([0, 1, 1, 0, 1]):
        load(i)
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")  # eager work between
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk).all()
        bits = out.view(torch.int16) if act == torch.bfloat16 else out.view(torch.int32)
        ref = eager[i].view(torch.int16) if act == torch.bfloat16 else eager[i].view(torch.int32)
        assert torch.equal(bits, ref), f"replay {rep} (input {i}) differs from the eager step"
        assert int(share.lay["status"].item()) == 0
    del g, share
    torch.cuda.empty_cache()
