"""GPU parity of the W8A8 path against the CPU oracle.

The 1 x 128 fp8 payload (quantization and dispatch) must match bit for bit:
the quantization rule is the oracle's (one fp32 scale per 128 columns =
block max / 448, RNE e4m3fn codes of value / scale) and both sides take every
rounding decision in fp32 from the same fp32 input.

The W8A8 grouped GEMM is compared with the oracle's W8A8 FFN on the same
codes (rel-L2 5e-3 overall, 5e-2 per row; see TOL_W8A8) and with the
unquantized SwiGLU on the same weights within the fp8 tolerance 5e-2.
"""
import numpy as np
import pytest
import torch

import combine_router_softmax_amd as moe
from combine_router_softmax_amd.layer import MoEShare
from oracle import (COMPACT, PADDED, dequant_blockwise, dispatch_layout, e4m3fn_table, moe_layer, moe_layer_w8a8,
                    quantize_1x128, route_topk, swiglu_ffn, w8a8_ffn_q, worst_case_rows)
from synth import get_config, make_inputs, make_routing_inputs, make_x
from synth.workloads import _quantize_blocks_e4m3
from util import f64, flush, i64, rel_l2

pytestmark = pytest.mark.gpu

TAB = e4m3fn_table()


def _quant_check(x: torch.Tensor):
    xq, xs = moe.moe_quantize_1x128(x.cuda())
    torch.cuda.synchronize()
    rq, rs = quantize_1x128(x.float().cpu().numpy())
    got_q, got_s = xq.cpu().numpy(), xs.cpu().numpy()
    bad = np.nonzero(got_q != rq)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}: " \
                             f"{got_q[bad][0]:#x} vs {rq[bad][0]:#x}"
    np.testing.assert_array_equal(got_s.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,H", [(1, 128), (37, 384), (300, 1024)])
def test_quantize_random(dt, N, H):
    g = torch.Generator().manual_seed(N * H)
    x = torch.randn((N, H), generator=g) * torch.exp2(torch.randint(-10, 10, (N, 1), generator=g).float())
    x[:, : min(H, 256)] *= 37.0                           # blocks of different magnitude in one row
    _quant_check(x.to(dt))


def test_quantize_ties_neighbours_and_special_blocks():
    # scale-1 blocks (largest magnitude 448) holding every midpoint between
    # adjacent codes, its float32 neighbours and their negatives; an all-zero
    # block; a block whose scale underflows; a block of subnormal float32 values
    pos = TAB[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))])
    vals = np.concatenate([vals, -vals])
    per = 127
    rows = []
    for i in range(0, len(vals), per):
        blk = np.zeros(128, dtype=np.float32)
        blk[0] = 448.0
        chunk = vals[i:i + per]
        blk[1:1 + len(chunk)] = chunk
        rows.append(blk)
    rows.append(np.zeros(128, dtype=np.float32))
    under = np.zeros(128, dtype=np.float32)
    under[3], under[7] = np.float32(2.0 ** -143), -np.float32(2.0 ** -145)
    rows.append(under)
    sub = (np.arange(128, dtype=np.float32) - 64) * np.float32(2.0 ** -135)
    rows.append(sub)
    x = np.stack(rows)
    pad = (-len(x)) % 3
    x = np.concatenate([x, np.zeros((pad, 128), dtype=np.float32)]).reshape(-1, 384)  # 3 blocks per row
    _quant_check(torch.from_numpy(x))
    # the same on-grid halves in bf16 (midpoints of e4m3 codes need 4 mantissa bits)
    _quant_check(torch.from_numpy(x).to(torch.bfloat16))


@pytest.mark.parametrize("name", ["kimi_k2_ep8", "dsv3_prefill_ep8"])
def test_quantize_full_size(name):
    cfg = get_config(name)
    d = make_routing_inputs(cfg, 0)
    x = make_x(cfg, 0, d["src_offsets"])
    n = min(x.shape[0], 8192)
    flush(f"quantize {name}: {n} x {x.shape[1]}")
    _quant_check(x[:n])


@pytest.mark.parametrize("layout", [0, 1])
def test_dispatch_fp8_bit_exact(layout):
    cfg = get_config("kimi_k2_ep8")
    d = make_routing_inputs(cfg, 0)
    off = d["src_offsets"]
    x = make_x(cfg, 0, off)
    N, H = x.shape
    idx, _ = route_topk(d["logits"], cfg.top_k)
    lo, L = 0, cfg.n_local
    cap = worst_case_rows(N, cfg.top_k, L) if layout == 0 else int(np.diff(off).max())
    lay = dispatch_layout(idx, off, lo, L, layout, cap)
    row_of = torch.from_numpy(lay["row_of"].astype(np.int32)).cuda()
    xq, xs = moe.moe_quantize_1x128(x.cuda())
    R = lay["rows"]
    xeq = torch.full((R, H), 0xAB, dtype=torch.uint8, device="cuda")
    xes = torch.full((R, H // 128), -7.0, dtype=torch.float32, device="cuda")
    moe.moe_dispatch_fp8(xq, xs, row_of, cfg.top_k, R, xeq, xes)
    torch.cuda.synchronize()
    rt = lay["row_token"]
    used = rt >= 0
    tok = torch.from_numpy(rt[used]).long().cuda()
    rows = torch.from_numpy(np.nonzero(used)[0]).cuda()
    assert torch.equal(xeq[rows], xq[tok]) and torch.equal(xes[rows].view(torch.int32), xs[tok].view(torch.int32))
    free = torch.from_numpy(np.nonzero(~used)[0]).cuda()
    assert bool((xeq[free] == 0xAB).all()) and bool((xes[free] == -7.0).all()), "an unused row was written"
    assert int(used.sum()) == int(i64(row_of).__ge__(0).sum())


# ----------------------------------------------------------------------------- W8A8 grouped GEMM

# GPU vs the W8A8 oracle. y is rounded to bf16 (about 1e-3 rel-L2). The fp8
# matrix instruction's own sum is not exact (measured up to ~3e-4 of the
# largest product per 64-deep instruction), so g and u carry ~1e-4 relative
# error, and an h value that close to a code midpoint takes the neighbouring
# code: one such step (6-12 % of |h_i|) moves a row of y by up to about
# 0.1 |h_i| / ||h||, a few percent of the row when I is a few hundred. Hence a
# tight aggregate bound and the fp8 tolerance per row.
TOL_W8A8 = 5e-3       # aggregate rel-L2
ROW_TOL_W8A8 = 5e-2   # per row
TOL_FP8 = 5e-2        # W8A8 vs the unquantized-activation FFN (fp8 tolerance)


def _fp8_expert_weights(rng, G, H, I):
    """e4m3 codes + 128x128 scales (blocks of different magnitude)."""
    def one(n, k):
        w = rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)
        w *= (2.0 ** rng.integers(-2, 3, (n // 128, k // 128))).repeat(128, 0).repeat(128, 1).astype(np.float32)
        return _quantize_blocks_e4m3(w)
    w13, s13, w2, s2 = [], [], [], []
    for _ in range(G):
        a, b = one(2 * I, H)
        c, d = one(H, I)
        w13.append(a); s13.append(b); w2.append(c); s2.append(d)
    return np.stack(w13), np.stack(s13), np.stack(w2), np.stack(s2)


def _check_rows(got, ref, what, tol=TOL_W8A8, row_tol=ROW_TOL_W8A8):
    err = rel_l2(got, ref)
    assert err <= tol, f"{what}: rel-L2 {err:.3e} > {tol}"
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    worst = float((num / den).max()) if len(ref) else 0.0
    assert worst <= row_tol, f"{what}: worst row rel-L2 {worst:.3e} > {row_tol}"
    return err


@pytest.mark.parametrize("layout", [COMPACT, PADDED])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("gather", [False, True])
def test_w8a8_grouped_gemm_small(layout, packed, gather):
    rng = np.random.default_rng(11 + 2 * layout + int(packed) + 4 * int(gather))
    H, I = 1024, 384 if layout == PADDED else 512     # I = 384: an odd number of 128-column blocks
    m = [0, 1, 33, 96, 97, 250]                        # ragged groups, several row tiles, a tail
    G = len(m)
    w13q, s13, w2q, s2 = _fp8_expert_weights(rng, G + 1, H, I)
    if layout == COMPACT:
        off = np.concatenate([[0], np.cumsum(m)]).astype(np.int32)
        R = int(off[-1])
        rows_of = [np.arange(off[g], off[g + 1]) for g in range(G)]
        S, C, counts_t, off_t = 1, 0, None, torch.from_numpy(off).cuda()
    else:
        S, C = 3, 100
        cnt = np.zeros((G, S), dtype=np.int32)
        for g, mg in enumerate(m):
            cut = np.sort(rng.integers(0, mg + 1, S - 1)) if mg else np.zeros(S - 1, int)
            cnt[g] = np.minimum(np.diff(np.concatenate([[0], cut, [mg]])), C)
        R = G * S * C
        rows_of = [np.concatenate([(g * S + s) * C + np.arange(cnt[g, s]) for s in range(S)]) for g in range(G)]
        S, counts_t, off_t = S, torch.from_numpy(cnt).cuda(), None
    T = 300                                            # source tokens (gather) or rows (no gather)
    x = (rng.standard_normal((T if gather else R, H)) * 2.0 ** rng.integers(-3, 3, (T if gather else R, 1)))
    x = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    xq, xs = quantize_1x128(x.float().numpy())
    a_rows_np = rng.integers(0, T, R).astype(np.int32) if gather else None
    B = 40
    sx = torch.from_numpy(rng.standard_normal((B, H)).astype(np.float32)).to(torch.bfloat16)
    sq, ss = quantize_1x128(sx.float().numpy())
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    W13, S13, W2, S2 = d(w13q[:G]), d(s13[:G]), d(w2q[:G]), d(s2[:G])
    if packed:
        W13, W2 = moe.moe_pack_weights(W13, W2, H, I)
        SW13, SW2 = moe.moe_pack_weights(d(w13q[G:]), d(w2q[G:]), H, I)
    else:
        SW13, SW2 = d(w13q[G:]), d(w2q[G:])
    shared = dict(a=d(sq), a_scales=d(ss), w13=SW13, w2=SW2, s13=d(s13[G:]), s2=d(s2[G:]),
                  y=torch.empty((B, H), dtype=torch.bfloat16, device="cuda"))
    y = torch.full((R, H), 7.0, dtype=torch.bfloat16, device="cuda")
    kw = dict(group_off=off_t, counts=counts_t, s13=S13, s2=S2, layout=layout, n_src=S, capacity=C, y=y,
              shared=shared, w_format=moe.W_PACKED if packed else moe.W_ROWMAJOR, a_scales=d(xs),
              rows=R, a_rows=d(a_rows_np) if gather else None)
    flush(f"w8a8 gemm layout={layout} packed={packed} gather={gather}")
    moe.moe_grouped_gemm(d(xq), W13, W2, **kw)
    torch.cuda.synchronize()
    got = f64(y)
    src = (lambda r: a_rows_np[r]) if gather else (lambda r: r)
    tot_ref, tot_got, tot_fp = [], [], []
    for g in range(G):
        rows = rows_of[g]
        if len(rows) == 0:
            continue
        ref = w8a8_ffn_q(xq[src(rows)], xs[src(rows)], w13q[g], s13[g], w2q[g], s2[g])
        fp = swiglu_ffn(x.float().numpy()[src(rows)], dequant_blockwise(w13q[g], s13[g]),
                        dequant_blockwise(w2q[g], s2[g]))
        _check_rows(got[rows], ref, f"group {g} ({len(rows)} rows)")
        tot_ref.append(ref); tot_got.append(got[rows]); tot_fp.append(fp)
    assert rel_l2(np.concatenate(tot_got), np.concatenate(tot_fp)) <= TOL_FP8
    sref = w8a8_ffn_q(sq, ss, w13q[G], s13[G], w2q[G], s2[G])
    _check_rows(f64(shared["y"]), sref, "shared expert")
    # rows no group owns keep their contents
    used = np.zeros(R, bool)
    for rows in rows_of:
        used[rows] = True
    assert bool((y[torch.from_numpy(np.nonzero(~used)[0]).cuda()] == 7.0).all())

    # a policy that asks for the wide-tile kernel (absent for W8A8) changes nothing
    y3 = torch.full_like(y, 7.0)
    moe.moe_grouped_gemm(d(xq), W13, W2, **dict(kw, y=y3, policy=moe.GEMM_WIDE,
                                                 shared=dict(shared, y=torch.empty_like(shared["y"]))))
    torch.cuda.synchronize()
    assert torch.equal(y3, y), "policy WIDE changed the W8A8 result"

    # the two stages in turn on one workspace give the same bits
    y2 = torch.zeros_like(y)
    ws = torch.zeros(1 << 28, dtype=torch.uint8, device="cuda")   # above the workspace size query
    sy2 = torch.empty_like(shared["y"])
    for stage in (moe.GG_UP, moe.GG_DOWN):
        kw2 = dict(kw, y=y2 if stage == moe.GG_DOWN else None, stage=stage, shared=dict(shared, y=sy2))
        moe.moe_grouped_gemm(d(xq), W13, W2, ws=ws, **kw2)
    torch.cuda.synchronize()
    for g in range(G):
        rows = torch.from_numpy(rows_of[g]).long().cuda()
        assert torch.equal(y2[rows], y[rows]), f"staged run differs in group {g}"
    assert torch.equal(sy2, shared["y"]), "staged run differs for the shared expert"


# ----------------------------------------------------------------------------- W8A8 layer


def _w8a8_share(d, layout, gather=None, cap=None):
    cfg = d["cfg"]
    off = d["src_offsets"]
    N, B0 = int(off[-1]), int(off[1])
    if cap is None and layout == PADDED:
        cap = int(np.diff(off).max())
    share = MoEShare(n_tokens=N, hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                     n_src=cfg.n_src, expert_lo=cfg.expert_lo, n_local=cfg.n_local, act_dtype=torch.bfloat16,
                     layout=layout, capacity=cap, self_range=(0, B0), gather=gather, w8a8=True)
    share.set_weights(d["routed"], d["shared"])
    return share


def _w8a8_run(share, d, shared_mode=None, sentinel=-9.0):
    logits = torch.from_numpy(d["logits"]).cuda()
    off = torch.from_numpy(d["src_offsets"]).cuda()
    x = d["x"].cuda()
    out = torch.full_like(x, sentinel)
    share.step(logits, off, x, out, shared_mode=shared_mode)
    torch.cuda.synchronize()
    return out


def _np(wd, k):
    return wd[k].numpy()


def _oracles(d, layout, capacity, n=None):
    """W8A8 oracle layer and the unquantized-activation oracle layer (same fp8
    weights) over the first n tokens (all by default)."""
    cfg = d["cfg"]
    off = np.asarray(d["src_offsets"])
    if n is not None:
        off = np.array([0, n])
    N = int(off[-1])
    B0 = int(off[1])
    x = d["x"][:N].float().numpy()
    r, s = d["routed"], d["shared"]
    args = (x, d["logits"][:N], off, cfg.top_k, cfg.expert_lo, cfg.n_local)
    q = moe_layer_w8a8(*args, _np(r, "w13"), _np(r, "w2"), _np(r, "s13"), _np(r, "s2"),
                       shared=(_np(s, "w13"), _np(s, "w2"), _np(s, "s13"), _np(s, "s2")), self_range=(0, B0),
                       layout=layout, capacity=capacity, out_init=np.full((N, cfg.hidden), -9.0))
    deq13 = [dequant_blockwise(r["w13"][g].numpy(), r["s13"][g].numpy()) for g in range(cfg.n_local)]
    deq2 = [dequant_blockwise(r["w2"][g].numpy(), r["s2"][g].numpy()) for g in range(cfg.n_local)]
    sh = (dequant_blockwise(s["w13"][0].numpy(), s["s13"][0].numpy())[None],
          dequant_blockwise(s["w2"][0].numpy(), s["s2"][0].numpy())[None], None, None)
    u = moe_layer(x.astype(np.float64), *args[1:], _Stack(deq13), _Stack(deq2), shared=sh, self_range=(0, B0),
                  layout=layout, capacity=capacity, out_init=np.full((N, cfg.hidden), -9.0))
    return q, u


class _Stack:
    """expert g -> its float64 matrix (a list that indexes like [G, ...])"""
    def __init__(self, mats):
        self.m = mats

    def __getitem__(self, g):
        return self.m[g]


def _compare_layer(got, q, u, what):
    touched = q["out"][:, 0] != -9.0
    assert np.all(got[~touched] == -9.0), f"{what}: an untouched row was written"
    err = _check_rows(got[touched], q["out"][touched], what)
    err_u = rel_l2(got[touched], u["out"][touched])
    flush(f"  {what}: {int(touched.sum())} rows, rel-L2 {err:.2e} vs W8A8 oracle, {err_u:.2e} vs unquantized")
    assert err_u <= TOL_FP8, f"{what}: rel-L2 {err_u:.3e} against the unquantized layer"


@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_w8a8_layer_mid_size_every_row(layout):
    # hidden 1024, 8 ranks x 96 tokens, 64 experts (8 local), top-8, intermediate
    # 512: several tiles per expert, stream-K ranges cut inside tiles (fix-ups)
    cfg = get_config("kimi_k2_ep8", hidden=1024, inter=512, n_experts=64, n_local=8, tokens_per_src=96)
    d = make_inputs(cfg, 7)
    outs = {}
    for gather in (True, False):
        share = _w8a8_share(d, layout, gather=gather)
        for mode in ("fused", "serial", "stream"):
            outs[(gather, mode)] = _w8a8_run(share, d, shared_mode=mode)
    # the gathered and the dispatched rows are the same codes: the same bits
    for mode in ("fused", "serial", "stream"):
        assert torch.equal(outs[(True, mode)].view(torch.int16), outs[(False, mode)].view(torch.int16)), mode
    assert torch.equal(outs[(True, "serial")].view(torch.int16), outs[(True, "stream")].view(torch.int16))
    q, u = _oracles(d, layout, share.capacity)
    np.testing.assert_array_equal(i64(share.lay["row_of"]), q["layout"]["row_of"])
    for mode in ("fused", "serial"):
        _compare_layer(f64(outs[(True, mode)]), q, u, f"mid layout={layout} shared={mode}")


def test_w8a8_layer_full_size_kimi():
    """kimi_k2_ep8 (fp8 weights) on the W8A8 path: every touched row of the
    whole layer against the W8A8 oracle and the unquantized-activation layer;
    the two layouts give the same bits."""
    cfg = get_config("kimi_k2_ep8")
    flush("generate kimi_k2_ep8")
    d = make_inputs(cfg, 0)
    outs = {}
    for layout in (COMPACT, PADDED):
        share = _w8a8_share(d, layout)
        outs[layout] = _w8a8_run(share, d)
        again = _w8a8_run(share, d)
        assert torch.equal(outs[layout].view(torch.int16), again.view(torch.int16)), "not deterministic"
        if layout == COMPACT:
            cap = share.capacity
        del share
        torch.cuda.empty_cache()
    assert torch.equal(outs[COMPACT].view(torch.int16), outs[PADDED].view(torch.int16))
    flush("  oracle layers")
    q, u = _oracles(d, COMPACT, cap)
    _compare_layer(f64(outs[COMPACT]), q, u, "kimi_k2_ep8 W8A8")


def test_w8a8_layer_full_size_prefill_own_tokens():
    """dsv3_prefill_ep8 with its weights quantized to fp8 (128 x 128 tiles), on
    the W8A8 path: the GPU's own 4096 tokens end to end (their routed rows,
    the shared expert and the combine) against the oracles run on those
    tokens alone (other sources' rows do not touch these outputs)."""
    cfg = get_config("dsv3_prefill_ep8", weight="fp8_e4m3")
    flush("generate dsv3_prefill_ep8 with fp8 weights")
    d = make_inputs(cfg, 0)
    off = d["src_offsets"]
    B0 = int(off[1])
    share = _w8a8_share(d, COMPACT)
    out = _w8a8_run(share, d)
    del share
    torch.cuda.empty_cache()
    flush(f"  oracle layers over the {B0} own tokens")
    q, u = _oracles(d, COMPACT, None, n=B0)
    _compare_layer(f64(out[:B0]), q, u, "dsv3_prefill_ep8 W8A8 own tokens")


def test_e4m3_encoder_on_every_float32():
    """The encoder behind every fp8 code (the conversion instruction, with
    magnitudes <= 2^-10 entered as +0) equals a bit-level encoder of the
    OCP e4m3fn format, round to nearest even, zero as 0x00, on every finite
    float32 clamped to [-448, 448] (probes/fp8_encode.hip, built by build.py)."""
    import os
    import re
    import subprocess
    exe = os.path.join(os.path.dirname(moe.__file__), "fp8_encode_check")
    assert os.path.exists(exe), "fp8_encode_check is built with the library (combine_router_softmax_amd/build.py)"
    flush("fp8 encoder probe over all float32")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    m = re.search(r"tested (\d+) mismatches (\d+)", out.stdout)
    assert m, out.stdout
    assert int(m.group(1)) == 2 ** 32 - 2 ** 24
    assert int(m.group(2)) == 0, out.stdout
