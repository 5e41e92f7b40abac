"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest

import combine_router_softmax_amd as moe
from combine_router_softmax_amd import GGemmDesc, LayoutDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.lib_path()):
        pytest.fail("libmoe.so is not built: run python combine_router_softmax_amd/build.py")
    return moe.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"moe_route_topk", "moe_dispatch_layout", "moe_dispatch", "moe_grouped_gemm", "moe_combine"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert moe.moe_abi_version() == 3
    for s, txt in [(0, b"ok"), (1, b"invalid argument"), (3, b"workspace missing or too small")]:
        assert lib.moe_status_string(s) == txt


def test_binding_exposes_the_same_names():
    for n in ("moe_route_topk", "moe_dispatch_layout", "moe_dispatch", "moe_grouped_gemm", "moe_combine"):
        assert callable(getattr(moe, n))


def test_route_argument_errors(lib):
    f = lib.moe_route_topk
    assert f(FAKE, 10, 16, 17, 1, FAKE, FAKE, None) == INVALID      # top_k > E
    assert f(FAKE, 10, 16, 0, 1, FAKE, FAKE, None) == INVALID       # top_k < 1
    assert f(FAKE, -1, 16, 2, 1, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 10, 2048, 8, 1, FAKE, FAKE, None) == UNSUPPORTED  # E > 1024
    assert f(FAKE, 10, 64, 20, 1, FAKE, FAKE, None) == UNSUPPORTED   # K > 16
    assert f(None, 10, 16, 2, 1, FAKE, FAKE, None) == INVALID       # null with work to do
    assert f(None, 0, 16, 2, 1, None, None, None) == OK             # nothing to do, nothing enqueued


def _ld(**kw):
    base = dict(n_tokens=100, top_k=2, n_experts=16, n_src=4, expert_lo=0, n_local=2, layout=0, capacity=200)
    base.update(kw)
    return LayoutDesc(**base)


def test_layout_rows_and_workspace(lib):
    assert lib.moe_layout_rows(ctypes.byref(_ld())) == 200
    assert lib.moe_layout_rows(ctypes.byref(_ld(layout=1, capacity=30))) == 2 * 4 * 30
    assert lib.moe_layout_rows(ctypes.byref(_ld(n_src=0))) == -1
    assert lib.moe_layout_rows(ctypes.byref(_ld(layout=7))) == -1
    ws = lib.moe_dispatch_layout_workspace(ctypes.byref(_ld()))
    assert ws > 0 and ws % 256 == 0
    assert lib.moe_dispatch_layout_workspace(ctypes.byref(_ld(top_k=0))) == 0


def test_layout_argument_errors(lib):
    f = lib.moe_dispatch_layout
    d = _ld()
    ws = lib.moe_dispatch_layout_workspace(ctypes.byref(d))
    args = [FAKE] * 7
    assert f(ctypes.byref(_ld(top_k=17)), *args, FAKE, ws, None) == INVALID
    assert f(ctypes.byref(_ld(n_local=2000)), *args, FAKE, ws, None) == UNSUPPORTED
    assert f(ctypes.byref(_ld(n_src=5000)), *args, FAKE, ws, None) == UNSUPPORTED
    assert f(ctypes.byref(d), *args, None, ws, None) == WORKSPACE
    assert f(ctypes.byref(d), *args, FAKE, ws - 4, None) == WORKSPACE
    assert f(ctypes.byref(d), FAKE, None, *([FAKE] * 5), FAKE, ws, None) == INVALID  # src_offsets NULL
    assert f(None, *args, FAKE, ws, None) == INVALID


def test_dispatch_and_combine_argument_errors(lib):
    assert lib.moe_dispatch(FAKE, 1, 10, 12, 2, FAKE, 100, FAKE, None) == INVALID     # 24-byte rows
    assert lib.moe_dispatch(FAKE, 2, 10, 64, 2, FAKE, 100, FAKE, None) == UNSUPPORTED  # fp8 rows
    assert lib.moe_dispatch(FAKE, 1, 10, 64, 17, FAKE, 100, FAKE, None) == UNSUPPORTED
    assert lib.moe_dispatch(ctypes.c_void_p(0x100008), 1, 10, 64, 2, FAKE, 100, FAKE, None) == INVALID  # misaligned
    assert lib.moe_dispatch(None, 1, 0, 64, 2, None, 100, None, None) == OK
    b = lib.moe_dispatch_blocked
    assert b(FAKE, 0, 10, 64, 2, FAKE, 100, FAKE, None) == UNSUPPORTED  # f32 rows
    assert b(FAKE, 1, 10, 48, 2, FAKE, 100, FAKE, None) == INVALID      # hidden % 32
    assert b(FAKE, 1, -1, 64, 2, FAKE, 100, FAKE, None) == INVALID
    assert b(FAKE, 1, 10, 64, 17, FAKE, 100, FAKE, None) == UNSUPPORTED  # K > 16
    assert b(FAKE, 1, 10, 64, 2, None, 100, FAKE, None) == INVALID      # no row_of
    assert b(None, 1, 0, 64, 2, None, 100, None, None) == OK
    c = lib.moe_combine
    assert c(FAKE, 1, 100, FAKE, FAKE, 10, 2, 12, None, 0, 0, FAKE, None) == INVALID  # 24-byte rows
    assert c(FAKE, 1, 100, FAKE, FAKE, 10, 2, 64, FAKE, 5, 20, FAKE, None) == INVALID  # self range past N
    assert c(FAKE, 1, 100, FAKE, None, 10, 2, 64, None, 0, 0, FAKE, None) == INVALID   # no weights
    assert c(None, 1, 0, None, None, 0, 2, 64, None, 0, 0, None, None) == OK
    m = lib.moe_combine_multi
    assert m(FAKE, 1, 100, FAKE, FAKE, 10, 2, 12, None, 0, 0, FAKE, None) == INVALID  # 24-byte rows
    # the scatter's self range is checked even without shared rows (it decides which tokens are left)
    assert m(FAKE, 1, 100, FAKE, FAKE, 10, 2, 64, None, 5, 20, FAKE, None) == INVALID
    assert m(FAKE, 1, 100, FAKE, FAKE, 10, 2, 64, None, 6, 5, FAKE, None) == INVALID
    assert m(None, 1, 0, None, None, 0, 2, 64, None, 0, 0, None, None) == OK


def _gd(**kw):
    base = dict(n_groups=4, hidden=256, inter=128, act_dt=1, w_dt=1, layout=0, n_src=1, capacity=0, rows=64, stage=0)
    shared = kw.pop("shared", None)
    base.update(kw)
    d = GGemmDesc(**base)
    if shared is not None:
        d.shared = ctypes.pointer(shared)
    return d


def test_grouped_gemm_workspace_and_errors(lib):
    ws = lib.moe_grouped_gemm_workspace(ctypes.byref(_gd()))
    assert ws >= 64 * 128 * 2
    assert lib.moe_grouped_gemm_workspace(ctypes.byref(_gd(act_dt=0, w_dt=0))) >= 64 * 128 * 4
    assert lib.moe_grouped_gemm_workspace(ctypes.byref(_gd(layout=1, n_src=4, capacity=8, rows=100))) == 0
    f = lib.moe_grouped_gemm
    ptrs = [FAKE] * 8
    assert f(ctypes.byref(_gd(hidden=200)), *ptrs, FAKE, ws, None) == UNSUPPORTED          # H % 128
    assert f(ctypes.byref(_gd(act_dt=0, w_dt=1)), *ptrs, FAKE, ws, None) == UNSUPPORTED    # f32 x bf16
    assert f(ctypes.byref(_gd(act_dt=1, w_dt=0)), *ptrs, FAKE, ws, None) == UNSUPPORTED    # bf16 x f32
    assert f(ctypes.byref(_gd(n_groups=600)), *ptrs, FAKE, ws, None) == UNSUPPORTED
    assert f(ctypes.byref(_gd(stage=5)), *ptrs, FAKE, ws, None) == INVALID
    assert f(ctypes.byref(_gd()), *ptrs, FAKE, ws - 1, None) == WORKSPACE
    assert f(ctypes.byref(_gd()), *ptrs, None, ws, None) == WORKSPACE
    # compact needs group_off, padded needs counts, fp8 needs scales
    assert f(ctypes.byref(_gd()), FAKE, FAKE, None, *([FAKE] * 5), FAKE, ws, None) == INVALID
    pd = _gd(layout=1, n_src=4, capacity=4, rows=64)
    pws = lib.moe_grouped_gemm_workspace(ctypes.byref(pd))
    assert f(ctypes.byref(pd), FAKE, None, FAKE, *([FAKE] * 5), FAKE, pws, None) == INVALID
    fd = _gd(w_dt=2)
    assert f(ctypes.byref(fd), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, ws, None) == INVALID
    assert f(ctypes.byref(_gd(rows=0)), *ptrs, FAKE, ws, None) == OK   # nothing to do


def test_grouped_gemm_gather_validation(lib):
    f = lib.moe_grouped_gemm
    ws = lib.moe_grouped_gemm_workspace(ctypes.byref(_gd()))
    ptrs = [FAKE] * 8
    assert f(ctypes.byref(_gd(a_rows=FAKE.value, a_nrows=0)), *ptrs, FAKE, ws, None) == INVALID   # no input rows
    wsf = lib.moe_grouped_gemm_workspace(ctypes.byref(_gd(act_dt=0, w_dt=0)))
    assert f(ctypes.byref(_gd(act_dt=0, w_dt=0, a_rows=FAKE.value, a_nrows=10)), *ptrs, FAKE, wsf,
             None) == UNSUPPORTED                                                                   # f32
    assert f(ctypes.byref(_gd(a_rows=FAKE.value, a_nrows=10, a_layout=1)), *ptrs, FAKE, ws, None) == UNSUPPORTED
    assert f(ctypes.byref(_gd(a_rows=FAKE.value, a_nrows=(1 << 23) + 1)), *ptrs, FAKE, ws, None) == UNSUPPORTED  # > 4 GiB
    assert f(ctypes.byref(_gd(rows=0, a_rows=FAKE.value, a_nrows=10)), *ptrs, FAKE, ws, None) == OK


def test_grouped_gemm_shared_expert_validation(lib):
    from combine_router_softmax_amd import SharedExpert
    f = lib.moe_grouped_gemm
    base = lib.moe_grouped_gemm_workspace(ctypes.byref(_gd()))
    se = SharedExpert(FAKE.value, 32, FAKE.value, FAKE.value, None, None, FAKE.value)
    ws = lib.moe_grouped_gemm_workspace(ctypes.byref(_gd(shared=se)))
    assert ws >= base + 32 * 128 * 2
    assert lib.moe_grouped_gemm_workspace(ctypes.byref(_gd(shared=SharedExpert(None, -1)))) == 0
    ptrs = [FAKE] * 8
    assert f(ctypes.byref(_gd(shared=se)), *ptrs, FAKE, base, None) == WORKSPACE      # sized without it
    bad = SharedExpert(None, 32, FAKE.value, FAKE.value, None, None, FAKE.value)
    assert f(ctypes.byref(_gd(shared=bad)), *ptrs, FAKE, ws, None) == INVALID        # no input rows
    fp8 = SharedExpert(FAKE.value, 32, FAKE.value, FAKE.value, None, None, FAKE.value)
    assert f(ctypes.byref(_gd(w_dt=2, shared=fp8)), *ptrs, FAKE, ws, None) == INVALID  # fp8 without scales
    assert f(ctypes.byref(_gd(n_groups=0, shared=SharedExpert(None, 0))), *ptrs, FAKE, ws, None) == OK


def test_grouped_gemm_scatter_validation(lib):
    from combine_router_softmax_amd import Scatter
    f = lib.moe_grouped_gemm
    ws = lib.moe_grouped_gemm_workspace(ctypes.byref(_gd()))
    ptrs = [FAKE] * 8

    def d(sc, **kw):
        g = _gd(**kw)
        g.scatter = ctypes.pointer(sc)
        return g
    good = dict(row_token=FAKE.value, row_of=FAKE.value, topk_w=FAKE.value, n_tokens=10, top_k=2, n_rows=64,
                self_lo=0, self_hi=4, out=FAKE.value)
    wsf = lib.moe_grouped_gemm_workspace(ctypes.byref(_gd(act_dt=0, w_dt=0)))
    assert f(ctypes.byref(d(Scatter(**good), act_dt=0, w_dt=0)), *ptrs, FAKE, wsf, None) == UNSUPPORTED  # f32 out
    for k, v in (("row_token", None), ("row_of", None), ("topk_w", None), ("out", None), ("out", FAKE.value + 8),
                 ("top_k", 0), ("top_k", 17), ("n_tokens", -1), ("n_rows", -1), ("self_lo", 5), ("self_hi", 11)):
        bad = dict(good, **{k: v})
        assert f(ctypes.byref(d(Scatter(**bad))), *ptrs, FAKE, ws, None) == INVALID, (k, v)
    # checked only where it is used: the up stage ignores it
    bad = dict(good, out=None)
    assert f(ctypes.byref(d(Scatter(**bad), stage=1)), *ptrs, FAKE, ws - 1, None) == WORKSPACE
    assert f(ctypes.byref(d(Scatter(**good), rows=0)), *ptrs, FAKE, ws, None) == OK


def test_pack_weights_and_format_validation(lib):
    f = lib.moe_pack_weights
    assert f(4, 256, 128, 0, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED      # f32 weights are not packed
    assert f(4, 200, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED      # H % 128
    assert f(4, 256, 128, 1, FAKE, FAKE, FAKE, ctypes.c_void_p(0x200000), None) == INVALID  # in place
    assert f(4, 256, 128, 1, FAKE, None, ctypes.c_void_p(0x300000), FAKE, None) == INVALID  # pairs mismatch
    assert f(-1, 256, 128, 1, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert f(0, 256, 128, 1, None, None, None, None, None) == OK
    bad = _gd()
    bad.w_format = 7
    assert lib.moe_grouped_gemm_workspace(ctypes.byref(bad)) == 0
    badp = _gd()
    badp.policy = 3
    assert lib.moe_grouped_gemm_workspace(ctypes.byref(badp)) == 0
    bada = _gd()
    bada.a_layout = 2
    assert lib.moe_grouped_gemm_workspace(ctypes.byref(bada)) == 0
    f32b = _gd(act_dt=0, w_dt=0)
    f32b.a_layout = 1
    ws = lib.moe_grouped_gemm_workspace(ctypes.byref(f32b))
    assert lib.moe_grouped_gemm(ctypes.byref(f32b), *([FAKE] * 8), FAKE, ws, None) == UNSUPPORTED
    f32p = _gd(act_dt=0, w_dt=0)
    f32p.w_format = 1
    ws = lib.moe_grouped_gemm_workspace(ctypes.byref(f32p))
    assert lib.moe_grouped_gemm(ctypes.byref(f32p), *([FAKE] * 8), FAKE, ws, None) == UNSUPPORTED


def test_product_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "combine_router_softmax_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), fn
                assert "oracle/" not in text, fn


def test_blocked_layout_helper_matches_the_documented_formula():
    # element (r, c) at ((r / 16) * (K / 32) + c / 32) * 512 + (r % 16) * 32 + c % 32
    import numpy as np
    from util import unblock16
    R, K = 37, 96
    a = np.arange(R * K).reshape(R, K)
    R16 = (R + 15) // 16 * 16
    flat = np.full(R16 * K, -1)
    for r in range(R):
        for c in range(K):
            flat[((r // 16) * (K // 32) + c // 32) * 512 + (r % 16) * 32 + c % 32] = a[r, c]
    np.testing.assert_array_equal(unblock16(flat.reshape(R16, K), R), a)
    assert moe.blocked_rows(37) == 48 and moe.blocked_rows(48) == 48 and moe.blocked_rows(0) == 0


def test_layer_gather_rule():
    # bf16 row-major rows: the up projection gathers from the tokens and no
    # expert-row copy is allocated; blocked rows and fp32 keep the dispatch
    import torch
    from combine_router_softmax_amd.layer import MoEShare
    kw = dict(n_tokens=64, hidden=256, inter=128, n_experts=16, top_k=2, n_src=2, expert_lo=0, n_local=4,
              device="cpu")
    s = MoEShare(act_dtype=torch.bfloat16, **kw)
    assert s.gather and s.xe is None
    s = MoEShare(act_dtype=torch.bfloat16, blocked=True, **kw)
    assert not s.gather and s.xe is not None
    s = MoEShare(act_dtype=torch.bfloat16, gather=False, **kw)
    assert not s.gather and s.xe is not None
    s = MoEShare(act_dtype=torch.float32, **kw)
    assert not s.gather
    with pytest.raises(ValueError):
        MoEShare(act_dtype=torch.float32, gather=True, **kw)


# The binding checks every size a kernel relies on before anything reaches the
# library: a short buffer raises ValueError on the host (these run on CPU
# tensors; the size checks come before the placement check).
def _t(*shape, dt=None):
    import torch
    return torch.zeros(shape, dtype=dt or torch.bfloat16)


def test_binding_rejects_short_buffers(lib):
    import torch
    i32, f32 = torch.int32, torch.float32
    with pytest.raises(ValueError, match="topk_idx and topk_w"):
        moe.moe_route_topk(_t(10, 16, dt=f32), 2, topk_idx=_t(9, 2, dt=i32), topk_w=_t(10, 2, dt=f32))
    # dispatch: xe rows / width, row_of length
    with pytest.raises(ValueError, match="xe must be"):
        moe.moe_dispatch(_t(4, 64), _t(8, dt=i32), 2, 10, xe=_t(9, 64))
    with pytest.raises(ValueError, match="xe must be"):
        moe.moe_dispatch(_t(4, 64), _t(8, dt=i32), 2, 10, xe=_t(10, 32))
    with pytest.raises(ValueError, match="row_of must hold"):
        moe.moe_dispatch(_t(4, 64), _t(7, dt=i32), 2, 10, xe=_t(10, 64))
    with pytest.raises(ValueError, match="blocked_rows"):
        moe.moe_dispatch_blocked(_t(4, 64), _t(8, dt=i32), 2, 17, xe=_t(17, 64))
    # layout outputs passed in by the caller
    out = {"row_of": _t(199, dt=i32)}
    with pytest.raises(ValueError, match="row_of holds"):
        moe.moe_dispatch_layout(_t(100, 2, dt=i32), _t(5, dt=i32), 16, 0, 2, moe.COMPACT, 200, out=out)
    with pytest.raises(ValueError, match="counts holds"):
        moe.moe_dispatch_layout(_t(100, 2, dt=i32), _t(5, dt=i32), 16, 0, 2, moe.COMPACT, 200,
                                out={"counts": _t(7, dt=i32)})
    with pytest.raises(ValueError, match="row_token holds"):
        moe.moe_dispatch_layout(_t(100, 2, dt=i32), _t(5, dt=i32), 16, 0, 2, moe.COMPACT, 200,
                                out={"row_token": _t(150, dt=i32)})
    # combine: ye width, shared rows, routing lengths
    with pytest.raises(ValueError, match="ye must be"):
        moe.moe_combine(_t(10, 32), _t(8, dt=i32), _t(4, 2, dt=f32), _t(4, 64))
    with pytest.raises(ValueError, match="shared_y must be"):
        moe.moe_combine(_t(10, 64), _t(8, dt=i32), _t(4, 2, dt=f32), _t(4, 64), _t(1, 64), 0, 2)
    with pytest.raises(ValueError, match="self range"):
        moe.moe_combine(_t(10, 64), _t(8, dt=i32), _t(4, 2, dt=f32), _t(4, 64), _t(9, 64), 0, 9)
    with pytest.raises(ValueError, match="row_of and topk_w"):
        moe.moe_combine(_t(10, 64), _t(7, dt=i32), _t(4, 2, dt=f32), _t(4, 64))


def test_binding_rejects_bad_gemm_shapes(lib):
    import torch
    i32, f32 = torch.int32, torch.float32
    G, H, I = 3, 256, 128
    a, w13, w2 = _t(40, H), _t(G, 2 * I, H), _t(G, H, I)
    off = _t(G + 1, dt=i32)
    with pytest.raises(ValueError, match="w2 has shape"):
        moe.moe_grouped_gemm(a, w13, _t(G, I, H), group_off=off)
    with pytest.raises(ValueError, match="group_off must hold"):
        moe.moe_grouped_gemm(a, w13, w2, group_off=_t(G, dt=i32))
    with pytest.raises(ValueError, match="counts must hold"):
        moe.moe_grouped_gemm(_t(3 * 2 * 4, H), w13, w2, counts=_t(5, dt=i32), layout=moe.PADDED, n_src=2,
                             capacity=4)
    with pytest.raises(ValueError, match="padded layout needs"):
        moe.moe_grouped_gemm(_t(20, H), w13, w2, counts=_t(6, dt=i32), layout=moe.PADDED, n_src=2, capacity=4)
    with pytest.raises(ValueError, match="a holds"):
        moe.moe_grouped_gemm(a, w13, w2, group_off=off, rows=41)
    with pytest.raises(ValueError, match="y must be"):
        moe.moe_grouped_gemm(a, w13, w2, group_off=off, y=_t(39, H))
    with pytest.raises(ValueError, match="ws holds"):
        moe.moe_grouped_gemm(a, w13, w2, group_off=off, ws=_t(16, dt=torch.uint8))
    u8 = torch.uint8
    with pytest.raises(ValueError, match="fp8 weights need"):
        moe.moe_grouped_gemm(a, _t(G, 2 * I, H, dt=u8), _t(G, H, I, dt=u8), group_off=off)
    with pytest.raises(ValueError, match="s13 has shape"):
        moe.moe_grouped_gemm(a, _t(G, 2 * I, H, dt=u8), _t(G, H, I, dt=u8), group_off=off,
                             s13=_t(G, 2, 1, dt=f32), s2=_t(G, 2, 1, dt=f32))
    with pytest.raises(ValueError, match="shared y must be"):
        moe.moe_grouped_gemm(a, w13, w2, group_off=off,
                             shared={"a": _t(9, H), "w13": w13[:1], "w2": w2[:1], "y": _t(8, H)})
    with pytest.raises(ValueError, match="shared w2 has shape"):
        moe.moe_grouped_gemm(a, w13, w2, group_off=off,
                             shared={"a": _t(9, H), "w13": w13[:1], "w2": _t(1, I, H), "y": _t(9, H)})
    with pytest.raises(ValueError, match="w13 has shape"):
        moe.moe_pack_weights(_t(G, I, H), None, H, I)
    # right sizes on host tensors: the placement check is the one that fails
    with pytest.raises(ValueError, match="must be a device tensor"):
        moe.moe_grouped_gemm(a, w13, w2, group_off=off)
