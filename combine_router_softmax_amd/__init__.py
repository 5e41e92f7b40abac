"""Python binding of ``libmoe.so``, the gfx950 MoE-layer share.

Argument marshalling only: each function checks tensor placement, shape and
dtype, allocates any output the caller did not pass (PyTorch device memory),
and calls the C entry point of the same name on the current HIP stream. Every
step of the computation runs in the library's HIP kernels; there is no other
implementation to fall back to, and a missing library raises
``MoeLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = [
    "COMPACT", "PADDED", "GG_FULL", "GG_UP", "GG_DOWN", "STATUS_OVERFLOW", "MoeError", "MoeLibraryMissing",
    "lib", "lib_path", "moe_route_topk", "moe_dispatch_layout", "moe_layout_rows", "moe_dispatch",
    "moe_grouped_gemm", "moe_combine", "moe_abi_version", "moe_pack_weights", "W_ROWMAJOR", "W_PACKED",
    "moe_quantize_1x128", "moe_dispatch_fp8",
]

COMPACT, PADDED = 0, 1
W_ROWMAJOR, W_PACKED = 0, 1
GG_FULL, GG_UP, GG_DOWN = 0, 1, 2
GEMM_AUTO, GEMM_WIDE, GEMM_STREAM_K = 0, 1, 2
ACT_ROWS, ACT_BLOCKED16 = 0, 1
STATUS_OVERFLOW = 1
ABI_VERSION = 3  # struct layouts of moe.h this binding mirrors
_F32, _BF16, _FP8 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(_HERE, "libmoe.so")
_lib = None


class MoeError(RuntimeError):
    pass


class MoeLibraryMissing(ImportError):
    pass


class LayoutDesc(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int), ("top_k", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("n_src", ctypes.c_int), ("expert_lo", ctypes.c_int), ("n_local", ctypes.c_int),
                ("layout", ctypes.c_int), ("capacity", ctypes.c_int)]


class SharedExpert(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("rows", ctypes.c_int), ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("s13", ctypes.c_void_p), ("s2", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("a_scales", ctypes.c_void_p)]


class Scatter(ctypes.Structure):
    _fields_ = [("row_token", ctypes.c_void_p), ("row_of", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("n_tokens", ctypes.c_int), ("top_k", ctypes.c_int), ("n_rows", ctypes.c_int64),
                ("self_lo", ctypes.c_int), ("self_hi", ctypes.c_int), ("out", ctypes.c_void_p)]


class GGemmDesc(ctypes.Structure):
    _fields_ = [("n_groups", ctypes.c_int), ("hidden", ctypes.c_int), ("inter", ctypes.c_int),
                ("act_dt", ctypes.c_int), ("w_dt", ctypes.c_int), ("layout", ctypes.c_int),
                ("n_src", ctypes.c_int), ("capacity", ctypes.c_int), ("rows", ctypes.c_int64),
                ("stage", ctypes.c_int), ("shared", ctypes.POINTER(SharedExpert)), ("w_format", ctypes.c_int),
                ("policy", ctypes.c_int), ("a_layout", ctypes.c_int), ("a_rows", ctypes.c_void_p),
                ("a_nrows", ctypes.c_int64), ("a_scales", ctypes.c_void_p),
                ("scatter", ctypes.POINTER(Scatter))]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "moe_abi_version": (_I, []),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_route_topk": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_layout_rows": (_I64, [ctypes.POINTER(LayoutDesc)]),
    "moe_dispatch_layout_workspace": (_SZ, [ctypes.POINTER(LayoutDesc)]),
    "moe_dispatch_layout": (_I, [ctypes.POINTER(LayoutDesc), _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_dispatch_layout_noalloc": (_I, [ctypes.POINTER(LayoutDesc), _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch": (_I, [_P, _I, _I, _I, _I, _P, _I64, _P, _P]),
    "moe_dispatch_blocked": (_I, [_P, _I, _I, _I, _I, _P, _I64, _P, _P]),
    "moe_quantize_1x128": (_I, [_P, _I, _I64, _I, _P, _P, _P]),
    "moe_dispatch_fp8": (_I, [_P, _P, _I, _I, _I, _P, _I64, _P, _P, _P]),
    "moe_grouped_gemm_workspace": (_SZ, [ctypes.POINTER(GGemmDesc)]),
    "moe_grouped_gemm": (_I, [ctypes.POINTER(GGemmDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_combine": (_I, [_P, _I, _I64, _P, _P, _I, _I, _I, _P, _I, _I, _P, _P]),
    "moe_combine_multi": (_I, [_P, _I, _I64, _P, _P, _I, _I, _I, _P, _I, _I, _P, _P]),
    "moe_pack_weights": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P]),
}


def lib_path() -> str:
    return _LIB_FILE


def lib():
    """The loaded library (ctypes), loading it on first use."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_FILE):
            raise MoeLibraryMissing(
                f"{_LIB_FILE} is not built; run `python combine_router_softmax_amd/build.py` "
                "(there is no CPU fallback)")
        l = ctypes.CDLL(_LIB_FILE)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        v = int(l.moe_abi_version())
        if v != ABI_VERSION:
            raise MoeError(f"{_LIB_FILE} has ABI version {v}, this binding expects {ABI_VERSION}; rebuild it")
        _lib = l
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        raise MoeError(f"{what}: {msg} (status {status})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    """Contiguity and dtype (placement is checked by _on_gpu right before the
    call, after every size check)."""
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def _need(ok: bool, msg: str):
    """Host-side size check: a short buffer must never reach a kernel."""
    if not ok:
        raise ValueError(msg)


def _shape_is(t: torch.Tensor, shape, name: str):
    _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _act_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return _F32
    if dt == torch.bfloat16:
        return _BF16
    raise ValueError(f"unsupported activation dtype {dt}")


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


# --------------------------------------------------------------------------- route
def moe_route_topk(logits: torch.Tensor, top_k: int, renormalize: bool = True,
                   topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None):
    """Top-K experts per token and their (renormalised) softmax weights."""
    _dev(logits, "logits", torch.float32)
    N, E = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty((N, top_k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((N, top_k), dtype=torch.float32, device=logits.device)
    _dev(topk_idx, "topk_idx", torch.int32)
    _dev(topk_w, "topk_w", torch.float32)
    _need(logits.dim() == 2, "logits must be [N, E]")
    _need(topk_idx.numel() == N * top_k and topk_w.numel() == N * top_k, "topk_idx and topk_w must hold N * top_k")
    _on_gpu(logits=logits, topk_idx=topk_idx, topk_w=topk_w)
    _check(lib().moe_route_topk(_ptr(logits), N, E, top_k, int(bool(renormalize)), _ptr(topk_idx), _ptr(topk_w),
                                _stream()), "moe_route_topk")
    return topk_idx, topk_w


# --------------------------------------------------------------------------- layout
def _layout_desc(n_tokens, top_k, n_experts, n_src, expert_lo, n_local, layout, capacity) -> LayoutDesc:
    return LayoutDesc(n_tokens, top_k, n_experts, n_src, expert_lo, n_local, layout, capacity)


def moe_layout_rows(n_tokens, top_k, n_experts, n_src, expert_lo, n_local, layout, capacity) -> int:
    d = _layout_desc(n_tokens, top_k, n_experts, n_src, expert_lo, n_local, layout, capacity)
    r = int(lib().moe_layout_rows(ctypes.byref(d)))
    if r < 0:
        raise MoeError("moe_layout_rows: invalid descriptor")
    return r


def moe_dispatch_layout(topk_idx: torch.Tensor, src_offsets: torch.Tensor, n_experts: int, expert_lo: int,
                        n_local: int, layout: int, capacity: int, out: Optional[dict] = None) -> dict:
    """Counts, offsets and a slot per (token, k). ``out`` may hold preallocated
    ``counts, expert_off, row_of, row_token, status, ws`` tensors."""
    _dev(topk_idx, "topk_idx", torch.int32)
    _dev(src_offsets, "src_offsets", torch.int32)
    N, K = topk_idx.shape
    S = src_offsets.numel() - 1
    d = _layout_desc(N, K, n_experts, S, expert_lo, n_local, layout, capacity)
    R = int(lib().moe_layout_rows(ctypes.byref(d)))
    if R < 0:
        raise MoeError("moe_dispatch_layout: invalid descriptor")
    wsb = int(lib().moe_dispatch_layout_workspace(ctypes.byref(d)))
    dev = topk_idx.device
    o = dict(out) if out else {}
    shapes = {"counts": ((n_local, S), torch.int32), "expert_off": ((n_local + 1,), torch.int32),
              "row_of": ((N * K,), torch.int32), "row_token": ((max(R, 1),), torch.int32),
              "status": ((1,), torch.int32), "ws": ((max(wsb, 256),), torch.uint8)}
    for k, (shape, dt) in shapes.items():
        if k not in o:   # allocate only what the caller did not bring
            o[k] = torch.empty(shape, dtype=dt, device=dev)
    for k in ("counts", "expert_off", "row_of", "row_token", "status"):
        _dev(o[k], k, torch.int32)
    _dev(o["ws"], "ws")
    for k, (shape, _) in shapes.items():
        need = int(np.prod(shape))
        _need(o[k].numel() * o[k].element_size() >= need * (1 if k == "ws" else 4),
              f"{k} holds {o[k].numel()} elements, fewer than the {need} the layout writes")
    _on_gpu(topk_idx=topk_idx, src_offsets=src_offsets, **{k: o[k] for k in shapes})
    _check(lib().moe_dispatch_layout(ctypes.byref(d), _ptr(topk_idx), _ptr(src_offsets), _ptr(o["counts"]),
                                     _ptr(o["expert_off"]), _ptr(o["row_of"]), _ptr(o["row_token"]),
                                     _ptr(o["status"]), _ptr(o["ws"]), o["ws"].numel(), _stream()),
           "moe_dispatch_layout")
    o["rows"] = R
    return o


def moe_dispatch_layout_noalloc(topk_idx: torch.Tensor, src_offsets: torch.Tensor, n_experts: int, expert_lo: int,
                                n_local: int, layout: int, capacity: int, out: Optional[dict] = None) -> dict:
    """moe_dispatch_layout without a workspace argument: the library's fixed
    per-GPU scratch array serves instead (calls that overlap on one GPU race).
    ``out`` may hold preallocated ``counts, expert_off, row_of, row_token,
    status``; the C call itself allocates nothing."""
    _dev(topk_idx, "topk_idx", torch.int32)
    _dev(src_offsets, "src_offsets", torch.int32)
    N, K = topk_idx.shape
    S = src_offsets.numel() - 1
    d = _layout_desc(N, K, n_experts, S, expert_lo, n_local, layout, capacity)
    R = int(lib().moe_layout_rows(ctypes.byref(d)))
    if R < 0:
        raise MoeError("moe_dispatch_layout_noalloc: invalid descriptor")
    dev = topk_idx.device
    o = dict(out) if out else {}
    shapes = {"counts": (n_local, S), "expert_off": (n_local + 1,), "row_of": (N * K,), "row_token": (max(R, 1),),
              "status": (1,)}
    for k, shape in shapes.items():
        if k not in o:
            o[k] = torch.empty(shape, dtype=torch.int32, device=dev)
        _dev(o[k], k, torch.int32)
        _need(o[k].numel() >= int(np.prod(shape)), f"{k} holds {o[k].numel()} elements, fewer than {np.prod(shape)}")
    _on_gpu(topk_idx=topk_idx, src_offsets=src_offsets, **{k: o[k] for k in shapes})
    _check(lib().moe_dispatch_layout_noalloc(ctypes.byref(d), _ptr(topk_idx), _ptr(src_offsets), _ptr(o["counts"]),
                                             _ptr(o["expert_off"]), _ptr(o["row_of"]), _ptr(o["row_token"]),
                                             _ptr(o["status"]), _stream()), "moe_dispatch_layout_noalloc")
    o["rows"] = R
    return o


# --------------------------------------------------------------------------- dispatch
def moe_dispatch(x: torch.Tensor, row_of: torch.Tensor, top_k: int, n_rows: int,
                 xe: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Copy token rows into their expert-grouped slots (unused rows untouched)."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _dev(row_of, "row_of", torch.int32)
    N, H = x.shape
    if xe is None:
        xe = torch.empty((n_rows, H), dtype=x.dtype, device=x.device)
    _dev(xe, "xe", x.dtype)
    _need(xe.dim() == 2 and xe.shape[1] == H and xe.shape[0] >= n_rows, f"xe must be [>= {n_rows}, {H}]")
    _need(row_of.numel() >= N * top_k, f"row_of must hold N * top_k = {N * top_k} entries")
    _on_gpu(x=x, row_of=row_of, xe=xe)
    _check(lib().moe_dispatch(_ptr(x), _act_code(x.dtype), N, H, top_k, _ptr(row_of), n_rows, _ptr(xe), _stream()),
           "moe_dispatch")
    return xe


def moe_quantize_1x128(x: torch.Tensor, xq: Optional[torch.Tensor] = None, xs: Optional[torch.Tensor] = None):
    """fp8 payload of token rows: e4m3fn codes ``xq`` (uint8 [N, H]) and one
    float32 scale per 128 columns ``xs`` ([N, H / 128])."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    _need(x.dim() == 2, "x must be [N, H]")
    N, H = x.shape
    _need(H % 128 == 0, f"hidden {H} must be a multiple of 128")
    if xq is None:
        xq = torch.empty((N, H), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = torch.empty((N, H // 128), dtype=torch.float32, device=x.device)
    _dev(xq, "xq", torch.uint8)
    _dev(xs, "xs", torch.float32)
    _need(xq.dim() == 2 and xq.shape[1] == H and xq.shape[0] >= N, f"xq must be [>= {N}, {H}]")
    _need(xs.dim() == 2 and xs.shape[1] == H // 128 and xs.shape[0] >= N, f"xs must be [>= {N}, {H // 128}]")
    _on_gpu(x=x, xq=xq, xs=xs)
    _check(lib().moe_quantize_1x128(_ptr(x), _act_code(x.dtype), N, H, _ptr(xq), _ptr(xs), _stream()),
           "moe_quantize_1x128")
    return xq, xs


def moe_dispatch_fp8(xq: torch.Tensor, xs: torch.Tensor, row_of: torch.Tensor, top_k: int, n_rows: int,
                     xeq: Optional[torch.Tensor] = None, xes: Optional[torch.Tensor] = None):
    """Copy fp8 payload rows (codes and scales) into their expert-grouped slots."""
    _dev(xq, "xq", torch.uint8)
    _dev(xs, "xs", torch.float32)
    _dev(row_of, "row_of", torch.int32)
    _need(xq.dim() == 2, "xq must be [N, H]")
    N, H = xq.shape
    _need(H % 128 == 0, f"hidden {H} must be a multiple of 128")
    _shape_is(xs, (N, H // 128), "xs")
    if xeq is None:
        xeq = torch.empty((n_rows, H), dtype=torch.uint8, device=xq.device)
    if xes is None:
        xes = torch.empty((n_rows, H // 128), dtype=torch.float32, device=xq.device)
    _dev(xeq, "xeq", torch.uint8)
    _dev(xes, "xes", torch.float32)
    _need(xeq.dim() == 2 and xeq.shape[1] == H and xeq.shape[0] >= n_rows, f"xeq must be [>= {n_rows}, {H}]")
    _need(xes.dim() == 2 and xes.shape[1] == H // 128 and xes.shape[0] >= n_rows,
          f"xes must be [>= {n_rows}, {H // 128}]")
    _need(row_of.numel() >= N * top_k, f"row_of must hold N * top_k = {N * top_k} entries")
    _on_gpu(xq=xq, xs=xs, row_of=row_of, xeq=xeq, xes=xes)
    _check(lib().moe_dispatch_fp8(_ptr(xq), _ptr(xs), N, H, top_k, _ptr(row_of), n_rows, _ptr(xeq), _ptr(xes),
                                  _stream()), "moe_dispatch_fp8")
    return xeq, xes


def blocked_rows(n_rows: int) -> int:
    """Rows a 16-row blocked buffer of n_rows rows holds."""
    return (n_rows + 15) // 16 * 16


def moe_dispatch_blocked(x: torch.Tensor, row_of: torch.Tensor, top_k: int, n_rows: int,
                         xe: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Copy token rows into their expert-grouped slots in the 16-row blocked
    layout (xe [blocked_rows(n_rows), H]; unused rows untouched)."""
    _dev(x, "x", torch.bfloat16)
    _dev(row_of, "row_of", torch.int32)
    N, H = x.shape
    if xe is None:
        xe = torch.empty((blocked_rows(n_rows), H), dtype=x.dtype, device=x.device)
    _dev(xe, "xe", x.dtype)
    _need(xe.dim() == 2 and xe.shape[1] == H and xe.shape[0] >= blocked_rows(n_rows),
          f"xe must be [>= blocked_rows({n_rows}), {H}]")
    _need(row_of.numel() >= N * top_k, f"row_of must hold N * top_k = {N * top_k} entries")
    _on_gpu(x=x, row_of=row_of, xe=xe)
    _check(lib().moe_dispatch_blocked(_ptr(x), _act_code(x.dtype), N, H, top_k, _ptr(row_of), n_rows, _ptr(xe),
                                      _stream()), "moe_dispatch_blocked")
    return xe


# --------------------------------------------------------------------------- grouped GEMM
_W_CODE = {torch.float32: _F32, torch.bfloat16: _BF16, torch.uint8: _FP8, torch.float8_e4m3fn: _FP8}


def gemm_desc(n_groups, hidden, inter, act_dtype, w_dtype, layout, n_src, capacity, rows, stage=GG_FULL,
              shared: "SharedExpert | None" = None, w_format: int = W_ROWMAJOR, policy: int = 0,
              a_layout: int = ACT_ROWS):
    w_code = _W_CODE[w_dtype]
    a_code = _FP8 if act_dtype in (torch.uint8, torch.float8_e4m3fn) else _act_code(act_dtype)
    d = GGemmDesc(n_groups, hidden, inter, a_code, w_code, layout, n_src, capacity, rows, stage)
    d.w_format = w_format
    d.policy = policy
    d.a_layout = a_layout
    if shared is not None:
        d.shared = ctypes.pointer(shared)
    return d


def shared_expert(a: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, y: Optional[torch.Tensor],
                  s13: Optional[torch.Tensor] = None, s2: Optional[torch.Tensor] = None,
                  a_scales: Optional[torch.Tensor] = None) -> SharedExpert:
    """Descriptor of the shared expert run inside a moe_grouped_gemm call
    (W8A8: ``a`` holds e4m3 codes and ``a_scales`` their 1 x 128 scales)."""
    _dev(a, "shared a")
    _dev(w13, "shared w13")
    _dev(w2, "shared w2")
    _need(a.dim() == 2 and w13.dim() == 3 and w13.shape[0] == 1 and w13.shape[2] == a.shape[1],
          "shared expert: a must be [B, H] and w13 [1, 2I, H]")
    B, H = a.shape
    I = w13.shape[1] // 2
    _shape_is(w2, (1, H, I), "shared w2")
    w8a8 = a.dtype == torch.uint8
    if y is not None:
        _dev(y, "shared y", torch.bfloat16 if w8a8 else a.dtype)
        _need(y.dim() == 2 and y.shape[1] == H and y.shape[0] >= B, f"shared y must be [>= {B}, {H}]")
    if w8a8:
        _need(a_scales is not None, "W8A8 shared rows need a_scales")
        _dev(a_scales, "shared a_scales", torch.float32)
        _need(a_scales.dim() == 2 and a_scales.shape[1] == H // 128 and a_scales.shape[0] >= B,
              f"shared a_scales must be [>= {B}, {H // 128}]")
    if s13 is not None or s2 is not None:
        _need(s13 is not None and s2 is not None, "fp8 shared weights need both scale tensors")
        _dev(s13, "shared s13", torch.float32)
        _dev(s2, "shared s2", torch.float32)
        _shape_is(s13, (1, 2 * I // 128, H // 128), "shared s13")
        _shape_is(s2, (1, H // 128, I // 128), "shared s2")
    return SharedExpert(a.data_ptr(), a.shape[0], w13.data_ptr(), w2.data_ptr(),
                        None if s13 is None else s13.data_ptr(), None if s2 is None else s2.data_ptr(),
                        None if y is None else y.data_ptr(), None if a_scales is None else a_scales.data_ptr())


def moe_grouped_gemm_workspace(desc: GGemmDesc) -> int:
    return int(lib().moe_grouped_gemm_workspace(ctypes.byref(desc)))


def moe_grouped_gemm(a: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, *, group_off=None, counts=None,
                     s13=None, s2=None, layout: int = COMPACT, n_src: int = 1, capacity: int = 0,
                     stage: int = GG_FULL, y: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, shared: Optional[dict] = None,
                     w_format: int = W_ROWMAJOR, policy: int = 0, a_layout: int = ACT_ROWS,
                     rows: Optional[int] = None, a_rows: Optional[torch.Tensor] = None,
                     a_scales: Optional[torch.Tensor] = None, scatter: Optional[dict] = None) -> torch.Tensor:
    """SwiGLU FFN per expert over the rows each expert holds (see moe.h).

    ``scatter`` = dict(row_token, row_of, topk_w, out, n_rows[, self_lo, self_hi]):
    the down projection writes the rows of tokens with exactly one kept entry
    and no shared-expert row straight into ``out`` as their combine (y rows of
    those tokens are then not written; finish with moe_combine_multi).

    ``shared`` = dict(a, w13, w2, y[, s13, s2, a_scales]) runs the shared expert in the same launches.
    ``a_rows`` (int32 [rows], e.g. the layout's row_token) gathers routed row r
    of the up projection from row a_rows[r] of ``a``; ``rows`` is then required.
    W8A8: ``a`` is uint8 e4m3 codes with ``a_scales`` [rows of a, H / 128]
    (moe_quantize_1x128 / moe_dispatch_fp8), the weights fp8 codes with
    scales; ``y`` is bf16."""
    _dev(a, "a", (torch.float32, torch.bfloat16, torch.uint8))
    w8a8 = a.dtype == torch.uint8
    _dev(w13, "w13")
    _dev(w2, "w2")
    _need(a.dim() == 2 and w13.dim() == 3, "a must be [rows, H] and w13 [G, 2I, H]")
    R, H = a.shape
    G, I2, H2 = w13.shape
    if H2 != H or I2 % 2:
        raise ValueError("w13 must be [G, 2I, H]")
    I = I2 // 2
    _shape_is(w2, (G, H, I), "w2")
    if w13.dtype in (torch.uint8, torch.float8_e4m3fn):
        _need(s13 is not None and s2 is not None, "fp8 weights need s13 and s2")
    if s13 is not None or s2 is not None:
        _need(s13 is not None and s2 is not None, "fp8 weights need both scale tensors")
        _shape_is(s13, (G, I2 // 128, H // 128), "s13")
        _shape_is(s2, (G, H // 128, I // 128), "s2")
    if w8a8:
        _need(w13.dtype in (torch.uint8, torch.float8_e4m3fn) and s13 is not None,
              "W8A8 needs fp8 weights with their scales")
        _need(a_scales is not None, "W8A8 rows need a_scales")
        _dev(a_scales, "a_scales", torch.float32)
        _need(a_scales.dim() == 2 and a_scales.shape[1] == H // 128 and a_scales.shape[0] >= a.shape[0],
              f"a_scales must be [>= {a.shape[0]}, {H // 128}]")
    else:
        _need(a_scales is None, "a_scales belong to fp8 (uint8) activations")
    se = None
    if shared is not None:
        se = shared_expert(shared["a"], shared["w13"], shared["w2"], shared.get("y"), shared.get("s13"),
                           shared.get("s2"), shared.get("a_scales"))
    if a_rows is not None:
        if rows is None:
            raise ValueError("a gathered input needs rows (the routed row count)")
        _dev(a_rows, "a_rows", torch.int32)
        if a_rows.numel() < rows:
            raise ValueError(f"a_rows holds {a_rows.numel()} entries, fewer than rows={rows}")
        _need(a.shape[0] >= 1, "a gathered input needs at least one row to gather from")
        R = rows
    elif a_layout == ACT_BLOCKED16:
        R = a.shape[0] // 16 * 16 if rows is None else rows
        _need(a.shape[0] >= blocked_rows(R), f"blocked a must hold blocked_rows({R}) rows")
    elif rows is not None:
        _need(a.shape[0] >= rows, f"a holds {a.shape[0]} rows, fewer than rows={rows}")
        R = rows
    if layout == COMPACT:
        _need(group_off is not None and group_off.numel() >= G + 1, f"group_off must hold G + 1 = {G + 1} entries")
    else:
        _need(counts is not None and counts.numel() >= G * n_src, f"counts must hold G * n_src = {G * n_src}")
        _need(R >= G * n_src * capacity, f"the padded layout needs {G * n_src * capacity} rows, got {R}")
    desc = gemm_desc(G, H, I, a.dtype, w13.dtype, layout, n_src, capacity, R, stage, se, w_format, policy, a_layout)
    if a_rows is not None:
        desc.a_rows = a_rows.data_ptr()
        desc.a_nrows = a.shape[0]
    if w8a8:
        desc.a_scales = a_scales.data_ptr()
    sc = None
    if scatter is not None:
        rt, ro, tw, so = scatter["row_token"], scatter["row_of"], scatter["topk_w"], scatter["out"]
        _dev(rt, "scatter row_token", torch.int32)
        _dev(ro, "scatter row_of", torch.int32)
        _dev(tw, "scatter topk_w", torch.float32)
        _dev(so, "scatter out", torch.bfloat16)
        _need(so.dim() == 2 and so.shape[1] == H, f"scatter out must be [N, {H}]")
        Nt = so.shape[0]
        Kt = tw.shape[-1] if tw.dim() == 2 else 1
        _need(rt.numel() >= R, f"scatter row_token must hold rows = {R} entries")
        _need(ro.numel() >= Nt * Kt and tw.numel() >= Nt * Kt, f"scatter row_of and topk_w must hold N * K = {Nt * Kt}")
        lo, hi = int(scatter.get("self_lo", 0)), int(scatter.get("self_hi", 0))
        _need(0 <= lo <= hi <= Nt, "the scatter self range must lie inside [0, N]")
        _on_gpu(**{"scatter row_token": rt, "scatter row_of": ro, "scatter topk_w": tw, "scatter out": so})
        sc = Scatter(rt.data_ptr(), ro.data_ptr(), tw.data_ptr(), Nt, Kt, int(scatter["n_rows"]), lo, hi,
                     so.data_ptr())
        desc.scatter = ctypes.pointer(sc)
    wsb = moe_grouped_gemm_workspace(desc)
    if wsb == 0:
        raise MoeError("moe_grouped_gemm: invalid descriptor")
    if ws is None:
        ws = torch.zeros(wsb, dtype=torch.uint8, device=a.device)
    _dev(ws, "ws")
    _need(ws.numel() * ws.element_size() >= wsb, f"ws holds {ws.numel() * ws.element_size()} bytes, needs {wsb}")
    y_dtype = torch.bfloat16 if w8a8 else a.dtype
    if y is None and stage != GG_UP:
        y = torch.empty((R, H), dtype=y_dtype, device=a.device)
    if y is not None:
        _dev(y, "y", y_dtype)
        _need(y.dim() == 2 and y.shape[1] == H and y.shape[0] >= R, f"y must be [>= {R}, {H}]")
    for name, t in (("group_off", group_off), ("counts", counts)):
        if t is not None:
            _dev(t, name, torch.int32)
    for name, t in (("s13", s13), ("s2", s2)):
        if t is not None:
            _dev(t, name, torch.float32)
    _on_gpu(a=a, w13=w13, w2=w2, group_off=group_off, counts=counts, s13=s13, s2=s2, y=y, ws=ws, a_rows=a_rows,
            a_scales=a_scales)
    if shared is not None:
        _on_gpu(**{f"shared {k}": v for k, v in shared.items() if isinstance(v, torch.Tensor)})
    _check(lib().moe_grouped_gemm(ctypes.byref(desc), _ptr(a), _ptr(counts), _ptr(group_off), _ptr(w13), _ptr(w2),
                                  _ptr(s13), _ptr(s2), _ptr(y), _ptr(ws), ws.numel(), _stream()),
           "moe_grouped_gemm")
    return y


def moe_pack_weights(w13: Optional[torch.Tensor], w2: Optional[torch.Tensor], hidden: int, inter: int):
    """Packed copies of expert weights (w13 [G,2I,H], w2 [G,H,I]; bf16 or fp8 codes)."""
    ref = w13 if w13 is not None else w2
    G = ref.shape[0]
    if w13 is not None:
        _shape_is(w13, (G, 2 * inter, hidden), "w13")
    if w2 is not None:
        _shape_is(w2, (G, hidden, inter), "w2")
    out13 = None if w13 is None else torch.empty_like(_dev(w13, "w13"))
    out2 = None if w2 is None else torch.empty_like(_dev(w2, "w2"))
    _on_gpu(w13=w13, w2=w2)
    _check(lib().moe_pack_weights(G, hidden, inter, _W_CODE[ref.dtype], _ptr(w13), _ptr(w2), _ptr(out13), _ptr(out2),
                                  _stream()), "moe_pack_weights")
    return out13, out2


# --------------------------------------------------------------------------- combine
def moe_combine(ye: torch.Tensor, row_of: torch.Tensor, topk_w: torch.Tensor, out: torch.Tensor,
                shared_y: Optional[torch.Tensor] = None, self_lo: int = 0, self_hi: int = 0,
                multi: bool = False) -> torch.Tensor:
    """Router-weighted sum of each token's expert rows (+ shared expert) into
    ``out``. ``multi``: only the tokens a down-projection scatter left
    (moe_combine_multi)."""
    _dev(ye, "ye", (torch.float32, torch.bfloat16))
    _dev(row_of, "row_of", torch.int32)
    _dev(topk_w, "topk_w", torch.float32)
    _dev(out, "out", ye.dtype)
    N, H = out.shape
    K = topk_w.shape[-1] if topk_w.dim() == 2 else (topk_w.numel() // N if N else 1)
    _need(ye.dim() == 2 and ye.shape[1] == H, f"ye must be [rows, {H}]")
    _need(row_of.numel() >= N * K and topk_w.numel() >= N * K, f"row_of and topk_w must hold N * K = {N * K}")
    if shared_y is not None or multi:
        _need(0 <= self_lo <= self_hi <= N, "the self range must lie inside [0, N]")
    if shared_y is not None:
        _dev(shared_y, "shared_y", ye.dtype)
        _need(shared_y.dim() == 2 and shared_y.shape[1] == H and shared_y.shape[0] >= self_hi - self_lo,
              f"shared_y must be [>= {self_hi - self_lo}, {H}]")
    _on_gpu(ye=ye, row_of=row_of, topk_w=topk_w, out=out, shared_y=shared_y)
    fn = lib().moe_combine_multi if multi else lib().moe_combine
    _check(fn(_ptr(ye), _act_code(ye.dtype), ye.shape[0], _ptr(row_of), _ptr(topk_w), N, K, H, _ptr(shared_y),
              self_lo, self_hi, _ptr(out), _stream()), "moe_combine_multi" if multi else "moe_combine")
    return out
