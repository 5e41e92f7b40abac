"""On-the-fly 1x128 activation quantization and the fp8 x fp8 expert FFN (W8A8).

Test infrastructure only (see the package docstring).

What the pages fix (Perplexity, "Lower latency and higher throughput with
multi-node DeepSeek deployment", section Quantization): weights are quantized
statically with one scale per 128 x 128 tile, activations on the fly with one
scale per 128-element vector; the scales of an (M, K) x (K, N) product are an
M x K/128 and a K/128 x N/128 matrix, i.e. they enter only along K, so the
product is a sum over 128-wide K blocks of (activation scale x weight scale x
the block's fp8 dot product); the SiLU kernel quantizes its output the same way
(per 128-element block, after a max reduction). The dispatch payload is fp8
and the return path bf16 (lehuy.net, "Decoding high-performance EP kernels",
section Latency: send without asking; Perplexity, "Enabling trillion-parameter
models on AWS EFA", section Evaluation).

Readings (the pages give neither the scale rule nor the rounding):
  * the scale of a 128-element block is its largest magnitude / 448 (the
    largest OCP e4m3fn value), computed in fp32; where that is 0 (an all-zero
    block, or a largest magnitude below 224 x 2^-149, whose quotient by
    448 rounds to 0) the scale is 1 (the same rule as the weight tiles), so every
    code stays finite;
  * codes are round-to-nearest-even of value / scale, computed in fp32 and
    clamped to +-448 first;
  * values are quantized from their fp32 form: the token rows are bf16 (exact
    in fp32); the SiLU output is held in fp32 (what the kernel accumulates)
    before it is quantized.

Pins: tests/test_oracle_w8a8.py (every code reproduced by the quantizer,
the scale's closed form, hand-derived ties, the half-step error bound, the
block-scaled product against a float64 matmul of the dequantized operands,
the whole FFN within the fp8 bound of the unquantized one).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3fn_table
from .moe_oracle import COMPACT, combine, dispatch_layout, route_topk, silu, worst_case_rows
from .moe_oracle import group_rows as _group_rows

E4M3_MAX = 448.0
_TABLE = e4m3fn_table()
# the finite non-negative codes 0x00..0x7E in increasing value order
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALS = _TABLE[:0x7F]


def encode_e4m3fn_rne(v) -> np.ndarray:
    """e4m3fn code nearest to each float32 value in [-448, 448], ties to the
    even code (mantissa bit 0 clear), from the table of code values."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    assert np.all(a <= E4M3_MAX), "clamp to +-448 before encoding"
    hi = np.searchsorted(_POS_VALS, a, side="left")      # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(a == _POS_VALS[hi], _POS_CODES[hi], code).astype(np.uint8)
    neg = np.signbit(v) & (code != 0)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_1x128(a):
    """Quantize each 128-element block of each row of ``a`` [R, K] (K a
    multiple of 128; values taken as fp32).

    Returns ``(codes uint8 [R, K], scales float32 [R, K / 128])`` with
    ``scale = fp32(max |block|) / 448`` (1 where that is 0) and
    ``code = RNE(clamp(fp32(value) / scale, +-448))``.
    """
    a32 = np.asarray(a, dtype=np.float32)
    R, K = a32.shape
    assert K % 128 == 0
    blk = a32.reshape(R, K // 128, 128)
    amax = np.abs(blk).max(axis=2)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (blk / scale[:, :, None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = encode_e4m3fn_rne(y).reshape(R, K)
    return codes, scale


def dequant_1x128(codes, scales) -> np.ndarray:
    """float64 values of 1x128-quantized rows: code value x its block's scale."""
    q = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.float64)
    return _TABLE[q] * np.repeat(s, 128, axis=1)


def gemm_w8a8(aq, a_s, wq, w_s) -> np.ndarray:
    """``out[r, n] = sum_kb a_s[r, kb] * w_s[n / 128, kb] * sum_{k in kb} a[r, k] w[n, k]``
    over fp8 codes: activations ``aq [R, K]`` with scales ``a_s [R, K/128]``,
    weights ``wq [N, K]`` with 128 x 128 tile scales ``w_s [N/128, K/128]``.
    Each 128-wide block's dot products are exact in float64 (products of two
    e4m3 values need 8 significant bits). Returns float64 ``[R, N]``."""
    aq = np.asarray(aq, dtype=np.uint8)
    wq = np.asarray(wq, dtype=np.uint8)
    a_s = np.asarray(a_s, dtype=np.float64)
    w_s = np.asarray(w_s, dtype=np.float64)
    R, K = aq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and K % 128 == 0 and N % 128 == 0
    out = np.zeros((R, N))
    ws_rows = np.repeat(w_s, 128, axis=0)  # [N, K/128]
    for kb in range(K // 128):
        sl = slice(128 * kb, 128 * (kb + 1))
        part = _TABLE[aq[:, sl]] @ _TABLE[wq[:, sl]].T
        out += a_s[:, kb][:, None] * ws_rows[:, kb][None, :] * part
    return out


def w8a8_ffn_q(xq, xs, w13q, s13, w2q, s2):
    """One SwiGLU expert (same form as ``swiglu_ffn``: gate rows ``0..I-1`` and
    up rows ``I..2I-1`` of ``w13``) on rows that arrive already quantized:
    block-scaled up product, ``h = silu(g) * u`` taken to fp32 and quantized
    1 x 128 (the SiLU step's quantization), block-scaled down product.
    Returns float64 ``[R, H]``."""
    gu = gemm_w8a8(xq, xs, w13q, s13)
    inter = gu.shape[1] // 2
    h = (silu(gu[:, :inter]) * gu[:, inter:]).astype(np.float32)
    hq, hs = quantize_1x128(h)
    return gemm_w8a8(hq, hs, w2q, s2)


def w8a8_ffn(x, w13q, s13, w2q, s2):
    """``w8a8_ffn_q`` on rows quantized 1 x 128 from their fp32 values."""
    xq, xs = quantize_1x128(x)
    return w8a8_ffn_q(xq, xs, w13q, s13, w2q, s2)


def moe_layer_w8a8(x, logits, src_offsets, top_k, expert_lo, n_local, w13q, w2q, s13, s2,
                   shared=None, self_range=None, layout=COMPACT, capacity=None, renormalize=True,
                   out_init=None):
    """The one-GPU share with an fp8 payload: route and layout as ``moe_layer``;
    every token row is quantized 1 x 128 once at its source, the dispatched
    rows carry its codes and scales, each expert runs ``w8a8_ffn_q``, the
    shared expert runs ``w8a8_ffn_q`` on the own tokens' codes, and the expert
    outputs return for the weighted combine (bf16 on the return path; the
    oracle keeps them in float64). Weights are e4m3fn codes with 128 x 128
    scales (``shared = (w13q [1,2I,H], w2q [1,H,I], s13, s2)``).

    Returns a dict of the intermediates, as ``moe_layer`` does, plus ``xq``
    and ``xs`` (the quantized token rows) and ``xe_q`` / ``xe_s`` (the
    dispatched codes and scales; unoccupied rows hold code 0 and scale NaN).
    """
    x32 = np.asarray(x, dtype=np.float32)
    N = x32.shape[0]
    off = np.asarray(src_offsets, dtype=np.int64)
    idx, w = route_topk(logits, top_k, renormalize)
    if capacity is None:
        capacity = worst_case_rows(N, top_k, n_local) if layout == COMPACT else int(np.diff(off).max(initial=0))
    lay = dispatch_layout(idx, off, expert_lo, n_local, layout, capacity)
    xq, xs = quantize_1x128(x32)
    R = lay["rows"]
    xe_q = np.zeros((R, x32.shape[1]), dtype=np.uint8)
    xe_s = np.full((R, xs.shape[1]), np.nan, dtype=np.float32)
    for e, r in enumerate(np.asarray(lay["row_of"], dtype=np.int64)):
        if r >= 0:
            xe_q[r] = xq[e // top_k]
            xe_s[r] = xs[e // top_k]
    ye = np.full((R, x32.shape[1]), np.nan)
    G = len(lay["expert_off"]) - 1
    for g in range(G):
        rows = _group_rows(lay, g)
        if len(rows):
            ye[rows] = w8a8_ffn_q(xe_q[rows], xe_s[rows], w13q[g], s13[g], w2q[g], s2[g])
    lo, hi = self_range if self_range is not None else (0, int(off[1]) if len(off) > 1 else 0)
    ys = None
    if shared is not None:
        sw13, sw2, ss13, ss2 = shared
        ys = w8a8_ffn_q(xq[lo:hi], xs[lo:hi], sw13[0], ss13[0], sw2[0], ss2[0])
    init = np.zeros(x32.shape) if out_init is None else out_init
    out = combine(ye, lay["row_of"], w, top_k, init, ys, lo, hi)
    return {"topk_idx": idx, "topk_w": w, "layout": lay, "xq": xq, "xs": xs, "xe_q": xe_q, "xe_s": xe_s,
            "ye": ye, "ys": ys, "out": out, "self_range": (lo, hi)}
