"""Plain CPU definition of the one-GPU share of an expert-parallel MoE layer.

Test infrastructure only (see the package docstring).

Notation: ``S`` logical source ranks holding ``B_s`` tokens each, contiguous
in the global token order (``src_offsets[S+1]``); ``E`` experts, top ``K`` per
token; this GPU owns the ``L`` experts ``[expert_lo, expert_lo + L)``; ``H``
hidden size, ``I`` SwiGLU intermediate size.

Steps, in the order the pages give them:

1. route (Perplexity, "Lower latency and higher throughput with multi-node
   DeepSeek deployment", sections Expert parallelism and MoE Router): pick the
   K highest-scoring experts per token, weights from a softmax over the router
   scores, renormalised over the K picked so that combine is a weighted average;
2. dispatch layout (lehuy.net, "Decoding high-performance EP kernels",
   sections Throughput > Dispatch and Latency: send without asking; Perplexity,
   "Enabling trillion-parameter models on AWS EFA", section Send and receive
   buffers): per-expert counts, their prefix sum, and a slot per (token, k),
   either packed by expert (count-first) or in a fixed region per
   (source rank, expert) with a static address;
3. dispatch: copy each token row into its slots;
4. expert FFN per local expert (GroupGEMM section of the first page, SiLU
   activation from its Quantization section; SwiGLU form as stated below),
   plus the shared expert on the GPU's own tokens (Expert parallelism section);
5. combine (lehuy.net, section Throughput > Combine; AWS EFA page, section
   MoE all-to-all over EFA): undo the permutation and sum the expert outputs
   weighted by the router weights, then add the shared expert.

Readings where the pages are silent are stated at each function.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import dequant_blockwise

COMPACT = 0
PADDED = 1
STATUS_OVERFLOW = 1


# --------------------------------------------------------------------------- route
def route_topk(logits, top_k: int, renormalize: bool = True):
    """Top-K routing.

    Selection: experts ordered by descending fp32 logit, equal logits broken by
    the lower expert index; the first K are kept in that order. Softmax is
    monotone, so selecting on logits selects the same experts as selecting on
    softmax scores (the router page says only that top-K indices and scores
    are produced; the softmax rule and the tie order are readings).

    Weights: ``p = softmax(logits)`` over all E in float64 (max subtracted);
    ``w_k = p[idx_k] / sum_j p[idx_j]`` when ``renormalize`` else ``p[idx_k]``.

    Returns ``(idx int32 [N, K], w float64 [N, K])``.

    Pins: brute force over all orderings for E <= 5, ``np.lexsort``, K = E and
    K = 1 special cases, softmax over the selected logits (closed form),
    overflow safety at large logits (tests/test_oracle_route.py).
    """
    z = np.asarray(logits, dtype=np.float32)
    assert z.ndim == 2
    assert np.all(np.isfinite(z)), "router logits must be finite"
    N, E = z.shape
    assert 1 <= top_k <= E
    # stable sort of -logit: equal values keep ascending expert index
    order = np.argsort(-z, axis=1, kind="stable")
    idx = order[:, :top_k].astype(np.int32)

    z64 = z.astype(np.float64)
    m = z64.max(axis=1, keepdims=True) if E else np.zeros((N, 1))
    ex = np.exp(z64 - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    w = sel / sel.sum(axis=1, keepdims=True) if renormalize else sel
    return idx, w


# --------------------------------------------------------------------------- layout
def worst_case_rows(n_tokens: int, top_k: int, n_local: int) -> int:
    """Most (token, k) entries that can land on one GPU's L experts.

    A token's K experts are distinct, so at most ``min(K, L)`` of them are
    local. (The AWS EFA page, section Send and receive buffers, prints the bound
    with a max over the same two quantities; min is the attained bound, see
    the brute-force pin in tests/test_oracle_layout.py.)
    """
    return int(n_tokens) * min(int(top_k), int(n_local))


def dispatch_layout(topk_idx, src_offsets, expert_lo: int, n_local: int, layout: int, capacity: int):
    """Slots of the local (token, k) entries in the expert-grouped buffer.

    ``counts[le, s]``: entries of source s routed to local expert ``le``.

    COMPACT (count-first, ragged): rows are ordered by local expert, then by
    global token index (= source rank, then token), i.e. a stable counting sort
    of the entries by expert; ``expert_off`` is the exclusive prefix sum of the
    per-expert totals, clipped to ``capacity`` (rows available). Entries whose
    row would reach ``capacity`` are dropped and the overflow bit is set.

    PADDED (fixed rectangle): a private region of ``capacity`` rows per
    (local expert, source), expert-major: entry j of (le, s) goes to row
    ``(le * S + s) * capacity + j``; entries with ``j >= capacity`` are dropped
    and the overflow bit is set. ``expert_off[le] = le * S * capacity``.

    Entries are visited in (token, k) order. ``row_of[t*K + k]`` is the row or
    -1 (not local, or dropped); ``row_token[r]`` is the token in row r or -1.

    Pins: counts sum to N*K over the full expert range and over any split into
    EP ranges, bijection onto [0, M), stability, agreement with a stable
    ``np.argsort``, padded closed form, overflow, adversarial worst case,
    hand-worked fixture tests/golden/layout_toy.json.
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    N, K = idx.shape
    off = np.asarray(src_offsets, dtype=np.int64)
    S = len(off) - 1
    L = int(n_local)
    C = int(capacity)
    assert off[0] == 0 and off[-1] == N and np.all(np.diff(off) >= 0)
    src_of = np.repeat(np.arange(S), np.diff(off))

    counts = np.zeros((L, S), dtype=np.int64)
    for t in range(N):
        for k in range(K):
            le = idx[t, k] - expert_lo
            if 0 <= le < L:
                counts[le, src_of[t]] += 1

    row_of = np.full(N * K, -1, dtype=np.int64)
    status = 0
    if layout == COMPACT:
        R = C
        totals = counts.sum(axis=1)
        starts = np.zeros(L + 1, dtype=np.int64)
        starts[1:] = np.cumsum(totals)
        expert_off = np.minimum(starts, C)
        row_token = np.full(R, -1, dtype=np.int64)
        cursor = np.zeros(L, dtype=np.int64)
        for t in range(N):
            for k in range(K):
                le = idx[t, k] - expert_lo
                if 0 <= le < L:
                    row = starts[le] + cursor[le]
                    cursor[le] += 1
                    if row < C:
                        row_of[t * K + k] = row
                        row_token[row] = t
                    else:
                        status |= STATUS_OVERFLOW
    elif layout == PADDED:
        R = L * S * C
        expert_off = np.arange(L + 1, dtype=np.int64) * S * C
        row_token = np.full(R, -1, dtype=np.int64)
        cursor = np.zeros((L, S), dtype=np.int64)
        for t in range(N):
            s = src_of[t]
            for k in range(K):
                le = idx[t, k] - expert_lo
                if 0 <= le < L:
                    j = cursor[le, s]
                    cursor[le, s] += 1
                    if j < C:
                        row = (le * S + s) * C + j
                        row_of[t * K + k] = row
                        row_token[row] = t
                    else:
                        status |= STATUS_OVERFLOW
    else:
        raise ValueError(layout)

    return {
        "counts": counts,
        "expert_off": expert_off,
        "row_of": row_of,
        "row_token": row_token,
        "status": status,
        "rows": R,
        "layout": layout,
        "n_src": S,
        "capacity": C,
    }


def group_rows(lay: dict, g: int) -> np.ndarray:
    """Occupied rows of local expert g, in row order."""
    if lay["layout"] == COMPACT:
        return np.arange(lay["expert_off"][g], lay["expert_off"][g + 1], dtype=np.int64)
    S, C = lay["n_src"], lay["capacity"]
    parts = [np.arange((g * S + s) * C, (g * S + s) * C + min(int(lay["counts"][g, s]), C), dtype=np.int64)
             for s in range(S)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


# --------------------------------------------------------------------------- dispatch
def dispatch(x, row_of, top_k: int, n_rows: int):
    """``xe[row_of[t*K+k]] = x[t]`` for every kept entry; other rows are NaN.

    Pins: equals ``np.take(x, row_token)`` on the occupied rows.
    """
    x = np.asarray(x, dtype=np.float64)
    xe = np.full((n_rows, x.shape[1]), np.nan)
    row_of = np.asarray(row_of, dtype=np.int64)
    for e, r in enumerate(row_of):
        if r >= 0:
            xe[r] = x[e // top_k]
    return xe


# --------------------------------------------------------------------------- expert FFN
def silu(z):
    """``z * sigmoid(z)`` in float64, written to stay finite for large |z|."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu_ffn(a, w13, w2):
    """One SwiGLU expert on the rows of ``a`` (float64).

    Reading (the pages name only the SiLU activation): ``w13 [2I, H]`` holds the
    gate projection in rows ``0..I-1`` and the up projection in rows
    ``I..2I-1``; ``w2 [H, I]``; no biases;
    ``y = w2 @ (silu(w_gate @ a) * (w_up @ a))`` per row.

    Pins: identity/permutation weights with a pure-Python closed form, and a
    triple-loop brute force (tests/test_oracle_ffn.py).
    """
    a = np.asarray(a, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    I = w13.shape[0] // 2
    g = a @ w13[:I].T
    u = a @ w13[I:].T
    return (silu(g) * u) @ w2.T


def expert_weights_f64(w13, w2, s13=None, s2=None, g: int = 0):
    """float64 weights of expert g from bf16/f32 values or e4m3fn codes + scales."""
    if s13 is None:
        return np.asarray(w13[g], dtype=np.float64), np.asarray(w2[g], dtype=np.float64)
    return dequant_blockwise(w13[g], s13[g]), dequant_blockwise(w2[g], s2[g])


def grouped_ffn(xe, lay: dict, w13, w2, s13=None, s2=None):
    """Expert FFN of every occupied row: row r of expert g gets
    ``swiglu_ffn(xe[r], W_g)``; unoccupied rows stay NaN.

    This is the GroupGEMM of the first page: g groups, group i a
    ``[m_i, k] x [k, n]`` product (here two, with SwiGLU between them).
    Experts with no rows contribute nothing.
    """
    xe = np.asarray(xe, dtype=np.float64)
    H = xe.shape[1]
    ye = np.full((lay["rows"], H), np.nan)
    G = len(lay["expert_off"]) - 1
    for g in range(G):
        rows = group_rows(lay, g)
        if len(rows) == 0:
            continue
        a13, a2 = expert_weights_f64(w13, w2, s13, s2, g)
        ye[rows] = swiglu_ffn(xe[rows], a13, a2)
    return ye


# --------------------------------------------------------------------------- combine
def combine(ye, row_of, topk_w, top_k: int, out_init, shared_y=None, self_lo: int = 0, self_hi: int = 0,
            tokens=None):
    """Weighted sum back in token order (sender-side partial over local experts).

    For a token t with at least one kept entry, or with ``self_lo <= t <
    self_hi`` when a shared-expert output is given:
    ``out[t] = sum_{k ascending, row_of[t,k] >= 0} w[t,k] * ye[row_of[t,k]]
    + [t in self] * shared_y[t - self_lo]``. Every other row keeps
    ``out_init``. With ``tokens`` only those rows are computed (others copied).

    Pins: identity experts give ``(sum of local weights) * x``; with all experts
    local and renormalised weights it gives ``x``; the sum of the partial
    outputs of all EP ranges equals the whole layer (tests/test_oracle_layer.py).
    """
    out = np.array(out_init, dtype=np.float64, copy=True)
    row_of = np.asarray(row_of, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64).reshape(-1)
    N = out.shape[0]
    it = range(N) if tokens is None else tokens
    for t in it:
        t = int(t)
        in_self = shared_y is not None and self_lo <= t < self_hi
        terms = [(k, row_of[t * top_k + k]) for k in range(top_k) if row_of[t * top_k + k] >= 0]
        if not terms and not in_self:
            continue
        acc = np.zeros(out.shape[1])
        for k, r in terms:
            acc = acc + w[t * top_k + k] * np.asarray(ye[r], dtype=np.float64)
        if in_self:
            acc = acc + np.asarray(shared_y[t - self_lo], dtype=np.float64)
        out[t] = acc
    return out


# --------------------------------------------------------------------------- layer
def moe_layer(x, logits, src_offsets, top_k, expert_lo, n_local, w13, w2, s13=None, s2=None,
              shared=None, self_range=None, layout=COMPACT, capacity=None, renormalize=True,
              out_init=None):
    """The whole one-GPU share: route, layout, dispatch, FFN, shared expert, combine.

    ``shared`` is ``(w13 [1,2I,H], w2 [1,H,I], s13, s2)`` or None; it runs on the
    tokens ``self_range = (lo, hi)`` (default: source rank 0's tokens).
    ``capacity`` defaults to the worst case (compact) or ``max B_s`` (padded).
    ``out_init`` defaults to zeros. Returns a dict of every intermediate.
    """
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[0]
    off = np.asarray(src_offsets, dtype=np.int64)
    idx, w = route_topk(logits, top_k, renormalize)
    if capacity is None:
        capacity = worst_case_rows(N, top_k, n_local) if layout == COMPACT else int(np.diff(off).max(initial=0))
    lay = dispatch_layout(idx, off, expert_lo, n_local, layout, capacity)
    xe = dispatch(x, lay["row_of"], top_k, lay["rows"])
    ye = grouped_ffn(xe, lay, w13, w2, s13, s2)
    lo, hi = self_range if self_range is not None else (0, int(off[1]) if len(off) > 1 else 0)
    ys = None
    if shared is not None:
        sw13, sw2, ss13, ss2 = shared
        a13, a2 = expert_weights_f64(sw13, sw2, ss13, ss2, 0)
        ys = swiglu_ffn(x[lo:hi], a13, a2)
    init = np.zeros_like(x) if out_init is None else out_init
    out = combine(ye, lay["row_of"], w, top_k, init, ys, lo, hi)
    return {"topk_idx": idx, "topk_w": w, "layout": lay, "xe": xe, "ye": ye, "ys": ys, "out": out,
            "self_range": (lo, hi)}
