"""One step of the one-GPU MoE-layer share, as a sequence of the five C-ABI calls.

Host orchestration only: buffers are allocated once (PyTorch device memory)
and every step enqueues route -> layout -> dispatch -> grouped GEMM (routed,
then shared expert) -> combine on the current stream. No host synchronisation
inside a step: the expert buffer is sized for the worst case (compact) or for
the fixed rectangle (padded), and the kernels read the real counts on the
device.

W8A8 (fp8 weights, ``w8a8=True``): the token rows are quantized 1 x 128 once
(moe_quantize_1x128, the fp8 payload), the dispatch moves codes and scales
(or the GEMM gathers them), the grouped GEMM runs fp8 x fp8 and returns bf16
rows, and the combine sums bf16 as before.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (ACT_BLOCKED16, ACT_ROWS, COMPACT, GEMM_STREAM_K, GEMM_WIDE, GG_DOWN, GG_FULL, GG_UP, PADDED, W_PACKED,
               W_ROWMAJOR, SharedExpert, blocked_rows, gemm_desc, moe_combine, moe_dispatch, moe_dispatch_blocked,
               moe_dispatch_fp8, moe_dispatch_layout, moe_grouped_gemm, moe_grouped_gemm_workspace, moe_layout_rows,
               moe_pack_weights, moe_quantize_1x128, moe_route_topk)


class MoEShare:
    """Buffers and weights for one GPU's share of the layer."""

    def __init__(self, *, n_tokens: int, hidden: int, inter: int, n_experts: int, top_k: int, n_src: int,
                 expert_lo: int, n_local: int, act_dtype: torch.dtype, layout: int = COMPACT,
                 capacity: Optional[int] = None, self_range=(0, 0), device="cuda",
                 blocked: Optional[bool] = None, policy: Optional[int] = None, gather: Optional[bool] = None,
                 w8a8: bool = False, scatter: Optional[bool] = None):
        self.N, self.H, self.I, self.E, self.K = n_tokens, hidden, inter, n_experts, top_k
        self.S, self.lo, self.L = n_src, expert_lo, n_local
        self.layout = layout
        if capacity is None:
            if layout != COMPACT:
                raise ValueError("the padded layout needs an explicit capacity (rows per expert and source)")
            capacity = n_tokens * min(top_k, n_local)
        self.capacity = capacity
        self.self_lo, self.self_hi = self_range
        self.act_dtype = act_dtype
        self.dev = torch.device(device)
        self.R = moe_layout_rows(n_tokens, top_k, n_experts, n_src, expert_lo, n_local, layout, capacity)
        # expert rows in the 16-row blocked layout when experts are expected to
        # hold enough rows for the wide-tile GEMM (the layout speeds up its loads)
        many_rows = n_tokens * top_k >= 128 * n_experts
        # expert rows row-major by default: the token-major dispatch into them
        # moves the fewest bytes; blocked rows speed the wide GEMM's loads but
        # cost the dispatch more than that saves on the prefill share
        if blocked is None:
            blocked = False
        self.w8a8 = bool(w8a8)
        if self.w8a8 and act_dtype != torch.bfloat16:
            raise ValueError("the W8A8 path takes bf16 token rows")
        # scatter: the down projection writes the tokens with one row here and
        # no shared-expert row straight into the output (bf16 outputs only) and
        # the combine takes the other tokens. Off by default: measured on
        # MI355X it costs the down projection more than it saves the combine
        # (the epilogue's reads of the token's K entries sit on the tile's
        # critical path): dsv3_prefill_ep8 3.25 -> 3.48 ms, kimi_k2_ep8
        # 0.664 -> 0.695 ms, dsv3_decode_ep128 0.189 -> 0.195 ms
        self.scatter = False if scatter is None else bool(scatter)
        if self.scatter and act_dtype != torch.bfloat16:
            raise ValueError("the down projection's scatter writes bf16 outputs")
        self.blocked = bool(blocked) and act_dtype == torch.bfloat16 and hidden % 32 == 0 and not self.w8a8
        self.a_layout = ACT_BLOCKED16 if self.blocked else ACT_ROWS
        # one kernel per product: batches whose experts are expected to hold
        # enough rows take the wide-tile kernel for every group (what the AUTO
        # rule picks for them) without an empty stream-K launch; decode-sized
        # batches take the stream-K kernel without an empty wide launch
        self.policy = (GEMM_WIDE if many_rows else GEMM_STREAM_K) if policy is None else policy
        # the bf16 GEMM kernels can read the routed rows straight from the
        # tokens (row_token of the layout), which leaves out the dispatch copy
        can_gather = (act_dtype == torch.bfloat16 and not self.blocked and
                      n_tokens * hidden * (1 if self.w8a8 else 2) <= 1 << 32)
        self.gather = can_gather if gather is None else bool(gather)
        if self.gather and not can_gather:
            raise ValueError("gathered rows need bf16 activations, row-major rows and tokens below 4 GiB")
        d = self.dev
        self.topk_idx = torch.empty((n_tokens, top_k), dtype=torch.int32, device=d)
        self.topk_w = torch.empty((n_tokens, top_k), dtype=torch.float32, device=d)
        self.lay = None
        # W8A8: the quantized token rows (codes, one scale per 128 columns)
        self.xq = torch.empty((n_tokens, hidden), dtype=torch.uint8, device=d) if self.w8a8 else None
        self.xs = torch.empty((n_tokens, hidden // 128), dtype=torch.float32, device=d) if self.w8a8 else None
        self.xes = None
        # the expert-grouped copy of the rows; gathering layers need none (made on first dispatch)
        self.xe = None if self.gather else self._new_xe()
        self.ye = torch.empty((max(self.R, 1), hidden), dtype=act_dtype, device=d)
        B0 = self.self_hi - self.self_lo
        self.ys = torch.empty((max(B0, 1), hidden), dtype=act_dtype, device=d)
        self.shared_off = torch.tensor([0, B0], dtype=torch.int32, device=d)
        self.w = None
        self.sw = None
        self.w_format = W_ROWMAJOR
        self.ws = None
        self.sws = None
        self.shared_mode = "fused"

    def _new_xe(self):
        if self.w8a8:
            self.xes = torch.empty((max(self.R, 1), self.H // 128), dtype=torch.float32, device=self.dev)
            return torch.empty((max(self.R, 1), self.H), dtype=torch.uint8, device=self.dev)
        return torch.empty((max(blocked_rows(self.R) if self.blocked else self.R, 1), self.H), dtype=self.act_dtype,
                           device=self.dev)

    @property
    def gemm_act_dtype(self):
        return torch.uint8 if self.w8a8 else self.act_dtype

    # weights: dict with w13 [G,2I,H], w2 [G,H,I], optional s13/s2 (host or device tensors)
    def set_weights(self, routed: dict, shared: Optional[dict] = None, pack: bool = True):
        """Upload weights; bf16/fp8 weights are packed once into the kernel's load order."""
        def todev(wd):
            if wd is None:
                return None
            out = {k: (v.to(self.dev).contiguous() if isinstance(v, torch.Tensor) else v)
                   for k, v in wd.items() if k in ("w13", "w2", "s13", "s2")}
            if self.w_format == W_PACKED:
                out["w13"], out["w2"] = moe_pack_weights(out["w13"], out["w2"], self.H, self.I)
            return out
        self.w_format = W_PACKED if (pack and routed["w13"].dtype != torch.float32) else W_ROWMAJOR
        self.w = todev(routed)
        self.sw = todev(shared)
        if self.w8a8 and self.w.get("s13") is None:
            raise ValueError("the W8A8 path needs fp8 weights with their 128 x 128 scales")
        self._default_shared_mode()
        wdt = self.w["w13"].dtype
        B0 = self.self_hi - self.self_lo
        se = SharedExpert(rows=B0 if self.sw is not None else 0)
        desc = gemm_desc(self.L, self.H, self.I, self.gemm_act_dtype, wdt, self.layout, self.S, self.capacity,
                         self.R, shared=se, w_format=self.w_format, a_layout=self.a_layout, policy=self.policy)
        self.ws = torch.zeros(moe_grouped_gemm_workspace(desc), dtype=torch.uint8, device=self.dev)
        if self.sw is not None:
            sdesc = gemm_desc(1, self.H, self.I, self.gemm_act_dtype, self.sw["w13"].dtype, COMPACT, 1, 0,
                              max(B0, 1), w_format=self.w_format)
            self.sws = torch.zeros(moe_grouped_gemm_workspace(sdesc), dtype=torch.uint8, device=self.dev)

    def _shared_arg(self, x):
        if self.sw is None or self.self_hi <= self.self_lo:
            return None
        sw = self.sw
        a = x[self.self_lo: self.self_hi]
        d = {"a": a, "w13": sw["w13"], "w2": sw["w2"], "s13": sw.get("s13"), "s2": sw.get("s2"),
             "y": self.ys[: a.shape[0]]}
        if self.w8a8:
            d["a"], d["a_scales"] = self.xq[self.self_lo: self.self_hi], self.xs[self.self_lo: self.self_hi]
        return d

    def quantize(self, x):
        """W8A8: the fp8 payload of the token rows."""
        moe_quantize_1x128(x, self.xq, self.xs)

    def route(self, logits):
        moe_route_topk(logits, self.K, True, self.topk_idx, self.topk_w)

    def layout_step(self, src_offsets):
        self.lay = moe_dispatch_layout(self.topk_idx, src_offsets, self.E, self.lo, self.L, self.layout,
                                       self.capacity, out=self.lay)

    def dispatch(self, x):
        if self.xe is None:
            self.xe = self._new_xe()
        if self.w8a8:
            moe_dispatch_fp8(self.xq, self.xs, self.lay["row_of"], self.K, self.R, self.xe, self.xes)
        elif self.blocked:
            moe_dispatch_blocked(x, self.lay["row_of"], self.K, self.R, self.xe)
        else:
            moe_dispatch(x, self.lay["row_of"], self.K, self.R, self.xe)

    def _self_range(self):
        # the tokens with a shared-expert row (the range the scatter and the
        # combine must agree on)
        has = self.sw is not None and self.self_hi > self.self_lo
        return (self.self_lo, self.self_hi) if has else (0, 0)

    def gemm(self, stage=GG_FULL, x=None, src=None, out=None):
        """Routed experts; with ``x`` the shared expert runs in the same launches.
        Gathering, the up projection reads its rows from ``src`` (the tokens).
        With ``out`` and the scatter on, the down projection writes the tokens
        with one row here (and no shared-expert row) into ``out``."""
        w = self.w
        extra = {}
        if out is not None and self.scatter and stage != GG_UP and self.R > 0:
            lo, hi = self._self_range()
            extra["scatter"] = dict(row_token=self.lay["row_token"], row_of=self.lay["row_of"], topk_w=self.topk_w,
                                    out=out, n_rows=max(self.R, 1), self_lo=lo, self_hi=hi)
        if self.gather:
            if src is None:
                raise ValueError("gathered rows need the tokens (src)")
            a, extra["a_rows"] = src, self.lay["row_token"]
            if self.w8a8:
                a, extra["a_scales"] = self.xq, self.xs
        else:
            a = self.xe if self.blocked else self.xe[: self.R]
            if self.w8a8:
                extra["a_scales"] = self.xes[: self.R]
        moe_grouped_gemm(a, w["w13"], w["w2"], group_off=self.lay["expert_off"],
                         counts=self.lay["counts"], s13=w.get("s13"), s2=w.get("s2"), layout=self.layout,
                         n_src=self.S, capacity=self.capacity, stage=stage, y=self.ye[: self.R], ws=self.ws,
                         shared=None if x is None else self._shared_arg(x), w_format=self.w_format,
                         a_layout=self.a_layout, rows=self.R, policy=self.policy, **extra)

    def _default_shared_mode(self):
        # where the shared expert runs by default (measured on MI355X): beside
        # route, layout and the routed GEMM on a second stream for bf16 decode
        # batches, whose streaming GEMM leaves HBM idle during the latency-bound
        # route and layout (dsv3_decode_ep8: 0.587 -> 0.548 ms); inside the
        # routed launches otherwise (kimi_k2_ep8, fp8: 0.684 fused against
        # 0.718 ms on the second stream)
        bf16_decode = self.w["w13"].dtype == torch.bfloat16 and self.policy == GEMM_STREAM_K
        self.shared_mode = "stream" if bf16_decode and self.sw is not None else "fused"

    def share_weights_from(self, other: "MoEShare"):
        """Use another share's (already uploaded and packed) weights: a second
        share over a different batch of the same layer, e.g. a microbatch."""
        self.w_format, self.w, self.sw = other.w_format, other.w, other.sw
        self._default_shared_mode()
        wdt = self.w["w13"].dtype
        B0 = self.self_hi - self.self_lo
        se = SharedExpert(rows=B0 if self.sw is not None else 0)
        desc = gemm_desc(self.L, self.H, self.I, self.gemm_act_dtype, wdt, self.layout, self.S, self.capacity,
                         self.R, shared=se, w_format=self.w_format, a_layout=self.a_layout, policy=self.policy)
        self.ws = torch.zeros(moe_grouped_gemm_workspace(desc), dtype=torch.uint8, device=self.dev)
        if self.sw is not None:
            sdesc = gemm_desc(1, self.H, self.I, self.gemm_act_dtype, self.sw["w13"].dtype, COMPACT, 1, 0,
                              max(B0, 1), w_format=self.w_format)
            self.sws = torch.zeros(moe_grouped_gemm_workspace(sdesc), dtype=torch.uint8, device=self.dev)

    def footprint_bytes(self) -> int:
        """Device bytes of the per-step expert buffers (xe, ye and the GEMM
        workspace with h and the partial sums): what the layout choice costs."""
        n = self.ye.numel() * self.ye.element_size() + self.ws.numel()
        for t in (self.xe, self.xes, self.xq, self.xs):
            if t is not None:
                n += t.numel() * t.element_size()
        return int(n)

    def shared_gemm(self, x, stage=GG_FULL):
        if self.sw is None or self.self_hi <= self.self_lo:
            return
        sw = self.sw
        a = x[self.self_lo: self.self_hi]
        extra = {}
        if self.w8a8:
            a, extra["a_scales"] = self.xq[self.self_lo: self.self_hi], self.xs[self.self_lo: self.self_hi]
        # a call of its own: with 128 or more rows of bf16 weights the wide
        # kernel takes it whole (what AUTO picks too), without AUTO's empty
        # stream-K launch and its fix-up
        wide = a.shape[0] >= 128 and sw["w13"].dtype == torch.bfloat16 and self.H % 256 == 0
        moe_grouped_gemm(a, sw["w13"], sw["w2"], group_off=self.shared_off, s13=sw.get("s13"), s2=sw.get("s2"),
                         layout=COMPACT, stage=stage, y=self.ys[: a.shape[0]], ws=self.sws, w_format=self.w_format,
                         policy=GEMM_WIDE if wide else 0, **extra)

    def combine(self, out, multi: bool = False):
        """Weighted sum into ``out``; ``multi``: only the tokens the down
        projection's scatter left."""
        sy = self.ys if (self.sw is not None and self.self_hi > self.self_lo) else None
        lo, hi = self._self_range() if multi else (self.self_lo, self.self_hi)
        moe_combine(self.ye[: max(self.R, 1)] if self.R else self.ye[:0], self.lay["row_of"], self.topk_w, out, sy,
                    lo, hi, multi=multi)

    def step(self, logits, src_offsets, x, out, events: Optional[dict] = None, fused_shared: bool = True,
             shared_mode: Optional[str] = None):
        """One full pass. ``events`` maps step names to (start, end) CUDA events
        recorded around each call. ``shared_mode`` places the shared expert
        (default: the share's ``shared_mode``, see _default_shared_mode):
        "fused" inside the routed grouped-GEMM launches; "serial" as
        calls of its own on the same stream after the routed GEMM; "stream" as
        calls of its own on a second stream, concurrent with route, layout and
        the routed GEMM, joined before the combine (the pages overlap it with
        the dispatch). ``fused_shared=False`` is "serial". Gathering, the
        dispatch copy is left out (its events, if any, enclose no work)."""
        mode = shared_mode or (self.shared_mode if fused_shared else "serial")
        if mode not in ("fused", "serial", "stream"):
            raise ValueError(f"unknown shared_mode {mode}")

        def run(name, fn):
            if events is not None and name in events:
                events[name][0].record()
                fn()
                events[name][1].record()
            else:
                fn()

        if self.w8a8:
            run("quantize", lambda: self.quantize(x))
        cur = side = None
        if mode == "stream" and self.sw is not None and self.self_hi > self.self_lo:
            if getattr(self, "_side", None) is None:
                self._side = torch.cuda.Stream(device=self.dev)  # default priority
            cur, side = torch.cuda.current_stream(self.dev), self._side
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                run("shared", lambda: self.shared_gemm(x, GG_FULL))
        run("route", lambda: self.route(logits))
        run("layout", lambda: self.layout_step(src_offsets))
        run("dispatch", (lambda: None) if self.gather else (lambda: self.dispatch(x)))
        xs = x if mode == "fused" else None
        sc = self.scatter and self.R > 0
        run("gemm_up", lambda: self.gemm(GG_UP, xs, src=x))
        run("gemm_down", lambda: self.gemm(GG_DOWN, xs, src=x, out=out if sc else None))
        if mode == "serial":
            run("shared_up", lambda: self.shared_gemm(x, GG_UP))
            run("shared_down", lambda: self.shared_gemm(x, GG_DOWN))
        if side is not None:
            cur.wait_stream(side)
        run("combine", lambda: self.combine(out, multi=sc))
        return out


__all__ = ["MoEShare", "COMPACT", "PADDED"]
