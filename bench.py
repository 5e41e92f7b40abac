#!/usr/bin/env python3
"""Throughput of one GPU's share of an expert-parallel MoE layer on MI355X.

One step = route top-K -> dispatch layout -> dispatch -> grouped SwiGLU GEMM
(routed experts, shared expert in the same launches) -> combine, over one
batch of seeded synthetic input already resident in HBM. Default workload (the
largest single-GPU configuration): DeepSeek-V3-shaped prefill, EP8 share
(8 source ranks x 4096 tokens, hidden 7168, 256 experts with Zipf-skewed
routing, top-8, local experts 0-31 + 1 shared, SwiGLU intermediate 2048, bf16,
count-first compact layout).

Prints one JSON line. ``value`` is MoE-layer tokens per second for this GPU
(its own tokens per step divided by the step time). ``roofline`` reports the
dominant kernel against MI355X's published peak, from HIP events around each
launch on the launching stream. ``cpu_baseline`` times the CPU oracle on the
host (rank 0, one GPU only) on the bounded sample it names, with all cores and
single-threaded. ``extras`` holds the other configurations (decode shares, the
fixed-rectangle layout of the prefill share), ``overlap`` the shared expert on
a second stream against the fused launch, and ``microbatch`` the cost of
running the grouped GEMM as two half batches.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--layout compact|padded] [--extras LIST|none]
                       [--no-cpu-baseline] [--copy-calib] [--ceilings]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, TFLOP/s
# the shared expert runs inside the gemm_up / gemm_down launches
STEP_NAMES = ("route", "layout", "dispatch", "gemm_up", "gemm_down", "combine")
KERNEL_OF_STEP = {"gemm_up": "ffn_wide_kernel<up> + ffn_wide_fixup_kernel<up> (or ffn_bf16_kernel<up> + "
                             "ffn_fixup_kernel<up> for decode batches)",
                  "gemm_down": "ffn_wide_kernel<down> + ffn_wide_fixup_kernel<down> (or ffn_bf16_kernel<down> + "
                               "ffn_fixup_kernel<down>)",
                  "dispatch": "dispatch_kernel", "combine": "combine_kernel", "route": "route_topk_kernel"}
KERNEL_OF_STEP_FP8 = {"gemm_up": "ffn_fp8_kernel<up> + ffn_fp8_fixup_kernel<up>",
                      "gemm_down": "ffn_fp8_kernel<down> + ffn_fp8_fixup_kernel<down>"}
KERNEL_OF_STEP_W8A8 = {"gemm_up": "ffn_w8a8_kernel<up> + ffn_w8a8_fixup_kernel<up>",
                       "gemm_down": "ffn_w8a8_kernel<down> + ffn_w8a8_fixup_kernel<down>",
                       "quantize": "quantize_1x128_kernel"}
# extra configurations: workload[:option+option], options padded (fixed-rectangle
# layout) and w8a8 (fp8 activations; bf16 checkpoints quantized to fp8 128 x 128 tiles)
DEFAULT_EXTRAS = ("dsv3_decode_ep8,dsv3_decode_ep128,kimi_k2_ep8,dsv3_prefill_ep8:padded,kimi_k2_ep8:w8a8,"
                  "dsv3_prefill_ep8:w8a8")


# --------------------------------------------------------------------------- perf model
def groupgemm_flops(g, m, k, n):
    """FLOP of a grouped GEMM with g groups of [m,k] x [k,n] (Perplexity DeepSeek page, GroupGEMM)."""
    return 2 * g * m * k * n


def groupgemm_bytes(g, m, k, n, a_bytes=1, b_bytes=1, c_bytes=1):
    """Memory traffic of the same grouped GEMM: each group reads A and B once and writes C."""
    return g * (m * k * a_bytes + n * k * b_bytes + m * n * c_bytes)


def tokens_per_expert(batch, qlen, top_k, ep, n_experts):
    """Average rows per expert under EP with DP = EP (same page, GroupGEMM)."""
    return batch * qlen * top_k * ep / n_experts


def algorithmic_model(cfg, counts, row_of, B0, w8a8=False, shared_apart=False, scatter=False):
    """Algorithmic bytes and FLOP per call from the actual routing of the step.

    counts [L, S] rows per local expert and source; row_of [N*K] (-1 = not local).
    W8A8: the GEMMs read fp8 rows (1 byte + 4 bytes per 128 columns) and the
    up projection writes fp8 h; y and the combine stay bf16.
    shared_apart: the shared expert runs as calls of its own (on a second
    stream), so gemm_up / gemm_down carry the routed rows only and the shared
    expert's bytes and FLOP go to a "shared" entry.
    scatter: the down projection writes the S1 tokens with exactly one row
    here and no shared-expert row straight to the output (their rows are
    written once, to out instead of y, after reading the token's K entries),
    and the combine neither reads their y rows nor writes their output rows.
    """
    H, I, K = cfg.hidden, cfg.inter, cfg.top_k
    wb = 1 if cfg.weight == "fp8_e4m3" else (4 if cfg.weight == "f32" else 2)
    ab = 4 if cfg.act == "f32" else 2
    qb = 1 + 4 / 128  # an fp8 payload element with its share of the scale
    N = len(row_of) // K
    m = counts.sum(axis=1)
    M = int(m.sum())
    active = int(np.count_nonzero(m))
    local_tok = (row_of.reshape(N, K) >= 0).any(axis=1)
    U = int(local_tok.sum())
    touched = local_tok.copy()
    touched[:B0] = True
    UT = int(touched.sum())
    n_local_entries = (row_of.reshape(N, K) >= 0).sum(axis=1)
    single = n_local_entries == 1
    if cfg.shared:
        single[:B0] = False
    S1 = int(single.sum()) if scatter else 0
    scale_bytes = (2 * I // 128) * (H // 128) * 4 if wb == 1 else 0
    up_w = active * (2 * I * H * wb + scale_bytes)
    down_w = active * (H * I * wb + (scale_bytes // 2))
    sh_up_w = (2 * I * H * wb + scale_bytes) if cfg.shared else 0
    sh_down_w = (H * I * wb + scale_bytes // 2) if cfg.shared else 0
    B0s = B0 if cfg.shared else 0
    MS = M + B0s  # rows through the expert FFN: routed plus the shared expert's
    model = {
        "M": M, "U": U, "touched": UT, "active_experts": active, "max_rows_per_expert": int(m.max(initial=0)),
        "single_row_tokens_scattered": S1,
        "bytes": {
            "route": N * cfg.n_experts * 4 + N * K * 8,
            "layout": 3 * N * K * 4 + M * 4,
            "dispatch": (U + M) * H * ab + N * K * 4,
            "gemm_up": up_w + sh_up_w + MS * H * ab + MS * I * ab,
            "gemm_down": down_w + sh_down_w + MS * I * ab + MS * H * ab,
            "combine": (M - S1 + B0s + UT - S1) * H * ab + N * K * 8,
        },
        "flops": {"gemm_up": 2 * MS * H * 2 * I, "gemm_down": 2 * MS * I * H},
    }
    if w8a8:
        b = model["bytes"]
        b["quantize"] = int(N * H * (ab + qb))
        b["dispatch"] = int((U + M) * H * qb + N * K * 4)
        b["gemm_up"] = int(up_w + sh_up_w + MS * H * qb + MS * I * qb)
        b["gemm_down"] = int(down_w + sh_down_w + MS * I * qb + MS * H * 2)
    if shared_apart and cfg.shared:
        b, f = model["bytes"], model["flops"]
        rb = qb if w8a8 else ab  # bytes of an fp8 or activation element of x and h
        sh = {"gemm_up": sh_up_w + B0 * H * rb + B0 * I * rb, "gemm_down": sh_down_w + B0 * I * rb + B0 * H * ab}
        for n in ("gemm_up", "gemm_down"):
            b[n] = int(b[n] - sh[n])
        b["shared"] = int(sh["gemm_up"] + sh["gemm_down"])
        f["gemm_up"], f["gemm_down"] = 2 * M * H * 2 * I, 2 * M * I * H
        f["shared"] = 2 * B0 * H * 2 * I + 2 * B0 * I * H
    return model


# --------------------------------------------------------------------------- helpers
def _kernel_source_hash():
    """Hash of the grouped-GEMM sources (traffic counters are valid for these only)."""
    import glob
    csrc = os.path.join(ROOT, "combine_router_softmax_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(csrc, "gemm_*"))) + [os.path.join(csrc, "grouped_gemm.hip"),
                                                                   os.path.join(csrc, "moe_common.hpp"),
                                                                   os.path.join(csrc, "fp8_quant.hpp")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload, kernel_step):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_step}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != _kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return None


def _oracle_weights(cfg, d):
    """The oracle's weight inputs: float64 arrays for bf16/f32 checkpoints
    (converted once, outside any timing), e4m3fn codes + scales for fp8 (the
    oracle decodes them itself)."""
    fp8 = cfg.weight == "fp8_e4m3"

    def conv(wd):
        if wd is None:
            return None
        if fp8:
            return (wd["w13"].numpy(), wd["w2"].numpy(), wd["s13"].numpy(), wd["s2"].numpy())
        return (wd["w13"].double().numpy(), wd["w2"].double().numpy(), None, None)

    return conv(d["routed"]), conv(d["shared"])


def _cpu_time(cfg, d, weights, n, sub_off, B0_sample, min_seconds):
    import oracle
    (w13, w2, s13, s2), sh = weights
    x = d["x"][:n].double().numpy()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(x, d["logits"][:n], sub_off, cfg.top_k, cfg.expert_lo, cfg.n_local, w13, w2, s13, s2,
                         shared=sh, self_range=(0, B0_sample))
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt / reps * (reps + 1) > 3 * min_seconds:
            return dt, reps


def _cpu_baseline(cfg, d, B0, max_tokens, min_seconds=10.0):
    """Time the CPU oracle (as it stands) on the host for one step of the same
    workload, on a bounded sample of it, and scale to tokens/s. Once with every
    BLAS thread, once single-threaded (a smaller sample)."""
    off = d["src_offsets"]
    N = int(off[-1])
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host_cores = os.cpu_count()
    weights = _oracle_weights(cfg, d)

    # all cores: whole source ranks (a prefix), so the sample has the layer's shape
    n = min(N, max_tokens)
    s_cnt = max(int(np.searchsorted(off, n, side="right") - 1), 1)
    n = int(off[s_cnt])
    dt, reps = _cpu_time(cfg, d, weights, n, off[: s_cnt + 1], int(off[1]), min_seconds)
    full_time = dt / reps * (N / n)
    res = {
        "value": B0 / full_time, "unit": "tokens/s", "cores": _blas_threads() or host_cores,
        "host_cores": host_cores, "kind": "oracle", "seconds": round(dt, 2), "passes": reps,
        "sample": (f"float64 NumPy oracle, one whole layer step over the first {s_cnt} of {len(off) - 1} source "
                   f"ranks ({n} of {N} tokens, all their local experts, shared expert on the GPU's own "
                   f"{int(off[1])} tokens), repeated {reps} times ({dt:.1f} s); time per pass scaled by {N}/{n}"),
    }
    # one thread: the first n1 tokens of source 0 (also the shared expert's rows)
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return res
    n1 = min(int(off[1]), 256)
    with threadpool_limits(limits=1):
        dt1, reps1 = _cpu_time(cfg, d, weights, n1, np.array([0, n1], dtype=np.int32), n1, min_seconds)
    t1 = dt1 / reps1 * (N / n1)
    res["single_thread"] = {
        "value": B0 / t1, "unit": "tokens/s", "cores": 1, "kind": "oracle", "seconds": round(dt1, 2),
        "passes": reps1,
        "sample": (f"the same oracle with one BLAS thread over the first {n1} tokens of source rank 0 (their local "
                   f"experts and the shared expert), repeated {reps1} times ({dt1:.1f} s); time per pass scaled "
                   f"by {N}/{n1}"),
    }
    return res


# --------------------------------------------------------------------------- GPU timing
class Bench:
    def __init__(self, torch, flush_mb):
        self.torch = torch
        self.flush_buf = (torch.ones((flush_mb << 20) // 8, dtype=torch.int64, device="cuda")
                          if flush_mb > 0 else None)
        self.flush_sink = torch.zeros((), dtype=torch.int64, device="cuda")

    def flush(self):
        # between timed steps (never inside the events): a read of a buffer
        # twice the Infinity Cache, so no step finds the previous one's weights
        # or activations in a cache. (A read, not a write: written flush data
        # would sit dirty in the cache and be written back during the next
        # step.) The previous step's own dirty lines are written back here.
        if self.flush_buf is not None:
            self.torch.sum(self.flush_buf, dim=0, out=self.flush_sink)

    def events(self, n):
        E = self.torch.cuda.Event
        return [(E(enable_timing=True), E(enable_timing=True)) for _ in range(n)]

    def time_step(self, share, logits, offs, x, out, steps, warmup, graph=True, shared_mode=None):
        """Eager steps with events around every call, then (graph) replays of
        one captured step; mean times."""
        torch = self.torch
        run = lambda ev=None: share.step(logits, offs, x, out, events=ev, shared_mode=shared_mode)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        names = STEP_NAMES + (("shared",) if (shared_mode or share.shared_mode) == "stream" else ()) + \
            (("quantize",) if share.w8a8 else ())
        ev = {n: self.events(steps) for n in names}
        est = self.events(steps)
        t0 = time.perf_counter()
        for i in range(steps):
            self.flush()
            est[i][0].record()
            run({n: ev[n][i] for n in names})
            est[i][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        eager_ms = float(np.mean([a.elapsed_time(b) for a, b in est]))
        per_call_us = {n: 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names}
        graph_ms = None
        if graph:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                run()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run()
            for _ in range(max(1, warmup)):
                g.replay()
            torch.cuda.synchronize()
            gst = self.events(steps)
            t0 = time.perf_counter()
            for i in range(steps):
                self.flush()
                gst[i][0].record()
                g.replay()
                gst[i][1].record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            graph_ms = float(np.mean([a.elapsed_time(b) for a, b in gst]))
            del g
        return {"ms": graph_ms if graph_ms is not None else eager_ms, "ms_eager": eager_ms,
                "timing": "hip_graph_replay" if graph_ms is not None else "eager", "per_call_us": per_call_us,
                "wall": wall, "shared_mode": shared_mode or share.shared_mode}


def _make_share(cfg, d, layout, *, policy=None, gather=None, blocked=None, weights_from=None, self_range=None,
                w8a8=False, scatter=None):
    import torch
    from combine_router_softmax_amd import COMPACT
    from combine_router_softmax_amd.layer import MoEShare
    off = d["src_offsets"]
    N, B0 = int(off[-1]), int(off[1])
    cap = None if layout == COMPACT else int(np.diff(off).max())
    act = torch.float32 if cfg.act == "f32" else torch.bfloat16
    share = MoEShare(n_tokens=N, hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                     n_src=cfg.n_src, expert_lo=cfg.expert_lo, n_local=cfg.n_local, act_dtype=act, layout=layout,
                     capacity=cap, self_range=self_range or (0, B0), blocked=blocked, gather=gather, policy=policy,
                     w8a8=w8a8, scatter=scatter)
    if weights_from is not None:
        share.share_weights_from(weights_from)
    else:
        share.set_weights(d["routed"], d["shared"])
    return share


def _dev_inputs(d):
    import torch
    return (torch.from_numpy(d["logits"]).cuda(), torch.from_numpy(d["src_offsets"]).cuda(), d["x"].cuda())


def _summarize(cfg, share, res, B0):
    """Algorithmic model of the step's actual routing, per-call rates and the
    dominant kernel's roofline."""
    counts = share.lay["counts"].cpu().numpy().astype(np.int64)
    row_of = share.lay["row_of"].cpu().numpy().astype(np.int64)
    apart = res.get("shared_mode") == "stream"
    model = algorithmic_model(cfg, counts, row_of, B0, w8a8=share.w8a8, shared_apart=apart, scatter=share.scatter)
    per_call_us = dict(res["per_call_us"])
    steps = STEP_NAMES + (("quantize",) if share.w8a8 else ()) + (("shared",) if "shared" in per_call_us else ())
    if share.gather:
        # the up projection reads its rows from the tokens: no dispatch copy
        # (its events enclosed no work)
        model["bytes"]["dispatch"] = 0
        per_call_us["dispatch"] = 0.0
    breakdown = {}
    for n in steps:
        us = per_call_us[n]
        b = model["bytes"].get(n, 0)
        f = model["flops"].get(n, 0)
        breakdown[n] = {"us": round(us, 2), "GB/s": round(b / us / 1e3, 1) if us > 0 and b else None,
                        "TFLOP/s": round(f / us / 1e6, 1) if f and us > 0 else None}
    if share.gather:
        breakdown["dispatch"]["fused_into"] = "gemm_up"
    dom = max(("gemm_up", "gemm_down", "dispatch", "combine"), key=lambda n: per_call_us[n])
    dom_us = per_call_us[dom]
    flops = model["flops"].get(dom, 0)
    byts = model["bytes"][dom]
    mfma_peak = FP8_PEAK_TFLOPS if share.w8a8 else BF16_PEAK_TFLOPS
    mfma_bound = flops > 0 and flops / byts > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(flops / dom_us / 1e6, 2), "peak": mfma_peak,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(byts / dom_us / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = _traffic(cfg.name + ("_w8a8" if share.w8a8 else ""), dom) if share.layout == 0 else None
    names = dict(KERNEL_OF_STEP)
    names.update(KERNEL_OF_STEP_FP8 if cfg.weight == "fp8_e4m3" else {})
    names.update(KERNEL_OF_STEP_W8A8 if share.w8a8 else {})
    roof["kernel"] = names.get(dom, dom)
    roof["step"] = dom
    roof["algorithmic_bytes_per_launch"] = int(byts)
    roof["flops_per_launch"] = int(flops)
    roof["avg_launch_us"] = round(dom_us, 2)
    # the GEMM's other bound, for context (decode GEMMs are graded on HBM, prefill on MFMA)
    gemm_us = per_call_us["gemm_up"] + per_call_us["gemm_down"]
    gb = model["bytes"]["gemm_up"] + model["bytes"]["gemm_down"]
    gf = model["flops"]["gemm_up"] + model["flops"]["gemm_down"]
    gemm = {"us": round(gemm_us, 2), "frac_hbm": round(gb / gemm_us / 1e3 / HBM_PEAK_GBS, 4),
            "frac_mfma_bf16": round(gf / gemm_us / 1e6 / BF16_PEAK_TFLOPS, 4)}
    if share.w8a8:
        gemm["frac_mfma_fp8"] = round(gf / gemm_us / 1e6 / FP8_PEAK_TFLOPS, 4)
    mv = {"combine": {"GB/s": breakdown["combine"]["GB/s"],
                      "frac_hbm": round(model["bytes"]["combine"] / per_call_us["combine"] / 1e3 / HBM_PEAK_GBS, 4)}}
    if not share.gather:
        dc_bytes = model["bytes"]["dispatch"] + model["bytes"]["combine"]
        dc_us = per_call_us["dispatch"] + per_call_us["combine"]
        mv["dispatch_combine"] = {"GB/s": round(dc_bytes / dc_us / 1e3, 1),
                                  "frac_hbm": round(dc_bytes / dc_us / 1e3 / HBM_PEAK_GBS, 4)}
    routing = {k: model[k] for k in ("M", "U", "touched", "active_experts", "max_rows_per_expert",
                                     "single_row_tokens_scattered")}
    return model, breakdown, roof, gemm, mv, routing


def _measure_extra(bench, name, steps, warmup, headline=None):
    """One more configuration: step time, per-call times, the dominant
    kernel's roofline, the expert-buffer footprint."""
    import torch
    from combine_router_softmax_amd import COMPACT, PADDED
    from synth import get_config, make_inputs
    wl, _, opts = name.partition(":")
    opts = set(opts.split("+")) - {""}
    if opts - {"padded", "w8a8"}:
        raise ValueError(f"unknown option in extra {name}")
    layout = PADDED if "padded" in opts else COMPACT
    w8a8 = "w8a8" in opts
    cfg = get_config(wl)
    if w8a8 and cfg.weight != "fp8_e4m3":
        cfg = get_config(wl, weight="fp8_e4m3")   # the checkpoint quantized to fp8 128 x 128 tiles
    same = headline is not None and headline[0] == cfg
    d = headline[1] if same else make_inputs(cfg, 0)
    off = d["src_offsets"]
    B0 = int(off[1])
    share = _make_share(cfg, d, layout, weights_from=headline[2] if same else None, w8a8=w8a8)
    logits, offs, x = _dev_inputs(d)
    out = torch.zeros_like(x)
    res = bench.time_step(share, logits, offs, x, out, steps, warmup)
    model, breakdown, roof, gemm, mv, routing = _summarize(cfg, share, res, B0)
    ent = {"workload": wl, "layout": "padded" if layout == PADDED else "compact", "shared_mode": share.shared_mode,
           "w8a8": w8a8, "weights": cfg.weight,
           "ms_per_step": round(res["ms"], 4),
           "tokens_per_s": round(B0 / (res["ms"] / 1e3), 1), "ms_per_step_eager": round(res["ms_eager"], 4),
           "roofline": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "kernel", "avg_launch_us")},
           "gemm": gemm, **mv, "breakdown": {k: v["us"] for k, v in breakdown.items()}, "routing": routing,
           "expert_buffer_bytes": share.footprint_bytes(), "status_word": int(share.lay["status"].item())}
    return cfg, d, share, ent


def _copy_rate(torch, launches=10):
    """A plain 1 GiB device copy: mean ms and read + write GB/s."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    return ms, 2 * (1 << 30) / ms / 1e6


def _ceilings(torch):
    """What the chip delivers in practice, for reading the rooflines: the
    probe program (matrix-core peak loops, LDS, L2 and HBM streams), a device
    copy, and the platform's dense GEMMs (torch.matmul, torch._scaled_mm) of
    the prefill share's two projection shapes, with M = the share's routed
    plus shared-expert rows under its seeded routing (from this library's
    route and layout calls)."""
    import subprocess
    import combine_router_softmax_amd as moe
    from synth import get_config, make_routing_inputs
    probe = os.path.join(ROOT, "combine_router_softmax_amd", "ceilings")
    if not os.path.exists(probe):
        print("the ceilings probe is not built (combine_router_softmax_amd/build.py builds it)", file=sys.stderr)
        return 1
    r = subprocess.run([probe], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        print(r.stdout + r.stderr, file=sys.stderr)
        return r.returncode
    out = {"probe": json.loads(r.stdout.strip().splitlines()[-1])}
    ms, gbs = _copy_rate(torch)
    out["copy_1GiB"] = {"ms": round(ms, 4), "GBps_read_plus_write": round(gbs, 1)}
    cfg = get_config("dsv3_prefill_ep8")
    d = make_routing_inputs(cfg, 0)
    idx, _ = moe.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), cfg.top_k)
    lay = moe.moe_dispatch_layout(idx, torch.from_numpy(d["src_offsets"]).cuda(), cfg.n_experts, cfg.expert_lo,
                                  cfg.n_local, moe.COMPACT, 0)
    M = int(lay["counts"].sum().item()) + int(d["src_offsets"][1])
    H, I = cfg.hidden, cfg.inter
    g = {}
    for name, (m, k, n) in {"up": (M, H, 2 * I), "down": (M, I, H)}.items():
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, k, device="cuda", dtype=torch.bfloat16)
        runs = {"bf16": lambda: torch.matmul(a, b.t())}
        try:
            a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
            one = torch.ones((), device="cuda")
            torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            runs["fp8"] = lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        except Exception as ex:  # pragma: no cover - depends on the platform build
            g[f"{name}_fp8"] = {"error": repr(ex)[:200]}
        for dt, fn in runs.items():
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / 20 * 1e3
            g[f"{name}_{dt}"] = {"M": m, "K": k, "N": n, "us": round(us, 1),
                                 "TFLOPs": round(2 * m * k * n / us / 1e6, 1)}
    out["dense_gemm_prefill_shapes"] = g
    print(json.dumps(out))
    return 0


def _overlap(bench, cfg, d, share, steps, warmup):
    """The shared expert fused into the routed launches, against its own calls
    on the same stream, and on a second stream beside the routed path."""
    import torch
    logits, offs, x = _dev_inputs(d)
    out = torch.zeros_like(x)
    r = {}
    for mode in ("fused", "serial", "stream"):
        res = bench.time_step(share, logits, offs, x, out, steps, warmup, shared_mode=mode)
        r[mode] = {"ms_per_step": round(res["ms"], 4), "ms_per_step_eager": round(res["ms_eager"], 4)}
    return r


def _microbatch(bench, cfg, d, share, steps, warmup):
    """The step as two microbatches, each holding half of every source rank's
    tokens (the pages' two-microbatch overlap), against one step over the whole
    batch: the grouped GEMM streams the weights once per microbatch."""
    import torch
    from combine_router_softmax_amd import COMPACT
    off = np.asarray(d["src_offsets"], dtype=np.int64)
    halves = []
    for h in range(2):
        idx = np.concatenate([np.arange(off[s] + (off[s + 1] - off[s]) // 2 * h,
                                        off[s] + ((off[s + 1] - off[s]) // 2 if h == 0 else off[s + 1] - off[s]))
                              for s in range(len(off) - 1)])
        b = np.array([((off[s + 1] - off[s]) // 2 if h == 0 else (off[s + 1] - off[s]) - (off[s + 1] - off[s]) // 2)
                      for s in range(len(off) - 1)])
        sub = {"logits": np.ascontiguousarray(d["logits"][idx]), "x": d["x"][torch.from_numpy(idx)],
               "src_offsets": np.concatenate([[0], np.cumsum(b)]).astype(np.int32), "routed": None, "shared": None}
        halves.append(sub)
    full = bench.time_step(share, *_dev_inputs(d), torch.zeros_like(d["x"]).cuda(), steps, warmup)
    r = {"full": {"ms_per_step": round(full["ms"], 4),
                  "gemm_us": round(full["per_call_us"]["gemm_up"] + full["per_call_us"]["gemm_down"], 2)}}
    tot_ms = tot_gemm = 0.0
    for h, sub in enumerate(halves):
        s = _make_share(cfg, sub, COMPACT, weights_from=share)
        res = bench.time_step(s, *_dev_inputs(sub), torch.zeros_like(sub["x"]).cuda(), steps, warmup)
        g = res["per_call_us"]["gemm_up"] + res["per_call_us"]["gemm_down"]
        r[f"half{h}"] = {"tokens": int(sub["src_offsets"][-1]), "ms_per_step": round(res["ms"], 4),
                         "gemm_us": round(g, 2)}
        tot_ms += res["ms"]
        tot_gemm += g
        del s
    r["two_halves_ms"] = round(tot_ms, 4)
    r["gemm_penalty"] = round(tot_gemm / (r["full"]["gemm_us"]) - 1.0, 4)
    return r


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3_prefill_ep8")
    ap.add_argument("--layout", choices=["compact", "padded"], default="compact")
    ap.add_argument("--gemm-policy", choices=["layer", "auto", "wide", "stream_k"], default="layer",
                    help="grouped-GEMM kernel choice (default: the layer's own, from its shape)")
    ap.add_argument("--gather", choices=["auto", "on", "off"], default="auto",
                    help="up projection reads its rows from the tokens (no dispatch copy); auto: the layer's choice")
    ap.add_argument("--xe-layout", choices=["auto", "rows", "blocked"], default="auto",
                    help="storage of the expert rows (auto: the layer's choice)")
    ap.add_argument("--shared-mode", choices=["layer", "fused", "serial", "stream"], default="layer",
                    help="shared expert inside the routed launches, after them, or on a second stream "
                         "(default: the layer's choice)")
    ap.add_argument("--scatter", action="store_true",
                    help="the down projection writes the tokens with one row on this GPU (and no shared-expert "
                         "row) straight to the output and the combine takes the rest (off by default: slower here)")
    ap.add_argument("--w8a8", action="store_true",
                    help="run the headline workload on the W8A8 path (fp8 activations; a bf16 checkpoint is "
                         "quantized to fp8 128 x 128 tiles), e.g. to profile the W8A8 kernels")
    ap.add_argument("--extras", default=DEFAULT_EXTRAS,
                    help="comma-separated workloads[:padded] measured after the headline, or 'none'")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--no-overlap", action="store_true", help="skip the shared-expert stream and microbatch study")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of a HIP graph of one step")
    ap.add_argument("--cpu-max-tokens", type=int, default=1024)
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="read a buffer of this size between timed steps (outside the timed events), so the 256 MB "
                         "Infinity Cache and L2 cannot carry data from one step to the next; 0: off")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--ceilings", action="store_true",
                    help="run only the measured ceilings: matrix-core, LDS, L2 and HBM probes, a device copy, and "
                         "dense library GEMMs of the prefill share's projection shapes")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer; runs on more than one GPU are not part of "
              "this build (other EP ranks are modelled as source partitions on the one GPU).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.ceilings:
        return _ceilings(torch)

    if args.copy_calib:
        # a plain 1 GiB device copy: the counter calibration for rocprofv3 --pmc,
        # and (timed) the practical streaming rate (read + write bytes / time)
        ms, gbs = _copy_rate(torch)
        print(json.dumps({"copy_calib_bytes": 1 << 30, "launches": 13, "copy_ms": round(ms, 4),
                          "copy_GBps_read_plus_write": round(gbs, 1)}))
        return 0

    import combine_router_softmax_amd as moe
    from combine_router_softmax_amd import COMPACT, PADDED
    from synth import get_config, make_inputs

    moe.lib()  # raises if the HIP library is missing: there is no other path
    cfg = get_config(args.workload)
    if args.w8a8 and cfg.weight != "fp8_e4m3":
        cfg = get_config(args.workload, weight="fp8_e4m3")
    t_gen = time.perf_counter()
    d = make_inputs(cfg, 0)
    t_gen = time.perf_counter() - t_gen
    off = d["src_offsets"]
    N, B0 = int(off[-1]), int(off[1])
    layout = COMPACT if args.layout == "compact" else PADDED
    share = _make_share(cfg, d, layout,
                        blocked=None if args.xe_layout == "auto" else args.xe_layout == "blocked",
                        gather=None if args.gather == "auto" else args.gather == "on",
                        policy={"layer": None, "auto": moe.GEMM_AUTO, "wide": moe.GEMM_WIDE,
                                "stream_k": moe.GEMM_STREAM_K}[args.gemm_policy], w8a8=args.w8a8,
                        scatter=True if args.scatter else None)
    logits, offs, x = _dev_inputs(d)
    out = torch.zeros_like(x)
    torch.cuda.synchronize()
    bench = Bench(torch, args.flush_mb)
    res = bench.time_step(share, logits, offs, x, out, args.steps, args.warmup, graph=not args.eager,
                          shared_mode=None if args.shared_mode == "layer" else args.shared_mode)
    print(f"# headline {cfg.name}: {res['ms']:.4f} ms/step", file=sys.stderr, flush=True)
    ms_per_step = res["ms"]
    st = int(share.lay["status"].item())
    model, breakdown, roof, gemm, mv, routing = _summarize(cfg, share, res, B0)

    extras = {}
    headline = (cfg, d, share)
    if args.extras and args.extras != "none":
        for name in args.extras.split(","):
            t0 = time.perf_counter()
            e_cfg, e_d, e_share, ent = _measure_extra(bench, name, args.extra_steps, 3, headline)
            ent["wall_s"] = round(time.perf_counter() - t0, 1)
            extras[name] = ent
            print(f"# extra {name}: {ent['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
            if not args.no_overlap and name in ("dsv3_decode_ep8", "kimi_k2_ep8"):
                ent["overlap"] = _overlap(bench, e_cfg, e_d, e_share, args.extra_steps, 3)
                ent["microbatch"] = _microbatch(bench, e_cfg, e_d, e_share, args.extra_steps, 3)
                print(f"# overlap and microbatch {name} done", file=sys.stderr, flush=True)
            del e_share
            if e_d is not d:
                del e_d
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(cfg, d, B0, args.cpu_max_tokens)

    value = B0 / (ms_per_step / 1e3)
    line = {
        "metric": "MoE-layer tokens/s per GPU",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "timing": res["timing"],
        "cache_flush_mb": args.flush_mb,
        "ms_per_step_eager": round(res["ms_eager"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if args.w8a8 else ("bf16" if cfg.act == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": cfg.name + (":w8a8" if args.w8a8 else ""), "layout": args.layout,
                   "xe_layout": "gathered" if share.gather else "blocked" if share.blocked else "rows",
                   "shared_mode": share.shared_mode if args.shared_mode == "layer" else args.shared_mode,
                   "global_batch": N, "tokens_per_gpu": B0,
                   "source_ranks": cfg.n_src, "hidden": cfg.hidden, "n_experts": cfg.n_experts,
                   "top_k": cfg.top_k, "local_experts": cfg.n_local, "shared_expert": cfg.shared,
                   "inter": cfg.inter, "weights": cfg.weight, "zipf": cfg.zipf,
                   "parallelism": f"ep{cfg.n_experts // cfg.n_local}"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "gemm": gemm,
        **mv,
        "breakdown": breakdown,
        "routing": routing,
        "expert_buffer_bytes": share.footprint_bytes(),
        "status_word": st,
        "extras": extras,
        "wall_s": round(res["wall"], 3),
        "input_gen_s": round(t_gen, 2),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
