#!/usr/bin/env python3
"""Throughput of one GPU's share of an expert-parallel MoE layer on MI355X.

One step = route top-K -> dispatch layout -> dispatch -> grouped SwiGLU GEMM
(routed experts) -> shared expert -> combine, over one batch of seeded
synthetic input already resident in HBM. Default workload: DeepSeek-V3-shaped
decode, single-node EP8 share (8 source ranks x 128 tokens, hidden 7168, 256
experts, top-8, local experts 0-31 + 1 shared, SwiGLU intermediate 2048, bf16).

Prints one JSON line. ``value`` is MoE-layer tokens per second for this GPU
(its own 128 tokens per step divided by the step time). ``roofline`` reports
the dominant kernel against MI355X's published peak, from HIP events around
each launch on the launching stream. ``cpu_baseline`` times the CPU oracle on
the host (rank 0, one GPU only) on the bounded sample it names.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--layout compact|padded] [--no-cpu-baseline] [--copy-calib]
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
# the shared expert runs inside the gemm_up / gemm_down launches
STEP_NAMES = ("route", "layout", "dispatch", "gemm_up", "gemm_down", "combine")
KERNEL_OF_STEP = {"gemm_up": "ffn_wide_kernel<up> + ffn_bf16_kernel<up> + ffn_fixup_kernel<up>",
                  "gemm_down": "ffn_wide_kernel<down> + ffn_bf16_kernel<down> + ffn_fixup_kernel<down>",
                  "dispatch": "dispatch_kernel", "combine": "combine_kernel", "route": "route_topk_kernel"}
KERNEL_OF_STEP_FP8 = {"gemm_up": "ffn_fp8_kernel<up> + ffn_fp8_fixup_kernel<up>",
                      "gemm_down": "ffn_fp8_kernel<down> + ffn_fp8_fixup_kernel<down>"}


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


def algorithmic_model(cfg, counts, row_of, B0):
    """Algorithmic bytes and FLOP per call from the actual routing of the step.

    counts [L, S] rows per local expert and source; row_of [N*K] (-1 = not local).
    """
    H, I, K = cfg.hidden, cfg.inter, cfg.top_k
    wb = 1 if cfg.weight == "fp8_e4m3" else (4 if cfg.weight == "f32" else 2)
    ab = 4 if cfg.act == "f32" else 2
    N = len(row_of) // K
    m = counts.sum(axis=1)
    M = int(m.sum())
    active = int(np.count_nonzero(m))
    local_tok = (row_of.reshape(N, K) >= 0).any(axis=1)
    U = int(local_tok.sum())
    touched = local_tok.copy()
    touched[:B0] = True
    UT = int(touched.sum())
    scale_bytes = (2 * I // 128) * (H // 128) * 4 if wb == 1 else 0
    up_w = active * (2 * I * H * wb + scale_bytes)
    down_w = active * (H * I * wb + (scale_bytes // 2))
    sh_up_w = (2 * I * H * wb + scale_bytes) if cfg.shared else 0
    sh_down_w = (H * I * wb + scale_bytes // 2) if cfg.shared else 0
    B0s = B0 if cfg.shared else 0
    MS = M + B0s  # rows through the expert FFN: routed plus the shared expert's
    model = {
        "M": M, "U": U, "active_experts": active, "max_rows_per_expert": int(m.max(initial=0)),
        "bytes": {
            "route": N * cfg.n_experts * 4 + N * K * 8,
            "layout": 3 * N * K * 4 + M * 4,
            "dispatch": (U + M) * H * ab + N * K * 4,
            "gemm_up": up_w + sh_up_w + MS * H * ab + MS * I * ab,
            "gemm_down": down_w + sh_down_w + MS * I * ab + MS * H * ab,
            "combine": (M + B0s + UT) * H * ab + N * K * 8,
        },
        "flops": {"gemm_up": 2 * MS * H * 2 * I, "gemm_down": 2 * MS * I * H},
    }
    return model


# --------------------------------------------------------------------------- helpers
def _kernel_source_hash():
    h = hashlib.sha256()
    for f in ("grouped_gemm.hip", "moe_common.hpp"):
        with open(os.path.join(ROOT, "combine_router_softmax_amd", "csrc", f), "rb") as fh:
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


def _cpu_baseline(cfg, d, B0, max_tokens, min_seconds=10.0):
    """Time the CPU oracle (as it stands) on the host for one step of the same
    workload, or a token-prefix sample of it, and scale to tokens/s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    off = d["src_offsets"]
    N = int(off[-1])
    n = min(N, max_tokens)
    # keep whole sources so the sample has the same shape: a prefix of source ranks
    s_cnt = int(np.searchsorted(off, n, side="right") - 1)
    s_cnt = max(s_cnt, 1)
    n = int(off[s_cnt])
    sub_off = off[: s_cnt + 1]

    class Lazy:
        def __init__(self, t, codes):
            self.t, self.codes = t, codes

        def __getitem__(self, g):
            v = self.t[g]
            return v.numpy() if self.codes else v.double().numpy()

    fp8 = cfg.weight == "fp8_e4m3"
    rw, sw = d["routed"], d["shared"]
    w13, w2 = Lazy(rw["w13"], fp8), Lazy(rw["w2"], fp8)
    s13 = rw["s13"].numpy() if fp8 else None
    s2 = rw["s2"].numpy() if fp8 else None
    sh = None
    if sw is not None:
        sh = (Lazy(sw["w13"], fp8), Lazy(sw["w2"], fp8), sw["s13"].numpy() if fp8 else None,
              sw["s2"].numpy() if fp8 else None)
    x = d["x"][:n].double().numpy()
    # the sample is repeated until about min_seconds of CPU work (a bounded
    # sample of 10-30 s), then timed per pass
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(x, d["logits"][:n], sub_off, cfg.top_k, cfg.expert_lo, cfg.n_local, w13, w2, s13, s2,
                         shared=sh, self_range=(0, int(off[1])))
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt / reps * (reps + 1) > 3 * min_seconds:
            break
    full_time = dt / reps * (N / n)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    return {
        "value": B0 / full_time, "unit": "tokens/s", "cores": blas_threads or cores,
        "host_cores": cores, "kind": "oracle", "seconds": dt, "passes": reps,
        "sample": (f"float64 NumPy oracle, one whole layer step over the first {s_cnt} of {len(off) - 1} source "
                   f"ranks ({n} of {N} tokens, all their local experts, shared expert on the GPU's own "
                   f"{int(off[1])} tokens), repeated {reps} times ({dt:.1f} s); time per pass scaled by {N}/{n}"),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3_decode_ep8")
    ap.add_argument("--layout", choices=["compact", "padded"], default="compact")
    ap.add_argument("--gemm-policy", choices=["layer", "auto", "wide", "stream_k"], default="layer",
                    help="grouped-GEMM kernel choice (default: the layer's own, from its shape)")
    ap.add_argument("--gather", choices=["auto", "on", "off"], default="auto",
                    help="up projection reads its rows from the tokens (no dispatch copy); auto: decode batches")
    ap.add_argument("--xe-layout", choices=["auto", "rows", "blocked"], default="auto",
                    help="storage of the expert rows (auto: the layer's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of a HIP graph of one step")
    ap.add_argument("--cpu-max-tokens", type=int, default=1024)
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="read a buffer of this size between timed steps (outside the timed events), so the 256 MB "
                         "Infinity Cache and L2 cannot carry data from one step to the next; 0: off")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer; runs on more than one GPU are not part of "
              "this build (other EP ranks are modelled as source partitions on the one GPU).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": 1 << 30, "launches": 3}))
        return 0

    import combine_router_softmax_amd as moe
    from combine_router_softmax_amd import COMPACT, PADDED
    from combine_router_softmax_amd.layer import MoEShare
    from synth import get_config, make_inputs

    cfg = get_config(args.workload)
    t_gen = time.perf_counter()
    d = make_inputs(cfg, 0)
    t_gen = time.perf_counter() - t_gen
    off = d["src_offsets"]
    N, B0 = int(off[-1]), int(off[1])
    layout = COMPACT if args.layout == "compact" else PADDED
    cap = None if layout == COMPACT else int(np.diff(off).max())
    act = torch.float32 if cfg.act == "f32" else torch.bfloat16
    share = MoEShare(n_tokens=N, hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts, top_k=cfg.top_k,
                     n_src=cfg.n_src, expert_lo=cfg.expert_lo, n_local=cfg.n_local, act_dtype=act, layout=layout,
                     capacity=cap, self_range=(0, B0),
                     blocked=None if args.xe_layout == "auto" else args.xe_layout == "blocked",
                     gather=None if args.gather == "auto" else args.gather == "on",
                     policy={"layer": None, "auto": moe.GEMM_AUTO, "wide": moe.GEMM_WIDE,
                             "stream_k": moe.GEMM_STREAM_K}[args.gemm_policy])
    share.set_weights(d["routed"], d["shared"])
    logits = torch.from_numpy(d["logits"]).cuda()
    offs = torch.from_numpy(off).cuda()
    x = d["x"].cuda()
    out = torch.zeros_like(x)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        share.step(logits, offs, x, out)
    torch.cuda.synchronize()

    # between timed steps (never inside the events): a read of a buffer twice
    # the Infinity Cache, so no step finds the previous one's weights or
    # activations in a cache. (A read, not a write: written flush data would
    # sit dirty in the cache and be written back during the next step.) The
    # previous step's own dirty lines are written back during the flush.
    flush_buf = torch.ones((args.flush_mb << 20) // 8, dtype=torch.int64, device="cuda") if args.flush_mb > 0 else None
    flush_sink = torch.zeros((), dtype=torch.int64, device="cuda")

    def flush():
        if flush_buf is not None:
            torch.sum(flush_buf, dim=0, out=flush_sink)

    def step_events(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    # per-call timing: eager steps with events around each call
    ev = {n: step_events(args.steps) for n in STEP_NAMES}
    est = step_events(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        est[i][0].record()
        share.step(logits, offs, x, out, events={n: ev[n][i] for n in STEP_NAMES})
        est[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_ms = float(np.mean([a.elapsed_time(b) for a, b in est]))
    per_call_us = {n: 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in STEP_NAMES}

    # the step as one HIP graph (one graph per batch shape, as the pages do with
    # CUDA graphs): same kernels, no host launch gaps
    graph_ms = None
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            share.step(logits, offs, x, out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            share.step(logits, offs, x, out)
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
        gst = step_events(args.steps)
        t0 = time.perf_counter()
        for i in range(args.steps):
            flush()
            gst[i][0].record()
            graph.replay()
            gst[i][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        graph_ms = float(np.mean([a.elapsed_time(b) for a, b in gst]))
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    st = int(share.lay["status"].item())

    counts = share.lay["counts"].cpu().numpy().astype(np.int64)
    row_of = share.lay["row_of"].cpu().numpy().astype(np.int64)
    model = algorithmic_model(cfg, counts, row_of, B0)
    if share.gather:
        # the up projection reads its rows from the tokens: no dispatch copy
        # (its events enclosed no work)
        model["bytes"]["dispatch"] = 0
        per_call_us["dispatch"] = 0.0
    breakdown = {}
    for n in STEP_NAMES:
        us = per_call_us[n]
        b = model["bytes"].get(n, 0)
        f = model["flops"].get(n, 0)
        breakdown[n] = {"us": round(us, 2), "GB/s": round(b / us / 1e3, 1) if us > 0 else None,
                        "TFLOP/s": round(f / us / 1e6, 1) if f and us > 0 else None}
    if share.gather:
        breakdown["dispatch"]["fused_into"] = "gemm_up"
    dc_bytes = model["bytes"]["dispatch"] + model["bytes"]["combine"]
    dc_us = per_call_us["dispatch"] + per_call_us["combine"]

    dom = max(("gemm_up", "gemm_down", "dispatch", "combine"), key=lambda n: per_call_us[n])
    dom_us = per_call_us[dom]
    flops = model["flops"].get(dom, 0)
    byts = model["bytes"][dom]
    mfma_bound = flops > 0 and flops / byts > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(flops / dom_us / 1e6, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(byts / dom_us / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = _traffic(cfg.name, dom)
    names = dict(KERNEL_OF_STEP, **(KERNEL_OF_STEP_FP8 if cfg.weight == "fp8_e4m3" else {}))
    roof["kernel"] = names.get(dom, dom)
    roof["algorithmic_bytes_per_launch"] = int(byts)
    roof["flops_per_launch"] = int(flops)
    roof["avg_launch_us"] = round(dom_us, 2)

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
        "timing": "hip_graph_replay" if graph_ms is not None else "eager",
        "cache_flush_mb": args.flush_mb,
        "ms_per_step_eager": round(eager_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layout": args.layout,
                   "xe_layout": "gathered" if share.gather else "blocked" if share.blocked else "rows",
                   "global_batch": N, "tokens_per_gpu": B0,
                   "source_ranks": cfg.n_src, "hidden": cfg.hidden, "n_experts": cfg.n_experts,
                   "top_k": cfg.top_k, "local_experts": cfg.n_local, "shared_expert": cfg.shared,
                   "inter": cfg.inter, "weights": cfg.weight, "parallelism": f"ep{cfg.n_experts // cfg.n_local}"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "dispatch_combine": {"GB/s": round(dc_bytes / dc_us / 1e3, 1), "frac_hbm": round(dc_bytes / dc_us / 1e3 /
                                                                                        HBM_PEAK_GBS, 4)},
        "breakdown": breakdown,
        "routing": {k: model[k] for k in ("M", "U", "active_experts", "max_rows_per_expert")},
        "status_word": st,
        "wall_s": round(wall, 3),
        "input_gen_s": round(t_gen, 2),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
