"""Workload shapes and seeded synthetic inputs.

The shapes follow the serving set-ups the pages discuss (Perplexity, "Lower
latency and higher throughput with multi-node DeepSeek deployment", sections
Expert parallelism and GroupGEMM; Perplexity, "Enabling trillion-parameter
models on AWS EFA", section Evaluation; lehuy.net, "Decoding high-performance
EP kernels", section Our task). No dataset, checkpoint or routing trace is
used: every tensor is drawn from a seeded generator.

Recipe (all draws from numpy PCG64 seeded by ``SeedSequence(20250418,
spawn_key=(config, seed, tensor, part))``):

* tokens per source rank ``B_s``: fixed, or uniform on ``{1..b_max}``;
* activations ``x``: N(0, 1), stored in the activation dtype (bf16 by
  round-to-nearest-even from the fp32 draw);
* router logits: N(0, 1) in fp32, plus an optional per-expert bias where a
  seeded permutation ranks the experts and rank ``i`` (0-based) gets
  ``3 * (i + 1) ** -1.1`` (Zipf s = 1.1 scaled to a maximum of +3);
* expert weights: N(0, 0.02); for the fp8 checkpoint each 128 x 128 block is
  stored as OCP e4m3fn codes ``q = RNE(clamp(W / s, +-448))`` with
  ``s = absmax(block) / 448`` (``s = 1`` for an all-zero block). That is the
  offline, static weight quantization the pages describe; the layer itself
  only consumes ``q`` and ``s``.

This module holds no routing, layout, FFN or combine arithmetic.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

ROOT_SEED = 20250418

# tensor codes inside the spawn key
_T_BATCH, _T_X, _T_LOGITS, _T_PERM, _T_W13, _T_W2, _T_SW13, _T_SW2 = range(8)


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    n_src: int                 # S logical source ranks
    tokens_per_src: int        # B_s when fixed; 0 = draw B_s uniformly on {1..b_max}
    b_max: int
    hidden: int                # H
    n_experts: int             # E
    top_k: int                 # K
    n_local: int               # L local experts [expert_lo, expert_lo + L)
    inter: int                 # I (SwiGLU intermediate size)
    act: str                   # "f32" | "bf16"
    weight: str                # "f32" | "bf16" | "fp8_e4m3"
    shared: bool               # one shared expert on the self tokens
    zipf: str = "none"         # "none" | "perm" | "identity"
    expert_lo: int = 0
    weight_std: float = 0.02

    @property
    def fixed_batch(self) -> bool:
        return self.tokens_per_src > 0


CONFIGS = {
    # lehuy.net toy problem: 8 ranks, variable B_i, E = 16, two experts per GPU, K = 2.
    "tiny": Config("tiny", 0, n_src=8, tokens_per_src=0, b_max=16, hidden=128,
                   n_experts=16, top_k=2, n_local=2, inter=256, act="f32",
                   weight="f32", shared=False),
    # DeepSeek-V3 decode, single-node EP8 share (128 tokens per rank, local experts 0-31).
    "dsv3_decode_ep8": Config("dsv3_decode_ep8", 1, n_src=8, tokens_per_src=128, b_max=128,
                              hidden=7168, n_experts=256, top_k=8, n_local=32, inter=2048,
                              act="bf16", weight="bf16", shared=True),
    # DeepSeek-V3 decode, EP128 share (64 tokens per rank, local experts 0-1).
    "dsv3_decode_ep128": Config("dsv3_decode_ep128", 2, n_src=128, tokens_per_src=64, b_max=64,
                                hidden=7168, n_experts=256, top_k=8, n_local=2, inter=2048,
                                act="bf16", weight="bf16", shared=True),
    # DeepSeek-V3 prefill, EP8 share with Zipf-skewed routing.
    "dsv3_prefill_ep8": Config("dsv3_prefill_ep8", 3, n_src=8, tokens_per_src=4096, b_max=4096,
                               hidden=7168, n_experts=256, top_k=8, n_local=32, inter=2048,
                               act="bf16", weight="bf16", shared=True, zipf="perm"),
    # Kimi-K2 EP8 share: 384 experts, fp8 e4m3 weights with 128x128 block scales.
    "kimi_k2_ep8": Config("kimi_k2_ep8", 4, n_src=8, tokens_per_src=512, b_max=512,
                          hidden=7168, n_experts=384, top_k=8, n_local=48, inter=2048,
                          act="bf16", weight="fp8_e4m3", shared=True),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


def tiny_config(**overrides) -> Config:
    return get_config("tiny", **overrides)


def _rng(cfg: Config, seed: int, tensor: int, part: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=(cfg.cfg_id, seed, tensor, part))
    return np.random.Generator(np.random.PCG64(ss))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def batch_sizes(cfg: Config, seed: int = 0) -> np.ndarray:
    if cfg.fixed_batch:
        return np.full(cfg.n_src, cfg.tokens_per_src, dtype=np.int64)
    return _rng(cfg, seed, _T_BATCH).integers(1, cfg.b_max + 1, size=cfg.n_src).astype(np.int64)


def src_offsets_from_batches(b: np.ndarray) -> np.ndarray:
    off = np.zeros(len(b) + 1, dtype=np.int32)
    off[1:] = np.cumsum(b)
    return off


def expert_bias(cfg: Config, seed: int = 0) -> np.ndarray:
    """Per-expert logit bias (float32). Zero unless the config asks for Zipf skew."""
    E = cfg.n_experts
    bias = np.zeros(E, dtype=np.float64)
    if cfg.zipf == "none":
        return bias.astype(np.float32)
    if cfg.zipf == "perm":
        order = _rng(cfg, seed, _T_PERM).permutation(E)
    elif cfg.zipf == "identity":
        order = np.arange(E)
    else:
        raise ValueError(cfg.zipf)
    bias[order] = 3.0 * np.arange(1, E + 1, dtype=np.float64) ** -1.1
    return bias.astype(np.float32)


def make_routing_inputs(cfg: Config, seed: int = 0, batches: Optional[np.ndarray] = None) -> dict:
    """``B_s``, ``src_offsets`` (int32, S+1) and fp32 logits ``[N, E]``."""
    b = batch_sizes(cfg, seed) if batches is None else np.asarray(batches, dtype=np.int64)
    off = src_offsets_from_batches(b)
    N, E = int(off[-1]), cfg.n_experts
    logits = np.empty((N, E), dtype=np.float32)
    bias = expert_bias(cfg, seed)

    def fill(s):
        lo, hi = int(off[s]), int(off[s + 1])
        if hi > lo:
            r = _rng(cfg, seed, _T_LOGITS, s)
            logits[lo:hi] = r.standard_normal((hi - lo, E), dtype=np.float32) + bias

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(b))))
    return {"batches": b, "src_offsets": off, "logits": logits}


def _to_act(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(dtype)


def make_x(cfg: Config, seed: int, src_offsets: np.ndarray) -> torch.Tensor:
    """Activations ``[N, H]`` in the activation dtype (host tensor)."""
    N, H = int(src_offsets[-1]), cfg.hidden
    out = torch.empty((N, H), dtype=torch.float32 if cfg.act == "f32" else torch.bfloat16)

    def fill(s):
        lo, hi = int(src_offsets[s]), int(src_offsets[s + 1])
        if hi > lo:
            r = _rng(cfg, seed, _T_X, s)
            out[lo:hi] = _to_act(r.standard_normal((hi - lo, H), dtype=np.float32), cfg.act)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(src_offsets) - 1)))
    return out


def _quantize_blocks_e4m3(w: np.ndarray):
    """Static 128x128 block quantization of a fp32 weight matrix to e4m3fn codes.

    Returns ``(codes uint8 [R, C], scales float32 [R/128, C/128])``.
    """
    R, C = w.shape
    assert R % 128 == 0 and C % 128 == 0, "fp8 block scales need multiples of 128"
    blk = w.reshape(R // 128, 128, C // 128, 128)
    amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = blk / scale[:, None, :, None]
    q = np.clip(q, -448.0, 448.0).astype(np.float32).reshape(R, C)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _one_matrix(cfg: Config, rng: np.random.Generator, rows: int, cols: int):
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(cfg.weight_std)
    if cfg.weight == "f32":
        return torch.from_numpy(w), None
    if cfg.weight == "bf16":
        return torch.from_numpy(w).to(torch.bfloat16), None
    if cfg.weight == "fp8_e4m3":
        codes, scale = _quantize_blocks_e4m3(w)
        return torch.from_numpy(codes), torch.from_numpy(scale)
    raise ValueError(cfg.weight)


def make_expert_weights(cfg: Config, seed: int = 0, experts=None, shared: bool = False) -> dict:
    """Weights of the given global experts (default: the local ones), stacked.

    ``w13 [G, 2I, H]`` holds the gate rows ``0..I-1`` then the up rows
    ``I..2I-1``; ``w2 [G, H, I]``. fp8 checkpoints add ``s13 [G, 2I/128, H/128]``
    and ``s2 [G, H/128, I/128]``. With ``shared=True`` the single shared expert
    is returned instead (G = 1).
    """
    H, I = cfg.hidden, cfg.inter
    if shared:
        ids = [0]
        codes = (_T_SW13, _T_SW2)
    else:
        ids = list(range(cfg.expert_lo, cfg.expert_lo + cfg.n_local)) if experts is None else list(experts)
        codes = (_T_W13, _T_W2)
    G = len(ids)

    def gen(i):
        e = ids[i]
        a = _one_matrix(cfg, _rng(cfg, seed, codes[0], e), 2 * I, H)
        b = _one_matrix(cfg, _rng(cfg, seed, codes[1], e), H, I)
        return a, b

    with ThreadPoolExecutor(_threads()) as ex:
        mats = list(ex.map(gen, range(G)))
    out = {
        "w13": torch.stack([m[0][0] for m in mats]) if G else None,
        "w2": torch.stack([m[1][0] for m in mats]) if G else None,
        "s13": None,
        "s2": None,
        "experts": ids,
    }
    if cfg.weight == "fp8_e4m3" and G:
        out["s13"] = torch.stack([m[0][1] for m in mats])
        out["s2"] = torch.stack([m[1][1] for m in mats])
    return out


def make_inputs(cfg: Config, seed: int = 0, with_weights: bool = True, batches=None) -> dict:
    """Everything one layer step needs, as host tensors / arrays."""
    d = make_routing_inputs(cfg, seed, batches)
    d["x"] = make_x(cfg, seed, d["src_offsets"])
    if with_weights:
        d["routed"] = make_expert_weights(cfg, seed)
        d["shared"] = make_expert_weights(cfg, seed, shared=True) if cfg.shared else None
    d["cfg"] = cfg
    d["seed"] = seed
    return d
