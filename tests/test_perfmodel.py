"""Bench arithmetic against the pages' worked numbers (no GPU)."""
import subprocess
import sys
import os

import numpy as np

import bench
from synth import get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tokens_per_expert_worked_example():
    # batch 128, query length 2, top-8, EP128 = DP128 over 256 experts: m = 1024
    assert bench.tokens_per_expert(128, 2, 8, 128, 256) == 1024
    # at EP8 the same formula gives 64 (the page's figure caption prints 128 for this
    # case; the formula, not the caption, is taken as the definition)
    assert bench.tokens_per_expert(128, 2, 8, 8, 256) == 64


def test_groupgemm_formulas():
    assert bench.groupgemm_flops(3, 5, 7, 11) == 2 * 3 * 5 * 7 * 11
    assert bench.groupgemm_bytes(3, 5, 7, 11) == 3 * (5 * 7 + 11 * 7 + 5 * 11)
    # SwiGLU FFN per row: 2*H*2I + 2*I*H = 6*H*I flop
    H, I = 7168, 2048
    assert bench.groupgemm_flops(1, 1, H, 2 * I) + bench.groupgemm_flops(1, 1, I, H) == 6 * H * I


def test_algorithmic_model_counts():
    cfg = get_config("dsv3_decode_ep8")
    L, S, K = 32, 8, 8
    counts = np.zeros((L, S), dtype=np.int64)
    counts[0, 0] = 2
    counts[5, 3] = 1
    N = 4
    row_of = -np.ones(N * K, dtype=np.int64)
    row_of[[0, 9, 30]] = [0, 1, 2]             # tokens 0, 1, 3 have a local entry
    m = bench.algorithmic_model(cfg, counts, row_of, B0=2)
    assert m["M"] == 3 and m["U"] == 3 and m["active_experts"] == 2
    H, I = 7168, 2048
    w_up = 2 * I * H * 2
    assert m["bytes"]["gemm_up"] == 3 * w_up + (3 + 2) * (H + I) * 2
    assert m["bytes"]["dispatch"] == (3 + 3) * H * 2 + N * K * 4
    assert m["bytes"]["combine"] == (3 + 2 + 3) * H * 2 + N * K * 8
    # the shared expert as calls of its own: the routed GEMMs keep the routed
    # rows and weights, the shared entry holds one expert over the B0 rows,
    # and nothing is lost or counted twice
    a = bench.algorithmic_model(cfg, counts, row_of, B0=2, shared_apart=True)
    assert a["bytes"]["gemm_up"] == 2 * w_up + 3 * (H + I) * 2
    assert a["bytes"]["gemm_down"] == 2 * (H * I * 2) + 3 * (I + H) * 2
    assert a["bytes"]["shared"] == w_up + H * I * 2 + 2 * 2 * (H + I) * 2
    assert a["flops"]["shared"] == 6 * 2 * H * I and a["flops"]["gemm_up"] == 2 * 3 * H * 2 * I
    for d in ("bytes", "flops"):
        tot = sum(m[d][n] for n in ("gemm_up", "gemm_down"))
        assert sum(a[d][n] for n in ("gemm_up", "gemm_down", "shared")) == tot
    # the down projection's scatter: tokens 1 and 3 have one local row each and
    # lie outside the shared expert's tokens [0, 2): token 3 is scattered
    # (token 1 is a shared-expert token), so the combine skips one y row read
    # and one output row write
    sc = bench.algorithmic_model(cfg, counts, row_of, B0=2, scatter=True)
    assert sc["single_row_tokens_scattered"] == 1
    assert sc["bytes"]["combine"] == m["bytes"]["combine"] - 2 * H * 2
    assert sc["bytes"]["gemm_down"] == m["bytes"]["gemm_down"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
