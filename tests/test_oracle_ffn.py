"""Pins of oracle.silu / swiglu_ffn / grouped_ffn."""
import math

import numpy as np

from oracle import COMPACT, PADDED, dispatch, dispatch_layout, group_rows, grouped_ffn, route_topk, silu, swiglu_ffn


def test_silu_closed_forms():
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(np.array([1.0, -1.0, 2.5])),
                               [1 / (1 + math.exp(-1)), -1 / (1 + math.exp(1)), 2.5 / (1 + math.exp(-2.5))],
                               rtol=1e-15)
    big = silu(np.array([60.0, -60.0, 800.0, -800.0]))
    assert abs(big[0] - 60.0) < 1e-20 and abs(big[1]) < 1e-24
    assert big[2] == 800.0
    assert big[3] == 0.0


def test_swiglu_identity_and_permutation_weights():
    # W_gate = c*Id, W_up = Id, W2 = P (a non-symmetric permutation):
    # y[i] = silu(c * a[P^-1 i]) * a[P^-1 i]; swapping gate/up or transposing W2 fails.
    H = I = 5
    c = 0.7
    perm = [2, 0, 4, 1, 3]          # y[i] = h[perm[i]]
    P = np.zeros((H, I))
    for i, j in enumerate(perm):
        P[i, j] = 1.0
    w13 = np.concatenate([c * np.eye(I, H), np.eye(I, H)])
    a = np.array([[0.3, -1.2, 2.0, 0.0, -0.4], [1.0, 1.0, -3.0, 0.5, 0.25]])
    y = swiglu_ffn(a, w13, P)
    for r in range(2):
        for i in range(H):
            v = a[r, perm[i]]
            expect = (c * v) / (1 + math.exp(-c * v)) * v
            assert abs(y[r, i] - expect) < 1e-15


def test_swiglu_brute_force_loops():
    rng = np.random.default_rng(0)
    H, I, m = 6, 3, 4
    a = rng.standard_normal((m, H))
    w13 = rng.standard_normal((2 * I, H))
    w2 = rng.standard_normal((H, I))
    y = swiglu_ffn(a, w13, w2)
    for r in range(m):
        h = []
        for j in range(I):
            g = sum(a[r, k] * w13[j, k] for k in range(H))
            u = sum(a[r, k] * w13[I + j, k] for k in range(H))
            h.append(g / (1 + math.exp(-g)) * u)
        for n in range(H):
            assert abs(y[r, n] - sum(h[j] * w2[n, j] for j in range(I))) < 1e-12


def test_grouped_ffn_per_group_and_holes():
    rng = np.random.default_rng(1)
    N, E, K, S, H, I, L = 30, 8, 2, 3, 4, 2, 3
    z = rng.standard_normal((N, E)).astype(np.float32)
    idx, _ = route_topk(z, K)
    off = np.array([0, 10, 10, 30])
    x = rng.standard_normal((N, H))
    w13 = rng.standard_normal((L, 2 * I, H))
    w2 = rng.standard_normal((L, H, I))
    for layout, cap in [(COMPACT, 60), (PADDED, 20)]:
        lay = dispatch_layout(idx, off, 0, L, layout, cap)
        xe = dispatch(x, lay["row_of"], K, lay["rows"])
        ye = grouped_ffn(xe, lay, w13, w2)
        occupied = np.zeros(lay["rows"], dtype=bool)
        for g in range(L):
            rows = group_rows(lay, g)
            occupied[rows] = True
            for r in rows:
                # brute-force loops for one row of group g
                t = lay["row_token"][r]
                h = [0.0] * I
                for j in range(I):
                    gv = sum(x[t, k] * w13[g, j, k] for k in range(H))
                    uv = sum(x[t, k] * w13[g, I + j, k] for k in range(H))
                    h[j] = gv / (1 + math.exp(-gv)) * uv
                for n in range(H):
                    assert abs(ye[r, n] - sum(h[j] * w2[g, n, j] for j in range(I))) < 1e-12
        assert np.all(np.isnan(ye[~occupied]))
