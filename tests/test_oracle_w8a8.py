"""Pins of the W8A8 oracle (oracle/w8a8.py): the e4m3fn encoder, the 1 x 128
activation quantizer, the block-scaled fp8 product and the fp8 expert FFN.

The 1 x 128 activation scales and 128 x 128 weight scales come from Perplexity,
"Lower latency and higher throughput with multi-node DeepSeek deployment",
section Quantization; the scale rule (block max / 448) and RNE rounding are the
oracle's stated readings.
"""
import numpy as np
import pytest
import torch

from oracle import (
    COMPACT,
    PADDED,
    dequant_1x128,
    dequant_blockwise,
    e4m3fn_table,
    encode_e4m3fn_rne,
    gemm_w8a8,
    moe_layer,
    moe_layer_w8a8,
    quantize_1x128,
    swiglu_ffn,
    w8a8_ffn,
)
from synth.workloads import _quantize_blocks_e4m3

TAB = e4m3fn_table()
FINITE = [c for c in range(256) if not np.isnan(TAB[c])]


def _torch_codes(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ----------------------------------------------------------------------------- encoder
def test_every_finite_code_encodes_to_itself():
    vals = TAB[FINITE].astype(np.float32)
    codes = encode_e4m3fn_rne(vals)
    # +0 and -0 both give code 0 (the sign of zero is dropped); every other code is reproduced
    for c, got in zip(FINITE, codes):
        assert got == (0 if c in (0x00, 0x80) else c), (hex(c), hex(got))


def test_encoder_ties_go_to_even_by_hand():
    # with scale 1: 17 lies halfway between 16 (0x58, mantissa 0) and 18 (0x59, mantissa 1)
    # -> 16; 19 lies between 18 (0x59) and 20 (0x5A) -> 20; 2**-10 is half the smallest
    # subnormal 2**-9 (0x01) -> 0; 3 * 2**-10 is halfway between 0x01 and 0x02 -> 0x02;
    # 464 is not reached (clamped to 448 first).
    got = encode_e4m3fn_rne(np.array([17.0, 19.0, -17.0, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, 432.0],
                                     dtype=np.float32))
    assert list(got) == [0x58, 0x5A, 0xD8, 0x00, 0x02, 0x7E, 0x7E]


def test_encoder_matches_torch_float8_conversion():
    # library routine (torch's RNE float32 -> float8_e4m3fn) on midpoints, their float32
    # neighbours and random values over the whole range, subnormals included
    pos = TAB[0:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(3)
    rnd = (rng.uniform(-1, 1, 200_000) * 2.0 ** rng.integers(-12, 9, 200_000)).astype(np.float32)
    v = np.concatenate([mids, up, dn, -mids, -up, -dn, rnd])
    v = np.clip(v, -448, 448).astype(np.float32)
    ours = encode_e4m3fn_rne(v)
    ref = _torch_codes(v)
    # torch keeps the sign of a value that rounds to zero; the oracle writes code 0
    ref = np.where((ref & 0x7F) == 0, 0, ref)
    np.testing.assert_array_equal(ours, ref)


# ----------------------------------------------------------------------------- quantizer
def test_quantizer_reproduces_every_code_exhaustively():
    # blocks whose largest magnitude is exactly 448 * 2**j have the exact scale 2**j, so
    # every finite code placed in them comes back unchanged
    others = [c for c in FINITE if c not in (0x7E, 0x00, 0x80)]
    per = 127
    rows = []
    for j in (0, -5, 3):
        for i in range(0, len(others), per):
            chunk = others[i:i + per]
            codes = [0x7E] + chunk + [0x00] * (per - len(chunk))
            rows.append((np.array(codes, dtype=np.uint8), j))
    x = np.stack([TAB[c] * 2.0 ** j for c, j in rows]).astype(np.float32)
    q, s = quantize_1x128(x)
    for (c, j), qr, sr in zip(rows, q, s):
        assert sr[0] == np.float32(2.0 ** j)
        np.testing.assert_array_equal(qr, c)


def test_scale_closed_form_and_extremes():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((5, 512)) * np.array([1e-3, 1, 30, 0.02, 7])[:, None]).astype(np.float32)
    x[2, 128:256] = 0.0                                      # an all-zero block
    x[3, 300] = -5.0                                         # a negative largest magnitude
    q, s = quantize_1x128(x)
    assert q.shape == x.shape and q.dtype == np.uint8 and s.shape == (5, 4) and s.dtype == np.float32
    for r in range(5):
        for b in range(4):
            blk = x[r, 128 * b:128 * (b + 1)]
            amax = np.float32(np.abs(blk).max())
            if amax == 0:
                assert s[r, b] == 1.0 and not q[r, 128 * b:128 * (b + 1)].any()
                continue
            assert s[r, b] == np.float32(amax / np.float32(448.0))
            i = int(np.abs(blk).argmax())
            # the block's largest magnitude maps to +-448
            assert q[r, 128 * b + i] == (0xFE if blk[i] < 0 else 0x7E)


def test_scale_underflow_gives_scale_one():
    # a block whose largest magnitude is a float32 subnormal below 224 * 2**-149: its
    # quotient by 448 rounds to 0, so the scale is 1 and every code is 0
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 5] = np.float32(2.0 ** -143)
    x[0, 9] = -np.float32(2.0 ** -145)
    q, s = quantize_1x128(x)
    assert s[0, 0] == 1.0 and not q.any()
    # just above that bound the scale is the smallest subnormal and the codes are finite
    x[0, 5] = np.float32(2.0 ** -140)
    q, s = quantize_1x128(x)
    assert s[0, 0] == np.float32(2.0 ** -149) and q[0, 5] != 0 and np.all(~np.isnan(TAB[q]))


def test_quantizer_error_within_half_step():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 1024)) * 2.0 ** rng.integers(-8, 6, (64, 1))).astype(np.float32)
    x[:, 512:640] *= 1e-4                                    # blocks far below their neighbours
    q, s = quantize_1x128(x)
    deq = dequant_1x128(q, s)
    sfull = np.repeat(s, 128, axis=1).astype(np.float64)
    err = np.abs(deq - x)
    # half an e4m3 step: 2**-4 relative in the normal range, 2**-10 * scale below 2**-6 * scale;
    # the float32 quotient adds one float32 rounding
    bound = np.maximum(np.abs(x) * 2.0 ** -4, sfull * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)
    assert err.max() > 0


def test_quantizer_matches_torch_quantization():
    # the same rule written with torch's float32 ops and float8 conversion
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((16, 768)) * 3).astype(np.float32)
    xt = torch.from_numpy(x).view(16, 6, 128)
    amax = xt.abs().amax(dim=2)
    st = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    yt = (xt / st[:, :, None]).clamp(-448, 448)
    ref = yt.to(torch.float8_e4m3fn).view(torch.uint8).reshape(16, 768).numpy()
    ref = np.where((ref & 0x7F) == 0, 0, ref)
    q, s = quantize_1x128(x)
    np.testing.assert_array_equal(s, st.numpy())
    np.testing.assert_array_equal(q, ref)


# ----------------------------------------------------------------------------- block-scaled product
def _rand_fp8_weight(rng, n, k, spread=True):
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    if spread:
        w *= (2.0 ** rng.integers(-3, 4, (n // 128, k // 128))).repeat(128, 0).repeat(128, 1).astype(np.float32)
    return _quantize_blocks_e4m3(w)


def test_block_scaled_product_equals_dequantized_matmul():
    rng = np.random.default_rng(4)
    R, N, K = 37, 256, 384                                   # weight scales 2 x 3: a transposition shows
    x = (rng.standard_normal((R, K)) * 2.0 ** rng.integers(-4, 4, (R, K // 128)).repeat(128, 1)).astype(np.float32)
    aq, a_s = quantize_1x128(x)
    wq, w_s = _rand_fp8_weight(rng, N, K)
    got = gemm_w8a8(aq, a_s, wq, w_s)
    ref = dequant_1x128(aq, a_s) @ dequant_blockwise(wq, w_s).T
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_block_scaled_product_brute_force():
    rng = np.random.default_rng(6)
    R, N, K = 2, 128, 256
    aq = rng.choice(FINITE, (R, K)).astype(np.uint8)
    a_s = np.array([[0.5, 3.0], [2.0, 0.25]], dtype=np.float32)
    wq = rng.choice(FINITE, (N, K)).astype(np.uint8)
    w_s = np.array([[1.5, 0.125]], dtype=np.float32)
    got = gemm_w8a8(aq, a_s, wq, w_s)
    for r in range(R):
        for n in (0, 1, 77, 127):
            acc = 0.0
            for k in range(K):
                acc += TAB[aq[r, k]] * float(a_s[r, k // 128]) * TAB[wq[n, k]] * float(w_s[n // 128, k // 128])
            assert got[r, n] == pytest.approx(acc, rel=1e-12, abs=1e-9)


# ----------------------------------------------------------------------------- FFN and layer
def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_w8a8_ffn_within_fp8_bound_of_unquantized():
    # the unquantized SwiGLU on the same (dequantized) weights is the reference; two
    # 1 x 128 quantizations of activations stay within the 5e-2 fp8 tolerance
    rng = np.random.default_rng(7)
    H, I, R = 512, 256, 48
    w13q, s13 = _rand_fp8_weight(rng, 2 * I, H)
    w2q, s2 = _rand_fp8_weight(rng, H, I)
    x = (rng.standard_normal((R, H))).astype(np.float32)
    x[:, :128] *= 40.0                                       # blocks of different magnitude
    got = w8a8_ffn(x, w13q, s13, w2q, s2)
    ref = swiglu_ffn(x, dequant_blockwise(w13q, s13), dequant_blockwise(w2q, s2))
    err = _rel_l2(got, ref)
    assert 1e-3 < err < 5e-2, err


def test_w8a8_ffn_exact_when_nothing_rounds():
    # identity-like weights (code 1.0, scale 1) and inputs on the e4m3 grid with a 448 in
    # every block: the up product reproduces x exactly, so y = dequant(quantize(silu(x) * x))
    H = I = 256
    eye = np.zeros((I, H), dtype=np.uint8)
    eye[np.arange(I), np.arange(H)] = 0x38
    w13q = np.concatenate([eye, eye])
    s13 = np.ones((2 * I // 128, H // 128), dtype=np.float32)
    w2q = eye.copy()
    s2 = np.ones((H // 128, I // 128), dtype=np.float32)
    rng = np.random.default_rng(8)
    x = TAB[rng.choice([c for c in FINITE if c < 0x60 or 0x80 <= c < 0xE0], (4, H))].astype(np.float32)
    x[:, 0] = 448.0
    x[:, 128] = -448.0
    got = w8a8_ffn(x, w13q, s13, w2q, s2)
    h = np.array([[float(np.float32(v / (1 + np.exp(-float(v))) * v)) for v in row] for row in x.astype(np.float64)],
                 dtype=np.float32)
    # per-block half-step bound of the second quantization, from h alone
    sh = np.repeat(np.abs(h).reshape(4, 2, 128).max(2) / 448.0, 128, axis=1)
    assert np.all(np.abs(got - h) <= np.maximum(np.abs(h) * 2.0 ** -4, sh * 2.0 ** -10) * (1 + 1e-6))
    # and the largest |h| of each block comes back exactly
    for r in range(4):
        for b in range(2):
            i = 128 * b + int(np.abs(h[r, 128 * b:128 * (b + 1)]).argmax())
            assert got[r, i] == pytest.approx(float(h[r, i]), rel=1e-6)


@pytest.mark.parametrize("layout", [COMPACT, PADDED])
def test_moe_layer_w8a8_matches_unquantized_layer(layout):
    rng = np.random.default_rng(9)
    H, I, E, L, K = 256, 128, 16, 4, 4
    S, B = 4, 24
    off = np.arange(S + 1) * B
    N = S * B
    x = rng.standard_normal((N, H)).astype(np.float32)
    logits = rng.standard_normal((N, E)).astype(np.float32)
    w13, s13, w2, s2 = [], [], [], []
    for _ in range(L + 1):
        a, b = _rand_fp8_weight(rng, 2 * I, H)
        c, d = _rand_fp8_weight(rng, H, I)
        w13.append(a); s13.append(b); w2.append(c); s2.append(d)
    w13, s13, w2, s2 = map(np.stack, (w13, s13, w2, s2))
    shared = (w13[L:], w2[L:], s13[L:], s2[L:])
    q = moe_layer_w8a8(x, logits, off, K, 4, L, w13[:L], w2[:L], s13[:L], s2[:L], shared=shared, layout=layout)
    ref = moe_layer(x, logits, off, K, 4, L, w13[:L], w2[:L], s13[:L], s2[:L], shared=shared, layout=layout)
    # routing and layout are the unquantized layer's
    np.testing.assert_array_equal(q["topk_idx"], ref["topk_idx"])
    np.testing.assert_array_equal(q["layout"]["row_of"], ref["layout"]["row_of"])
    # dispatched codes are the source rows' codes
    row_of = q["layout"]["row_of"]
    for e in range(N * K):
        if row_of[e] >= 0:
            np.testing.assert_array_equal(q["xe_q"][row_of[e]], q["xq"][e // K])
    touched = np.unique(np.nonzero(row_of.reshape(N, K) >= 0)[0])
    lo, hi = q["self_range"]
    rows = np.union1d(touched, np.arange(lo, hi))
    err = _rel_l2(q["out"][rows], ref["out"][rows])
    assert 1e-3 < err < 5e-2, err
