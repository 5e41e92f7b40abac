"""Pins of oracle.decode_e4m3fn / dequant_blockwise."""
import math

import numpy as np
import torch

from oracle import decode_e4m3fn, dequant_blockwise, e4m3fn_table
from synth import get_config
from synth.workloads import _quantize_blocks_e4m3


def test_all_codes_match_torch_float8_e4m3fn():
    ours = e4m3fn_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_known_codes():
    assert decode_e4m3fn(0x7E) == 448.0
    assert decode_e4m3fn(0xFE) == -448.0
    assert decode_e4m3fn(0x01) == 2.0 ** -9
    assert decode_e4m3fn(0x08) == 2.0 ** -6
    assert decode_e4m3fn(0x38) == 1.0
    assert decode_e4m3fn(0x00) == 0.0 and math.copysign(1, decode_e4m3fn(0x80)) == -1
    assert math.isnan(decode_e4m3fn(0x7F)) and math.isnan(decode_e4m3fn(0xFF))


def test_block_indexing():
    R, C = 256, 384
    codes = np.full((R, C), 0x38, dtype=np.uint8)           # every code decodes to 1.0
    scales = (10 * np.arange(2)[:, None] + np.arange(3)[None, :] + 1).astype(np.float32)
    w = dequant_blockwise(codes, scales)
    for (i, j) in [(0, 0), (127, 127), (128, 0), (0, 128), (255, 383), (130, 300), (127, 256)]:
        assert w[i, j] == scales[i // 128, j // 128]


def test_checkpoint_quantization_round_trip_error():
    # Dequantized synthetic fp8 weights sit within half an e4m3 step of the fp32 draw:
    # relative error <= 2**-4 for normal codes, absolute <= scale * 2**-10 near zero.
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[:128, :128] *= 50.0                                   # blocks with different scales
    codes, scales = _quantize_blocks_e4m3(w)
    deq = dequant_blockwise(codes, scales)
    sfull = np.repeat(np.repeat(scales, 128, 0), 128, 1).astype(np.float64)
    err = np.abs(deq - w)
    assert np.all(err <= np.maximum(np.abs(w) * 2.0 ** -4, sfull * 2.0 ** -10) * (1 + 1e-6))
    # the largest magnitude of each block maps to the largest code
    for bi in range(2):
        for bj in range(3):
            blk = codes[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] & 0x7F
            assert blk.max() == 0x7E
    assert get_config("kimi_k2_ep8").weight == "fp8_e4m3"
