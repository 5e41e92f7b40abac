"""OCP FP8 E4M3 ("e4m3fn") decoding and 128x128 block dequantization.

Test infrastructure only (see the package docstring).

Format (OCP 8-bit floating point specification, E4M3 variant): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; no infinities; the codes with
exponent 1111 and mantissa 111 are NaN; largest finite magnitude 448; exponent
field 0 encodes subnormals ``m/8 * 2**-6``.

Block scaling follows Perplexity, "Lower latency and higher throughput with
multi-node DeepSeek deployment", section Quantization: weights are quantized
statically with one scale per 128 x 128 tile, so a weight element is its decoded
code times the scale of the tile that contains it.

Pins: ``tests/test_oracle_fp8.py`` checks all 256 codes against
``torch.float8_e4m3fn`` and hand-derived values, and the block indexing against
hand-built scale patterns.
"""
from __future__ import annotations

import math

import numpy as np


def decode_e4m3fn(code: int) -> float:
    """Value of one e4m3fn code, from the bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3fn_table() -> np.ndarray:
    """float64[256]: decoded value of every code."""
    return np.array([decode_e4m3fn(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3fn_table()


def dequant_blockwise(codes, scales, block: int = 128) -> np.ndarray:
    """float64 weights from e4m3fn codes ``[R, C]`` and per-tile scales.

    ``W[i, j] = decode(codes[i, j]) * scales[i // block, j // block]``.
    """
    q = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.float64)
    R, C = q.shape
    assert s.shape == ((R + block - 1) // block, (C + block - 1) // block), (q.shape, s.shape)
    vals = _TABLE[q]
    rs = np.repeat(s, block, axis=0)[:R]
    return vals * np.repeat(rs, block, axis=1)[:, :C]
