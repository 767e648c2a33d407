"""FP8 block-scaled weights for the oracle (test infrastructure only).

The pages' serving engine ran the gpt-oss experts on Hopper as FP8 weights with
128x128 block scales, converted once from the released MXFP4 weights
(Perplexity, "GPT-OSS el dia 0", section "GPT-OSS a Hopper"). The element format
is not on the pages; it is the OCP 8-bit floating point E4M3 encoding:
  * bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  * exponent field 0 is subnormal: (m/8) * 2^-6; otherwise 2^(e-7) * (1 + m/8);
  * exponent 15 with mantissa 7 (0x7F, 0xFF) is NaN; there are no infinities
    (largest finite magnitude 448).
Block scaling (a reading of "128x128 block scales"): one float32 scale per
128 rows x 128 columns of a matrix W[N][K]; blocks at the edges are partial, so
the scale array is [ceil(N/128)][ceil(K/128)]:
  W[n][k] = E4M3(codes[n][k]) * scales[n // 128][k // 128].
Storage: codes [..., N, K] one byte per element, K contiguous.
"""
from __future__ import annotations

import numpy as np


def e4m3_value(code: int) -> float:
    """Value of one 8-bit E4M3 code, from its bit fields."""
    sign = (code >> 7) & 1
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = 2.0 ** (exp - 7) * (1.0 + man / 8.0)
    return -mag if sign else mag


E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequant_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 value of a block-scaled FP8 matrix: codes [..., N, K] (uint8),
    scales [..., ceil(N/128), ceil(K/128)] (float32) -> [..., N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape[-2:]
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    assert sc.shape[-2:] == ((N + 127) // 128, (K + 127) // 128), "one scale per 128x128 block"
    full = np.repeat(np.repeat(sc, 128, axis=-2), 128, axis=-1)[..., :N, :K]
    return E4M3[codes] * full
