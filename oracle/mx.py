"""MXFP4 decoding for the oracle (test infrastructure only).

Format (OCP Microscaling Formats (MX) v1.0; the pages only say the MoE weights
are MXFP4 -- Perplexity, "GPT-OSS el dia 0", section "GPT-OSS a Hopper"; Unsloth
tutorial mirror, paragraph "解释"):
  * element: FP4 E2M1 -- bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
    exponent field 0 is subnormal (value m/2), otherwise 2^(e-1) * (1 + m/2);
    no infinities or NaNs.
  * scale: E8M0 byte s -> 2^(s-127); s = 255 is NaN.
  * one scale per 32 consecutive elements along K.
Storage layout used throughout (a choice; the pages give none): a matrix row of
K elements is K/2 bytes, element k in byte k>>1, low nibble when k is even.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code, from its bit fields."""
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = man * 0.5
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + man * 0.5)
    return -mag if sign else mag


def e8m0_value(s: int) -> float:
    """Value of one E8M0 scale byte: 2^(s-127); 255 encodes NaN."""
    if s == 255:
        return float("nan")
    return 2.0 ** (s - 127)


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0 = np.array([e8m0_value(s) for s in range(256)], dtype=np.float64)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] packed bytes -> [..., K] 4-bit codes (even k = low nibble)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 value of an MXFP4 matrix: codes [..., N, K/2], scales [..., N, K/32]
    -> [..., N, K]; element (n, k) = E2M1[code(n, k)] * 2^(scales[n, k // 32] - 127)."""
    codes = unpack_codes(packed)
    K = codes.shape[-1]
    assert scales.shape[-1] * 32 == K, "one scale per 32 elements along K"
    vals = E2M1[codes]
    sc = E8M0[np.asarray(scales, dtype=np.uint8)]
    vals = vals.reshape(vals.shape[:-1] + (K // 32, 32)) * sc[..., None]
    return vals.reshape(codes.shape)
