"""CPU emulation of the two-term MXFP6 activation encoding (test infrastructure).

The expert GEMMs of the HIP path feed the activations (x, then h) to gfx950's
block-scaled matrix cores as two MXFP6-E2M3 terms per 32-element block. This
module restates that encoding in numpy, from its definition, so that the error
it adds can be studied on the CPU at sizes a GPU test cannot sweep:

  s1 = max(floor(log2 max|v|) - 2, -126)
  hi = RNE_E2M3(v / 2^s1), saturated at +-7.5
  r  = v - hi * 2^s1                       (exact)
  s2 = max(floor(log2 max|r|) - 2, -126)
  lo = RNE_E2M3(r / 2^s2), saturated at +-7.5
  v ~ hi * 2^s1 + lo * 2^s2

E2M3 (OCP Microscaling Formats v1.0): sign, 2 exponent bits with bias 1, 3
mantissa bits, no Inf/NaN; magnitudes k/8 below 2, steps of 1/4 in [2, 4) and
of 1/2 in [4, 7.5].

It shares no code with the HIP library (whose encoder uses the hardware's
scaled conversion instructions) and none with the oracle's arithmetic; the
layer emulation below takes the oracle's dequantised weights and exact
reference only as inputs.
"""
from __future__ import annotations

import numpy as np

import oracle


def e2m3_round(a: np.ndarray) -> np.ndarray:
    """Nearest E2M3 magnitude to a >= 0, ties to the even code, saturating at
    7.5. In each binade the codes are consecutive integers a/step, so rounding
    a/step half to even is rounding the code half to even."""
    a = np.asarray(a, np.float64)
    step = np.where(a < 2.0, 0.125, np.where(a < 4.0, 0.25, 0.5))
    return np.minimum(np.rint(a / step) * step, 7.5)


def _block_exp(amax: np.ndarray) -> np.ndarray:
    _, e = np.frexp(amax)  # amax = m 2^e, m in [0.5, 1): floor(log2 amax) = e - 1
    s = np.where(amax > 0, e - 1 - 2, -126)
    return np.maximum(s, -126)


def _term(v: np.ndarray):
    """One E2M3 term of blocks v [..., 32]: (value of the term, its exponent)."""
    s = _block_exp(np.abs(v).max(axis=-1, keepdims=True))
    q = np.sign(v) * e2m3_round(np.abs(v) / np.ldexp(1.0, s))
    return q * np.ldexp(1.0, s), s


def encode2(v: np.ndarray) -> np.ndarray:
    """Value of the two-term encoding of rows v [..., K] (K a multiple of 32),
    as float64. v is taken as float32 first (the kernels encode fp32 values)."""
    v = np.asarray(v, np.float32).astype(np.float64)
    shp = v.shape
    b = v.reshape(*shp[:-1], shp[-1] // 32, 32)
    hi, _ = _term(b)
    lo, _ = _term(b - hi)
    return (hi + lo).reshape(shp)


def expert_outputs(x: np.ndarray, layer, e: int, encode: bool = True):
    """One expert on rows x [m][d] (float64 values of bf16 inputs): the exact
    float64 output and, with `encode`, the output with x and h passed through
    the two-term encoding (h rounded to float32 first, as the kernels hold it);
    accumulation in float64 (the kernels' fp32 accumulation adds ~1e-7)."""
    wg, wu, wd, bg, bu, bd = oracle.moe._expert_weights(layer, e)
    y_ref = oracle.expert_ffn(x, wg, wu, wd, bg, bu, bd)
    if not encode:
        return y_ref, None
    g, u = oracle.gate_up(encode2(x), wg, wu, bg, bu)
    h = oracle.swiglu(g, u).astype(np.float32)
    return y_ref, oracle.down(encode2(h), wd, bd)
