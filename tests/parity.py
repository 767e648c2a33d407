"""Parity metrics shared by the GPU tests (test infrastructure).

Tolerance on bf16 outputs (ref is the unrounded float64 oracle value):
  * excess error: max_i (|out_i - ref_i| - half_ulp_bf16(ref_i))^+ <= 2e-2 * RMS(ref),
    where half_ulp_bf16(v) = 2^(floor(log2|v|) - 8) is the rounding error that even a
    correctly rounded bf16 result may carry. The literal max|err| <= 2e-2 * RMS(ref)
    cannot be met by any bf16 output on the wide-expert workload (a correctly rounded
    result already scores 2.5e-2 there), so the excess form is the gate and the
    literal figure is reported beside it.
  * mean relative error: sum|out - ref| / sum|ref| <= 5e-3.
RMS is over every element of the checked tensor.

Attention outputs (assert_attention_close) carry a per-element bound instead of
the RMS-relative one, because their magnitudes span orders of magnitude along a
causal sequence (an early query averages a few values, a late one thousands).
The kernel rounds each probability to bf16 (relative error <= 2^-9) before the
probability-times-value product and sums the row total from the unrounded fp32
probabilities, so out = sum_j p~_j v_j / l with |p~_j - p_j| <= 2^-9 p_j, and

    |out - ref| <= half_ulp_bf16(out) + 2^-9 * sum_j p_j |v_j| / l + (fp32 terms).

The gate is that bound with the 2^-9 term doubled (the fp32 score, exponential
and accumulation errors are near 2^-20 of the same sum), where
sum_j p_j |v_j| / l is the oracle's attention with |v| as the values; the mean
relative error bar above applies as well.
"""
from __future__ import annotations

import numpy as np

from oracle import bf16_to_f64

EXCESS_TOL = 2e-2
MEAN_REL_TOL = 5e-3


def half_ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(ref, np.float64))
    _, e = np.frexp(a)  # a = m * 2^e with m in [0.5, 1): floor(log2 a) = e - 1
    return np.ldexp(1.0, e - 1 - 8)


def error_metrics(out: np.ndarray, ref: np.ndarray, bf16_out: bool = True) -> dict:
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(out - ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    slack = half_ulp_bf16(ref) if bf16_out else 0.0
    excess = np.maximum(err - slack, 0.0)
    return dict(
        rms=rms,
        literal=float(err.max() / rms) if err.size else 0.0,
        excess=float(excess.max() / rms) if err.size else 0.0,
        mean_rel=float(err.sum() / np.abs(ref).sum()) if err.size else 0.0,
    )


def assert_close(out, ref, what: str = "", bf16_out: bool = True) -> dict:
    m = error_metrics(out, ref, bf16_out)
    assert m["excess"] <= EXCESS_TOL and m["mean_rel"] <= MEAN_REL_TOL, (what, m)
    return m


def bf16_out_to_f64(bits) -> np.ndarray:
    return bf16_to_f64(np.asarray(bits, np.uint16))


def assert_attention_close(out, ref, abs_ref, what: str = "") -> dict:
    """out: bf16 results as float64; ref: the oracle's attention; abs_ref: the
    oracle's attention of the same queries and keys with |v| as the values."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    m = error_metrics(out, ref)
    err = np.abs(out - ref)
    bound = half_ulp_bf16(np.maximum(np.abs(out), np.abs(ref))) + 2.0 ** -8 * np.asarray(abs_ref, np.float64)
    ratio = err / bound
    m["bound_ratio"] = float(ratio.max()) if err.size else 0.0
    assert m["bound_ratio"] <= 1.0 and m["mean_rel"] <= MEAN_REL_TOL, (what, m)
    return m
