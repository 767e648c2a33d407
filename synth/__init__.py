"""Seeded synthetic inputs for the sparse-MoE block.

This module is the only code shared by the CPU oracle and the HIP path. It draws
random numbers, casts them to their storage types (bf16 bit patterns, packed
MXFP4 nibbles, E8M0 scale bytes) and nothing else: no step of the method
(router, top-k, softmax, dispatch, expert FFN, combine, normalisation) is
computed here, and no decoding of the formats either.

Shapes and distributions follow gpt-oss MoE layers: hidden width 2880 (Perplexity,
"GPT-OSS el dia 0", section "Ajustaments de rendiment"), 32 experts with top-4 for
the 20b model and 128 experts with top-4 for the 120b model (Unsloth tutorial
mirror, "第39章 使用 Unsloth 微调 gpt-oss", paragraph "解释").

Generator contract (stated once, used by tests and the bench):
  x          bf16 bits  [T][d]       ~ N(0, 1)
  w_router   fp32       [d][E]       ~ N(0, 0.02)       (std, not variance)
  b_router   fp32       [E] or None  -1.1 * ln(rank), rank a random permutation of 1..E
                                     (only the 120b-like workload: a log-Zipf(1.1) prior)
  gate, up   MXFP4      [E][F][d]    codes: uniform random bytes, i.e. two independent
  down       MXFP4      [E][d][F]    uniform nibbles 0..15 per byte; element k of a row
                                     is the low nibble of byte k>>1 when k is even, the
                                     high nibble when odd; scales: E8M0 bytes uniform in
                                     121..124 (exponents -6..-3), one per 32 K-elements
  b_gate/up  bf16 bits  [E][F]       ~ N(0, 0.01)
  b_down     bf16 bits  [E][d]       ~ N(0, 0.01)
  gain       bf16 bits  [d]          ~ N(1, 0.02)       (stacked workload only)
bf16 casting: float64 -> float32 (round to nearest even) -> bf16 (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterator, List, Optional

import numpy as np

__all__ = [
    "bf16_bits", "MX4", "LayerParams", "Workload", "WORKLOADS", "draw_layer",
    "workload", "stack_layer", "tiny_workload", "fp8_weights", "attention_inputs", "ATTN_WORKLOADS",
]


def bf16_bits(a) -> np.ndarray:
    """Storage cast: float64 -> float32 (RNE) -> bf16 bit pattern (RNE), as uint16."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    # round-to-nearest-even on the 16 dropped bits (inputs here are finite)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


@dataclass
class MX4:
    """One MXFP4 weight tensor for all experts: packed E2M1 codes and E8M0 scales."""
    codes: np.ndarray   # uint8 [E][N][K/2]
    scales: np.ndarray  # uint8 [E][N][K/32]

    @property
    def nbytes(self) -> int:
        return self.codes.nbytes + self.scales.nbytes


@dataclass
class LayerParams:
    w_router: np.ndarray             # float32 [d][E]
    b_router: Optional[np.ndarray]   # float32 [E] or None
    gate: MX4                        # N=F, K=d
    up: MX4                          # N=F, K=d
    down: MX4                        # N=d, K=F
    b_gate: np.ndarray               # bf16 bits [E][F]
    b_up: np.ndarray                 # bf16 bits [E][F]
    b_down: np.ndarray               # bf16 bits [E][d]
    gain: Optional[np.ndarray] = None  # bf16 bits [d] (pre-norm gain, stacked workload)

    @property
    def expert_bytes(self) -> int:
        """Bytes of one expert's MXFP4 weights and bf16 biases."""
        E = self.w_router.shape[1]
        tot = self.gate.nbytes + self.up.nbytes + self.down.nbytes
        tot += self.b_gate.nbytes + self.b_up.nbytes + self.b_down.nbytes
        return tot // E


@dataclass
class Workload:
    name: str
    T: int
    d: int
    F: int
    E: int
    k: int
    seed: int
    x: np.ndarray                          # bf16 bits [T][d]
    layers: List[LayerParams] = field(default_factory=list)
    n_layers: int = 1
    eps: float = 1e-5


def _mx4(rng: np.random.Generator, E: int, N: int, K: int) -> MX4:
    assert K % 32 == 0
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(121, 125, (E, N, K // 32), dtype=np.uint8)
    return MX4(codes, scales)


def draw_layer(rng: np.random.Generator, d: int, F: int, E: int, zipf: bool = False,
               with_gain: bool = False) -> LayerParams:
    """Draw one MoE layer's parameters in a fixed order from `rng`."""
    gain = None
    if with_gain:
        gain = bf16_bits(1.0 + 0.02 * rng.standard_normal(d))
    w_r = (rng.standard_normal((d, E)) * 0.02).astype(np.float32)
    b_r = None
    if zipf:
        b_r = (-1.1 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)
    gate = _mx4(rng, E, F, d)
    up = _mx4(rng, E, F, d)
    down = _mx4(rng, E, d, F)
    b_gate = bf16_bits(rng.standard_normal((E, F)) * 0.01)
    b_up = bf16_bits(rng.standard_normal((E, F)) * 0.01)
    b_down = bf16_bits(rng.standard_normal((E, d)) * 0.01)
    return LayerParams(w_r, b_r, gate, up, down, b_gate, b_up, b_down, gain)


# The five workloads: tiny, decode (20b-like), prefill (20b-like), 120b-like wide
# experts with a skewed router, and a 24-block pre-norm stack.
WORKLOADS = {
    0: dict(name="tiny", T=128, d=512, F=512, E=32, k=4, seed=0, zipf=False, n_layers=1),
    1: dict(name="decode-20b", T=16, d=2880, F=2880, E=32, k=4, seed=1, zipf=False, n_layers=1),
    2: dict(name="prefill-20b", T=8192, d=2880, F=2880, E=32, k=4, seed=2, zipf=False, n_layers=1),
    3: dict(name="wide-120b", T=4096, d=2880, F=2880, E=128, k=4, seed=3, zipf=True, n_layers=1),
    4: dict(name="stack24-20b", T=2048, d=2880, F=2880, E=32, k=4, seed=4, zipf=False, n_layers=24),
}


def workload(i: int, with_layers: bool = True) -> Workload:
    """Build workload `i`. For the stacked workload only layer 0 is drawn here
    (its stream continues after x); other layers come from `stack_layer`."""
    c = WORKLOADS[i]
    rng = np.random.default_rng(c["seed"])
    x = bf16_bits(rng.standard_normal((c["T"], c["d"])))
    w = Workload(c["name"], c["T"], c["d"], c["F"], c["E"], c["k"], c["seed"], x,
                 n_layers=c["n_layers"])
    if with_layers:
        w.layers.append(draw_layer(rng, c["d"], c["F"], c["E"], zipf=c["zipf"],
                                   with_gain=c["n_layers"] > 1))
    return w


def stack_layer(i: int, l: int) -> LayerParams:
    """Layer l (0-based) of a stacked workload: layer 0 continues the workload's
    own stream after x; layer l >= 1 uses its own generator seeded seed+l."""
    c = WORKLOADS[i]
    if l == 0:
        return workload(i).layers[0]
    rng = np.random.default_rng(c["seed"] + l)
    return draw_layer(rng, c["d"], c["F"], c["E"], zipf=c["zipf"], with_gain=True)


def stack_layers(i: int) -> Iterator[LayerParams]:
    for l in range(WORKLOADS[i]["n_layers"]):
        yield stack_layer(i, l)


def fp8_weights(rng: np.random.Generator, E: int, N: int, K: int):
    """Random FP8-E4M3 block-scaled weights for one [E][N][K] tensor: codes with a
    uniform sign, a uniform exponent field in 4..11 and a uniform mantissa (no
    NaN codes), and one float32 scale per 128x128 block drawn as 2^u * (1 + v),
    u uniform in -9..-7, v uniform in [0, 1). Returns (codes uint8 [E][N][K],
    scales float32 [E][ceil(N/128)][ceil(K/128)])."""
    sign = rng.integers(0, 2, (E, N, K), dtype=np.uint8)
    expf = rng.integers(4, 12, (E, N, K), dtype=np.uint8)
    man = rng.integers(0, 8, (E, N, K), dtype=np.uint8)
    codes = (sign << 7) | (expf << 3) | man
    nb, kb = (N + 127) // 128, (K + 127) // 128
    u = rng.integers(-9, -6, (E, nb, kb))
    v = rng.random((E, nb, kb))
    scales = (np.exp2(u) * (1.0 + v)).astype(np.float32)
    return codes.astype(np.uint8), scales


def attention_inputs(seed: int, B: int, Tq: int, S: int, Hq: int, Hkv: int, D: int):
    """Seeded inputs of one attention call: q [B][Tq][Hq][D], k and v [B][S][Hkv][D]
    as bf16 bits, each element ~ N(0, 1); sinks [Hq] float32 ~ N(1, 1) (one per
    query head). Drawn in that order from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    q = bf16_bits(rng.standard_normal((B, Tq, Hq, D)))
    k = bf16_bits(rng.standard_normal((B, S, Hkv, D)))
    v = bf16_bits(rng.standard_normal((B, S, Hkv, D)))
    sinks = (1.0 + rng.standard_normal(Hq)).astype(np.float32)
    return q, k, v, sinks


# Attention workloads of the gpt-oss-20b shape (64 query heads, 8 KV heads,
# head size 64): an 8192-token prefill (causal; the full-attention layers) and
# a decode step of 16 sequences against 8192-token KV caches.
ATTN_WORKLOADS = {
    "attn-prefill": dict(B=1, Tq=8192, S=8192, Hq=64, Hkv=8, D=64, window=0, seed=80),
    "attn-decode": dict(B=16, Tq=1, S=8192, Hq=64, Hkv=8, D=64, window=0, seed=81),
}


def tiny_workload(T: int, d: int, F: int, E: int, k: int, seed: int, zipf: bool = False,
                  scale_lo: int = 121, scale_hi: int = 124) -> Workload:
    """A workload of arbitrary small shape with the same distributions."""
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((T, d)))
    w = Workload(f"T{T}-d{d}-F{F}-E{E}-k{k}-s{seed}", T, d, F, E, k, seed, x)
    lay = draw_layer(rng, d, F, E, zipf=zipf)
    if (scale_lo, scale_hi) != (121, 124):
        for m in (lay.gate, lay.up, lay.down):
            m.scales[...] = rng.integers(scale_lo, scale_hi + 1, m.scales.shape, dtype=np.uint8)
    w.layers.append(lay)
    return w
