"""The MoE block, stage by stage, in float64 (test infrastructure only).

Each function names the passage it follows. Page keys used below:
  [P3] Perplexity, "GPT-OSS el dia 0"
  [P4] Unsloth tutorial mirror, "第39章 使用 Unsloth 微调 gpt-oss"
  [P5] CSDN, "GPT-OSS-120B 4-bit 量化技术深度解析"
Readings of points the pages leave open are stated where they are used.
"""
from __future__ import annotations

import numpy as np

from .fp8 import dequant_fp8
from .mx import dequant


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- routing

def router_logits(x: np.ndarray, w_router: np.ndarray, b_router=None) -> np.ndarray:
    """l[t,e] = sum_k x[t,k] * W_r[k,e] + b_r[e], in float64.

    [P3] section "Nuclis per a GPT-OSS / MoE": the routing scheme scores every
    expert for every token; [P5] section "Unsloth 4-bit量化技术解析": the router is
    left unquantised, so W_r is plain fp32. The bias is present only where a
    workload supplies one."""
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64)
    if b_router is not None:
        l = l + np.asarray(b_router, np.float64)[None, :]
    return l


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, ordered by (logit descending,
    expert index ascending); exact ties go to the lower index first.

    [P4] paragraph "解释": top-4 of 32 (20b) / of 128 (120b) experts per token.
    The tie rule is a reading (the pages are silent)."""
    # a stable sort of -l keeps equal logits in ascending expert order
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def softmax_selected(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over the k selected logits only (not over all experts).

    [P3] section "MLP" ("Softmax després de Top-K") and section "Nuclis per a
    GPT-OSS / MoE" (softmax only across the top-k selected experts, unlike
    models that softmax over every expert). Max-subtracted; no temperature."""
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ex / ex.sum(axis=1, keepdims=True)


def route(x, w_router, b_router, k: int):
    """Router GEMM -> top-k -> softmax over the selected logits."""
    l = router_logits(x, w_router, b_router)
    idx = topk_select(l, k)
    return idx, softmax_selected(l, idx), l


# --------------------------------------------------------------------------- dispatch

def permute(idx: np.ndarray, E: int):
    """Group the (token, slot) pairs by expert.

    [P3] section "Nuclis per a GPT-OSS / MoE": dispatch selects the tokens of each
    expert. Pair q = t*k + j. Reading: inside an expert, pairs are in ascending
    token order (a token meets an expert at most once), i.e. the unique stable
    counting sort by expert.
    Returns counts[E], offsets[E+1] (exclusive prefix, offsets[E] = P),
    sorted_pair[P] (value q) and pair_row[P] (its inverse: row of pair q)."""
    flat = np.asarray(idx, np.int64).reshape(-1)
    P = flat.size
    sorted_pair = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    pair_row = np.empty(P, np.int64)
    pair_row[sorted_pair] = np.arange(P)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_pair.astype(np.int32), pair_row.astype(np.int32))


# --------------------------------------------------------------------------- experts

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z), with sigmoid evaluated without overflow."""
    z = np.asarray(z, np.float64)
    e = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return z * sig


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """[P3] section "MLP": SwiGLU activation, taken as silu(g) * u exactly
    (no clamp, no scaling constant, no offset on u)."""
    return silu(g) * u


def gate_up(xr: np.ndarray, wg: np.ndarray, wu: np.ndarray, bg: np.ndarray,
            bu: np.ndarray):
    """Pre-activation projections g = xr Wg^T + bg, u = xr Wu^T + bu
    (W [N][K] dequantised; xr [m][K]).

    [P3] section "MLP" ("Els experts tenen biaixos") and section "Nuclis per a
    GPT-OSS / MoE" (the bias enters the expert GEMM through its accumulators,
    i.e. it is added to each projection's output before the activation)."""
    g = xr @ wg.T + bg[None, :]
    u = xr @ wu.T + bu[None, :]
    return g, u


def down(h: np.ndarray, wd: np.ndarray, bd: np.ndarray) -> np.ndarray:
    """y = h Wd^T + bd (the down projection, bias added before routing weights)."""
    return h @ wd.T + bd[None, :]


def expert_ffn(xr: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
               bg: np.ndarray, bu: np.ndarray, bd: np.ndarray) -> np.ndarray:
    """One expert on rows xr [m][d]: y = (silu(g) * u) Wd^T + bd."""
    g, u = gate_up(xr, wg, wu, bg, bu)
    return down(swiglu(g, u), wd, bd)


def _expert_weights(layer, e: int):
    wg = dequant(layer.gate.codes[e], layer.gate.scales[e])
    wu = dequant(layer.up.codes[e], layer.up.scales[e])
    wd = dequant(layer.down.codes[e], layer.down.scales[e])
    return (wg, wu, wd, bf16_to_f64(layer.b_gate[e]), bf16_to_f64(layer.b_up[e]),
            bf16_to_f64(layer.b_down[e]))


def ffn_sorted(x: np.ndarray, sorted_pair: np.ndarray, offsets: np.ndarray, k: int,
               layer) -> np.ndarray:
    """Expert outputs in dispatch order: row p of expert e (offsets[e] <= p <
    offsets[e+1]) is FFN_e(x[sorted_pair[p] // k]). One expert is dequantised at
    a time (float64 copies of all experts would not fit in memory at full size)."""
    x = np.asarray(x, np.float64)
    E = offsets.size - 1
    d_out = layer.down.codes.shape[1]
    y = np.zeros((sorted_pair.size, d_out), np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        rows = x[np.asarray(sorted_pair[a:b], np.int64) // k]
        y[a:b] = expert_ffn(rows, *_expert_weights(layer, e))
    return y


def expert_ffn_fp8(xr, layer8, e: int, b_gate, b_up, b_down) -> np.ndarray:
    """One expert on rows xr with FP8 block-scaled weights (layer8: gate/up/down
    each (codes [E][N][K], scales [E][ceil(N/128)][ceil(K/128)])); the biases
    as bf16 bits [E][N]. The FFN itself is the same as expert_ffn.

    [P3] section "GPT-OSS a Hopper": the experts run as FP8 with 128x128 block
    scales; section "Nuclis per a GPT-OSS / MoE": biases in the accumulators."""
    wg = dequant_fp8(*[a[e] for a in layer8["gate"]])
    wu = dequant_fp8(*[a[e] for a in layer8["up"]])
    wd = dequant_fp8(*[a[e] for a in layer8["down"]])
    return expert_ffn(xr, wg, wu, wd, bf16_to_f64(b_gate[e]), bf16_to_f64(b_up[e]),
                      bf16_to_f64(b_down[e]))


def ffn_sorted_fp8(x, sorted_pair, offsets, k: int, layer8, b_gate, b_up, b_down) -> np.ndarray:
    """ffn_sorted with FP8 block-scaled expert weights."""
    x = np.asarray(x, np.float64)
    E = offsets.size - 1
    d_out = layer8["down"][0].shape[1]
    y = np.zeros((sorted_pair.size, d_out), np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        y[a:b] = expert_ffn_fp8(x[np.asarray(sorted_pair[a:b], np.int64) // k], layer8, e,
                                b_gate, b_up, b_down)
    return y


def round_bf16(w: np.ndarray) -> np.ndarray:
    """Routing weights as the GPU holds them (float32), rounded to the nearest
    bf16 (ties to even), as float64.

    [P3] section "Nuclis per a GPT-OSS / MoE": computing the expert (routing)
    weights in bfloat16 was critical for matching the reference numerics."""
    f = np.ascontiguousarray(np.asarray(w, np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def combine(y_sorted: np.ndarray, pair_row: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t,j] * y_sorted[pair_row[t*k + j]]  (float64, unrounded).

    [P3] section "Nuclis per a GPT-OSS / MoE": combine performs the weighted
    accumulation of the experts' outputs. The down-projection bias is inside
    y, so it is weighted too."""
    T, k = w.shape
    rows = np.asarray(pair_row, np.int64).reshape(T, k)
    out = np.zeros((T, y_sorted.shape[1]), np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y_sorted[rows[:, j]]
    return out


def moe_layer(x_bits: np.ndarray, layer, k: int) -> dict:
    """The whole block on bf16 input bits: every stage's output, float64."""
    x = bf16_to_f64(x_bits)
    E = layer.w_router.shape[1]
    idx, w, logits = route(x, layer.w_router, layer.b_router, k)
    counts, offsets, sorted_pair, pair_row = permute(idx, E)
    y = ffn_sorted(x, sorted_pair, offsets, k, layer)
    out = combine(y, pair_row, w)
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                sorted_pair=sorted_pair, pair_row=pair_row, y_sorted=y, out=out)


def dense_moe(x_bits: np.ndarray, layer, k: int) -> np.ndarray:
    """The same block written densely, with no dispatch: every expert runs on
    every token and the result is masked by the routing. Tiny shapes only."""
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    E = layer.w_router.shape[1]
    idx, w, _ = route(x, layer.w_router, layer.b_router, k)
    gate = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            gate[t, idx[t, j]] = w[t, j]
    out = np.zeros((T, layer.down.codes.shape[1]))
    for e in range(E):
        out += gate[:, e:e + 1] * expert_ffn(x, *_expert_weights(layer, e))
    return out


# --------------------------------------------------------------------------- stack

def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """n = x / sqrt(mean(x^2) + eps) * gain, per row, float64.

    [P5] section "推理优化": rms_norm_eps = 1e-05."""
    x = np.asarray(x, np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(gain, np.float64)
