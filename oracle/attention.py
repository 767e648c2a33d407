"""Attention with sinks for the oracle (test infrastructure only).

Perplexity, "GPT-OSS el dia 0", section "Atenció: GQA amb Attention Sinks":
every attention head has a pretrained sink parameter that takes part in the
softmax; section "Nuclis per a GPT-OSS / Atenció de buidatge": the sink is an
extra term before the softmax, and an online softmax takes it into account by
starting its running maximum at the head's sink value (and its running
denominator at 1), in the first KV chunk only when the keys are split into
chunks. (The page's formula itself was lost in extraction.)

Reading used here: for query q of head h and keys k_j, values v_j of its KV
head (grouped-query attention: query head h uses KV head h // (Hq / Hkv)),
  z_j = scale * <q, k_j>   for the keys the query may see, -inf otherwise,
  out = sum_j exp(z_j) v_j / (exp(s_h) + sum_j exp(z_j)),
i.e. a softmax over [s_h, z_1, ..., z_S] whose sink entry has no value vector.
Visibility: queries are the last Tq of S positions (query i sits at position
S - Tq + i) and see keys j <= their position (causal); with a sliding window W
> 0, only keys j > position - W.
"""
from __future__ import annotations

import numpy as np


def visible(Tq: int, S: int, window: int = 0) -> np.ndarray:
    """[Tq][S] boolean mask of the keys each query sees."""
    qpos = S - Tq + np.arange(Tq)[:, None]
    j = np.arange(S)[None, :]
    m = j <= qpos
    if window > 0:
        m &= j > qpos - window
    return m


def attention_sink(q, k, v, sinks, scale: float, window: int = 0) -> np.ndarray:
    """q [B][Tq][Hq][D], k and v [B][S][Hkv][D], sinks [Hq] -> out [B][Tq][Hq][D],
    float64, with the sink entering each softmax's denominator only."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Tq, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    mask = visible(Tq, S, window)
    out = np.zeros((B, Tq, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            z = (q[b, :, h, :] @ k[b, :, g, :].T) * scale
            z = np.where(mask, z, -np.inf)
            s = float(sinks[h])
            m = np.maximum(z.max(axis=1, keepdims=True), s)
            p = np.exp(z - m)
            den = np.exp(s - m) + p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (p @ v[b, :, g, :]) / den
    return out


def attention_sink_chunked(q, k, v, sinks, scale: float, window: int, chunk: int) -> np.ndarray:
    """The same attention computed the way a split-KV kernel does: keys in chunks
    of `chunk`, each chunk an online-softmax partial (running max m, running
    denominator l, unnormalised output o), the sink taken in the first chunk
    only (m starts at the sink and l at 1 there; at -inf and 0 elsewhere), and
    the partials merged in chunk order. Equal to attention_sink up to rounding."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Tq, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    mask = visible(Tq, S, window)
    out = np.zeros((B, Tq, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            M, L, O = None, None, None
            for c0 in range(0, S, chunk):
                sl = slice(c0, min(S, c0 + chunk))
                z = (q[b, :, h, :] @ k[b, sl, g, :].T) * scale
                z = np.where(mask[:, sl], z, -np.inf)
                if c0 == 0:
                    m = np.full((Tq, 1), float(sinks[h]))
                    l = np.ones((Tq, 1))
                else:
                    m = np.full((Tq, 1), -np.inf)
                    l = np.zeros((Tq, 1))
                mn = np.maximum(m, z.max(axis=1, keepdims=True))
                safe = np.where(np.isfinite(mn), mn, 0.0)
                p = np.exp(z - safe)
                l = l * np.exp(m - safe) + p.sum(axis=1, keepdims=True)
                o = p @ v[b, sl, g, :]
                if M is None:
                    M, L, O = mn, l, o
                else:
                    Mn = np.maximum(M, mn)
                    sM = np.where(np.isfinite(Mn), Mn, 0.0)
                    a, c = np.exp(M - sM), np.exp(mn - sM)
                    L, O, M = L * a + l * c, O * a + o * c, Mn
            out[b, :, h, :] = O / L
    return out
