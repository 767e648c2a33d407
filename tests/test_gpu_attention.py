"""Attention with per-head sinks through the C ABI against the CPU oracle
(oracle/attention.py): every output element, under the attention bars of
parity.py (each element within half a bf16 ulp plus 2^-8 of the oracle's
sum_j p_j |v_j| / l, the error that bf16 probabilities in the value product can
cause; mean relative error <= 5e-3), on ragged shapes, grouped heads, a sliding window, the split-KV path
(few queries: the keys are cut into chunks and merged, the sink in the first
chunk only) and the gpt-oss-20b-shaped decode and prefill workloads."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import parity  # noqa: E402
import synth  # noqa: E402


@pytest.fixture(scope="module")
def gu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gpu_util
    return gpu_util


def _check(gu, B, Tq, S, Hq, Hkv, window, seed, sinks=None):
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    q, k, v, s = synth.attention_inputs(seed, B, Tq, S, Hq, Hkv, 64)
    if sinks is not None:
        s = np.asarray(sinks, np.float32)
    print(f"[attn] B={B} Tq={Tq} S={S} Hq={Hq} Hkv={Hkv} window={window} chunks-ws="
          f"{moe.attention_workspace_bytes(B, Tq, S, Hq, Hkv, 64, window)}", flush=True)
    out = moe.attention_sink(gu.bf16_dev(q), gu.bf16_dev(k), gu.bf16_dev(v),
                             torch.from_numpy(s).cuda(), 0.125, window)
    torch.cuda.synchronize()
    f = oracle.bf16_to_f64
    qf, kf, vf, sf = f(q), f(k), f(v), s.astype(np.float64)
    ref = oracle.attention_sink(qf, kf, vf, sf, 0.125, window)
    abs_ref = oracle.attention_sink(qf, kf, np.abs(vf), sf, 0.125, window)
    m = parity.assert_attention_close(f(gu.bits_host(out)), ref, abs_ref, "attention out")
    print(f"[attn] {m}", flush=True)
    return out


@pytest.mark.parametrize("shape", [
    dict(B=2, Tq=37, S=100, Hq=16, Hkv=2, window=0, seed=90),     # ragged, grouped heads
    dict(B=1, Tq=64, S=64, Hq=8, Hkv=8, window=0, seed=91),       # one head per KV head
    dict(B=1, Tq=300, S=300, Hq=16, Hkv=2, window=128, seed=92),  # sliding window
    dict(B=4, Tq=1, S=3000, Hq=16, Hkv=2, window=0, seed=93),     # decode: split keys, merged
    dict(B=3, Tq=5, S=777, Hq=64, Hkv=8, window=0, seed=94),      # a few queries, split keys
    dict(B=2, Tq=3, S=5, Hq=4, Hkv=1, window=2, seed=95),         # tiny, window 2, G = 4
    dict(B=3, Tq=4, S=1000, Hq=16, Hkv=2, window=0, seed=99),     # 4 queries x 8 heads = 32 slots, causal in-tile
    dict(B=2, Tq=2, S=900, Hq=6, Hkv=2, window=300, seed=100),    # G = 3 packed, sliding window
    dict(B=1, Tq=1, S=8192, Hq=64, Hkv=8, window=128, seed=101),  # decode with a 128-key window
    dict(B=1, Tq=70, S=70, Hq=6, Hkv=2, window=0, seed=102),      # G = 3: two pieces per thread
    dict(B=2, Tq=50, S=120, Hq=2, Hkv=2, window=0, seed=103),     # G = 1: four pieces per thread
    dict(B=1, Tq=200, S=1000, Hq=8, Hkv=1, window=100, seed=104), # queries at the end, window
], ids=lambda d: f"B{d['B']}-Tq{d['Tq']}-S{d['S']}-H{d['Hq']}/{d['Hkv']}-w{d['window']}")
def test_attention_shapes(gu, shape):
    _check(gu, **shape)


def test_attention_without_sinks(gu):
    """A sink of -inf: plain causal softmax attention (split and unsplit)."""
    _check(gu, 2, 1, 2000, 16, 2, 0, 96, sinks=np.full(16, -np.inf))
    _check(gu, 1, 100, 100, 16, 2, 0, 97, sinks=np.full(16, -np.inf))


def test_attention_large_sinks(gu):
    """Sinks that dominate the softmax: outputs near zero, still within the bars."""
    _check(gu, 2, 1, 1500, 16, 2, 0, 98, sinks=np.full(16, 12.0))


@pytest.mark.parametrize("name", ["attn-decode", "attn-prefill"])
def test_attention_gpt_oss_workloads(gu, name):
    """The gpt-oss-20b attention shape (64 query heads, 8 KV heads, head size 64):
    16 decode queries against 8192-key caches, and a causal 8192-token prefill;
    every output compared."""
    c = synth.ATTN_WORKLOADS[name]
    _check(gu, c["B"], c["Tq"], c["S"], c["Hq"], c["Hkv"], c["window"], c["seed"])


def test_attention_deterministic(gu):
    import torch
    a = _check(gu, 4, 1, 3000, 16, 2, 0, 93)
    b = _check(gu, 4, 1, 3000, 16, 2, 0, 93)
    torch.cuda.synchronize()
    assert np.array_equal(gu.bits_host(a), gu.bits_host(b))
