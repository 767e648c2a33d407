"""GPU parity on seeded random shapes: the whole block through moe_forward
against the oracle, every output compared (the bars of test_gpu_parity). The
shapes are drawn from the range the calls accept (d, F multiples of 64 from
512, E up to 256, k up to 8, T from 1 to 600) so that the paths mix in ways the
hand-picked cases do not: decode and prefill kernels, the router's K split,
expert pairs with clamped passes, odd E, a half last K step, several passes or
row tiles per expert. The oracle's work is bounded so each case runs in
seconds."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import synth  # noqa: E402
from test_gpu_parity import _full_check  # noqa: E402


@pytest.fixture(scope="module")
def gu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gpu_util
    return gpu_util


def _shapes(n: int = 14, seed: int = 2026, many: bool = False):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 601))]))
        if many:   # the prefill kernels only
            T = int(rng.integers(65, 601))
        d = 64 * int(rng.integers(8, 57))          # 512 .. 3584
        F = 64 * int(rng.integers(8, 41))          # 512 .. 2560
        E = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 257))]))
        k = int(rng.integers(1, min(8, E) + 1))
        # the oracle dequantises every expert it touches: bound its work
        if T * k * d * F * 3 > 6e10 or E * d * F > 6e8:
            continue
        out.append(dict(T=T, d=d, F=F, E=E, k=k, seed=int(rng.integers(1000, 2000)),
                        zipf=bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("shape", _shapes() + _shapes(10, 7, many=True),
                         ids=lambda s: f"T{s['T']}-d{s['d']}-F{s['F']}-E{s['E']}-k{s['k']}")
def test_random_shape(gu, shape):
    _full_check(gu, synth.tiny_workload(**shape))


def _fp8_shapes(n: int = 8, seed: int = 31):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.integers(1, 65)) if len(out) % 2 else int(rng.integers(65, 601))
        d, F = 64 * int(rng.integers(8, 41)), 64 * int(rng.integers(8, 41))
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(8, E) + 1))
        if T * k * d * F * 3 > 4e10 or E * d * F > 4e8:
            continue
        out.append(dict(T=T, d=d, F=F, E=E, k=k, seed=int(rng.integers(3000, 4000))))
    return out


@pytest.mark.parametrize("shape", _fp8_shapes(), ids=lambda s: f"fp8-T{s['T']}-d{s['d']}-F{s['F']}-E{s['E']}-k{s['k']}")
def test_random_shape_fp8(gu, shape):
    """The FP8 expert FFN on MXFP4 weights converted on the GPU (the same numbers,
    so the MXFP4 oracle is the reference)."""
    import oracle
    from test_gpu_fp8 import _ffn_fp8_check, _fp8_layer_from_mxfp4
    w = synth.tiny_workload(**shape)
    L = w.layers[0]
    wt8 = _fp8_layer_from_mxfp4(gu, L)
    x = oracle.bf16_to_f64(w.x)
    _ffn_fp8_check(gu, w, wt8, lambda g: oracle.ffn_sorted(x, g["sorted_pair"], g["offsets"], w.k, L))


def _attn_shapes(n: int = 10, seed: int = 41):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B = int(rng.integers(1, 5))
        S = int(rng.integers(1, 3001))
        Tq = int(rng.integers(1, min(S, 400) + 1)) if len(out) % 2 else int(rng.integers(1, min(S, 6) + 1))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.integers(1, 9))
        window = 0 if rng.integers(0, 2) else int(rng.integers(1, S + 1))
        if B * Hq * Tq * S > 3e8:
            continue
        out.append(dict(B=B, Tq=Tq, S=S, Hq=Hq, Hkv=Hkv, window=window, seed=int(rng.integers(5000, 6000))))
    return out


@pytest.mark.parametrize("shape", _attn_shapes(),
                         ids=lambda d: f"attn-B{d['B']}-Tq{d['Tq']}-S{d['S']}-H{d['Hq']}/{d['Hkv']}-w{d['window']}")
def test_random_shape_attention(gu, shape):
    """Attention with sinks (causal, grouped heads, optional window, split or
    unsplit keys) against the oracle under the per-element bound."""
    from test_gpu_attention import _check
    _check(gu, **shape)
