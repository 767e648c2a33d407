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
