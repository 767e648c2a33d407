"""The allocation-free whole-block call (moe_forward_noalloc) through the C ABI:
its scratch is the library's own device array instead of a caller workspace,
and every output must be the same bytes as moe_forward's on the same inputs.
Two calls in a row on each path, the second with fewer tokens, so the second
runs on what the first left in the shared array."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import synth  # noqa: E402


@pytest.fixture(scope="module")
def gu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gpu_util
    return gpu_util


def _host(r: dict) -> dict:
    import torch
    torch.cuda.synchronize()
    out = {k: r[k].cpu().numpy() for k in ("topk_idx", "topk_w", "y_sorted")}
    out["out"] = r["out"].view(torch.int16).cpu().numpy()
    for i, name in enumerate(("counts", "offsets", "sorted_pair", "pair_row")):
        out[name] = r["perm"][i].cpu().numpy()
    return out


@pytest.mark.parametrize("shape,T2", [
    (dict(T=16, d=2880, F=2880, E=32, k=4, seed=1), 5),      # decode: fused front end
    (dict(T=200, d=512, F=576, E=16, k=4, seed=52), 130),    # separate launches (T > 64)
], ids=["decode", "prefill-path"])
def test_noalloc_equals_forward(gu, shape, T2):
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    w = synth.tiny_workload(**shape)
    L = w.layers[0]
    wt = gu.weights_dev(L)
    rng = np.random.default_rng(53)
    for T in (w.T, T2):
        xb = w.x if T == w.T else synth.bf16_bits(rng.standard_normal((T, w.d)))
        x = gu.bf16_dev(xb)
        print(f"[noalloc] {w.name} T={T}", flush=True)
        bufs = moe._outputs(T, w.d, w.E, w.k, x.device, None)
        for v in bufs.values():
            for t in (v if isinstance(v, tuple) else (v,)):
                t.view(torch.uint8).fill_(0xA5)   # stale bytes: every output must be written
        got = _host(moe.forward_noalloc(x, wt, w.k, bufs))
        ws = gu.workspace(T, w.d, w.F, w.E, w.k)
        ref = _host(moe.forward(x, wt, w.k, ws))
        for key in ref:
            assert np.array_equal(got[key].view(np.uint8), ref[key].view(np.uint8)), (T, key)


def test_noalloc_rejects_beyond_its_scratch(gu):
    """A batch whose scratch would not fit the array is refused before any
    launch, with the sizes in the message."""
    import sparse_moe_transformer_gemm_amd as moe
    L = moe.lib()
    cap = L.moe_forward_noalloc_max_bytes()
    assert cap == 32 << 20
    T = 4096
    assert L.moe_workspace_bytes(moe.Dims(T, 2880, 2880, 32, 4)) > cap
    w = synth.tiny_workload(T=16, d=2880, F=2880, E=32, k=4, seed=1)
    wt = gu.weights_dev(w.layers[0])
    x = gu.bf16_dev(np.zeros((T, 2880), np.uint16))
    with pytest.raises(moe.MoeError, match="scratch"):
        moe.forward_noalloc(x, wt, 4)
