"""The whole-block call (moe_forward) against the four separate calls, through
the C ABI: every output -- routing, permutation, y and out -- must be the same
bytes. At decode sizes moe_forward takes the fused front end (router partials
with the activation encode, then per-token selection with the permutation and
the pass table built by the last workgroup); elsewhere it chains the separate
launches. Its parity with the oracle is covered by test_gpu_parity.py, whose
layer runs go through moe_forward."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import synth  # noqa: E402

SHAPES = [
    dict(T=16, d=2880, F=2880, E=32, k=4, seed=1),   # decode-20b shape (fused front end)
    dict(T=1, d=512, F=512, E=4, k=4, seed=30),      # one token, E = k
    dict(T=37, d=512, F=704, E=8, k=2, seed=31),     # ragged T, d != F
    dict(T=50, d=512, F=640, E=16, k=1, seed=32),    # switch routing
    dict(T=64, d=576, F=640, E=256, k=8, seed=34),   # largest fused T, E and k
    dict(T=40, d=768, F=512, E=64, k=4, seed=44),    # F < d
    dict(T=8, d=4608, F=512, E=4, k=2, seed=38),     # K beyond the decode kernels: separate launches
    dict(T=128, d=512, F=512, E=32, k=4, seed=40),   # T above the decode limit: separate launches
    dict(T=200, d=2304, F=512, E=16, k=2, seed=52),  # many tokens, router K split in two
    dict(T=150, d=832, F=576, E=12, k=2, seed=57),   # many tokens, streaming down GEMM (pass table from the permutation)
]


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


def _same(a: dict, b: dict, what: str) -> None:
    for key in a:
        assert a[key].dtype == b[key].dtype and a[key].shape == b[key].shape, (what, key)
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (what, key)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"T{s['T']}-d{s['d']}-F{s['F']}-E{s['E']}-k{s['k']}")
def test_forward_equals_separate_calls(gu, shape):
    import sparse_moe_transformer_gemm_amd as moe
    w = synth.tiny_workload(**shape)
    L = w.layers[0]
    print(f"[forward] {w.name}", flush=True)
    wt = gu.weights_dev(L)
    ws = gu.workspace(w.T, w.d, w.F, w.E, w.k)
    x = gu.bf16_dev(w.x)
    fused = _host(moe.forward(x, wt, w.k, ws))
    ws2 = gu.workspace(w.T, w.d, w.F, w.E, w.k)
    sep = _host(moe.forward_calls(x, wt, w.k, ws2))
    _same(fused, sep, w.name)


@pytest.mark.parametrize("E", [16, 64])
def test_forward_reuses_workspace(gu, E):
    """Consecutive calls on one workspace with different tokens and batch sizes
    (the fused front end's arrival counter is cleared on every call)."""
    import sparse_moe_transformer_gemm_amd as moe
    w = synth.tiny_workload(T=48, d=512, F=512, E=E, k=4, seed=41)
    L = w.layers[0]
    wt = gu.weights_dev(L)
    ws = gu.workspace(w.T, w.d, w.F, w.E, w.k)
    ws_ref = gu.workspace(w.T, w.d, w.F, w.E, w.k)
    rng = np.random.default_rng(42)
    for T in (48, 5, 48, 17):
        xb = synth.bf16_bits(rng.standard_normal((T, w.d)))
        x = gu.bf16_dev(xb)
        print(f"[forward] reuse E={E} T={T}", flush=True)
        a = _host(moe.forward(x, wt, w.k, ws))
        b = _host(moe.forward_calls(x, wt, w.k, ws_ref))
        _same(a, b, f"T={T}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2], SHAPES[6], SHAPES[7],
                                   dict(T=300, d=576, F=640, E=12, k=4, seed=47)],
                         ids=["decode", "ragged", "wide-K", "prefill-path", "prefill-ragged"])
def test_ffn_stages_equal_the_call(gu, shape):
    """moe_expert_ffn_mxfp4_stage 0, 1, 2 in order write y_sorted byte for byte
    as moe_expert_ffn_mxfp4 does (decode and prefill kernels, ragged shapes)."""
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    w = synth.tiny_workload(**shape)
    L = w.layers[0]
    print(f"[stages] {w.name}", flush=True)
    wt = gu.weights_dev(L)
    ws = gu.workspace(w.T, w.d, w.F, w.E, w.k)
    x = gu.bf16_dev(w.x)
    idx, _ = moe.route(x, wt.w_router, wt.b_router, w.k, ws)
    perm = moe.permute(idx, w.E, ws)
    P = w.T * w.k
    y_call = moe.expert_ffn_mxfp4(x, perm[2], perm[1], wt, w.k, ws,
                                  torch.full((P, w.d), float("nan"), device=x.device))
    ws2 = gu.workspace(w.T, w.d, w.F, w.E, w.k)
    y_st = torch.full((P, w.d), float("nan"), device=x.device)
    for stage in range(3):
        moe.expert_ffn_mxfp4_stage(x, perm[2], perm[1], wt, w.k, ws2, y_st, stage)
    torch.cuda.synchronize()
    assert np.array_equal(y_call.cpu().numpy().view(np.uint32), y_st.cpu().numpy().view(np.uint32))
