"""The whole-block call under HIP graph capture: moe_forward allocates nothing,
never synchronises the host and clears its one counter with a kernel (no memset
node), so a serving loop can capture it once and replay it. The graph is
replayed several times, with the program's own eager calls and synchronisations
between the replays and new inputs copied into the captured buffers; every
replay must give the same bytes as an eager call on the same inputs."""
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


def _snapshot(r: dict) -> dict:
    import torch
    out = {k: r[k].clone() for k in ("topk_idx", "topk_w", "y_sorted")}
    out["out"] = r["out"].view(torch.int16).clone()
    for i, name in enumerate(("counts", "offsets", "sorted_pair", "pair_row")):
        out[name] = r["perm"][i].clone()
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("shape", [
    dict(T=16, d=2880, F=2880, E=32, k=4, seed=1),   # decode-20b shape: the fused front end
    dict(T=200, d=512, F=576, E=16, k=4, seed=48),   # separate launches (T > 64)
    dict(T=200, d=2304, F=512, E=16, k=2, seed=52),  # router K split (partials, then the selection launch)
    dict(T=150, d=832, F=576, E=12, k=2, seed=57),   # streaming down GEMM, pass table from the permutation
], ids=["decode", "prefill-path", "k-split", "streaming-down"])
def test_forward_graph_replays(gu, shape):
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    w = synth.tiny_workload(**shape)
    L = w.layers[0]
    T, d, E, k = w.T, w.d, w.E, w.k
    wt = gu.weights_dev(L)
    ws = gu.workspace(T, d, w.F, E, k)
    x = gu.bf16_dev(w.x)
    bufs = moe._outputs(T, d, E, k, x.device, None)
    print(f"[graph] {w.name}", flush=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up on the capture stream
        moe.forward(x, wt, k, ws, bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(x, wt, k, ws, bufs)
    torch.cuda.synchronize()

    rng = np.random.default_rng(49)
    ws_eager = gu.workspace(T, d, w.F, E, k)
    for rep in range(4):
        xb = w.x if rep == 0 else synth.bf16_bits(rng.standard_normal((T, d)))
        x.copy_(gu.bf16_dev(xb))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(bufs)
        # the program's own eager work between replays, on other buffers
        ref = _snapshot(moe.forward(gu.bf16_dev(xb), wt, k, ws_eager))
        for key in ref:
            assert np.array_equal(got[key].view(np.uint8), ref[key].view(np.uint8)), (rep, key)
        print(f"[graph] {w.name} replay {rep} equal to eager", flush=True)


@pytest.mark.parametrize("shape", [
    dict(T=16, d=2880, F=2880, E=32, k=4, seed=1),   # decode front end
    dict(T=200, d=2304, F=512, E=16, k=2, seed=52),  # many tokens, router K split
], ids=["decode", "k-split"])
def test_stack_block_graph_replays(gu, shape):
    """One stack block with its fused glue (moe_forward_residual_rmsnorm: the
    block, then combine + residual add + next pre-norm in one pass), captured
    with the residual stream and the normalised activations updated in place,
    as a captured decode loop would run it. Each replay advances the stream by
    one block; it must equal the same block run eagerly on copies."""
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    w = synth.tiny_workload(**shape)
    L = w.layers[0]
    T, d, E, k = w.T, w.d, w.E, w.k
    wt = gu.weights_dev(L)
    ws = gu.workspace(T, d, w.F, E, k)
    rng = np.random.default_rng(53)
    n = gu.bf16_dev(w.x)
    resid = gu.bf16_dev(synth.bf16_bits(rng.standard_normal((T, d)) * 3))
    gain = gu.bf16_dev(synth.bf16_bits(1 + 0.02 * rng.standard_normal(d)))
    bufs = moe._outputs(T, d, E, k, n.device, None, store_out=False)
    print(f"[graph] stack block {w.name}", flush=True)

    def block():
        moe.forward_residual_rmsnorm(n, wt, k, ws, resid, gain, 1e-5, resid_out=resid, n_out=n,
                                     bufs=bufs)

    n0, r0 = n.clone(), resid.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up on the capture stream
        block()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        block()
    torch.cuda.synchronize()

    n.copy_(n0)
    resid.copy_(r0)
    n_e, r_e = n0.clone(), r0.clone()
    ws_eager = gu.workspace(T, d, w.F, E, k)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        # the same block eagerly on the eager copies, with the program's own
        # synchronisations between
        moe.forward_residual_rmsnorm(n_e, wt, k, ws_eager, r_e, gain, 1e-5, resid_out=r_e, n_out=n_e)
        torch.cuda.synchronize()
        assert np.array_equal(gu.bits_host(n), gu.bits_host(n_e)), rep
        assert np.array_equal(gu.bits_host(resid), gu.bits_host(r_e)), rep
        print(f"[graph] stack block {w.name} replay {rep} equal to eager", flush=True)
