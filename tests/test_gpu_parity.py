"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing: exact ordered indices (ties only where the oracle's own margin is below
1e-6), |w - w_ref| <= 1e-6. Dispatch: bitwise equal to the oracle's permutation
of the GPU's routing. Expert outputs and the layer output: excess error <= 2e-2 *
RMS(ref) and mean relative error <= 5e-3 (see parity.py)."""
import os

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


def _full_check(gu, w: synth.Workload, check_y: bool = True):
    L = w.layers[0]
    print(f"[parity] {w.name} T={w.T} d={w.d} F={w.F} E={w.E} k={w.k}", flush=True)
    g = gu.run_layer(w.x, L, w.k)
    ref = oracle.moe_layer(w.x, L, w.k)
    stats = gu.check_routing(g["idx"], g["w"], ref["logits"], w.k)
    gu.check_permute(g, w.E)
    if check_y:
        y_ref = oracle.ffn_sorted(oracle.bf16_to_f64(w.x), g["sorted_pair"], g["offsets"], w.k, L)
        parity.assert_close(g["y_sorted"], y_ref, "y_sorted", bf16_out=False)
    # the layer output with the GPU's routing (identical to the oracle's when no ties)
    out_ref = gu.oracle_tokens(w.x, L, w.k, np.arange(w.T), g["idx"])
    m = parity.assert_close(parity.bf16_out_to_f64(g["out"]), out_ref, "out")
    print(f"[parity] {w.name} routing {stats} out {m}", flush=True)
    return g, m


def test_tiny_workload(gu):
    _full_check(gu, synth.workload(0))


def test_decode_workload(gu):
    _full_check(gu, synth.workload(1))


@pytest.mark.parametrize("shape", [
    dict(T=1, d=64, F=64, E=4, k=4, seed=30),            # one token, E = k (dense gating)
    dict(T=37, d=128, F=192, E=8, k=2, seed=31),         # ragged T, d != F
    dict(T=50, d=64, F=128, E=16, k=1, seed=32),         # switch routing
    dict(T=300, d=256, F=64, E=64, k=4, seed=33, zipf=True),  # skewed: empty + hot experts
    dict(T=129, d=192, F=320, E=256, k=8, seed=34),      # largest E and k
    dict(T=8, d=4608, F=256, E=4, k=2, seed=38),         # decode path, K beyond the unrolled stage counts
    dict(T=96, d=320, F=4160, E=6, k=3, seed=39),        # prefill path, F not a multiple of 128
    dict(T=300, d=128, F=64, E=8, k=1, seed=43),         # prefill path, switch routing, K = 64
    dict(T=5, d=64, F=64, E=1, k=1, seed=45),            # a single expert (E = k = 1)
])
def test_edge_shapes(gu, shape):
    _full_check(gu, synth.tiny_workload(**shape))


def test_max_tokens(gu):
    """The largest T the calls accept (65536 tokens, 131072 pairs): routing and the
    permutation on every token; y's mean relative error on every row; the
    maximum-error bars on 256 sampled tokens, a sample of the size the other
    cases check (the largest of 33M errors is a tail statistic that grows with
    the sample, while a misplaced row would be off by O(1))."""
    w = synth.tiny_workload(T=65536, d=256, F=256, E=8, k=2, seed=46)
    L = w.layers[0]
    print(f"[parity] {w.name}", flush=True)
    g = gu.run_layer(w.x, L, w.k)
    ref = oracle.moe_layer(w.x, L, w.k)
    stats = gu.check_routing(g["idx"], g["w"], ref["logits"], w.k)
    gu.check_permute(g, w.E)
    y_ref = oracle.ffn_sorted(oracle.bf16_to_f64(w.x), g["sorted_pair"], g["offsets"], w.k, L)
    err = np.abs(g["y_sorted"] - y_ref)
    mean_rel_all = float(err.sum() / np.abs(y_ref).sum())
    assert mean_rel_all <= 5e-3, mean_rel_all   # every row: a misplaced row would be O(1)
    tok = np.sort(np.random.default_rng(47).choice(w.T, 256, replace=False))
    rows = g["pair_row"].reshape(w.T, w.k)[tok].ravel()
    parity.assert_close(g["y_sorted"][rows], y_ref[rows], "y_sorted", bf16_out=False)
    out_ref = gu.oracle_tokens(w.x, L, w.k, tok, g["idx"])
    m = parity.assert_close(parity.bf16_out_to_f64(g["out"][tok]), out_ref, "out")
    print(f"[parity] {w.name} routing {stats} y mean rel (all rows) {mean_rel_all:.3g} sampled out {m}",
          flush=True)


def test_prefill_handover_across_tiles(gu):
    """Both prefill GEMMs with three K steps per tile (d = F = 384) and about two
    tiles per workgroup (32768 dispatch rows, 512 tiles each): every tile but a
    workgroup's last copies the next tile's first two steps among its own last
    two, through the rotating step buffers. y on every row (mean relative
    error), the error bars on 256 sampled tokens."""
    w = synth.tiny_workload(T=8192, d=384, F=384, E=4, k=4, seed=48)
    L = w.layers[0]
    print(f"[parity] {w.name}", flush=True)
    g = gu.run_layer(w.x, L, w.k)
    ref = oracle.moe_layer(w.x, L, w.k)
    stats = gu.check_routing(g["idx"], g["w"], ref["logits"], w.k)
    gu.check_permute(g, w.E)
    y_ref = oracle.ffn_sorted(oracle.bf16_to_f64(w.x), g["sorted_pair"], g["offsets"], w.k, L)
    err = np.abs(g["y_sorted"] - y_ref)
    mean_rel_all = float(err.sum() / np.abs(y_ref).sum())
    assert mean_rel_all <= 5e-3, mean_rel_all
    tok = np.sort(np.random.default_rng(49).choice(w.T, 256, replace=False))
    rows = g["pair_row"].reshape(w.T, w.k)[tok].ravel()
    parity.assert_close(g["y_sorted"][rows], y_ref[rows], "y_sorted", bf16_out=False)
    out_ref = gu.oracle_tokens(w.x, L, w.k, tok, g["idx"])
    m = parity.assert_close(parity.bf16_out_to_f64(g["out"][tok]), out_ref, "out")
    print(f"[parity] {w.name} routing {stats} y mean rel (all rows) {mean_rel_all:.3g} sampled out {m}",
          flush=True)


def test_all_tokens_to_one_expert_set(gu):
    """W_r = 0 and an ordered bias: every token picks experts 5, 2, 7, 0 (hot experts,
    the rest empty); the weights are the closed-form softmax of the biases."""
    w = synth.tiny_workload(T=200, d=128, F=128, E=12, k=4, seed=35)
    L = w.layers[0]
    L.w_router[:] = 0
    L.b_router = np.zeros(12, np.float32)
    L.b_router[[5, 2, 7, 0]] = [3.0, 2.0, 1.0, 0.5]
    g, _ = _full_check(gu, w)
    assert np.all(g["idx"] == np.array([5, 2, 7, 0]))
    assert np.array_equal(g["counts"], np.bincount([5, 2, 7, 0], minlength=12) * 200)


def test_decode_path_hot_expert(gu):
    """Decode-sized batch (T=60) where four experts take every token: more rows per
    expert than one 32-row pass of the weight-streaming kernel."""
    w = synth.tiny_workload(T=60, d=256, F=192, E=16, k=4, seed=37)
    L = w.layers[0]
    L.w_router[:] = 0
    L.b_router = np.zeros(16, np.float32)
    L.b_router[[9, 3, 14, 6]] = [2.0, 1.5, 1.0, 0.25]
    g, _ = _full_check(gu, w)
    assert g["counts"][9] == 60


def test_identity_experts_closed_form(gu):
    """W = I (code 2 at scale 127), zero biases: out = bf16(silu(x) * x)."""
    import pins
    d, E, k = 128, 8, 4
    L = pins._identity_layer(d, E)
    rng = np.random.default_rng(36)
    xb = synth.bf16_bits(rng.standard_normal((64, d)) * 2)
    g = gu.run_layer(xb, L, k)
    x = oracle.bf16_to_f64(xb)
    ref = x * x * 0.5 * (1 + np.tanh(0.5 * x))
    parity.assert_close(parity.bf16_out_to_f64(g["out"]), ref, "identity")


def test_deterministic(gu):
    w = synth.workload(0)
    a = gu.run_layer(w.x, w.layers[0], w.k)
    b = gu.run_layer(w.x, w.layers[0], w.k)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_sampled(gu, cfg):
    """Prefill (T=8192, E=32) and wide-expert (T=4096, E=128, skewed router)
    workloads at full size: routing and dispatch on every token, the layer output
    on a seeded sample of tokens (the block is per-token)."""
    w = synth.workload(cfg)
    L = w.layers[0]
    print(f"[parity] {w.name} full size", flush=True)
    g = gu.run_layer(w.x, L, w.k, keep_y=False)
    logits = oracle.router_logits(oracle.bf16_to_f64(w.x), L.w_router, L.b_router)
    stats = gu.check_routing(g["idx"], g["w"], logits, w.k)
    gu.check_permute(g, w.E)
    rng = np.random.default_rng(100 + cfg)
    tokens = np.sort(rng.choice(w.T, 48, replace=False))
    ref = gu.oracle_tokens(w.x, L, w.k, tokens, g["idx"])
    m = parity.assert_close(parity.bf16_out_to_f64(g["out"][tokens]), ref, "out")
    print(f"[parity] {w.name} routing {stats} sampled out {m}", flush=True)
