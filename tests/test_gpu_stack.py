"""The 24-block pre-norm stack on the GPU (x <- x + MoE(RMSNorm(x)), T=2048,
d=F=2880, E=32, top-4, layer l drawn from seed 4+l), checked teacher-forced after
blocks 1, 12 and 24: each checked block is compared with the oracle fed the
GPU's own input to that block. A free-running comparison would be meaningless:
rounding the block outputs to bf16 alone flips routing decisions that then
compound over 24 blocks."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import parity
import synth

pytestmark = pytest.mark.gpu

CHECKED = (0, 11, 23)   # blocks 1, 12, 24 (0-based)


@pytest.fixture(scope="module")
def gu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gpu_util
    return gpu_util


def _bf16_ulp(v: np.ndarray) -> np.ndarray:
    """One bf16 unit in the last place of |v| (8 significant bits)."""
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, e - 8)


def test_rmsnorm_and_residual_small(gu):
    """The two stack kernels alone on a ragged shape, against the fp64 definitions."""
    import torch
    import sparse_moe_transformer_gemm_amd as moe
    rng = np.random.default_rng(50)
    T, d = 37, 320
    xb = synth.bf16_bits(rng.standard_normal((T, d)) * 3)
    gb = synth.bf16_bits(1 + 0.02 * rng.standard_normal(d))
    mb = synth.bf16_bits(rng.standard_normal((T, d)) * 50)
    n = moe.rmsnorm(gu.bf16_dev(xb), gu.bf16_dev(gb))
    s = moe.residual_add(gu.bf16_dev(xb), gu.bf16_dev(mb))
    torch.cuda.synchronize()
    n_ref = oracle.rmsnorm(oracle.bf16_to_f64(xb), oracle.bf16_to_f64(gb))
    n_gpu = oracle.bf16_to_f64(gu.bits_host(n))
    assert np.all(np.abs(n_gpu - n_ref) <= _bf16_ulp(n_ref))
    s_ref = oracle.bf16_to_f64(xb) + oracle.bf16_to_f64(mb)
    s_gpu = oracle.bf16_to_f64(gu.bits_host(s))
    # one rounding of an exact fp32 sum: at most half an ulp
    assert np.all(np.abs(s_gpu - s_ref) <= 0.5 * _bf16_ulp(s_ref))


def test_stack24_teacher_forced(gu):
    import torch
    import sparse_moe_transformer_gemm_amd as moe
    w = synth.workload(4, with_layers=False)
    T, d, F, E, k = w.T, w.d, w.F, w.E, w.k
    x = gu.bf16_dev(w.x)
    ws = gu.workspace(T, d, F, E, k)
    saved = {}
    for l in range(w.n_layers):
        L = synth.stack_layer(4, l)
        wt = gu.weights_dev(L)
        n = moe.rmsnorm(x, gu.bf16_dev(L.gain), w.eps)
        r = moe.forward(n, wt, k, ws)
        x_new = moe.residual_add(x, r["out"])
        if l in CHECKED:
            torch.cuda.synchronize()
            saved[l] = dict(x=gu.bits_host(x), n=gu.bits_host(n), m=gu.bits_host(r["out"]),
                            x_new=gu.bits_host(x_new), idx=r["topk_idx"].cpu().numpy(),
                            w=r["topk_w"].cpu().numpy(), counts=r["perm"][0].cpu().numpy(),
                            offsets=r["perm"][1].cpu().numpy(),
                            sorted_pair=r["perm"][2].cpu().numpy(),
                            pair_row=r["perm"][3].cpu().numpy())
        x = x_new
        del wt
    torch.cuda.synchronize()

    rng = np.random.default_rng(104)
    for l in CHECKED:
        s = saved[l]
        L = synth.stack_layer(4, l)
        # (a) the norm of the GPU's block input, to one bf16 ulp
        n_ref = oracle.rmsnorm(oracle.bf16_to_f64(s["x"]), oracle.bf16_to_f64(L.gain), w.eps)
        n_gpu = oracle.bf16_to_f64(s["n"])
        assert np.all(np.abs(n_gpu - n_ref) <= _bf16_ulp(n_ref)), f"norm, block {l + 1}"
        # (b) the MoE block on the GPU's normalised input: routing and dispatch of
        # every token, the output on a seeded sample of tokens
        logits = oracle.router_logits(oracle.bf16_to_f64(s["n"]), L.w_router, L.b_router)
        stats = gu.check_routing(s["idx"], s["w"], logits, k)
        gu.check_permute(s, E)
        tokens = np.sort(rng.choice(T, 48, replace=False))
        m_ref = gu.oracle_tokens(s["n"], L, k, tokens, s["idx"])
        mm = parity.assert_close(oracle.bf16_to_f64(s["m"][tokens]), m_ref, f"block {l + 1} moe")
        # (c) the residual stream after the block
        x_ref = oracle.bf16_to_f64(s["x"][tokens]) + m_ref
        mx = parity.assert_close(oracle.bf16_to_f64(s["x_new"][tokens]), x_ref, f"block {l + 1} x")
        print(f"[parity] stack block {l + 1}: routing {stats} moe {mm} residual {mx}", flush=True)
