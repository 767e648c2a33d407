"""The FP8 weight variant through the C ABI: FP8-E4M3 expert weights with one
float32 scale per 128x128 block (the pages' Hopper serving path), and routing
weights rounded to bf16.

  * moe_convert_mxfp4_to_fp8: the converted tensors, decoded by the oracle's own
    FP8 decoder, equal the MXFP4 weights exactly (bitwise float64 equality).
  * moe_pack_fp8: byte for byte the documented packed layout, written out with
    numpy index arithmetic here.
  * moe_expert_ffn_fp8 on converted weights: the same oracle as the MXFP4 path
    (the weights are the same numbers), y_sorted on every row and the layer
    output on every token, under the bars of parity.py.
  * moe_expert_ffn_fp8 on general FP8 weights (random codes, random float32
    block scales): against the oracle's FP8 expert FFN.
  * moe_round_weights_bf16: bit-exact against the oracle's rounding of the same
    float32 weights, and the combine with bf16 weights against the oracle."""
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


def _u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _fp8_layer_from_mxfp4(gu, L):
    import sparse_moe_transformer_gemm_amd as moe
    return moe.fp8_from_mxfp4(
        w_router=_u8(L.w_router), b_router=None if L.b_router is None else _u8(L.b_router),
        gate_codes=_u8(L.gate.codes), gate_scales=_u8(L.gate.scales),
        up_codes=_u8(L.up.codes), up_scales=_u8(L.up.scales),
        down_codes=_u8(L.down.codes), down_scales=_u8(L.down.scales),
        b_gate=gu.bf16_dev(L.b_gate), b_up=gu.bf16_dev(L.b_up), b_down=gu.bf16_dev(L.b_down))


@pytest.mark.parametrize("E,N,K", [(3, 512, 640), (2, 2880, 2880), (1, 4160, 576)])
def test_convert_is_exact(gu, E, N, K):
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    rng = np.random.default_rng(E + N + K)
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(121, 125, (E, N, K // 32), dtype=np.uint8)
    print(f"[fp8] convert E={E} N={N} K={K}", flush=True)
    c8, s8 = moe.convert_mxfp4_to_fp8(_u8(codes), _u8(scales))
    torch.cuda.synchronize()
    c8, s8 = c8.cpu().numpy(), s8.cpu().numpy()
    for e in range(E):
        assert np.array_equal(oracle.dequant_fp8(c8[e], s8[e]), oracle.dequant(codes[e], scales[e])), e


def pack_fp8_reference(codes: np.ndarray) -> np.ndarray:
    """Packed FP8 layout of include/moe.h from codes [E][N][K]: entry (g, j, s, l)
    = 16 codes of block 4j + s, then 16 of block 4j + 2 + s, each starting at
    element 16 (l // 32)."""
    E, N, K = codes.shape
    S, G, nblk = (K + 127) // 128, N // 32, K // 32
    blocks = np.zeros((E, N, 4 * S, 2, 16), np.uint8)        # [block][16-element piece]
    blocks[:, :, :nblk] = codes.reshape(E, N, nblk, 2, 16)
    l = np.arange(64)
    out = np.zeros((E, G, S, 2, 64, 2, 16), np.uint8)
    for g in range(G):
        for j in range(S):
            for s in range(2):
                for p in range(2):
                    out[:, g, j, s, :, p] = blocks[:, 32 * g + l % 32, 4 * j + 2 * p + s, l // 32]
    return out.reshape(-1)


@pytest.mark.parametrize("E,N,K", [(2, 64, 128), (3, 320, 192), (1, 2880, 2880)])
def test_pack_fp8_matches_layout(E, N, K):
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    codes = np.random.default_rng(N + K).integers(0, 256, (E, N, K), dtype=np.uint8)
    p = moe.pack_fp8(_u8(codes))
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), pack_fp8_reference(codes))


def _ffn_fp8_check(gu, w, wt8, y_ref_fn):
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    L = w.layers[0]
    x = gu.bf16_dev(w.x)
    ws = gu.workspace(w.T, w.d, w.F, w.E, w.k)
    idx, tw = moe.route(x, wt8.w_router, wt8.b_router, w.k, ws)
    perm = moe.permute(idx, w.E, ws)
    y = moe.expert_ffn_fp8(x, perm[2], perm[1], wt8, w.k, ws)
    out = moe.combine(y, perm[3], tw)
    torch.cuda.synchronize()
    g = dict(idx=idx.cpu().numpy(), w=tw.cpu().numpy(), counts=perm[0].cpu().numpy(),
             offsets=perm[1].cpu().numpy(), sorted_pair=perm[2].cpu().numpy(),
             pair_row=perm[3].cpu().numpy())
    logits = oracle.router_logits(oracle.bf16_to_f64(w.x), L.w_router, L.b_router)
    gu.check_routing(g["idx"], g["w"], logits, w.k)
    gu.check_permute(g, w.E)
    y_ref = y_ref_fn(g)
    my = parity.assert_close(y.cpu().numpy(), y_ref, f"{w.name} fp8 y_sorted", bf16_out=False)
    wref = oracle.softmax_selected(logits, g["idx"])
    out_ref = oracle.combine(y_ref, g["pair_row"], wref)
    m = parity.assert_close(parity.bf16_out_to_f64(gu.bits_host(out)), out_ref, f"{w.name} fp8 out")
    print(f"[fp8] {w.name} y {my} out {m}", flush=True)


@pytest.mark.parametrize("shape", [
    dict(T=16, d=2880, F=2880, E=32, k=4, seed=1),       # decode-20b shape
    dict(T=128, d=512, F=512, E=32, k=4, seed=0),        # tiny
    dict(T=37, d=512, F=704, E=8, k=2, seed=31),         # ragged, F % 128 = 64
    dict(T=600, d=576, F=640, E=8, k=4, seed=55),        # several 32-row tiles per expert, d % 128 = 64
    dict(T=260, d=2880, F=1472, E=6, k=2, seed=58),      # many rows at d = 2880: 96-column down tiles, F % 128 = 64
    dict(T=150, d=1024, F=704, E=5, k=3, seed=59),       # many rows, 128-column down tiles, F % 128 = 64
], ids=lambda s: f"T{s['T']}-d{s['d']}-F{s['F']}-E{s['E']}-k{s['k']}")
def test_ffn_fp8_converted(gu, shape):
    """MXFP4 weights converted to FP8 on the GPU are the same numbers, so the
    MXFP4 oracle is the reference."""
    w = synth.tiny_workload(**shape)
    L = w.layers[0]
    print(f"[fp8] converted {w.name}", flush=True)
    wt8 = _fp8_layer_from_mxfp4(gu, L)
    x = oracle.bf16_to_f64(w.x)
    _ffn_fp8_check(gu, w, wt8, lambda g: oracle.ffn_sorted(x, g["sorted_pair"], g["offsets"], w.k, L))


@pytest.mark.parametrize("shape", [
    dict(T=200, d=512, F=576, E=8, k=4, seed=56),
    dict(T=9, d=640, F=512, E=4, k=2, seed=57),
], ids=["T200", "T9"])
def test_ffn_fp8_general_scales(gu, shape):
    """FP8 weights with arbitrary float32 block scales (not powers of two) against
    the oracle's FP8 expert FFN."""
    import sparse_moe_transformer_gemm_amd as moe
    w = synth.tiny_workload(**shape)
    L = w.layers[0]
    rng = np.random.default_rng(shape["seed"] + 1000)
    l8 = {"gate": synth.fp8_weights(rng, w.E, w.F, w.d), "up": synth.fp8_weights(rng, w.E, w.F, w.d),
          "down": synth.fp8_weights(rng, w.E, w.d, w.F)}
    print(f"[fp8] general scales {w.name}", flush=True)
    wt8 = moe.load_fp8_weights(_u8(L.w_router), None, *[(_u8(l8[n][0]), _u8(l8[n][1]))
                                                         for n in ("gate", "up", "down")],
                               gu.bf16_dev(L.b_gate), gu.bf16_dev(L.b_up), gu.bf16_dev(L.b_down))
    x = oracle.bf16_to_f64(w.x)
    _ffn_fp8_check(gu, w, wt8, lambda g: oracle.ffn_sorted_fp8(x, g["sorted_pair"], g["offsets"], w.k, l8,
                                                              L.b_gate, L.b_up, L.b_down))


def test_round_weights_bf16(gu):
    """The bf16 routing-weight option: the rounded weights are exactly the
    oracle's rounding of the GPU's float32 weights, and the layer output with
    them meets the bars against the oracle with bf16-rounded weights."""
    import torch

    import sparse_moe_transformer_gemm_amd as moe
    w = synth.workload(0)
    L = w.layers[0]
    g = gu.run_layer(w.x, L, w.k)
    wt = gu.weights_dev(L)
    ws = gu.workspace(w.T, w.d, w.F, w.E, w.k)
    x = gu.bf16_dev(w.x)
    idx, tw = moe.route(x, wt.w_router, wt.b_router, w.k, ws)
    w32 = tw.cpu().numpy().copy()
    moe.round_weights_bf16(tw)
    perm = moe.permute(idx, w.E, ws)
    y = moe.expert_ffn_mxfp4(x, perm[2], perm[1], wt, w.k, ws)
    out = moe.combine(y, perm[3], tw)
    torch.cuda.synchronize()
    wb = tw.cpu().numpy().astype(np.float64)
    assert np.array_equal(wb, oracle.round_bf16(w32))
    logits = oracle.router_logits(oracle.bf16_to_f64(w.x), L.w_router, L.b_router)
    wref = oracle.round_bf16(oracle.softmax_selected(logits, g["idx"]))
    y_ref = oracle.ffn_sorted(oracle.bf16_to_f64(w.x), g["sorted_pair"], g["offsets"], w.k, L)
    out_ref = oracle.combine(y_ref, g["pair_row"], wref)
    m = parity.assert_close(parity.bf16_out_to_f64(gu.bits_host(out)), out_ref, "bf16 weights out")
    print(f"[bf16 weights] out {m}", flush=True)
