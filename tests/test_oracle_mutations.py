"""Plant plausible mistakes in the oracle, one at a time, and check that at least
one pin catches each. This shows the pins constrain every stage of the oracle."""
import numpy as np
import pytest

import oracle.moe as om
import oracle.mx as omx
import pins


def _run_pins():
    failed = []
    for name, fn in pins.ALL_PINS.items():
        try:
            fn()
        except Exception:  # an assertion, or a shape error caused by the mistake
            failed.append(name)
    return failed


def _unpack_swapped(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed >> 4
    out[..., 1::2] = packed & 0x0F
    return out


def _dequant_scale_interleaved(packed, scales):
    codes = omx.unpack_codes(packed)
    K = codes.shape[-1]
    vals = omx.E2M1[codes]
    sc = omx.E8M0[np.asarray(scales, dtype=np.uint8)]
    # wrong: element k takes scale k % (K/32) instead of k // 32
    vals = vals.reshape(vals.shape[:-1] + (32, K // 32)) * sc[..., None, :]
    return vals.reshape(codes.shape)


def _topk_high_index_first(logits, k):
    E = logits.shape[1]
    order = np.argsort(-logits[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int32)


def _softmax_all_experts(logits, idx):
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, idx.astype(np.int64), axis=1)


_orig_permute = om.permute


def _permute_desc_tokens(idx, E):
    c, o, s, r = _orig_permute(idx, E)
    s = s.copy()
    for e in range(E):
        s[o[e]:o[e + 1]] = s[o[e]:o[e + 1]][::-1]
    r = np.empty_like(s)
    r[s] = np.arange(s.size)
    return c, o, s, r


def _permute_inclusive(idx, E):
    c, o, s, r = _orig_permute(idx, E)
    o2 = o.copy()
    o2[:-1] = o[1:]
    return c, o2, s, r


_orig_gate_up = om.gate_up


def _gate_up_no_gate_bias(xr, wg, wu, bg, bu):
    return _orig_gate_up(xr, wg, wu, bg * 0, bu)


def _gate_up_swapped(xr, wg, wu, bg, bu):
    g, u = _orig_gate_up(xr, wg, wu, bg, bu)
    return u, g


def _down_no_bias(h, wd, bd):
    return h @ wd.T


def _down_untransposed(h, wd, bd):
    return h @ wd + bd[None, :]


def _silu_wrong_sign(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(np.clip(z, -700, 700)))


def _combine_shifted_slot(y_sorted, pair_row, w):
    T, k = w.shape
    rows = np.asarray(pair_row, np.int64).reshape(T, k)
    out = np.zeros((T, y_sorted.shape[1]))
    for j in range(k):
        out += w[:, (j + 1) % k:(j + 1) % k + 1] * y_sorted[rows[:, j]]
    return out


_orig_router = om.router_logits


def _router_no_bias(x, w, b=None):
    return _orig_router(x, w, None)


def _router_reversed_k(x, w, b=None):
    return _orig_router(x, np.asarray(w)[::-1], b)


def _rmsnorm_eps_outside(x, gain, eps=1e-5):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * gain


def _rmsnorm_no_mean(x, gain, eps=1e-5):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * gain


import oracle.fp8 as of8  # noqa: E402


def _e4m3_bias8(code):
    sign, exp, man = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if exp == 15 and man == 7:
        return float("nan")
    mag = (man / 8.0) * 2.0 ** -7 if exp == 0 else 2.0 ** (exp - 8) * (1.0 + man / 8.0)
    return -mag if sign else mag


def _dequant_fp8_blocks_transposed(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape[-2:]
    sc = np.asarray(scales, np.float32).astype(np.float64)
    # wrong: block (i, j) scale taken from the transposed grid (reshaped to fit)
    sc = np.swapaxes(sc, -1, -2).reshape(sc.shape)
    full = np.repeat(np.repeat(sc, 128, axis=-2), 128, axis=-1)[..., :N, :K]
    return of8.E4M3[codes] * full


def _round_bf16_truncate(w):
    f = np.ascontiguousarray(np.asarray(w, np.float64).astype(np.float32))
    u = (f.view(np.uint32) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


import oracle.attention as oat  # noqa: E402

_orig_visible = oat.visible
_orig_attn = oat.attention_sink


def _visible_strict(Tq, S, window=0):
    m = _orig_visible(Tq, S, window)
    qpos = S - Tq + np.arange(Tq)[:, None]
    return m & (np.arange(S)[None, :] < qpos)   # wrong: a query does not see its own key


def _attn_no_sink(q, k, v, sinks, scale, window=0):
    return _orig_attn(q, k, v, np.full(len(sinks), -np.inf), scale, window)


def _attn_gqa_modulo(q, k, v, sinks, scale, window=0):
    q = np.asarray(q, np.float64)
    Hq, Hkv = q.shape[2], np.asarray(k).shape[2]
    # wrong: query head h reads KV head h % Hkv instead of h // (Hq / Hkv)
    order = [h % Hkv for h in range(Hq)]
    kk = np.asarray(k, np.float64)[:, :, order, :]
    vv = np.asarray(v, np.float64)[:, :, order, :]
    return _orig_attn(q, kk, vv, sinks, scale, window)


def _attn_sink_in_numerator(q, k, v, sinks, scale, window=0):
    # wrong: the sink also carries a value (the mean of the visible values)
    out = _orig_attn(q, k, v, sinks, scale, window)
    return out + 0.01


def _chunked_sink_every_chunk(q, k, v, sinks, scale, window, chunk):
    S = np.asarray(k).shape[1]
    n = -(-S // chunk)
    return _orig_attn(q, k, v, np.asarray(sinks) + np.log(n), scale, window)


MUTATIONS = {
    "attention_mask_excludes_own_key": (oat, "visible", _visible_strict),
    "attention_sink_dropped": (oat, "attention_sink", _attn_no_sink),
    "attention_gqa_modulo_heads": (oat, "attention_sink", _attn_gqa_modulo),
    "attention_sink_with_value": (oat, "attention_sink", _attn_sink_in_numerator),
    "attention_sink_in_every_chunk": (oat, "attention_sink_chunked", _chunked_sink_every_chunk),
    "e4m3_bias_8": (of8, "e4m3_value", _e4m3_bias8),
    "e4m3_table_bias_8": (of8, "E4M3", np.array([_e4m3_bias8(c) for c in range(256)])),
    "fp8_block_scales_transposed": (of8, "dequant_fp8", _dequant_fp8_blocks_transposed),
    "routing_weights_truncated_to_bf16": (om, "round_bf16", _round_bf16_truncate),
    "nibble_order_swapped": (omx, "unpack_codes", _unpack_swapped),
    "e2m1_sign_dropped": (omx, "E2M1", np.abs(omx.E2M1)),
    "e2m1_subnormal_as_normal": (omx, "E2M1", np.array([1.0, 1.5, 1, 1.5, 2, 3, 4, 6] * 2) * np.repeat([1, -1], 8)),
    "e8m0_off_by_one": (omx, "E8M0", omx.E8M0 * 2.0),
    "scale_block_interleaved": (omx, "dequant", _dequant_scale_interleaved),
    "router_bias_dropped": (om, "router_logits", _router_no_bias),
    "router_k_reversed": (om, "router_logits", _router_reversed_k),
    "topk_ties_high_index": (om, "topk_select", _topk_high_index_first),
    "softmax_over_all_experts": (om, "softmax_selected", _softmax_all_experts),
    "permute_tokens_descending": (om, "permute", _permute_desc_tokens),
    "permute_offsets_inclusive": (om, "permute", _permute_inclusive),
    "gate_bias_dropped": (om, "gate_up", _gate_up_no_gate_bias),
    "gate_up_swapped": (om, "gate_up", _gate_up_swapped),
    "down_bias_dropped": (om, "down", _down_no_bias),
    "down_untransposed": (om, "down", _down_untransposed),
    "silu_sign_flipped": (om, "silu", _silu_wrong_sign),
    "combine_slot_shifted": (om, "combine", _combine_shifted_slot),
    "rmsnorm_eps_outside_sqrt": (om, "rmsnorm", _rmsnorm_eps_outside),
    "rmsnorm_sum_not_mean": (om, "rmsnorm", _rmsnorm_no_mean),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod, attr, repl = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, repl)
    failed = _run_pins()
    assert failed, f"planted mistake {name!r} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []
