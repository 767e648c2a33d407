"""CPU oracle for the sparse-MoE block with MXFP4 expert weights.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link or
execute anything here: only the tests, the smoke check and the bench's CPU
baseline use it. It shares no code with the HIP library (no kernels, headers,
tables, constants or pre/post-processing); it decodes every input format itself.

What it computes is the plain per-token definition of the layer, in numpy float64,
with MXFP4 weights dequantised exactly and every sum accumulated in float64, with
no intermediate rounding:

  router logits   l[t,e] = sum_k x[t,k] W_r[k,e] + b_r[e]
  top-k           the k largest logits, ordered by (logit desc, expert index asc)
  softmax         over the k selected logits only ("softmax after top-k")
  dispatch        rows grouped per expert, ascending token index inside an expert
  expert FFN      g = x Wg^T + bg, u = x Wu^T + bu, h = silu(g) * u, y = h Wd^T + bd
  combine         out[t] = sum_j w[t,j] y[t, expert j]

Sources: Perplexity, "GPT-OSS el dia 0", section "MLP: barreja d'experts dispersos
(MoE)" (SwiGLU, softmax after top-k, experts with biases) and section "Nuclis per
a GPT-OSS / MoE" (routing scheme; biases in the expert GEMM accumulators; dispatch
selects each expert's tokens; combine is a weighted accumulation); Unsloth tutorial
mirror "第39章 使用 Unsloth 微调 gpt-oss", paragraph "解释" (top-4 of 32 / of 128
experts, MoE weights in MXFP4). The MXFP4 bit format itself is not on the pages:
it is the OCP Microscaling Formats (MX) v1.0 encoding (E2M1 elements, one E8M0
scale per 32 consecutive elements).

A second weight format, FP8-E4M3 with one float32 scale per 128x128 block
(oracle/fp8.py), serves the same expert FFN (ffn_sorted_fp8); and routing
weights may be rounded to bf16 before the combine (round_bf16). The other
kernel the pages build for gpt-oss, attention whose softmax includes a
per-head sink logit, is in oracle/attention.py.

Every function here is pinned by `-m "not gpu"` tests against closed forms, exact
rational arithmetic, published format tables or invariants; none is "parity
unpinned".
"""
from .mx import E2M1, E8M0, e2m1_value, e8m0_value, unpack_codes, dequant
from .fp8 import E4M3, e4m3_value, dequant_fp8
from .attention import visible, attention_sink, attention_sink_chunked
from .moe import (
    bf16_to_f64, router_logits, topk_select, softmax_selected, route, permute,
    silu, swiglu, gate_up, down, expert_ffn, ffn_sorted, combine, moe_layer, dense_moe, rmsnorm,
    expert_ffn_fp8, ffn_sorted_fp8, round_bf16,
)

__all__ = [
    "E2M1", "E8M0", "e2m1_value", "e8m0_value", "unpack_codes", "dequant",
    "E4M3", "e4m3_value", "dequant_fp8", "expert_ffn_fp8", "ffn_sorted_fp8", "round_bf16",
    "visible", "attention_sink", "attention_sink_chunked",
    "bf16_to_f64", "router_logits", "topk_select", "softmax_selected", "route",
    "permute", "silu", "swiglu", "gate_up", "down", "expert_ffn", "ffn_sorted", "combine", "moe_layer",
    "dense_moe", "rmsnorm",
]
