/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts MLP block with
 * MXFP4 expert weights.
 *
 * The layer, as the pages state it (Perplexity, "GPT-OSS el dia 0", section
 * "MLP: barreja d'experts dispersos (MoE)" and section "Nuclis per a GPT-OSS /
 * MoE"): a router scores every expert for every token, the top-k experts are
 * kept and their weights are a softmax over the selected logits only; dispatch
 * groups each expert's tokens; each expert is a SwiGLU MLP whose projections
 * carry biases; the combine is the routing-weighted sum of the expert outputs.
 * gpt-oss-20b keeps 4 of 32 experts, gpt-oss-120b 4 of 128 (Unsloth tutorial
 * mirror, "第39章 使用 Unsloth 微调 gpt-oss", paragraph "解释"), and the expert
 * weights are MXFP4 (same paragraph; "GPT-OSS el dia 0", section "GPT-OSS a Hopper").
 *
 * Calling convention, common to every entry point:
 *   - Pointers marked [device] are HIP device pointers; the caller allocates and
 *     owns every buffer, including the workspace. The library allocates nothing,
 *     frees nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *     call only enqueues kernels on it and returns; no call synchronises the
 *     host, and no call reads device data on the host (expert counts stay on
 *     the device). Order between calls comes from the stream.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call returns an error and enqueues nothing. Device-side data are
 *     trusted: an expert index >= E in topk_idx, or a scale byte of 255 (NaN),
 *     is undefined behaviour.
 *   - A launch failure returns MOE_ERR_HIP; moe_last_error() then holds the
 *     runtime's message (thread-local, valid until the next call on the thread).
 *   - Outputs are bitwise reproducible run to run: no floating-point atomics.
 *   - Calls are thread-safe; concurrent calls need distinct workspaces.
 *
 * Data formats:
 *   bf16    raw bfloat16 bit patterns in uint16_t.
 *   MXFP4   (OCP Microscaling Formats v1.0) a matrix W[N][K] is stored as
 *           codes[N][K/2]: element k in byte k>>1, low nibble when k is even,
 *           high nibble when odd, each a 4-bit E2M1 code (sign, 2 exponent bits
 *           with bias 1, 1 mantissa bit: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6);
 *           scales[N][K/32]: one E8M0 byte s per 32 consecutive K elements,
 *           value 2^(s-127). Element (n,k) = E2M1(code) * 2^(scales[n][k/32]-127).
 *           For all E experts the arrays are [E][N][K/2] and [E][N][K/32].
 *   pair    q = t*k + j names slot j of token t; P = T*k pairs.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer        */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement      */
  MOE_ERR_WORKSPACE = -3,   /* ws_bytes smaller than moe_workspace_bytes(dims)   */
  MOE_ERR_HIP = -4          /* the HIP runtime reported an error on launch       */
} moe_status;

/* Layer dimensions: T tokens, model width d, expert FFN width F, E experts,
 * k experts per token. Supported: T >= 1, d and F multiples of 64 (MX blocks of
 * 32 and the kernels' K step), d <= 16384, F <= 16384, 1 <= k <= 8, k <= E <= 256.
 * The calls that run the expert FFN (moe_expert_ffn_mxfp4, its staged form and
 * moe_forward) also need d >= MOE_MIN_FFN_K and F >= MOE_MIN_FFN_K, and return
 * MOE_ERR_UNSUPPORTED below: they feed the activations to the matrix cores as two
 * MXFP6-E2M3 terms per 32-element block, and with fewer than 512 elements per dot
 * product the tail of the error that encoding adds reaches the layer's tolerance
 * (max error <= 2e-2 RMS of the exact result) over large tensors. From 512 on its
 * largest value over 4e7 outputs stays below two thirds of that bound (at
 * d = F = 2880, about a third). moe_route and moe_permute accept d >= 64. */
#define MOE_MIN_FFN_K 512

typedef struct {
  int32_t T, d, F, E, k;
} moe_dims;

/* One MXFP4 weight tensor for all experts in the OCP layout above, [device]
 * pointers. */
typedef struct {
  const uint8_t* codes;  /* [E][N][K/2]  */
  const uint8_t* scales; /* [E][N][K/32] */
} moe_mxfp4;

/* The same tensor repacked by moe_pack_mxfp4 into the order in which gfx950's
 * scaled matrix cores take their B operand, [device] pointers. With
 * S = ceil(K/128) steps and G = N/32 row groups:
 *   codes  [E][G][S][2][64][16 B]: entry (e,g,j,s,l) = the 16 code bytes of row
 *          32g + l%32, 32-element block 4j + 2*(l/32) + s (byte order as in
 *          moe_mxfp4); zero for blocks past K.
 *   scales [E][G][S][64][2 B]: entry (e,g,j,l) = the scale bytes of row 32g + l%32,
 *          blocks 4j + 2*(l/32) and 4j + 2*(l/32) + 1; zero for blocks past K.
 * Every code nibble and scale byte is kept; only their order changes. */
typedef struct {
  const uint8_t* codes;  /* moe_mxfp4_packed_bytes(E, N, K, 0) bytes */
  const uint8_t* scales; /* moe_mxfp4_packed_bytes(E, N, K, 1) bytes */
} moe_mxfp4_packed;

typedef uint16_t moe_bf16;

/* Bytes of workspace that moe_route, moe_permute, moe_expert_ffn_mxfp4 and
 * moe_forward need for `dims` (one buffer serves all of them; it may be reused
 * across calls on one stream). Pure host function; returns 0 for invalid dims. */
size_t moe_workspace_bytes(moe_dims dims);

/* Router GEMM, top-k, softmax over the selected logits.
 * ("GPT-OSS el dia 0", section "MLP": softmax after top-k; section "Nuclis per a
 * GPT-OSS / MoE": the softmax runs over the top-k selected experts only. The
 * router is not quantised: CSDN "GPT-OSS-120B 4-bit 量化技术深度解析", section
 * "Unsloth 4-bit量化技术解析".)
 *   x         [device] bf16  [T][d]   token activations
 *   w_router  [device] fp32  [d][E]   router weight (row k holds all experts)
 *   b_router  [device] fp32  [E]      router bias, or NULL for none
 *   topk_idx  [device] int32 [T][k]   out: selected experts, ordered by logit
 *                                     descending; exact ties -> lower index first
 *   topk_w    [device] fp32  [T][k]   out: softmax of the selected logits
 * Logits are computed in float64 on the device, so the selection is the exact
 * top-k of the real-valued logits except where two logits differ by less than
 * ~1e-12 (relative to their magnitude). */
moe_status moe_route(moe_dims dims, const moe_bf16* x, const float* w_router,
                     const float* b_router, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream);

/* Dispatch: token-to-expert histogram, exclusive scan and a stable permutation.
 * ("GPT-OSS el dia 0", section "Nuclis per a GPT-OSS / MoE": dispatch selects
 * each expert's tokens.)
 *   topk_idx    [device] int32 [T][k]  routing from moe_route (values in [0,E))
 *   counts      [device] int32 [E]     out: pairs routed to each expert
 *   offsets     [device] int32 [E+1]   out: exclusive prefix sum, offsets[E] = P
 *   sorted_pair [device] int32 [P]     out: pairs grouped by expert, ascending
 *                                      token order inside an expert (value q)
 *   pair_row    [device] int32 [P]     out: inverse, pair_row[sorted_pair[p]] = p
 * Each token must name distinct experts (as moe_route guarantees). */
moe_status moe_permute(moe_dims dims, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_row,
                       void* ws, size_t ws_bytes, void* stream);

/* Bytes of the packed form of an [E][N][K] MXFP4 tensor: its codes when
 * `which` is 0, its scales when 1. Pure host function; 0 for sizes that no
 * moe_dims can use (E outside 1..256, N or K not a positive multiple of 64, or
 * above 16384). */
size_t moe_mxfp4_packed_bytes(int32_t E, int32_t N, int32_t K, int32_t which);

/* Repack an MXFP4 tensor [E][N][K] (OCP layout) into the packed layout that
 * moe_expert_ffn_mxfp4 streams: a byte permutation, run once when the weights
 * are loaded (the expert weights are fixed across calls). The layout is the
 * operand order of gfx950's scaled MFMA, so that every weight load of the
 * expert GEMMs is a contiguous run (this library's own choice; the pages give
 * only the MXFP4 format: "GPT-OSS el dia 0", section "GPT-OSS a Hopper", and
 * "第39章 使用 Unsloth 微调 gpt-oss", paragraph "解释").
 *   src            [device] codes [E][N][K/2], scales [E][N][K/32], 16-byte aligned
 *   codes_out      [device] moe_mxfp4_packed_bytes(E, N, K, 0) bytes, 16-byte aligned
 *   scales_out     [device] moe_mxfp4_packed_bytes(E, N, K, 1) bytes, 16-byte aligned
 * Output must not overlap the input. Enqueued on `stream` like every call. */
moe_status moe_pack_mxfp4(int32_t E, int32_t N, int32_t K, moe_mxfp4 src, uint8_t* codes_out,
                          uint8_t* scales_out, void* stream);

/* Grouped expert FFN in dispatch order, MXFP4 weights.
 * Two departures from a call that would take the weights as stored (the OCP
 * layout of moe_mxfp4) with d and F any multiple of 32:
 *   - the weights are passed packed (moe_mxfp4_packed, made once per matrix by
 *     moe_pack_mxfp4). The library allocates nothing and keeps no state, so it
 *     cannot repack on the caller's behalf without paying a full pass over the
 *     weights on every call; the packed bytes are the stored bytes reordered;
 *   - d and F are multiples of 64 (the MFMA step covers two 32-element blocks)
 *     and at least MOE_MIN_FFN_K.
 * With more than 64 tokens the down GEMM tiles its d output columns by 320, 192
 * or 128; a d that none of them divides (64 mod 128 and a multiple of neither
 * 192 nor 320, e.g. 704, 832, 2752) takes the weight-streaming kernel of the
 * small batches instead (correct, slower: it reads each expert's weights once
 * per 16 rows), which needs F <= 4096: otherwise MOE_ERR_UNSUPPORTED. This also
 * holds for moe_expert_ffn_mxfp4_stage, moe_forward and moe_forward_noalloc.
 * For every expert e and row p in [offsets[e], offsets[e+1]), with
 * t = sorted_pair[p] / k:
 *   g = x[t] Wg[e]^T + b_gate[e],  u = x[t] Wu[e]^T + b_up[e],
 *   h = silu(g) * u,               y_sorted[p] = h Wd[e]^T + b_down[e].
 * ("GPT-OSS el dia 0", section "MLP": SwiGLU, experts with biases; section
 * "Nuclis per a GPT-OSS / MoE": biases loaded into the GEMM accumulators.)
 *   x         [device] bf16 [T][d]
 *   sorted_pair, offsets  [device] from moe_permute
 *   w_gate, w_up          MXFP4 [E][F][d] (N = F, K = d), packed by moe_pack_mxfp4
 *   w_down                MXFP4 [E][d][F] (N = d, K = F), packed by moe_pack_mxfp4
 *   b_gate, b_up [device] bf16 [E][F];  b_down [device] bf16 [E][d]
 *   y_sorted  [device] fp32 [P][d]  out: per-pair expert output, bias included
 * The activations are re-encoded on the device for the matrix cores (two-term
 * MXFP6 per 32-element block); accumulation is fp32. Code and scale pointers
 * must be 16-byte aligned. The weights are read in place: the library keeps
 * no copy of them. */
moe_status moe_expert_ffn_mxfp4(moe_dims dims, const moe_bf16* x,
                                const int32_t* sorted_pair, const int32_t* offsets,
                                moe_mxfp4_packed w_gate, moe_mxfp4_packed w_up,
                                moe_mxfp4_packed w_down,
                                const moe_bf16* b_gate, const moe_bf16* b_up,
                                const moe_bf16* b_down, float* y_sorted,
                                void* ws, size_t ws_bytes, void* stream);

/* moe_expert_ffn_mxfp4 as three separately enqueued stages, for callers that
 * time or schedule the two GEMMs on their own (same arguments, plus `stage`):
 *   stage 0  encodes x for the matrix cores and builds the expert tile tables
 *            (into ws)
 *   stage 1  the gate/up GEMM with its biases and SwiGLU: h, encoded, into ws
 *   stage 2  the down GEMM with its bias: y_sorted
 * Stages 0, 1, 2 enqueued in that order on one stream with the same arguments
 * and workspace write exactly the bytes moe_expert_ffn_mxfp4 writes. Stage 1
 * reads what stage 0 left in ws and stage 2 what stage 1 left: running a stage
 * without the earlier ones of the same call (same dims, inputs and ws, nothing
 * else using ws in between) is undefined. Errors: MOE_ERR_INVALID_ARG for a
 * stage outside 0..2, otherwise as moe_expert_ffn_mxfp4. */
moe_status moe_expert_ffn_mxfp4_stage(moe_dims dims, const moe_bf16* x,
                                      const int32_t* sorted_pair, const int32_t* offsets,
                                      moe_mxfp4_packed w_gate, moe_mxfp4_packed w_up,
                                      moe_mxfp4_packed w_down,
                                      const moe_bf16* b_gate, const moe_bf16* b_up,
                                      const moe_bf16* b_down, float* y_sorted, int32_t stage,
                                      void* ws, size_t ws_bytes, void* stream);

/* Atomic-free weighted combine back to token order:
 *   out[t] = bf16( sum_{j=0..k-1} topk_w[t][j] * y_sorted[pair_row[t*k+j]] ),
 * summed in fp32 in fixed j order, rounded once to nearest even.
 * ("GPT-OSS el dia 0", section "Nuclis per a GPT-OSS / MoE": combine is the
 * weighted accumulation of the expert outputs.)
 *   y_sorted [device] fp32 [P][d]; pair_row [device] int32 [P];
 *   topk_w   [device] fp32 [T][k]; out [device] bf16 [T][d]. */
moe_status moe_combine(moe_dims dims, const float* y_sorted, const int32_t* pair_row,
                       const float* topk_w, moe_bf16* out, void* stream);

/* The whole block in one call: moe_route, moe_permute, moe_expert_ffn_mxfp4 and
 * moe_combine in that order, with the same arguments and the same output bytes
 * (every intermediate output is written as those calls write it). For
 * decode-sized batches (T <= 64 and d, F <= 4096) routing, permutation and the
 * activation encode are fused into two launches, so the block takes five
 * launches instead of eight. ("GPT-OSS el dia 0", section "MLP" and section
 * "Nuclis per a GPT-OSS / MoE": route, dispatch, expert FFNs, combine.)
 *   x, w_router, b_router          as for moe_route (b_router may be NULL)
 *   w_gate, w_up, w_down, biases   as for moe_expert_ffn_mxfp4 (packed weights)
 *   topk_idx, topk_w               [device] out, as from moe_route
 *   counts, offsets, sorted_pair, pair_row  [device] out, as from moe_permute
 *   y_sorted                       [device] out, fp32 [P][d]
 *   out                            [device] out, bf16 [T][d]
 *   ws, ws_bytes                   workspace of at least moe_workspace_bytes(dims)
 * Errors as for the four calls; all checks happen before the first launch. */
moe_status moe_forward(moe_dims dims, const moe_bf16* x, const float* w_router,
                       const float* b_router, moe_mxfp4_packed w_gate, moe_mxfp4_packed w_up,
                       moe_mxfp4_packed w_down, const moe_bf16* b_gate, const moe_bf16* b_up,
                       const moe_bf16* b_down, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_row,
                       float* y_sorted, moe_bf16* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * FP8 expert weights: the pages' serving variant ("GPT-OSS el dia 0", section
 * "GPT-OSS a Hopper": the MXFP4 experts converted once to FP8 with 128x128
 * block scales and run on FP8 GEMMs extended with a bias term; section "Nuclis
 * per a GPT-OSS / MoE": the bias goes into the GEMM accumulators).
 * A matrix W[N][K] is stored as codes[N][K], one OCP FP8 E4M3 byte per element
 * (bias 7, subnormals, no infinities, 0x7F/0xFF NaN), and scales
 * [ceil(N/128)][ceil(K/128)] float32, one per 128 x 128 block:
 *   W[n][k] = E4M3(codes[n][k]) * scales[n/128][k/128].
 * For all E experts: codes [E][N][K], scales [E][ceil(N/128)][ceil(K/128)]. */
typedef struct {
  const uint8_t* codes;  /* [E][N][K] (moe_convert_mxfp4_to_fp8), or packed (moe_pack_fp8) */
  const float* scales;   /* [E][ceil(N/128)][ceil(K/128)] */
} moe_fp8;

/* Convert MXFP4 weights (OCP layout, [device]) to FP8 with 128x128 block
 * scales, once, as the pages' engine did: each block's scale is 2^(its largest
 * E8M0 exponent - 127) and each element is rounded to the nearest E4M3 value
 * (ties to even) of element / block scale. When the E8M0 exponents inside a
 * 128x128 block differ by at most 8 (the gpt-oss-like weights here differ by 3)
 * every element is exact, so the FP8 layer computes the same function.
 *   codes_out  [device] E * N * K bytes;  scales_out [device] float32
 *   E * ceil(N/128) * ceil(K/128). N, K positive multiples of 64, <= 16384. */
moe_status moe_convert_mxfp4_to_fp8(int32_t E, int32_t N, int32_t K, moe_mxfp4 src,
                                    uint8_t* codes_out, float* scales_out, void* stream);

/* Bytes of the packed form of [E][N][K] FP8 codes (0 for unusable sizes). */
size_t moe_fp8_packed_bytes(int32_t E, int32_t N, int32_t K);

/* Repack FP8 codes [E][N][K] into the B-operand order of gfx950's scaled MFMA
 * with an FP8 operand (a byte permutation, once at load time):
 *   [E][N/32][ceil(K/128)][2][64][32 B]: entry (e,g,j,s,l), row 32g + l%32,
 *   h = l/32, holds in bytes 0..15 the codes of elements 16h..16h+15 of the
 *   32-element block 4j + s and in bytes 16..31 those of block 4j + 2 + s
 *   (the instruction takes an 8-bit operand in 16-element pieces); zero past K.
 * The block scales are used as stored. Output must not overlap the input. */
moe_status moe_pack_fp8(int32_t E, int32_t N, int32_t K, const uint8_t* codes,
                        uint8_t* packed_out, void* stream);

/* moe_expert_ffn_mxfp4 with FP8 block-scaled expert weights: the same
 * arguments, dims checks and outputs, with each moe_fp8 holding codes packed by
 * moe_pack_fp8 and the float32 block scales. Accumulators start at the bias;
 * each 128-deep K step is scaled by its block scale as it is added. */
moe_status moe_expert_ffn_fp8(moe_dims dims, const moe_bf16* x, const int32_t* sorted_pair,
                              const int32_t* offsets, moe_fp8 w_gate, moe_fp8 w_up,
                              moe_fp8 w_down, const moe_bf16* b_gate, const moe_bf16* b_up,
                              const moe_bf16* b_down, float* y_sorted, void* ws,
                              size_t ws_bytes, void* stream);

/* Routing weights in bfloat16 ("GPT-OSS el dia 0", section "Nuclis per a
 * GPT-OSS / MoE": computing the expert weights in bf16 was critical to match
 * the reference numerics): rounds topk_w [device] fp32 [T][k] in place to the
 * nearest bf16 value (ties to even), still stored as fp32, for moe_combine. */
moe_status moe_round_weights_bf16(int32_t T, int32_t k, float* topk_w, void* stream);

/* ---------------------------------------------------------------------------
 * Attention with per-head sinks, the other kernel the pages build for gpt-oss
 * ("GPT-OSS el dia 0", section "Atenció: GQA amb Attention Sinks": every head
 * has a pretrained sink that takes part in the softmax; section "Nuclis per a
 * GPT-OSS / Atenció de buidatge": an online softmax starts its running maximum
 * at the sink, in the first KV chunk only). For query q of head h:
 *   out = sum_j exp(z_j) v_j / (exp(sinks[h]) + sum_j exp(z_j)),  z_j = scale * <q, k_j>,
 * over the keys j the query sees, with KV head h / (Hq / Hkv) (grouped queries).
 * Queries are the last Tq of the S positions (query i at position S - Tq + i) and
 * see keys j <= their position; with window > 0 only keys j > position - window. */
typedef struct {
  int32_t B;       /* batch entries (sequences) */
  int32_t Tq;      /* queries per entry, 1 <= Tq <= S, Tq <= 2^20 */
  int32_t S;       /* keys per entry */
  int32_t Hq, Hkv; /* query and KV heads; Hq a multiple of Hkv, Hq / Hkv <= 8 */
  int32_t D;       /* head size: 64 */
  int32_t window;  /* sliding window, 0 for none */
} moe_attn_dims;

/* Workspace bytes of moe_attention_sink (0 when it needs none; also 0 for dims
 * it does not support, which moe_attention_sink rejects). */
size_t moe_attention_workspace_bytes(moe_attn_dims dims);

/*   q      [device] bf16 [B][Tq][Hq][D];  k, v [device] bf16 [B][S][Hkv][D]
 *   sinks  [device] fp32 [Hq] (in logit units)
 *   scale  softmax scale (1/sqrt(D) for gpt-oss)
 *   out    [device] bf16 [B][Tq][Hq][D]
 * fp32 accumulation; the probabilities enter the P V product as bf16. When the
 * keys are split into chunks (few queries), each chunk's partial softmax is kept
 * in the workspace and merged in chunk order (deterministic). */
moe_status moe_attention_sink(moe_attn_dims dims, const moe_bf16* q, const moe_bf16* k,
                              const moe_bf16* v, const float* sinks, float scale, moe_bf16* out,
                              void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, checks, launches and output bytes as
 * moe_forward, minus ws and ws_bytes: the scratch those calls need lives in a
 * fixed device array inside the library, moe_forward_noalloc_max_bytes() bytes
 * (32 MiB) per GPU, which each GPU the library runs on holds until the process
 * ends. The call itself allocates nothing and frees nothing; its first call on
 * a device looks up that device's copy of the array.
 *   Limit: dims whose moe_workspace_bytes(dims) exceeds the array return
 *   MOE_ERR_UNSUPPORTED (at d = F = 2880, E = 32 that is T above ~1400 tokens;
 *   decode batches need well under 5 MiB).
 *   Sharing: every call on one GPU uses the same array and leaves its
 *   contents behind (what must start at zero is cleared by the call's own
 *   kernels). Calls that may overlap on one GPU -- on different streams, or
 *   from several threads without ordering -- race on it and give undefined
 *   results; order them on one stream. */
moe_status moe_forward_noalloc(moe_dims dims, const moe_bf16* x, const float* w_router,
                               const float* b_router, moe_mxfp4_packed w_gate,
                               moe_mxfp4_packed w_up, moe_mxfp4_packed w_down,
                               const moe_bf16* b_gate, const moe_bf16* b_up,
                               const moe_bf16* b_down, int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                               int32_t* pair_row, float* y_sorted, moe_bf16* out, void* stream);

/* Bytes of the scratch array moe_forward_noalloc uses (per GPU). */
size_t moe_forward_noalloc_max_bytes(void);

/* RMSNorm of each row (the pre-norm of a transformer block; rms_norm_eps = 1e-5
 * per CSDN "GPT-OSS-120B 4-bit 量化技术深度解析", section "推理优化"):
 *   out[t] = bf16( x[t] / sqrt(mean_i x[t][i]^2 + eps) * gain ), fp32 arithmetic.
 *   x, out [device] bf16 [T][d]; gain [device] bf16 [d]. d a multiple of 8. */
moe_status moe_rmsnorm(int32_t T, int32_t d, const moe_bf16* x, const moe_bf16* gain,
                       float eps, moe_bf16* out, void* stream);

/* Residual add: out = bf16(x + m), fp32 add, round to nearest even. out may
 * alias x. x, m, out [device] bf16 [T][d]; d a multiple of 8. */
moe_status moe_residual_add(int32_t T, int32_t d, const moe_bf16* x, const moe_bf16* m,
                            moe_bf16* out, void* stream);

/* Residual add and the next pre-norm in one pass (the glue between two blocks
 * of a pre-norm stack, x <- x + MoE(RMSNorm(x))):
 *   x_out[t] = bf16(x[t] + m[t])                       as moe_residual_add,
 *   n_out[t] = RMSNorm(x_out[t]) with gain and eps     as moe_rmsnorm,
 * the same bytes as those two calls in that order, reading each row once.
 * x_out may alias x; n_out must alias none of the others. x, m, x_out, n_out
 * [device] bf16 [T][d]; gain [device] bf16 [d]; d a multiple of 8. Errors as
 * for moe_rmsnorm. */
moe_status moe_residual_rmsnorm(int32_t T, int32_t d, const moe_bf16* x, const moe_bf16* m,
                                const moe_bf16* gain, float eps, moe_bf16* x_out,
                                moe_bf16* n_out, void* stream);

/* The block's weighted combine, its residual add and the next block's pre-norm
 * in one pass over each token row, so that the block output never makes a round
 * trip through memory (the combine is the weighted accumulation of "GPT-OSS el
 * dia 0", section "Nuclis per a GPT-OSS / MoE"; the norm as for moe_rmsnorm):
 *   m[t]         = bf16(sum_j topk_w[t][j] * y_sorted[pair_row[t*k+j]])  as moe_combine,
 *   resid_out[t] = bf16(resid[t] + m[t])                                 as moe_residual_add,
 *   n_out[t]     = RMSNorm(resid_out[t]) with gain and eps               as moe_rmsnorm,
 * the same bytes as those calls in that order.
 *   y_sorted, pair_row, topk_w  as for moe_combine (dims.T, dims.d, dims.k used)
 *   resid      [device] bf16 [T][d]  the residual stream before the block
 *   gain       [device] bf16 [d]     the next block's norm gain, or NULL: then no
 *                                    norm is taken and n_out is not used
 *   m_out      [device] bf16 [T][d]  out: the block output m, or NULL (not stored)
 *   resid_out  [device] bf16 [T][d]  out: may alias resid
 *   n_out      [device] bf16 [T][d]  out: aliases none of the others
 * Errors as for moe_combine, plus MOE_ERR_INVALID_ARG for a negative eps or an
 * alias other than resid_out == resid. */
moe_status moe_combine_residual_rmsnorm(moe_dims dims, const float* y_sorted,
                                        const int32_t* pair_row, const float* topk_w,
                                        const moe_bf16* resid, const moe_bf16* gain, float eps,
                                        moe_bf16* m_out, moe_bf16* resid_out, moe_bf16* n_out,
                                        void* stream);

/* moe_forward whose last step is moe_combine_residual_rmsnorm instead of
 * moe_combine: one block of a pre-norm stack x <- x + MoE(RMSNorm(x)) after its
 * norm (x is the normalised block input, resid the residual stream). Arguments
 * as moe_forward, except that `out` (the block output m) may be NULL, followed
 * by those of moe_combine_residual_rmsnorm. Same bytes as moe_forward followed
 * by moe_residual_rmsnorm (or moe_residual_add when gain is NULL). n_out may be
 * the block input x itself (x is not read after the expert GEMMs), so a stack
 * can keep its normalised activations and its residual stream in place. */
moe_status moe_forward_residual_rmsnorm(moe_dims dims, const moe_bf16* x, const float* w_router,
                                        const float* b_router, moe_mxfp4_packed w_gate,
                                        moe_mxfp4_packed w_up, moe_mxfp4_packed w_down,
                                        const moe_bf16* b_gate, const moe_bf16* b_up,
                                        const moe_bf16* b_down, int32_t* topk_idx, float* topk_w,
                                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                        int32_t* pair_row, float* y_sorted, moe_bf16* out,
                                        const moe_bf16* resid, const moe_bf16* gain, float eps,
                                        moe_bf16* resid_out, moe_bf16* n_out, void* ws,
                                        size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);

/* Detail of the last error on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
