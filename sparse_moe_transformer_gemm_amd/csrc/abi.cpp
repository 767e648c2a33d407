// extern "C" entry points: host-side validation, then launches on the caller's
// stream. Nothing here allocates device memory or synchronises the host.
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "moe.h"
#include "common.hpp"
#include "glue.hpp"
#include "layout.hpp"

namespace {

thread_local char g_last_error[512] = "";

void set_error(const char* fmt, const char* detail) {
  snprintf(g_last_error, sizeof(g_last_error), fmt, detail);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxT = 65536;

moe_status check_dims(const moe_dims& m) {
  if (m.T < 1 || m.d < 64 || m.F < 64 || m.k < 1 || m.E < 1) {
    set_error("%s", "dims: need T >= 1, d >= 64, F >= 64, k >= 1, E >= 1");
    return MOE_ERR_INVALID_ARG;
  }
  if (m.d % 64 || m.F % 64) {
    set_error("%s", "dims: d and F must be multiples of 64");
    return MOE_ERR_INVALID_ARG;
  }
  if (m.k > m.E) {
    set_error("%s", "dims: k must not exceed E");
    return MOE_ERR_INVALID_ARG;
  }
  if (m.k > 8 || m.E > 256 || m.d > 16384 || m.F > 16384 || m.T > kMaxT) {
    set_error("%s", "dims: supported k <= 8, E <= 256, d,F <= 16384, T <= 65536");
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// The expert FFN encodes its activations as two MXFP6-E2M3 terms per 32-element
// block. Over large tensors the error that encoding adds stays within the
// layer's tolerance (max error <= 2e-2 RMS, mean relative error <= 5e-3) only
// when the contraction length K = min(d, F) is at least MOE_MIN_FFN_K: with
// fewer blocks per dot product the tail of the error distribution reaches the
// bound (at K = 64 about 18 in a million outputs of y exceed it; at K = 256 a
// few of 4e7 do), while at K >= 512 its largest value over 4e7 outputs stays
// below two thirds of it.
// The MXFP4 expert GEMMs: for T > 64 an output width d that no prefill column
// tile divides (d = 64 mod 128, a multiple of neither 192 nor 320) takes the
// weight-streaming down kernel, which unrolls K = F up to 4096.
moe_status check_mxfp4_tiles(const moe_dims& m) {
  if (!moe::ffn_supported(m.T, m.d, m.F)) {
    set_error("%s", "dims: for T > 64, a d that 128, 192 and 320 do not divide needs F <= 4096");
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

moe_status check_ffn_k(const moe_dims& m) {
  if (m.d < MOE_MIN_FFN_K || m.F < MOE_MIN_FFN_K) {
    set_error("%s", "dims: the expert FFN needs d >= 512 and F >= 512 (MOE_MIN_FFN_K)");
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

moe_status check_ptrs(std::initializer_list<const void*> ptrs, const char* what) {
  for (const void* p : ptrs) {
    if (!p) {
      set_error("null pointer argument in %s", what);
      return MOE_ERR_INVALID_ARG;
    }
    if (!aligned16(p)) {
      set_error("pointer not 16-byte aligned in %s", what);
      return MOE_ERR_INVALID_ARG;
    }
  }
  return MOE_OK;
}

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  set_error("HIP launch failed: %s", hipGetErrorString(e));
  return MOE_ERR_HIP;
}

size_t workspace_for(const moe_dims& m) {
  size_t a = moe::route_workspace_bytes(m.T, m.d, m.E);
  size_t b = moe::ffn_workspace_bytes(m.T, m.d, m.F, m.E, m.k);
  size_t r = a > b ? a : b;
  const size_t c = moe::permute_workspace_bytes(m.T, m.E, m.k);
  r = r > c ? r : c;
  if (moe::forward_front_fits(m.T, m.d, m.F, m.k)) {
    const size_t f = moe::forward_front_bytes(m.T, m.d, m.F, m.E, m.k);
    r = r > f ? r : f;
  } else if (m.T > 64) {
    // the whole-block call keeps the router's partial logits, then the
    // permutation's histograms, past the FFN's regions
    const size_t f = b + (a > c ? a : c);
    r = r > f ? r : f;
  }
  return (r + 255) & ~static_cast<size_t>(255);
}

#define MOE_TRY(expr)              \
  do {                             \
    moe_status s_ = (expr);        \
    if (s_ != MOE_OK) return s_;   \
  } while (0)

}  // namespace

extern "C" {

size_t moe_workspace_bytes(moe_dims dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return workspace_for(dims);
}

static moe_status check_ws(const moe_dims& dims, void* ws, size_t ws_bytes) {
  if (!ws || !aligned16(ws)) {
    set_error("%s", "workspace pointer null or not 16-byte aligned");
    return MOE_ERR_INVALID_ARG;
  }
  if (ws_bytes < workspace_for(dims)) {
    set_error("%s", "workspace smaller than moe_workspace_bytes(dims)");
    return MOE_ERR_WORKSPACE;
  }
  return MOE_OK;
}

moe_status moe_route(moe_dims dims, const moe_bf16* x, const float* w_router,
                     const float* b_router, int32_t* topk_idx, float* topk_w, void* ws,
                     size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_ptrs({x, w_router, topk_idx, topk_w}, "moe_route"));
  if (b_router && !aligned16(b_router)) {
    set_error("%s", "b_router not 16-byte aligned");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ws(dims, ws, ws_bytes));
  return hip_status(moe::launch_route(x, w_router, b_router, dims.T, dims.d, dims.E, dims.k,
                                      topk_idx, topk_w, ws,
                                      static_cast<hipStream_t>(stream)));
}

moe_status moe_permute(moe_dims dims, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_row, void* ws,
                       size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_ptrs({topk_idx, counts, offsets, sorted_pair, pair_row}, "moe_permute"));
  MOE_TRY(check_ws(dims, ws, ws_bytes));
  return hip_status(moe::launch_permute(topk_idx, dims.T, dims.E, dims.k, counts, offsets,
                                        sorted_pair, pair_row, ws,
                                        static_cast<hipStream_t>(stream)));
}

static bool packable(int32_t E, int32_t N, int32_t K) {
  return E >= 1 && E <= 256 && N >= 64 && K >= 64 && N % 64 == 0 && K % 64 == 0 && N <= 16384 &&
         K <= 16384;
}

size_t moe_mxfp4_packed_bytes(int32_t E, int32_t N, int32_t K, int32_t which) {
  if (!packable(E, N, K) || (which != 0 && which != 1)) return 0;
  return which == 0 ? moe::packed_codes_bytes(E, N, K) : moe::packed_scales_bytes(E, N, K);
}

moe_status moe_pack_mxfp4(int32_t E, int32_t N, int32_t K, moe_mxfp4 src, uint8_t* codes_out,
                          uint8_t* scales_out, void* stream) {
  g_last_error[0] = 0;
  if (!packable(E, N, K)) {
    set_error("%s", "moe_pack_mxfp4: need 1 <= E <= 256 and N, K positive multiples of 64, <= 16384");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ptrs({src.codes, src.scales, codes_out, scales_out}, "moe_pack_mxfp4"));
  return hip_status(moe::launch_pack_mxfp4(src.codes, src.scales, E, N, K, codes_out, scales_out,
                                           static_cast<hipStream_t>(stream)));
}

static moe_status ffn_args(moe_dims dims, const moe_bf16* x, const int32_t* sorted_pair,
                           const int32_t* offsets, moe_mxfp4_packed w_gate, moe_mxfp4_packed w_up,
                           moe_mxfp4_packed w_down, const moe_bf16* b_gate, const moe_bf16* b_up,
                           const moe_bf16* b_down, float* y_sorted, void* ws, size_t ws_bytes,
                           const char* who, moe::FfnArgs& a) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_ffn_k(dims));
  MOE_TRY(check_ptrs({x, sorted_pair, offsets, w_gate.codes, w_gate.scales, w_up.codes,
                      w_up.scales, w_down.codes, w_down.scales, b_gate, b_up, b_down, y_sorted},
                     who));
  MOE_TRY(check_ws(dims, ws, ws_bytes));
  a.T = dims.T;
  a.d = dims.d;
  a.F = dims.F;
  a.E = dims.E;
  a.k = dims.k;
  a.x = x;
  a.sorted_pair = sorted_pair;
  a.offsets = offsets;
  a.wg_codes = w_gate.codes;
  a.wg_scales = w_gate.scales;
  a.wu_codes = w_up.codes;
  a.wu_scales = w_up.scales;
  a.wd_codes = w_down.codes;
  a.wd_scales = w_down.scales;
  a.b_gate = b_gate;
  a.b_up = b_up;
  a.b_down = b_down;
  a.y_sorted = y_sorted;
  a.ws = ws;
  return MOE_OK;
}

moe_status moe_expert_ffn_mxfp4(moe_dims dims, const moe_bf16* x, const int32_t* sorted_pair,
                                const int32_t* offsets, moe_mxfp4_packed w_gate,
                                moe_mxfp4_packed w_up, moe_mxfp4_packed w_down,
                                const moe_bf16* b_gate, const moe_bf16* b_up,
                                const moe_bf16* b_down, float* y_sorted, void* ws,
                                size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  moe::FfnArgs a;
  MOE_TRY(check_mxfp4_tiles(dims));
  MOE_TRY(ffn_args(dims, x, sorted_pair, offsets, w_gate, w_up, w_down, b_gate, b_up, b_down,
                   y_sorted, ws, ws_bytes, "moe_expert_ffn_mxfp4", a));
  return hip_status(moe::launch_expert_ffn(a, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn_mxfp4_stage(moe_dims dims, const moe_bf16* x, const int32_t* sorted_pair,
                                      const int32_t* offsets, moe_mxfp4_packed w_gate,
                                      moe_mxfp4_packed w_up, moe_mxfp4_packed w_down,
                                      const moe_bf16* b_gate, const moe_bf16* b_up,
                                      const moe_bf16* b_down, float* y_sorted, int32_t stage,
                                      void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (stage < 0 || stage > 2) {
    set_error("%s", "moe_expert_ffn_mxfp4_stage: stage not in 0..2");
    return MOE_ERR_INVALID_ARG;
  }
  moe::FfnArgs a;
  MOE_TRY(check_mxfp4_tiles(dims));
  MOE_TRY(ffn_args(dims, x, sorted_pair, offsets, w_gate, w_up, w_down, b_gate, b_up, b_down,
                   y_sorted, ws, ws_bytes, "moe_expert_ffn_mxfp4_stage", a));
  return hip_status(moe::launch_expert_ffn_stage(a, static_cast<hipStream_t>(stream), (int)stage));
}

// The residual stream and next norm of moe_combine_residual_rmsnorm and
// moe_forward_residual_rmsnorm.
struct ResidNorm {
  const moe_bf16* resid;
  const moe_bf16* gain;  // null: no norm
  float eps;
  moe_bf16* resid_out;
  moe_bf16* n_out;
};

static moe_status resid_norm_checks(const ResidNorm& r, const moe_bf16* m_out, const char* who) {
  MOE_TRY(check_ptrs({r.resid, r.resid_out}, who));
  if (m_out && (m_out == r.resid || m_out == r.resid_out)) {
    set_error("%s: the block output must not alias resid or resid_out", who);
    return MOE_ERR_INVALID_ARG;
  }
  if (r.gain) {
    MOE_TRY(check_ptrs({r.gain, r.n_out}, who));
    if (!(r.eps >= 0.0f)) {
      set_error("%s: need eps >= 0", who);
      return MOE_ERR_INVALID_ARG;
    }
    if (r.n_out == r.resid || r.n_out == r.resid_out || (m_out && r.n_out == m_out)) {
      set_error("%s: n_out must not alias resid, resid_out or the block output", who);
      return MOE_ERR_INVALID_ARG;
    }
  }
  return MOE_OK;
}

// moe_forward and moe_forward_noalloc: argument checks other than the
// workspace's, then the launches on `ws`.
static moe_status forward_checks(const moe_dims& dims, const moe_bf16* x, const float* w_router,
                                 const float* b_router, moe_mxfp4_packed w_gate,
                                 moe_mxfp4_packed w_up, moe_mxfp4_packed w_down,
                                 const moe_bf16* b_gate, const moe_bf16* b_up,
                                 const moe_bf16* b_down, int32_t* topk_idx, float* topk_w,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                 int32_t* pair_row, float* y_sorted, moe_bf16* out,
                                 const char* who, bool out_optional = false) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_ffn_k(dims));
  MOE_TRY(check_mxfp4_tiles(dims));
  MOE_TRY(check_ptrs({x, w_router, w_gate.codes, w_gate.scales, w_up.codes, w_up.scales,
                      w_down.codes, w_down.scales, b_gate, b_up, b_down, topk_idx, topk_w,
                      counts, offsets, sorted_pair, pair_row, y_sorted},
                     who));
  if (!(out_optional && out == nullptr)) MOE_TRY(check_ptrs({out}, who));
  if (b_router && !aligned16(b_router)) {
    set_error("%s", "b_router not 16-byte aligned");
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

static moe_status forward_launch(const moe_dims& dims, const moe_bf16* x, const float* w_router,
                                 const float* b_router, moe_mxfp4_packed w_gate,
                                 moe_mxfp4_packed w_up, moe_mxfp4_packed w_down,
                                 const moe_bf16* b_gate, const moe_bf16* b_up,
                                 const moe_bf16* b_down, int32_t* topk_idx, float* topk_w,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                 int32_t* pair_row, float* y_sorted, moe_bf16* out, void* ws,
                                 hipStream_t s, const ResidNorm* rn = nullptr) {
  moe::FfnArgs a;
  a.T = dims.T;
  a.d = dims.d;
  a.F = dims.F;
  a.E = dims.E;
  a.k = dims.k;
  a.x = x;
  a.sorted_pair = sorted_pair;
  a.offsets = offsets;
  a.wg_codes = w_gate.codes;
  a.wg_scales = w_gate.scales;
  a.wu_codes = w_up.codes;
  a.wu_scales = w_up.scales;
  a.wd_codes = w_down.codes;
  a.wd_scales = w_down.scales;
  a.b_gate = b_gate;
  a.b_up = b_up;
  a.b_down = b_down;
  a.y_sorted = y_sorted;
  a.ws = ws;
  // decode sizes: route + encode, then select + permute + pass table (two
  // launches); many tokens: route + select + encode (one launch), then the
  // permutation with the GEMMs' tile table; otherwise the separate calls' launches
  const bool front = moe::forward_front_fits(dims.T, dims.d, dims.F, dims.k);
  const bool many = !front && !moe::ffn_decode_shape(dims.T, dims.d, dims.F) && dims.T > 64;
  if (front) {
    MOE_TRY(hip_status(moe::launch_forward_front(x, w_router, b_router, dims.T, dims.d, dims.F,
                                                 dims.E, dims.k, topk_idx, topk_w, counts, offsets,
                                                 sorted_pair, pair_row, ws, s)));
  } else if (many) {
    MOE_TRY(hip_status(moe::launch_route_encode(x, w_router, b_router, dims.T, dims.d, dims.E,
                                                dims.k, topk_idx, topk_w, moe::ffn_xenc(a),
                                                moe::ffn_ws_end(a), s)));
    MOE_TRY(hip_status(moe::launch_permute(
        topk_idx, dims.T, dims.E, dims.k, counts, offsets, sorted_pair, pair_row, moe::ffn_ws_end(a), s,
        moe::ffn_tiles(a),
        moe::ffn_down_decode(dims.T, dims.d, dims.F) ? moe::ffn_passes(a) : nullptr)));
  } else {
    MOE_TRY(hip_status(moe::launch_route(x, w_router, b_router, dims.T, dims.d, dims.E, dims.k,
                                         topk_idx, topk_w, ws, s)));
    MOE_TRY(hip_status(moe::launch_permute(topk_idx, dims.T, dims.E, dims.k, counts, offsets,
                                           sorted_pair, pair_row, ws, s)));
  }
  MOE_TRY(hip_status(moe::launch_expert_ffn(a, s, front || many)));
  if (rn)
    return hip_status(moe::launch_combine_residual_rmsnorm(y_sorted, pair_row, topk_w, rn->resid,
                                                           rn->gain, dims.T, dims.d, dims.k, rn->eps,
                                                           out, rn->resid_out, rn->n_out, s));
  return hip_status(moe::launch_combine(y_sorted, pair_row, topk_w, dims.T, dims.d, dims.k, out, s));
}

moe_status moe_forward(moe_dims dims, const moe_bf16* x, const float* w_router,
                       const float* b_router, moe_mxfp4_packed w_gate, moe_mxfp4_packed w_up,
                       moe_mxfp4_packed w_down, const moe_bf16* b_gate, const moe_bf16* b_up,
                       const moe_bf16* b_down, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_row,
                       float* y_sorted, moe_bf16* out, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  MOE_TRY(forward_checks(dims, x, w_router, b_router, w_gate, w_up, w_down, b_gate, b_up, b_down,
                         topk_idx, topk_w, counts, offsets, sorted_pair, pair_row, y_sorted, out,
                         "moe_forward"));
  MOE_TRY(check_ws(dims, ws, ws_bytes));
  return forward_launch(dims, x, w_router, b_router, w_gate, w_up, w_down, b_gate, b_up, b_down,
                        topk_idx, topk_w, counts, offsets, sorted_pair, pair_row, y_sorted, out,
                        ws, static_cast<hipStream_t>(stream));
}

size_t moe_forward_noalloc_max_bytes(void) { return moe::kNoAllocScratchBytes; }

moe_status moe_forward_noalloc(moe_dims dims, const moe_bf16* x, const float* w_router,
                               const float* b_router, moe_mxfp4_packed w_gate,
                               moe_mxfp4_packed w_up, moe_mxfp4_packed w_down,
                               const moe_bf16* b_gate, const moe_bf16* b_up,
                               const moe_bf16* b_down, int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                               int32_t* pair_row, float* y_sorted, moe_bf16* out, void* stream) {
  g_last_error[0] = 0;
  MOE_TRY(forward_checks(dims, x, w_router, b_router, w_gate, w_up, w_down, b_gate, b_up, b_down,
                         topk_idx, topk_w, counts, offsets, sorted_pair, pair_row, y_sorted, out,
                         "moe_forward_noalloc"));
  if (workspace_for(dims) > moe::kNoAllocScratchBytes) {
    snprintf(g_last_error, sizeof(g_last_error),
             "moe_forward_noalloc: these dims need %zu bytes of scratch, more than the %zu "
             "bytes the library holds per GPU (use moe_forward with a workspace)",
             workspace_for(dims), moe::kNoAllocScratchBytes);
    return MOE_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  MOE_TRY(hip_status(moe::noalloc_scratch(&ws)));
  return forward_launch(dims, x, w_router, b_router, w_gate, w_up, w_down, b_gate, b_up, b_down,
                        topk_idx, topk_w, counts, offsets, sorted_pair, pair_row, y_sorted, out,
                        ws, static_cast<hipStream_t>(stream));
}

moe_status moe_forward_residual_rmsnorm(moe_dims dims, const moe_bf16* x, const float* w_router,
                                        const float* b_router, moe_mxfp4_packed w_gate,
                                        moe_mxfp4_packed w_up, moe_mxfp4_packed w_down,
                                        const moe_bf16* b_gate, const moe_bf16* b_up,
                                        const moe_bf16* b_down, int32_t* topk_idx, float* topk_w,
                                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                        int32_t* pair_row, float* y_sorted, moe_bf16* out,
                                        const moe_bf16* resid, const moe_bf16* gain, float eps,
                                        moe_bf16* resid_out, moe_bf16* n_out, void* ws,
                                        size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  const char* who = "moe_forward_residual_rmsnorm";
  MOE_TRY(forward_checks(dims, x, w_router, b_router, w_gate, w_up, w_down, b_gate, b_up, b_down,
                         topk_idx, topk_w, counts, offsets, sorted_pair, pair_row, y_sorted, out,
                         who, true));
  const ResidNorm rn{resid, gain, eps, resid_out, n_out};
  MOE_TRY(resid_norm_checks(rn, out, who));
  MOE_TRY(check_ws(dims, ws, ws_bytes));
  return forward_launch(dims, x, w_router, b_router, w_gate, w_up, w_down, b_gate, b_up, b_down,
                        topk_idx, topk_w, counts, offsets, sorted_pair, pair_row, y_sorted, out,
                        ws, static_cast<hipStream_t>(stream), &rn);
}

moe_status moe_convert_mxfp4_to_fp8(int32_t E, int32_t N, int32_t K, moe_mxfp4 src,
                                    uint8_t* codes_out, float* scales_out, void* stream) {
  g_last_error[0] = 0;
  if (!packable(E, N, K)) {
    set_error("%s", "moe_convert_mxfp4_to_fp8: need 1 <= E <= 256 and N, K positive multiples of 64, <= 16384");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ptrs({src.codes, src.scales, codes_out, scales_out}, "moe_convert_mxfp4_to_fp8"));
  return hip_status(moe::launch_convert_mxfp4_to_fp8(src.codes, src.scales, E, N, K, codes_out,
                                                     scales_out, static_cast<hipStream_t>(stream)));
}

size_t moe_fp8_packed_bytes(int32_t E, int32_t N, int32_t K) {
  return packable(E, N, K) ? moe::fp8_packed_bytes(E, N, K) : 0;
}

moe_status moe_pack_fp8(int32_t E, int32_t N, int32_t K, const uint8_t* codes, uint8_t* packed_out,
                        void* stream) {
  g_last_error[0] = 0;
  if (!packable(E, N, K)) {
    set_error("%s", "moe_pack_fp8: need 1 <= E <= 256 and N, K positive multiples of 64, <= 16384");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ptrs({codes, packed_out}, "moe_pack_fp8"));
  return hip_status(moe::launch_pack_fp8(codes, E, N, K, packed_out, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn_fp8(moe_dims dims, const moe_bf16* x, const int32_t* sorted_pair,
                              const int32_t* offsets, moe_fp8 w_gate, moe_fp8 w_up, moe_fp8 w_down,
                              const moe_bf16* b_gate, const moe_bf16* b_up, const moe_bf16* b_down,
                              float* y_sorted, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  moe::FfnArgs a;
  const moe_mxfp4_packed g{w_gate.codes, reinterpret_cast<const uint8_t*>(w_gate.scales)};
  const moe_mxfp4_packed u{w_up.codes, reinterpret_cast<const uint8_t*>(w_up.scales)};
  const moe_mxfp4_packed dn{w_down.codes, reinterpret_cast<const uint8_t*>(w_down.scales)};
  MOE_TRY(ffn_args(dims, x, sorted_pair, offsets, g, u, dn, b_gate, b_up, b_down, y_sorted, ws,
                   ws_bytes, "moe_expert_ffn_fp8", a));
  return hip_status(moe::launch_expert_ffn_fp8(a, static_cast<hipStream_t>(stream)));
}

moe_status moe_round_weights_bf16(int32_t T, int32_t k, float* topk_w, void* stream) {
  g_last_error[0] = 0;
  if (T < 1 || k < 1 || k > 8 || T > kMaxT) {
    set_error("%s", "moe_round_weights_bf16: need 1 <= T <= 65536, 1 <= k <= 8");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ptrs({topk_w}, "moe_round_weights_bf16"));
  return hip_status(moe::launch_round_bf16(topk_w, T * k, static_cast<hipStream_t>(stream)));
}

static moe_status check_attn(const moe_attn_dims& m) {
  if (m.B < 1 || m.Tq < 1 || m.S < 1 || m.Tq > m.S || m.Hq < 1 || m.Hkv < 1 || m.window < 0) {
    set_error("%s", "attention dims: need B, Tq, S, Hq, Hkv >= 1, Tq <= S, window >= 0");
    return MOE_ERR_INVALID_ARG;
  }
  if (m.Hq % m.Hkv) {
    set_error("%s", "attention dims: Hq must be a multiple of Hkv");
    return MOE_ERR_INVALID_ARG;
  }
  if (m.D != 64 || m.Hq / m.Hkv > 8 || (size_t)m.B * m.S > ((size_t)1 << 26) || m.Hq > 1024 ||
      m.Tq > (1 << 20)) {
    set_error("%s", "attention dims: supported D = 64, Hq / Hkv <= 8, B * S <= 2^26, Hq <= 1024, "
                    "Tq <= 2^20");
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

size_t moe_attention_workspace_bytes(moe_attn_dims dims) {
  if (check_attn(dims) != MOE_OK) return 0;
  return moe::attention_workspace_bytes(dims.B, dims.Tq, dims.S, dims.Hq, dims.Hkv, dims.window);
}

moe_status moe_attention_sink(moe_attn_dims dims, const moe_bf16* q, const moe_bf16* k,
                              const moe_bf16* v, const float* sinks, float scale, moe_bf16* out,
                              void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  MOE_TRY(check_attn(dims));
  MOE_TRY(check_ptrs({q, k, v, sinks, out}, "moe_attention_sink"));
  if (!(scale > 0.0f)) {
    set_error("%s", "moe_attention_sink: scale must be positive");
    return MOE_ERR_INVALID_ARG;
  }
  const size_t need = moe::attention_workspace_bytes(dims.B, dims.Tq, dims.S, dims.Hq, dims.Hkv, dims.window);
  if (need) {
    if (!ws || !aligned16(ws)) {
      set_error("%s", "workspace pointer null or not 16-byte aligned");
      return MOE_ERR_INVALID_ARG;
    }
    if (ws_bytes < need) {
      set_error("%s", "workspace smaller than moe_attention_workspace_bytes(dims)");
      return MOE_ERR_WORKSPACE;
    }
  }
  return hip_status(moe::launch_attention_sink(q, k, v, sinks, dims.B, dims.Tq, dims.S, dims.Hq,
                                               dims.Hkv, dims.window, scale, out, ws,
                                               static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(moe_dims dims, const float* y_sorted, const int32_t* pair_row,
                       const float* topk_w, moe_bf16* out, void* stream) {
  g_last_error[0] = 0;
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_ptrs({y_sorted, pair_row, topk_w, out}, "moe_combine"));
  return hip_status(moe::launch_combine(y_sorted, pair_row, topk_w, dims.T, dims.d, dims.k, out,
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_combine_residual_rmsnorm(moe_dims dims, const float* y_sorted,
                                        const int32_t* pair_row, const float* topk_w,
                                        const moe_bf16* resid, const moe_bf16* gain, float eps,
                                        moe_bf16* m_out, moe_bf16* resid_out, moe_bf16* n_out,
                                        void* stream) {
  g_last_error[0] = 0;
  const char* who = "moe_combine_residual_rmsnorm";
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_ptrs({y_sorted, pair_row, topk_w}, who));
  if (m_out) MOE_TRY(check_ptrs({m_out}, who));
  const ResidNorm rn{resid, gain, eps, resid_out, n_out};
  MOE_TRY(resid_norm_checks(rn, m_out, who));
  return hip_status(moe::launch_combine_residual_rmsnorm(
      y_sorted, pair_row, topk_w, resid, gain, dims.T, dims.d, dims.k, eps, m_out, resid_out,
      gain ? n_out : nullptr, static_cast<hipStream_t>(stream)));
}

moe_status moe_rmsnorm(int32_t T, int32_t d, const moe_bf16* x, const moe_bf16* gain, float eps,
                       moe_bf16* out, void* stream) {
  g_last_error[0] = 0;
  if (T < 1 || d < 8 || d % 8 || T > (1 << 24) || d > (1 << 20) || !(eps >= 0.0f)) {
    set_error("%s", "moe_rmsnorm: need T >= 1, d a positive multiple of 8, eps >= 0");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ptrs({x, gain, out}, "moe_rmsnorm"));
  return hip_status(moe::launch_rmsnorm(x, gain, T, d, eps, out, static_cast<hipStream_t>(stream)));
}

moe_status moe_residual_add(int32_t T, int32_t d, const moe_bf16* x, const moe_bf16* m,
                            moe_bf16* out, void* stream) {
  g_last_error[0] = 0;
  if (T < 1 || d < 8 || d % 8 || T > (1 << 24) || d > (1 << 20)) {
    set_error("%s", "moe_residual_add: need T >= 1, d a positive multiple of 8");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ptrs({x, m, out}, "moe_residual_add"));
  return hip_status(
      moe::launch_residual_add(x, m, T, d, out, static_cast<hipStream_t>(stream)));
}

moe_status moe_residual_rmsnorm(int32_t T, int32_t d, const moe_bf16* x, const moe_bf16* m,
                                const moe_bf16* gain, float eps, moe_bf16* x_out,
                                moe_bf16* n_out, void* stream) {
  g_last_error[0] = 0;
  if (T < 1 || d < 8 || d % 8 || T > (1 << 24) || d > (1 << 20) || !(eps >= 0.0f)) {
    set_error("%s", "moe_residual_rmsnorm: need T >= 1, d a positive multiple of 8, eps >= 0");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ptrs({x, m, gain, x_out, n_out}, "moe_residual_rmsnorm"));
  if (n_out == x || n_out == m || n_out == x_out) {
    set_error("%s", "moe_residual_rmsnorm: n_out must not alias x, m or x_out");
    return MOE_ERR_INVALID_ARG;
  }
  return hip_status(moe::launch_residual_rmsnorm(x, m, gain, T, d, eps, x_out, n_out,
                                                 static_cast<hipStream_t>(stream)));
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dimensions";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error; }

}  // extern "C"
