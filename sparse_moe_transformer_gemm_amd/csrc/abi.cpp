// extern "C" entry points: host-side validation, then launches on the caller's
// stream. Nothing here allocates device memory or synchronises the host.
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "moe.h"
#include "common.hpp"
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
  MOE_TRY(ffn_args(dims, x, sorted_pair, offsets, w_gate, w_up, w_down, b_gate, b_up, b_down,
                   y_sorted, ws, ws_bytes, "moe_expert_ffn_mxfp4_stage", a));
  return hip_status(moe::launch_expert_ffn_stage(a, static_cast<hipStream_t>(stream), (int)stage));
}

moe_status moe_forward(moe_dims dims, const moe_bf16* x, const float* w_router,
                       const float* b_router, moe_mxfp4_packed w_gate, moe_mxfp4_packed w_up,
                       moe_mxfp4_packed w_down, const moe_bf16* b_gate, const moe_bf16* b_up,
                       const moe_bf16* b_down, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_row,
                       float* y_sorted, moe_bf16* out, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_ptrs({x, w_router, w_gate.codes, w_gate.scales, w_up.codes, w_up.scales,
                      w_down.codes, w_down.scales, b_gate, b_up, b_down, topk_idx, topk_w,
                      counts, offsets, sorted_pair, pair_row, y_sorted, out},
                     "moe_forward"));
  if (b_router && !aligned16(b_router)) {
    set_error("%s", "b_router not 16-byte aligned");
    return MOE_ERR_INVALID_ARG;
  }
  MOE_TRY(check_ws(dims, ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
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
  const bool front = moe::forward_front_fits(dims.T, dims.d, dims.F, dims.k);
  if (front) {
    MOE_TRY(hip_status(moe::launch_forward_front(x, w_router, b_router, dims.T, dims.d, dims.F,
                                                 dims.E, dims.k, topk_idx, topk_w, counts, offsets,
                                                 sorted_pair, pair_row, ws, s)));
  } else {
    MOE_TRY(hip_status(moe::launch_route(x, w_router, b_router, dims.T, dims.d, dims.E, dims.k,
                                         topk_idx, topk_w, ws, s)));
    MOE_TRY(hip_status(moe::launch_permute(topk_idx, dims.T, dims.E, dims.k, counts, offsets,
                                           sorted_pair, pair_row, ws, s)));
  }
  MOE_TRY(hip_status(moe::launch_expert_ffn(a, s, front)));
  return hip_status(moe::launch_combine(y_sorted, pair_row, topk_w, dims.T, dims.d, dims.k, out, s));
}

moe_status moe_combine(moe_dims dims, const float* y_sorted, const int32_t* pair_row,
                       const float* topk_w, moe_bf16* out, void* stream) {
  g_last_error[0] = 0;
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_ptrs({y_sorted, pair_row, topk_w, out}, "moe_combine"));
  return hip_status(moe::launch_combine(y_sorted, pair_row, topk_w, dims.T, dims.d, dims.k, out,
                                        static_cast<hipStream_t>(stream)));
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
