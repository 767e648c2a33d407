// Weighted combine back to token order (Perplexity, "GPT-OSS el dia 0", section
// "Nuclis per a GPT-OSS / MoE": combine is the weighted accumulation of the
// experts' outputs). Atomic-free: each output element is owned by one thread,
// which gathers the token's k expert rows through pair_row and sums them in
// fixed slot order in fp32, then rounds once to bf16 (nearest even).
// Memory-bound: 16-byte loads of y, 8-byte stores of out; one block per (token
// row, 1024 columns), one 4-column chunk per thread, so all of a thread's k
// loads are in flight at once.
#include "common.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ topk_w, int d,
                                                      int k, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const float4* rows[8];
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      rows[j] = reinterpret_cast<const float4*>(y + (size_t)pair_row[(size_t)t * k + j] * d);
      w[j] = topk_w[(size_t)t * k + j];
    }
  }
  uint2* o = reinterpret_cast<uint2*>(out + (size_t)t * d);
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c < d / 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        const float4 v = rows[j][c];
        acc.x = fmaf(w[j], v.x, acc.x);
        acc.y = fmaf(w[j], v.y, acc.y);
        acc.z = fmaf(w[j], v.z, acc.z);
        acc.w = fmaf(w[j], v.w, acc.w);
      }
    }
    uint2 r;
    r.x = f32_to_bf16(acc.x) | (static_cast<uint32_t>(f32_to_bf16(acc.y)) << 16);
    r.y = f32_to_bf16(acc.z) | (static_cast<uint32_t>(f32_to_bf16(acc.w)) << 16);
    o[c] = r;
  }
}

}  // namespace

hipError_t launch_combine(const float* y_sorted, const int32_t* pair_row, const float* topk_w,
                          int T, int d, int k, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(T, (d / 4 + 255) / 256), dim3(256), 0, stream, y_sorted,
                     pair_row, topk_w, d, k, out);
  return hipGetLastError();
}

}  // namespace moe
