// Pre-norm and residual for a stack of MoE blocks.
// RMSNorm: out = bf16(x / sqrt(mean(x^2) + eps) * gain) with fp32 arithmetic
// (rms_norm_eps = 1e-5: CSDN "GPT-OSS-120B 4-bit 量化技术深度解析", section "推理优化").
// Residual: out = bf16(x + m), fp32 add, round to nearest even.
// Both memory-bound, one block per row for the norm (16-byte loads), a flat grid
// for the add.
#include "common.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ gain, int d,
                                                      float eps, uint16_t* __restrict__ out) {
  __shared__ float red[256 / kWave];
  const int t = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * d);
  const int n8 = d / 8;
  float ss = 0.f;
  for (int c = threadIdx.x; c < n8; c += blockDim.x) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_to_f32(w[i] & 0xffff), b = bf16_to_f32(w[i] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
  const uint4* gr = reinterpret_cast<const uint4*>(gain);
  uint4* orow = reinterpret_cast<uint4*>(out + (size_t)t * d);
  for (int c = threadIdx.x; c < n8; c += blockDim.x) {
    const uint4 v = xr[c], g = gr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_to_f32(w[i] & 0xffff) * inv * bf16_to_f32(gw[i] & 0xffff);
      const float b = bf16_to_f32(w[i] >> 16) * inv * bf16_to_f32(gw[i] >> 16);
      r[i] = f32_to_bf16(a) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
    }
    orow[c] = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

// out may alias x or m (each element is read, then written, by one thread), so
// none of the three is declared __restrict__.
__global__ __launch_bounds__(256) void residual_kernel(const uint4* x, const uint4* m, size_t n8,
                                                       uint4* out) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint4 a = x[i], b = m[i];
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_to_f32(aw[j] & 0xffff) + bf16_to_f32(bw[j] & 0xffff);
      const float hi = bf16_to_f32(aw[j] >> 16) + bf16_to_f32(bw[j] >> 16);
      r[j] = f32_to_bf16(lo) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
    out[i] = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gain, int T, int d, float eps,
                          uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, x, gain, d, eps, out);
  return hipGetLastError();
}

hipError_t launch_residual_add(const uint16_t* x, const uint16_t* m, int T, int d, uint16_t* out,
                               hipStream_t stream) {
  const size_t n8 = (size_t)T * d / 8;
  size_t blocks = (n8 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(residual_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(x), reinterpret_cast<const uint4*>(m), n8,
                     reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
