// Pre-norm and residual for a stack of MoE blocks.
// RMSNorm: out = bf16(x / sqrt(mean(x^2) + eps) * gain) with fp32 arithmetic
// (rms_norm_eps = 1e-5: CSDN "GPT-OSS-120B 4-bit 量化技术深度解析", section "推理优化").
// Residual: out = bf16(x + m), fp32 add, round to nearest even.
// Residual + RMSNorm: the residual add of one block and the pre-norm of the
// next in one pass over the row.
// All memory-bound. The norms take one wavefront per row (four rows per
// workgroup, no workgroup barrier): lane l holds 16-byte chunks l, l + 64, ...
// of its row, the first kRegChunks of them in registers between the sum of
// squares and the scaling (the rest are read again), and sums its squares in
// chunk order before a butterfly over the wavefront, so both norm kernels sum
// in the same order and give the same bytes for the same row.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kRegChunks = 8;   // d <= 4096 stays in registers

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xffff);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// eight floats to bf16, round to nearest even, by the hardware's paired
// conversion (V_CVT_PK_BF16_F32; the same results as f32_to_bf16 for every
// non-NaN input)
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f[2 * i], f[2 * i + 1]}, bf16x2));
  return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ uint4 add8(const uint4& a, const uint4& b) {
  float fa[8], fb[8];
  unpack8(a, fa);
  unpack8(b, fb);
#pragma unroll
  for (int i = 0; i < 8; ++i) fa[i] += fb[i];
  return pack8(fa);
}

__device__ __forceinline__ float sumsq8(const uint4& v, float ss) {
  float f[8];
  unpack8(v, f);
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
  return ss;
}

__device__ __forceinline__ uint4 scale8(const uint4& v, const uint4& g, float inv) {
  float f[8], gf[8];
  unpack8(v, f);
  unpack8(g, gf);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = f[i] * inv * gf[i];
  return pack8(f);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// One row: with RESID, s = bf16(x + m) is stored to xout and normalised;
// otherwise x itself is.
template <bool RESID>
__device__ __forceinline__ void norm_row(const uint4* x, const uint4* m, const uint4* gain, int n8,
                                         float eps, float dn, uint4* xout, uint4* nout) {
  const int lane = threadIdx.x & (kWave - 1);
  // every load of the cached chunks is issued before the first store (x may
  // alias xout, so the compiler could not move them past it)
  uint4 reg[kRegChunks], mr[kRegChunks];
#pragma unroll
  for (int i = 0; i < kRegChunks; ++i) {
    const int c = lane + kWave * i;
    if (c < n8) {
      reg[i] = x[c];
      if constexpr (RESID) mr[i] = m[c];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kRegChunks; ++i) {
    const int c = lane + kWave * i;
    if (c < n8) {
      if constexpr (RESID) {
        reg[i] = add8(reg[i], mr[i]);
        xout[c] = reg[i];
      }
      ss = sumsq8(reg[i], ss);
    }
  }
  for (int c = lane + kWave * kRegChunks; c < n8; c += kWave) {
    uint4 v = x[c];
    if constexpr (RESID) {
      v = add8(v, m[c]);
      xout[c] = v;
    }
    ss = sumsq8(v, ss);
  }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / dn + eps);
#pragma unroll
  for (int i = 0; i < kRegChunks; ++i) {
    const int c = lane + kWave * i;
    if (c < n8) nout[c] = scale8(reg[i], gain[c], inv);
  }
  // past the cache: read back what this lane itself wrote (RESID) or x
  const uint4* src = RESID ? xout : x;
  for (int c = lane + kWave * kRegChunks; c < n8; c += kWave) nout[c] = scale8(src[c], gain[c], inv);
}

__global__ __launch_bounds__(kRowsPerBlock * kWave) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                                        const uint16_t* __restrict__ gain,
                                                                        int T, int d, float eps,
                                                                        uint16_t* __restrict__ out) {
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t o = (size_t)t * d;
  norm_row<false>(reinterpret_cast<const uint4*>(x + o), nullptr, reinterpret_cast<const uint4*>(gain),
                  d / 8, eps, static_cast<float>(d), nullptr, reinterpret_cast<uint4*>(out + o));
}

// xout may alias x (each chunk is read, then written, by one lane); nout
// aliases neither.
__global__ __launch_bounds__(kRowsPerBlock * kWave) void residual_rmsnorm_kernel(
    const uint16_t* x, const uint16_t* __restrict__ m, const uint16_t* __restrict__ gain, int T, int d,
    float eps, uint16_t* xout, uint16_t* __restrict__ nout) {
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t o = (size_t)t * d;
  norm_row<true>(reinterpret_cast<const uint4*>(x + o), reinterpret_cast<const uint4*>(m + o),
                 reinterpret_cast<const uint4*>(gain), d / 8, eps, static_cast<float>(d),
                 reinterpret_cast<uint4*>(xout + o), reinterpret_cast<uint4*>(nout + o));
}

// out may alias x or m (each element is read, then written, by one thread), so
// none of the three is declared __restrict__.
__global__ __launch_bounds__(256) void residual_kernel(const uint4* x, const uint4* m, size_t n8,
                                                       uint4* out) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x)
    out[i] = add8(x[i], m[i]);
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gain, int T, int d, float eps,
                          uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((T + kRowsPerBlock - 1) / kRowsPerBlock), dim3(kRowsPerBlock * kWave),
                     0, stream, x, gain, T, d, eps, out);
  return hipGetLastError();
}

hipError_t launch_residual_rmsnorm(const uint16_t* x, const uint16_t* m, const uint16_t* gain, int T,
                                   int d, float eps, uint16_t* xout, uint16_t* nout,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3((T + kRowsPerBlock - 1) / kRowsPerBlock),
                     dim3(kRowsPerBlock * kWave), 0, stream, x, m, gain, T, d, eps, xout, nout);
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
