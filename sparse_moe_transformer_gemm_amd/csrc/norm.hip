// Pre-norm and residual for a stack of MoE blocks.
// RMSNorm: out = bf16(x / sqrt(mean(x^2) + eps) * gain) with fp32 arithmetic
// (rms_norm_eps = 1e-5: CSDN "GPT-OSS-120B 4-bit 量化技术深度解析", section "推理优化").
// Residual: out = bf16(x + m), fp32 add, round to nearest even.
// Residual + RMSNorm: the residual add of one block and the pre-norm of the
// next in one pass over the row.
// Combine + residual + RMSNorm: the block's weighted combine (Perplexity, "GPT-OSS
// el dia 0", section "Nuclis per a GPT-OSS / MoE": the weighted accumulation of
// the experts' outputs), the residual add and the next block's pre-norm in one
// pass, so the block output m never makes a round trip through memory.
// All memory-bound. The norms take one wavefront per row (four rows per
// workgroup, no workgroup barrier): lane l holds 16-byte chunks l, l + 64, ...
// of its row, the first kRegChunks of them in registers between the sum of
// squares and the scaling (the rest are read again), and sums its squares in
// chunk order before a butterfly over the wavefront, so both norm kernels sum
// in the same order and give the same bytes for the same row.
#include "glue.hpp"
#include "mx6.hpp"

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

// One token row per workgroup of four wavefronts: m = bf16(sum over j of w_j *
// y_j), the fp32 multiply-adds in slot order from zero and one rounding (the
// arithmetic of the combine kernel); s = bf16(resid + m) is stored to resid_out
// (and m to mout when it is given) and kept in LDS; with NORM, wavefront 0 then
// sums the squares as norm_row does (lane l over the 8-column chunks l, l + 64,
// ... in order, then the butterfly), and every thread scales its share of s. So
// every output has the bytes of the separate combine, residual and norm kernels,
// while the loads of a row are spread over four wavefronts: wavefront v takes
// the chunk rounds i = v, v + 4, ... (chunk l + 64 i for lane l), kGlueChunks
// rounds at a time with all of their loads (2k quarter rows of y and the
// residual) issued before their sums. resid_out may alias resid (each chunk is
// read, then written, by one thread).
constexpr int kGlueWaves = 4;
constexpr int kGlueChunks = 2;
constexpr int kGlueMaxD = 16384;

template <int K, bool NORM>
__global__ __launch_bounds__(kGlueWaves * kWave) void combine_residual_norm_kernel(
    const float* __restrict__ y, const int32_t* __restrict__ pair_row,
    const float* __restrict__ topk_w, const uint16_t* resid, const uint16_t* __restrict__ gain,
    int d, float eps, uint16_t* __restrict__ mout, uint16_t* resid_out,
    uint16_t* __restrict__ nout) {
  extern __shared__ uint4 srow[];  // the row's s (NORM only): d / 8 chunks
  __shared__ float sinv;
  const int t = blockIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int n8 = d / 8;
  rsrc_t rows[K];
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int row = __builtin_amdgcn_readfirstlane(pair_row[(size_t)t * K + j]);
    rows[j] = make_rsrc(y + (size_t)row * d, (uint32_t)d * 4u);
    w[j] = topk_w[(size_t)t * K + j];
  }
  const size_t o = (size_t)t * d;
  const rsrc_t rx = make_rsrc(resid + o, (uint32_t)d * 2u);
  uint4* ro = reinterpret_cast<uint4*>(resid_out + o);
  uint4* mo = mout ? reinterpret_cast<uint4*>(mout + o) : nullptr;
  for (int i0 = wv; kWave * i0 < n8; i0 += kGlueWaves * kGlueChunks) {
    uint4 va[kGlueChunks][K], vb[kGlueChunks][K], vx[kGlueChunks];
#pragma unroll
    for (int u = 0; u < kGlueChunks; ++u) {
      const int c = lane + kWave * (i0 + kGlueWaves * u);
      const uint32_t off = c < n8 ? (uint32_t)c * 32u : kOutOfRange;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        va[u][j] = bload16nt(rows[j], off);
        vb[u][j] = bload16nt(rows[j], off, 16u);
      }
      vx[u] = bload16(rx, c < n8 ? (uint32_t)c * 16u : kOutOfRange);
    }
#pragma unroll
    for (int u = 0; u < kGlueChunks; ++u) {
      const int c = lane + kWave * (i0 + kGlueWaves * u);
      if (c < n8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j) {
          acc[0] = fmaf(w[j], __uint_as_float(va[u][j].x), acc[0]);
          acc[1] = fmaf(w[j], __uint_as_float(va[u][j].y), acc[1]);
          acc[2] = fmaf(w[j], __uint_as_float(va[u][j].z), acc[2]);
          acc[3] = fmaf(w[j], __uint_as_float(va[u][j].w), acc[3]);
          acc[4] = fmaf(w[j], __uint_as_float(vb[u][j].x), acc[4]);
          acc[5] = fmaf(w[j], __uint_as_float(vb[u][j].y), acc[5]);
          acc[6] = fmaf(w[j], __uint_as_float(vb[u][j].z), acc[6]);
          acc[7] = fmaf(w[j], __uint_as_float(vb[u][j].w), acc[7]);
        }
        uint4 m;
        m.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
        m.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
        m.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
        m.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
        const uint4 sv = add8(vx[u], m);
        ro[c] = sv;
        if (mo) mo[c] = m;
        if constexpr (NORM) srow[c] = sv;
      }
    }
  }
  if constexpr (NORM) {
    __syncthreads();
    if (wv == 0) {
      float ss = 0.f;
      for (int c = lane; c < n8; c += kWave) ss = sumsq8(srow[c], ss);
      const float inv = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(d) + eps);
      if (lane == 0) sinv = inv;
    }
    __syncthreads();
    const float inv = sinv;
    const uint4* g = reinterpret_cast<const uint4*>(gain);
    uint4* no = reinterpret_cast<uint4*>(nout + o);
    for (int c = threadIdx.x; c < n8; c += kGlueWaves * kWave) no[c] = scale8(srow[c], g[c], inv);
  }
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

template <int K>
static void launch_crn(int T, hipStream_t stream, const float* y, const int32_t* pair_row,
                       const float* topk_w, const uint16_t* resid, const uint16_t* gain, int d,
                       float eps, uint16_t* mout, uint16_t* resid_out, uint16_t* nout) {
  const dim3 g(T), b(kGlueWaves * kWave);
  if (gain)
    hipLaunchKernelGGL((combine_residual_norm_kernel<K, true>), g, b, (size_t)d * 2, stream, y, pair_row, topk_w,
                       resid, gain, d, eps, mout, resid_out, nout);
  else
    hipLaunchKernelGGL((combine_residual_norm_kernel<K, false>), g, b, 0, stream, y, pair_row, topk_w,
                       resid, gain, d, eps, mout, resid_out, nout);
}

hipError_t launch_combine_residual_rmsnorm(const float* y_sorted, const int32_t* pair_row,
                                           const float* topk_w, const uint16_t* resid,
                                           const uint16_t* gain, int T, int d, int k, float eps,
                                           uint16_t* mout, uint16_t* resid_out, uint16_t* nout,
                                           hipStream_t stream) {
  if (d > kGlueMaxD) return hipErrorInvalidValue;
#define MOE_CRN(KK) launch_crn<KK>(T, stream, y_sorted, pair_row, topk_w, resid, gain, d, eps, mout, resid_out, nout)
  switch (k) {
    case 1: MOE_CRN(1); break;
    case 2: MOE_CRN(2); break;
    case 3: MOE_CRN(3); break;
    case 4: MOE_CRN(4); break;
    case 5: MOE_CRN(5); break;
    case 6: MOE_CRN(6); break;
    case 7: MOE_CRN(7); break;
    default: MOE_CRN(8); break;
  }
#undef MOE_CRN
  return hipGetLastError();
}

}  // namespace moe
