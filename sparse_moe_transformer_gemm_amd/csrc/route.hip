// Router: logits = x W_r + b_r in float64, then per token the top-k experts and a
// softmax over the k selected logits only (Perplexity, "GPT-OSS el dia 0",
// section "MLP" and section "Nuclis per a GPT-OSS / MoE").
//
// Two kernels:
//   route_logits  grid (token tiles, K slices). Each block holds 16 tokens and all
//                 E experts; x and W_r are staged through LDS in 32-deep K tiles and
//                 accumulated in float64. When there are few token tiles (decode)
//                 K is split across blocks so the chip fills; partial sums go to
//                 the workspace as [slice][T][E].
//   route_topk    one wavefront per token: sums the slices in fixed order, then k
//                 rounds of a wave-wide (max logit, min index) reduction pick the
//                 experts; the softmax is taken in float64 and stored as fp32.
// Logits in float64 make the selection exact except where two logits differ by
// less than ~1e-12 relative; the summation order is fixed, so the result is
// deterministic.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kTM = 16;       // tokens per block
constexpr int kKT = 32;       // K depth of one LDS tile
constexpr int kMaxE = 256;

int route_kslices(int T, int d) {
  int tiles = (T + kTM - 1) / kTM;
  int ktiles = d / kKT;
  if (tiles >= 256) return 1;
  int want = (512 + tiles - 1) / tiles;
  return want < ktiles ? want : ktiles;
}

__global__ __launch_bounds__(256) void route_logits(const uint16_t* __restrict__ x,
                                                    const float* __restrict__ w, int T, int d,
                                                    int E, int kslice,
                                                    double* __restrict__ partial) {
  __shared__ double xs[kTM][kKT + 1];
  __shared__ double wt[kKT][kMaxE];
  const int t0 = blockIdx.x * kTM;
  const int kbeg = blockIdx.y * kslice;
  const int kend = min(d, kbeg + kslice);
  const int tid = threadIdx.x;
  const int tt = tid >> 4;   // token of this thread inside the tile
  const int el = tid & 15;   // experts el, el+16, ...
  const int ne = (E + 15) >> 4;

  double acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0;

  for (int k0 = kbeg; k0 < kend; k0 += kKT) {
    for (int i = tid; i < kTM * kKT; i += 256) {
      int r = i / kKT, c = i % kKT, t = t0 + r, kk = k0 + c;
      xs[r][c] = (t < T && kk < kend) ? static_cast<double>(bf16_to_f32(x[(size_t)t * d + kk])) : 0.0;
    }
    for (int i = tid; i < kKT * E; i += 256) {
      int r = i / E, c = i % E, kk = k0 + r;
      wt[r][c] = (kk < kend) ? static_cast<double>(w[(size_t)kk * E + c]) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kKT; ++kk) {
      const double xv = xs[tt][kk];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = el + 16 * i;
        if (i < ne && e < E) acc[i] = fma(xv, wt[kk][e], acc[i]);
      }
    }
    __syncthreads();
  }
  const int t = t0 + tt;
  if (t < T) {
    double* dst = partial + ((size_t)blockIdx.y * T + t) * E;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = el + 16 * i;
      if (i < ne && e < E) dst[e] = acc[i];
    }
  }
}

__device__ __forceinline__ bool better(double va, int ea, double vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

__global__ __launch_bounds__(256) void route_topk(const double* __restrict__ partial, int KS,
                                                  const float* __restrict__ bias, int T, int E,
                                                  int k, int32_t* __restrict__ topk_idx,
                                                  float* __restrict__ topk_w) {
  const int t = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (t >= T) return;  // uniform per wavefront

  double v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    double s = -INFINITY;
    if (e < E) {
      s = 0.0;
      for (int ks = 0; ks < KS; ++ks) s += partial[((size_t)ks * T + t) * E + e];
      if (bias) s += static_cast<double>(bias[e]);
    }
    v[i] = s;
  }

  unsigned taken = 0;
  double sel_v[8];
  int sel_e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_v[j] = 0.0;
    sel_e[j] = 0;
    if (j < k) {
      double bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + kWave * i;
        if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, be)) {
          bv = v[i];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      sel_v[j] = bv;
      sel_e[j] = be;
      if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    }
  }

  double den = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) den += exp(sel_v[j] - sel_v[0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k && lane == j) {
      topk_idx[(size_t)t * k + j] = sel_e[j];
      topk_w[(size_t)t * k + j] = static_cast<float>(exp(sel_v[j] - sel_v[0]) / den);
    }
  }
}

}  // namespace

size_t route_workspace_bytes(int T, int d, int E) {
  return (size_t)route_kslices(T, d) * T * E * sizeof(double);
}

hipError_t launch_route(const uint16_t* x, const float* w_router, const float* b_router, int T,
                        int d, int E, int k, int32_t* topk_idx, float* topk_w, void* ws,
                        hipStream_t stream) {
  const int KS = route_kslices(T, d);
  const int ktiles = d / kKT;
  const int kslice = ((ktiles + KS - 1) / KS) * kKT;
  const int KSeff = (d + kslice - 1) / kslice;
  double* partial = static_cast<double*>(ws);
  dim3 g1((T + kTM - 1) / kTM, KSeff);
  hipLaunchKernelGGL(route_logits, g1, dim3(256), 0, stream, x, w_router, T, d, E, kslice, partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 g2((T + 3) / 4);
  hipLaunchKernelGGL(route_topk, g2, dim3(256), 0, stream, partial, KSeff, b_router, T, E, k,
                     topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
