// Router device functions shared by the routing kernels (route.hip) and the
// fused decode front end (front.hip): the small-batch K-slice partial logits and
// the per-token reduce + top-k + softmax (Perplexity, "GPT-OSS el dia 0",
// section "MLP": softmax over the selected experts; section "Nuclis per a
// GPT-OSS / MoE": the routing scheme).
#pragma once

#include "common.hpp"

namespace moe {
namespace rt {

constexpr int kMaxE = 256;

__device__ __forceinline__ bool better(double va, int ea, double vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

// Top-k of the E logits in `logit` (LDS, float64) for token t, by the whole
// workgroup: the rank of expert e is the number of experts that come before it
// in the order (larger logit first, lower index on equal logits). Ranks are
// distinct, so the experts of rank < k are the top k in order; a NaN logit has
// been stored as -inf. Then the softmax over the picked logits in float64, each
// of the k lanes summing the k exponentials in rank order, stored as fp32.
// Every thread of the workgroup must call it (it contains barriers).
__device__ __forceinline__ void select_topk(const double* logit, int t, int E, int k,
                                            double* sel_v, int* sel_e,
                                            int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_w) {
  const int tid = threadIdx.x;
  if (tid < E) {
    const double v = logit[tid];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < E; ++j) rank += better(logit[j], j, v, tid) ? 1 : 0;
    if (rank < k) {
      sel_v[rank] = v;
      sel_e[rank] = tid;
    }
  }
  __syncthreads();
  // each of the k lanes takes one exponential (float64 exp is long), then each
  // sums all k in rank order
  __shared__ double sel_x[8];
  if (tid < k) sel_x[tid] = exp(sel_v[tid] - sel_v[0]);
  __syncthreads();
  if (tid < k) {
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += sel_x[j];
    topk_idx[(size_t)t * k + tid] = sel_e[tid];
    topk_w[(size_t)t * k + tid] = static_cast<float>(sel_x[tid] / den);
  }
}

// Logits of token t from the K-slice partials [KS][T][E], reduced in a fixed
// order (+ bias), then its top-k and softmax; one workgroup of 256 threads.
__device__ __forceinline__ void select_token(const double* __restrict__ partial, int KS,
                                             const float* __restrict__ bias, int T, int E, int k,
                                             int t, int32_t* __restrict__ topk_idx,
                                             float* __restrict__ topk_w) {
  __shared__ double part[256];
  __shared__ double logit[kMaxE];
  __shared__ double sel_v[8];
  __shared__ int sel_e[8];
  const int tid = threadIdx.x;
  const int G = 256 / E;
  if (tid < G * E) {
    const int e = tid % E, g = tid / E;
    double s = 0.0;
    // the slices g, g + G, ... are loaded eight at a time before any is added
    // (one memory round trip per eight), then added in slice order
    for (int k0 = g; k0 < KS; k0 += 8 * G) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ks = k0 + u * G;
        v[u] = ks < KS ? partial[((size_t)ks * T + t) * E + e] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u * G < KS) s += v[u];
    }
    part[g * E + e] = s;
  }
  __syncthreads();
  if (tid < E) {
    double v = 0.0;
    for (int g = 0; g < G; ++g) v += part[g * E + tid];
    if (bias) v += static_cast<double>(bias[tid]);
    logit[tid] = v == v ? v : -INFINITY;
  }
  __syncthreads();
  select_topk(logit, t, E, k, sel_v, sel_e, topk_idx, topk_w);
}

// Few tokens (decode): the workgroup of 64-deep K slice `slice` computes every
// (token, expert) partial dot product of its slice in float64, with the slice of
// W_r (read once, coalesced) and of x held in LDS; select_token then reduces the
// d/64 slices in order. No widened copy of W_r is needed.
constexpr int kSmallT = 64;

__device__ __forceinline__ void partial_slice(const uint16_t* __restrict__ x,
                                              const float* __restrict__ w, int T, int d, int E,
                                              int slice, double* __restrict__ partial) {
  __shared__ float ws[64 * kMaxE];      // W_r rows k0..k0+63, all experts (fp32 is exact)
  __shared__ float xs[kSmallT * 65];    // x[t][k0..k0+63] as fp32 (bf16 is exact in fp32)
  const int k0 = slice * 64;
  const int tid = threadIdx.x;
  // all loads of the slice are issued before any is used: W rows k0..k0+63 are
  // 16*E float4 (E is a multiple of 4 here or handled by the scalar tail),
  // x[t][k0..k0+63] is 8 uint4 per token
  const int nw4 = (64 * E) / 4;
  float4 wv[kMaxE / 16];
#pragma unroll
  for (int i = 0; i < kMaxE / 16; ++i) {
    const int c = tid + 256 * i;
    wv[i] = c < nw4 ? reinterpret_cast<const float4*>(w + (size_t)k0 * E)[c] : make_float4(0, 0, 0, 0);
  }
  uint4 xv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;        // (token, 8-element chunk)
    const int t = c >> 3, ch = c & 7;
    xv[i] = t < T ? reinterpret_cast<const uint4*>(x + (size_t)t * d + k0)[ch] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kMaxE / 16; ++i) {
    const int c = tid + 256 * i;
    if (c < nw4) reinterpret_cast<float4*>(ws)[c] = wv[i];
  }
  for (int i = nw4 * 4 + tid; i < 64 * E; i += 256) ws[i] = w[(size_t)k0 * E + i];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int t = c >> 3, ch = c & 7;
    if (t < T) {
      const uint32_t u[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        xs[t * 65 + ch * 8 + 2 * h] = bf16_to_f32(u[h] & 0xffffu);
        xs[t * 65 + ch * 8 + 2 * h + 1] = bf16_to_f32(u[h] >> 16);
      }
    }
  }
  __syncthreads();
  for (int p = tid; p < T * E; p += 256) {
    const int t = p / E, e = p - t * E;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};   // four chains (kk mod 4), summed in a fixed order
#pragma unroll
    for (int kk = 0; kk < 64; ++kk)
      acc[kk & 3] = fma(static_cast<double>(xs[t * 65 + kk]), static_cast<double>(ws[kk * E + e]),
                        acc[kk & 3]);
    partial[((size_t)slice * T + t) * E + e] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
}

}  // namespace rt
}  // namespace moe
