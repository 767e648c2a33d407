// Router: logits = x W_r + b_r in float64, then per token the top-k experts and a
// softmax over the k selected logits only (Perplexity, "GPT-OSS el dia 0",
// section "MLP" and section "Nuclis per a GPT-OSS / MoE"; the router weight is
// not quantised: CSDN "GPT-OSS-120B 4-bit 量化技术深度解析", section
// "Unsloth 4-bit量化技术解析").
//
// Float64 logits make the selection the exact top-k of the real-valued logits
// except where two logits differ by less than ~1e-12 relative, and the fixed
// summation order makes it deterministic.
//
// Few tokens (T <= 64): route_partial_small + route_select (below):
//   route_partial_small  one workgroup per 64-deep K slice: float64 partial
//                 logits of every (token, expert) of the slice.
//   route_select  one workgroup per token: the K-slice partials are reduced in a
//                 fixed order (+ bias), each expert's rank in (logit desc, index
//                 asc) order picks the top k, and the softmax over the picked
//                 logits is taken in float64.
// Many tokens: one launch, route_mfma. A workgroup takes 16 tokens; its eight
// wavefronts each take an eighth of K and accumulate the 16 x 16-expert tiles
// of logits with the float64 matrix instruction V_MFMA_F64_16X16X4_F64 (the
// bf16 x fp32 products are exact in float64, the sums are float64); the four
// ranges are added in wavefront order through LDS, the bias after them, and
// the workgroup then picks each token's top k and takes the softmax as above.
// (In each pass the ranges' sums are added in wavefront order, so the result
// does not depend on timing.)
#include "common.hpp"
#include "route_dev.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void route_select(const double* __restrict__ partial, int KS,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  rt::select_token(partial, KS, bias, T, E, k, blockIdx.x, topk_idx, topk_w);
}

// Many tokens: 16 tokens per workgroup, float64 matrix instructions.
//
// V_MFMA_F64_16X16X4_F64 multiplies a 16x4 A by a 4x16 B into 16x16 float64
// accumulators: lane l supplies A[l%16][l/16] and B[l/16][l%16], and holds
// D[l/16 + 4j][l%16] in register pair j (checked on gfx950 with one-hot B). Here A[m][q] is x of token t0+m and
// B[q][n] is W_r of expert 16b+n, both at K index k = 32c + 8q + s: in step s of
// 32-deep chunk c the lanes of quad q cover K elements 32c+8q+s, so that a lane
// reads its token's 8 consecutive bf16 of the chunk with one 16-byte load. The
// chunk's 8 steps cover its 32 K elements once each. The W_r reads are fp32
// (exact in float64), 16 experts = 64 contiguous bytes per quad.
typedef double v4d __attribute__((ext_vector_type(4)));
constexpr int kRtTok = 16;    // tokens per workgroup
constexpr int kRtWaves = 8;   // wavefronts per workgroup, one K range each
constexpr int kRtMaxNB = 4;   // 16-expert blocks per pass over K (more: further passes)

template <int NB>
__global__ __launch_bounds__(kRtWaves * 64) void route_mfma(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias, int T,
                                                            int d, int E, int k,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w) {
  __shared__ double red[kRtTok][16 * NB + 1];     // one pass: the K ranges, added in order
  __shared__ double logit[kRtTok][rt::kMaxE + 1];
  __shared__ double sel_v[kRtTok][8], sel_x[kRtTok][8];
  __shared__ int sel_e[kRtTok][8];
  constexpr int NT = kRtWaves * 64;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * kRtTok;
  const bool tv = t0 + r < T;
  const int nchunk = d / 32;
  const int c0 = wave * nchunk / kRtWaves, c1 = (wave + 1) * nchunk / kRtWaves;
  // rows past T read the last token (and count as zero); columns past E read the last expert
  const uint4* xrow = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + r, T - 1) * d + 8 * q);
  const int nbt = (E + 15) / 16;

  for (int eb0 = 0; eb0 < nbt; eb0 += NB) {
    // two accumulator chains per block (even and odd steps), added at the end
    v4d acc[2][NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[0][b] = acc[1][b] = v4d{0.0, 0.0, 0.0, 0.0};
    int col[NB];
    bool live[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      live[b] = 16 * (eb0 + b) + r < E;
      col[b] = min(16 * (eb0 + b) + r, E - 1);
    }
    auto load = [&](int c, uint4& xv, float (&wv)[8][NB]) __attribute__((always_inline)) {
      xv = xrow[c * 4];
      const float* wr = w + (size_t)(32 * c + 8 * q) * E;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
        for (int b = 0; b < NB; ++b) wv[s2][b] = wr[(size_t)s2 * E + col[b]];
    };
    auto compute = [&](const uint4& xv, const float (&wv)[8][NB]) __attribute__((always_inline)) {
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const float xf = bf16_to_f32(s2 & 1 ? (xw[s2 >> 1] >> 16) : (xw[s2 >> 1] & 0xffffu));
        const double a = static_cast<double>(tv ? xf : 0.0f);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[s2 & 1][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(
              a, static_cast<double>(live[b] ? wv[s2][b] : 0.0f), acc[s2 & 1][b], 0, 0, 0);
      }
    };
    // two chunks in flight: the loads of chunk c+1 are issued before chunk c is computed
    uint4 xa, xb;
    float wa[8][NB], wb[8][NB];
    int c = c0;
    if (c < c1) load(c, xa, wa);
    for (; c + 1 < c1; c += 2) {
      load(c + 1, xb, wb);
      compute(xa, wa);
      if (c + 2 < c1) load(c + 2, xa, wa);
      compute(xb, wb);
    }
    if (c < c1) compute(xa, wa);

    // the K ranges, added in wavefront order
    for (int wv2 = 0; wv2 < kRtWaves; ++wv2) {
      if (wave == wv2) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            double& dst = red[q + 4 * j][16 * b + r];
            const double v = acc[0][b][j] + acc[1][b][j];
            dst = wv2 == 0 ? v : dst + v;
          }
      }
      __syncthreads();
    }
    for (int i = tid; i < kRtTok * 16 * NB; i += NT) {
      const int m = i / (16 * NB), n = i - m * (16 * NB);
      const int e = 16 * eb0 + n;
      if (e < E) {
        double v = red[m][n];
        if (bias) v += static_cast<double>(bias[e]);
        logit[m][e] = v == v ? v : -INFINITY;
      }
    }
    __syncthreads();
  }

  // top k of each token: the rank of expert e is the number of experts before it
  // in (logit descending, index ascending) order; ranks are distinct
  for (int i = tid; i < kRtTok * E; i += NT) {
    const int m = i / E, e = i - m * E;
    const double v = logit[m][e];
    int rank = 0;
    for (int j = 0; j < E; ++j) rank += rt::better(logit[m][j], j, v, e) ? 1 : 0;
    if (rank < k) {
      sel_v[m][rank] = v;
      sel_e[m][rank] = e;
    }
  }
  __syncthreads();
  // softmax over the picks in float64: one exponential per (token, pick), then
  // each pick's lane sums the token's k exponentials in rank order
  const int m = tid / 8, j = tid & 7;
  if (m < kRtTok && j < k) sel_x[m][j] = exp(sel_v[m][j] - sel_v[m][0]);
  __syncthreads();
  if (m < kRtTok && j < k && t0 + m < T) {
    double den = 0.0;
    for (int i = 0; i < k; ++i) den += sel_x[m][i];
    topk_idx[(size_t)(t0 + m) * k + j] = sel_e[m][j];
    topk_w[(size_t)(t0 + m) * k + j] = static_cast<float>(sel_x[m][j] / den);
  }
}

__global__ __launch_bounds__(256) void route_partial_small(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ w, int T,
                                                           int d, int E,
                                                           double* __restrict__ partial) {
  rt::partial_slice(x, w, T, d, E, blockIdx.x, partial);
}

size_t al256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t route_workspace_bytes(int T, int d, int E) {
  // the many-token kernel needs no scratch
  if (T <= rt::kSmallT) return al256((size_t)(d / 64) * T * E * sizeof(double));
  return 0;
}

hipError_t launch_route(const uint16_t* x, const float* w_router, const float* b_router, int T,
                        int d, int E, int k, int32_t* topk_idx, float* topk_w, void* ws,
                        hipStream_t stream) {
  hipError_t err;
  if (T <= rt::kSmallT) {
    double* partial = static_cast<double*>(ws);
    hipLaunchKernelGGL(route_partial_small, dim3(d / 64), dim3(256), 0, stream, x, w_router, T, d,
                       E, partial);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(route_select, dim3(T), dim3(256), 0, stream, partial, d / 64, b_router, T,
                       E, k, topk_idx, topk_w);
    return hipGetLastError();
  }
  const dim3 grid((T + kRtTok - 1) / kRtTok);
  const int nbt = (E + 15) / 16;
  if (nbt <= 1)
    hipLaunchKernelGGL(route_mfma<1>, grid, dim3(kRtWaves * 64), 0, stream, x, w_router, b_router, T, d, E, k, topk_idx, topk_w);
  else if (nbt <= 2)
    hipLaunchKernelGGL(route_mfma<2>, grid, dim3(kRtWaves * 64), 0, stream, x, w_router, b_router, T, d, E, k, topk_idx, topk_w);
  else
    hipLaunchKernelGGL(route_mfma<kRtMaxNB>, grid, dim3(kRtWaves * 64), 0, stream, x, w_router, b_router, T, d, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
