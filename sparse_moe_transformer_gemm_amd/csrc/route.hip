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
// Few tokens (T <= 64): route_partial_small + route_select (below). Otherwise
// three kernels (route_select_many in place of route_select):
//   route_widen   W_r (fp32 [d][E]) -> float64 [d][Epad] in the workspace
//                 (Epad = E rounded up to 32, zero padded).
//   route_logits  grid (256-token blocks, K slices, 32-expert groups). One lane
//                 per token, 32 float64 accumulators per lane; each 64-deep K
//                 chunk of W is staged once in LDS and read as broadcasts by all
//                 four wavefronts. Partial sums [slice][T][E] are written through
//                 an LDS transpose so the stores coalesce.
//   route_select  one workgroup per token: the K-slice partials are reduced in a
//                 fixed order (+ bias), each expert's rank in (logit desc, index
//                 asc) order picks the top k, and the softmax over the picked
//                 logits is taken in float64.
#include "common.hpp"
#include "route_dev.hpp"

namespace moe {
namespace {

constexpr int kTok = 256;     // tokens per logits block (4 wavefronts, one lane per token)
constexpr int kEG = 32;       // experts per group (accumulators per lane)
constexpr int kKC = 64;       // K depth of one LDS stage
constexpr int kTargetBlocks = 480;

struct RoutePlan {
  int Epad, ngroups, tblocks, kslice, nslices;
};

RoutePlan route_plan(int T, int d, int E) {
  RoutePlan p;
  p.Epad = (E + kEG - 1) / kEG * kEG;
  p.ngroups = p.Epad / kEG;
  p.tblocks = (T + kTok - 1) / kTok;
  const int base = p.tblocks * p.ngroups;
  int want = (kTargetBlocks + base - 1) / base;
  const int kstages = d / kKC;
  if (want > kstages) want = kstages;
  if (want < 1) want = 1;
  p.kslice = (kstages + want - 1) / want * kKC;
  p.nslices = (d + p.kslice - 1) / p.kslice;
  return p;
}

__global__ __launch_bounds__(256) void route_widen(const float* __restrict__ w, int d, int E,
                                                   int Epad, double* __restrict__ w64) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= (size_t)d * Epad) return;
  const int k = static_cast<int>(i / Epad), e = static_cast<int>(i % Epad);
  w64[i] = e < E ? static_cast<double>(w[(size_t)k * E + e]) : 0.0;
}

__global__ __launch_bounds__(256) void route_logits(const uint16_t* __restrict__ x,
                                                    const double* __restrict__ w64, int T, int d,
                                                    int E, int Epad, int kslice,
                                                    double* __restrict__ partial) {
  // two W stages of [kKC][kEG] doubles (32 KB) during the K loop; the same memory
  // then holds the [kTok][kEG+1] transpose of the accumulators (67.6 KB)
  __shared__ __attribute__((aligned(16))) double smem[kTok * (kEG + 1)];
  const int tid = threadIdx.x;
  const int t = blockIdx.x * kTok + tid;
  const int slice = blockIdx.y, eg = blockIdx.z;
  const int k0 = slice * kslice;
  const int k1 = min(d, k0 + kslice);
  const bool valid = t < T;
  const bool wave_live = blockIdx.x * kTok + (tid & ~63) < T;  // uniform per wavefront

  double acc[kEG];
#pragma unroll
  for (int e = 0; e < kEG; ++e) acc[e] = 0.0;

  // stage loader: the 64x32 W chunk is 1024 double2 = 4 per thread
  const double* wsrc = w64 + (size_t)eg * kEG;
  double2 pre[4];
  auto load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;           // double2 index in the chunk
      const int kk = c >> 4, e2 = (c & 15) * 2;
      pre[i] = (kb + kk < k1) ? *reinterpret_cast<const double2*>(wsrc + (size_t)(kb + kk) * Epad + e2)
                              : make_double2(0.0, 0.0);
    }
  };
  auto store = [&](int buf) {
    double2* dst = reinterpret_cast<double2*>(smem + buf * kKC * kEG);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[tid + 256 * i] = pre[i];
  };

  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)(valid ? t : 0) * d);
  const int nst = (k1 - k0 + kKC - 1) / kKC;
  load(k0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int kb = k0 + s * kKC;
    if (s + 1 < nst) load(kb + kKC);
    if (wave_live) {
      const double2* ws2 = reinterpret_cast<const double2*>(smem + (s & 1) * kKC * kEG);
      const int kend = min(kKC, k1 - kb);
      for (int k8 = 0; k8 < kend; k8 += 8) {
        const uint4 xv = valid ? xr[(kb + k8) >> 3] : make_uint4(0, 0, 0, 0);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const double xd = static_cast<double>(bf16_to_f32(h & 1 ? (xw[h >> 1] >> 16) : (xw[h >> 1] & 0xffffu)));
          const double2* wrow = ws2 + (k8 + h) * (kEG / 2);
#pragma unroll
          for (int e2 = 0; e2 < kEG / 2; ++e2) {
            const double2 wv = wrow[e2];
            acc[2 * e2] = fma(xd, wv.x, acc[2 * e2]);
            acc[2 * e2 + 1] = fma(xd, wv.y, acc[2 * e2 + 1]);
          }
        }
      }
    }
    if (s + 1 < nst) store((s + 1) & 1);
    __syncthreads();
  }

  // transpose through LDS so that the partial stores are contiguous
#pragma unroll
  for (int e = 0; e < kEG; ++e) smem[tid * (kEG + 1) + e] = acc[e];
  __syncthreads();
  const int ebase = eg * kEG;
  const int ne = min(kEG, E - ebase);
  for (int i = tid; i < kTok * kEG; i += 256) {
    const int tl = i / kEG, e = i % kEG;
    const int tt = blockIdx.x * kTok + tl;
    if (tt < T && e < ne)
      partial[((size_t)slice * T + tt) * E + ebase + e] = smem[tl * (kEG + 1) + e];
  }
}

__global__ __launch_bounds__(256) void route_select(const double* __restrict__ partial, int KS,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  rt::select_token(partial, KS, bias, T, E, k, blockIdx.x, topk_idx, topk_w);
}

// Many tokens: 256 / Ep tokens per workgroup (Ep = E rounded up to a power of
// two), one thread per (token, expert): the logit sums the token's K-slice
// partials in slice order (+ bias), the expert's rank among the token's E
// logits picks the top k, and the k picked lanes' softmax is taken in float64
// as in rt::select_topk.
__global__ __launch_bounds__(256) void route_select_many(const double* __restrict__ partial, int KS,
                                                         const float* __restrict__ bias, int T,
                                                         int E, int Ep, int k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  __shared__ double logit[256];
  __shared__ double sel_v[256 * 8];   // [token slot][rank]: up to 256 slots (E = 1), k <= 8
  __shared__ int sel_e[256 * 8];
  const int tid = threadIdx.x;
  const int j = tid / Ep, e = tid - j * Ep;     // token slot in the workgroup, expert
  const int tpw = 256 / Ep;
  const int t = blockIdx.x * tpw + j;
  const bool live = t < T && e < E;
  if (live) {
    double v = 0.0;
    const double* p = partial + (size_t)t * E + e;
#pragma unroll 8
    for (int ks = 0; ks < KS; ++ks) v += p[(size_t)ks * T * E];
    if (bias) v += static_cast<double>(bias[e]);
    logit[tid] = v == v ? v : -INFINITY;
  }
  __syncthreads();
  if (live) {
    const double* row = logit + j * Ep;
    const double v = row[e];
    int rank = 0;
    for (int i = 0; i < E; ++i) rank += rt::better(row[i], i, v, e) ? 1 : 0;
    if (rank < k) {
      sel_v[j * 8 + rank] = v;
      sel_e[j * 8 + rank] = e;
    }
  }
  __syncthreads();
  if (t < T && e < k) {
    const double m = sel_v[j * 8];
    double den = 0.0;
    for (int i = 0; i < k; ++i) den += exp(sel_v[j * 8 + i] - m);
    topk_idx[(size_t)t * k + e] = sel_e[j * 8 + e];
    topk_w[(size_t)t * k + e] = static_cast<float>(exp(sel_v[j * 8 + e] - m) / den);
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
  if (T <= rt::kSmallT) return al256((size_t)(d / 64) * T * E * sizeof(double));
  const RoutePlan p = route_plan(T, d, E);
  return al256((size_t)d * p.Epad * sizeof(double)) +
         al256((size_t)p.nslices * T * E * sizeof(double));
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
  const RoutePlan p = route_plan(T, d, E);
  double* w64 = static_cast<double*>(ws);
  double* partial = reinterpret_cast<double*>(static_cast<uint8_t*>(ws) +
                                              al256((size_t)d * p.Epad * sizeof(double)));
  const size_t nw = (size_t)d * p.Epad;
  hipLaunchKernelGGL(route_widen, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream,
                     w_router, d, E, p.Epad, w64);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_logits, dim3(p.tblocks, p.nslices, p.ngroups), dim3(256), 0, stream, x,
                     w64, T, d, E, p.Epad, p.kslice, partial);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int tpw = 256 / Ep;
  hipLaunchKernelGGL(route_select_many, dim3((T + tpw - 1) / tpw), dim3(256), 0, stream, partial,
                     p.nslices, b_router, T, E, Ep, k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
