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
#include "mx6.hpp"
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
// D[l/16 + 4j][l%16] in register pair j (checked on gfx950 with one-hot B).
// Here A[m][q] is x of token t0+m and B[q][n] is W_r of expert 16b+n, both at K
// index k = 128c + 32q + s: in step s of 128-deep chunk c the lanes of quad q
// cover 32-element block 4c+q, so a lane holds one whole block of its token's
// x (four 16-byte loads) and the chunk's 32 steps cover its 128 K elements once
// each. The W_r reads are fp32 (exact in float64), 16 experts = 64 contiguous
// bytes per quad. A lane holding a whole block can also encode it for the
// expert GEMMs (two MXFP6-E2M3 terms, the encoding of encode_block), which the
// whole-block call uses to skip a separate pass over x.
typedef double v4d __attribute__((ext_vector_type(4)));
constexpr int kRtTok = 16;    // tokens per workgroup
// Wavefronts per workgroup, one K range each: four for up to 64 experts, eight
// above. With four, two workgroups share a CU (198 registers per lane allow two
// wavefronts per SIMD), so one workgroup's loads, top-k and softmax overlap the
// other's matrix work (measured: prefill-20b 1036.7 -> 1032.9 us per layer, the
// 24-block stack 8.17 -> 8.12 ms per pass); with 128 experts the eight-wavefront
// workgroup is faster (wide-120b 829 against 844 us). One shape always takes
// the same count, so the routing call and the whole-block call sum alike.
constexpr int kRtWaves = 8;       // K-split threshold unit (below)
inline int rt_waves(int E) { return E <= 64 ? 4 : 8; }
constexpr int kRtHalf = 16;   // K steps per half chunk (the unit of the load pipeline)

// K ranges per 16-token group: two when the groups are fewer than the 256 CUs
// of the MI355X and K has at least two chunks per wavefront in each range
// (d >= 2048), else one (a pure function of T and d: the separate routing call
// and the whole-block call make the same choice, so their logits are summed in
// the same order).
int route_ksplit(int T, int d) {
  const int groups = (T + kRtTok - 1) / kRtTok;
  const int nchunk = (d / 32 + 3) / 4;
  return groups < 256 && nchunk >= 2 * kRtWaves ? 2 : 1;
}

// PAIR (NB = 2, E even): lane r of a pass holds experts 2r and 2r + 1 instead of
// r and 16 + r, so each K row of W_r is one 8-byte load per lane (half the load
// instructions of 4-byte loads, which the texture addresser takes at the same rate).
//
// K split (partial non-null, gridDim.y = KS > 1): workgroup (g, s) takes the
// s-th of KS equal ranges of the K chunks for its 16 tokens and stores their
// logit sums without bias to partial[s][t][e]; route_select then adds the KS
// ranges in order, the bias, and takes the top k and the softmax. Used when the
// 16-token groups are fewer than the CUs, so that K keeps every CU busy.
template <int NB, bool ENC, bool PAIR, int WV>
__global__ __launch_bounds__(WV * 64) void route_mfma(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias, int T,
                                                            int d, int E, int k,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w,
                                                            uint8_t* __restrict__ xenc,
                                                            double* __restrict__ partial) {
  __shared__ double red[kRtTok][16 * NB + 1];     // one pass: the K ranges, added in order
  __shared__ double logit[kRtTok][rt::kMaxE + 1];
  __shared__ double sel_v[kRtTok][8], sel_x[kRtTok][8];
  __shared__ int sel_e[kRtTok][8];
  constexpr int NT = WV * 64;
  const int tid = threadIdx.x;
  // the wavefront index made uniform (SGPR), so the K-range loop needs no exec masks
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15,
            q = lane >> 4;
  const int t0 = blockIdx.x * kRtTok;
  const bool tv = t0 + r < T;
  const int nblk = d / 32;
  const int nchunk = (nblk + 3) / 4;               // the last one may hold two blocks
  // this workgroup's K chunks [kc0, kc1), dealt over its wavefronts
  const int ks = blockIdx.y, nks = gridDim.y;
  const int kc0 = ks * nchunk / nks, kc1 = (ks + 1) * nchunk / nks;
  const int c0 = kc0 + wave * (kc1 - kc0) / WV, c1 = kc0 + (wave + 1) * (kc1 - kc0) / WV;
  // columns past E read the last expert and blocks past K the last block of W_r:
  // valid addresses, and x is zero there
  // the workgroup's rows of x as a buffer: a row past T, a block past K or a chunk
  // past the wavefront's range reads zero through the range check, so no select
  // on the loaded values (which would wait for every load in flight) is needed
  const rsrc_t xr = make_rsrc(x + (size_t)t0 * d, (uint32_t)(min(kRtTok, T - t0) * d * 2));
  const int nbt = (E + 15) / 16;
  const uint32_t pitch = (uint32_t)nsteps_of(d) * kChunk;

  for (int eb0 = 0; eb0 < nbt; eb0 += NB) {
    // two accumulator chains per block (even and odd steps), added at the end
    v4d acc[2][NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[0][b] = acc[1][b] = v4d{0.0, 0.0, 0.0, 0.0};
    static_assert(!PAIR || NB == 2, "expert pairs need two blocks per pass");
    // the output column of block b held by lane r (the expert past 16 eb0)
    auto ncol = [&](int b) { return PAIR ? 2 * r + b : 16 * b + r; };
    int col[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) col[b] = min(16 * eb0 + ncol(b), E - 1);
    const int cpair = min(16 * eb0 + 2 * r, E - 2);   // PAIR: an even index, so 8-byte aligned
    auto load_x = [&](int c, uint4 (&xv)[4]) __attribute__((always_inline)) {
      const int blk = 4 * c + q;
      const bool ok = tv && blk < nblk && c < c1;
      const uint32_t off = (uint32_t)(r * d + 32 * blk) * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = bload16(xr, ok ? off + 16 * i : kOutOfRange);
    };
    auto load_w = [&](int hc, float (&wv)[kRtHalf][NB]) __attribute__((always_inline)) {
      const int c = hc >> 1, h = hc & 1;
      const int blk = min(4 * c + q, nblk - 1);
      const float* wr = w + (size_t)(32 * blk + kRtHalf * h) * E;
#pragma unroll
      for (int s2 = 0; s2 < kRtHalf; ++s2) {
        if constexpr (PAIR) {
          const float2 v2 = *reinterpret_cast<const float2*>(wr + (size_t)s2 * E + cpair);
          wv[s2][0] = v2.x;
          wv[s2][1] = v2.y;
        } else {
#pragma unroll
          for (int b = 0; b < NB; ++b) wv[s2][b] = wr[(size_t)s2 * E + col[b]];
        }
      }
    };
    auto compute = [&](int hc, const uint4 (&xv)[4], const float (&wv)[kRtHalf][NB])
                       __attribute__((always_inline)) {
      const int h = hc & 1;
      const uint32_t xw[8] = {xv[2 * h].x, xv[2 * h].y, xv[2 * h].z, xv[2 * h].w,
                              xv[2 * h + 1].x, xv[2 * h + 1].y, xv[2 * h + 1].z, xv[2 * h + 1].w};
#pragma unroll
      for (int s2 = 0; s2 < kRtHalf; ++s2) {
        const float xf = bf16_to_f32(s2 & 1 ? (xw[s2 >> 1] >> 16) : (xw[s2 >> 1] & 0xffffu));
        const double a = static_cast<double>(xf);
        // columns past E read the last expert's weights: finite, and their
        // logits are never stored
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[s2 & 1][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, static_cast<double>(wv[s2][b]),
                                                                acc[s2 & 1][b], 0, 0, 0);
      }
    };
    auto encode = [&](int c, const uint4 (&xv)[4]) __attribute__((always_inline)) {
      const int blk = 4 * c + q;
      if (!tv || blk >= nblk) return;
      float v[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
        for (int h2 = 0; h2 < 4; ++h2) {
          v[8 * i + 2 * h2] = bf16_to_f32(u[h2] & 0xffffu);
          v[8 * i + 2 * h2 + 1] = bf16_to_f32(u[h2] >> 16);
        }
      }
      uint32_t hi[6], lo[6], sc;
      encode_block(v, hi, lo, sc);
      uint8_t* rowp = xenc + (size_t)(t0 + r) * pitch;
      store_enc(rowp + (uint32_t)(blk >> 2) * kChunk + (blk & 3) * kEncBytes, hi, lo);
      *reinterpret_cast<uint16_t*>(rowp + (uint32_t)(blk >> 2) * kChunk + kChunkScales + (blk & 3) * 2) =
          static_cast<uint16_t>(sc);
    };
    // half chunks hc = 2c + h; the W_r loads of the next half and the x loads of
    // the next chunk are issued before the current half is computed
    const int h0 = 2 * c0, h1 = 2 * c1;
    uint4 xa[4], xb[4];
    float wa[kRtHalf][NB], wb[kRtHalf][NB];
    if (h0 < h1) {
      load_x(c0, xa);
      load_w(h0, wa);
    }
    for (int hc = h0; hc < h1; hc += 2) {
      // half 0 of chunk c (x in xa): prefetch half 1's weights and the next chunk's x
      const int c = hc >> 1;
      load_w(hc + 1, wb);
      load_x(c + 1, xb);
      compute(hc, xa, wa);
      if (ENC && eb0 == 0) encode(c, xa);
      load_w(min(hc + 2, h1 - 1), wa);   // past the range: a valid reload, unused
      compute(hc + 1, xa, wb);
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = xb[i];
    }

    // the K ranges, added in wavefront order
    for (int wv2 = 0; wv2 < WV; ++wv2) {
      if (wave == wv2) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            double& dst = red[q + 4 * j][ncol(b)];
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
        if (partial) {
          if (t0 + m < T) partial[((size_t)ks * T + t0 + m) * E + e] = v;
        } else {
          if (bias) v += static_cast<double>(bias[e]);
          logit[m][e] = v == v ? v : -INFINITY;
        }
      }
    }
    __syncthreads();
  }
  if (partial) return;   // the selection is route_select's

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

template <bool ENC>
hipError_t launch_route_mfma(const uint16_t* x, const float* w_router, const float* b_router, int T,
                             int d, int E, int k, int32_t* topk_idx, float* topk_w, uint8_t* xenc,
                             double* partial, hipStream_t stream) {
  const int KS = route_ksplit(T, d);
  double* part = KS > 1 ? partial : nullptr;
  const dim3 grid((T + kRtTok - 1) / kRtTok, KS);
  if (rt_waves(E) == 4) {
    const dim3 block(4 * 64);
    if (E <= 16)
      hipLaunchKernelGGL((route_mfma<1, ENC, false, 4>), grid, block, 0, stream, x, w_router, b_router, T,
                         d, E, k, topk_idx, topk_w, xenc, part);
    else if (E % 2 == 0)
      hipLaunchKernelGGL((route_mfma<2, ENC, true, 4>), grid, block, 0, stream, x, w_router, b_router, T,
                         d, E, k, topk_idx, topk_w, xenc, part);
    else
      hipLaunchKernelGGL((route_mfma<2, ENC, false, 4>), grid, block, 0, stream, x, w_router, b_router, T,
                         d, E, k, topk_idx, topk_w, xenc, part);
  } else {
    const dim3 block(8 * 64);
    if (E % 2 == 0)
      hipLaunchKernelGGL((route_mfma<2, ENC, true, 8>), grid, block, 0, stream, x, w_router, b_router, T,
                         d, E, k, topk_idx, topk_w, xenc, part);
    else
      hipLaunchKernelGGL((route_mfma<2, ENC, false, 8>), grid, block, 0, stream, x, w_router, b_router, T,
                         d, E, k, topk_idx, topk_w, xenc, part);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || KS == 1) return err;
  hipLaunchKernelGGL(route_select, dim3(T), dim3(256), 0, stream, part, KS, b_router, T, E, k, topk_idx,
                     topk_w);
  return hipGetLastError();
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
  // the many-token kernel's partial logits when it splits K
  const int KS = route_ksplit(T, d);
  return KS > 1 ? al256((size_t)KS * T * E * sizeof(double)) : 0;
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
  return launch_route_mfma<false>(x, w_router, b_router, T, d, E, k, topk_idx, topk_w, nullptr,
                                  static_cast<double*>(ws), stream);
}

hipError_t launch_route_encode(const uint16_t* x, const float* w_router, const float* b_router,
                               int T, int d, int E, int k, int32_t* topk_idx, float* topk_w,
                               uint8_t* xenc, void* ws, hipStream_t stream) {
  return launch_route_mfma<true>(x, w_router, b_router, T, d, E, k, topk_idx, topk_w, xenc,
                                 static_cast<double*>(ws), stream);
}

}  // namespace moe
