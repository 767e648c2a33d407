// Fused front end of the whole-block call for decode-sized batches (T <= 64,
// both expert GEMMs on the weight-streaming kernels). The separate calls route
// (two kernels), permute (one) and the FFN's activation encode (one) become two
// launches:
//   front_partials_encode  workgroups [0, d/64): the router's K-slice partial
//                          logits (Perplexity, "GPT-OSS el dia 0", section
//                          "MLP"); workgroups after them: the MXFP6 encode of
//                          x for the expert GEMMs. Neither depends on the other.
//   front_select_permute   one workgroup per token: reduce its partials, top-k,
//                          softmax over the picks; the last workgroup to finish
//                          (arrival counter, cleared by the first launch) then
//                          builds the stable permutation of all pairs (section
//                          "Nuclis per a GPT-OSS / MoE": dispatch selects each
//                          expert's tokens) and the 16-row pass table of the
//                          decode GEMMs (with at most 64 pairs, one wavefront
//                          does both).
// Each workgroup publishes its top-k with a device-scope release before it
// counts itself in, and the last one acquires before it reads them, so the
// permutation sees every token's choice whichever XCD computed it. The outputs
// are the same bytes that the separate calls produce.
#include "ffn_dev.hpp"
#include "permute_dev.hpp"
#include "route_dev.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void front_partials_encode(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ w_router,
                                                             int T, int d, int E,
                                                             double* __restrict__ partial,
                                                             int nslices, uint8_t* __restrict__ xenc,
                                                             int* __restrict__ counter) {
  const int b = blockIdx.x;
  if (b < nslices) {
    if (b == 0 && threadIdx.x == 0) *counter = 0;
    rt::partial_slice(x, w_router, T, d, E, b, partial);
  } else {
    encode_rows_group(x, T, d, xenc, b - nslices);
  }
}

// The stable permutation and the decode pass table of at most 64 pairs, by the
// workgroup's first wavefront from one load of the routing table (the other
// wavefronts only take part in the barriers): lane q holds pair q; lanes with
// the same expert are found with one ballot per expert-index bit, as in
// permute_chunk, and ranked by popcount of the lower lanes; per-expert counts
// and pass counts go through LDS, and each lane scans four experts' worth
// before a wavefront scan. The outputs are the bytes of permute_chunk followed
// by build_tile_table<kDecRows> (the unique stable counting sort and its table).
constexpr int kWavePairs = 64;

__device__ __forceinline__ void permute_wave(const int32_t* __restrict__ idx, int P, int E,
                                             int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                             int32_t* __restrict__ sorted_pair,
                                             int32_t* __restrict__ pair_row, int4* __restrict__ passes) {
  __shared__ int cnt[rt::kMaxE], npass[rt::kMaxE], off[rt::kMaxE], pst[rt::kMaxE];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const bool w0 = tid < kWave, valid = w0 && lane < P;
  for (int i = tid; i < rt::kMaxE; i += blockDim.x) {
    cnt[i] = 0;
    npass[i] = 0;
  }
  const int e = valid ? idx[lane] : 0;
  int rank = 0, c = 0;
  __syncthreads();
  if (w0) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t set = __ballot(valid && bit);
      same &= bit ? set : ~set;
    }
    const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    rank = __popcll(same & lower);
    c = __popcll(same);
    if (valid && rank == 0) {
      cnt[e] = c;
      npass[e] = (c + kDecRows - 1) / kDecRows;
    }
  }
  __syncthreads();
  if (w0) {
    // experts 4 lane .. 4 lane + 3, then an exclusive scan over the wavefront
    int cs[4], ps[4], sc = 0, sp = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = 4 * lane + j;
      cs[j] = x < E ? cnt[x] : 0;
      ps[j] = x < E ? npass[x] : 0;
      sc += cs[j];
      sp += ps[j];
    }
    int ic = sc, ip = sp;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t1 = __shfl_up(ic, o), t2 = __shfl_up(ip, o);
      if (lane >= o) {
        ic += t1;
        ip += t2;
      }
    }
    int ec = ic - sc, ep = ip - sp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = 4 * lane + j;
      if (x < E) {
        counts[x] = cs[j];
        offsets[x] = ec;
        off[x] = ec;
        pst[x] = ep;
        if (x == E - 1) offsets[E] = ec + cs[j];
      }
      ec += cs[j];
      ep += ps[j];
    }
    const int total = __shfl(ip, kWave - 1);
    if (lane == 0) passes[0] = make_int4(total, 0, 0, 0);
  }
  __syncthreads();
  if (valid) {
    const int pos = off[e] + rank;
    sorted_pair[pos] = lane;
    pair_row[lane] = pos;
    if (rank == 0)
      for (int p = 0; p < npass[e]; ++p)
        passes[1 + pst[e] + p] = make_int4(e, p * kDecRows, off[e], c);
  }
}

__global__ __launch_bounds__(256) void front_select_permute(
    const double* __restrict__ partial, int nslices, const float* __restrict__ b_router, int T,
    int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_row, int4* __restrict__ passes, int* __restrict__ counter) {
  __shared__ int last;
  __shared__ int s[257];
  __shared__ int offs[rt::kMaxE + 1];
  rt::select_token(partial, nslices, b_router, T, E, k, blockIdx.x, topk_idx, topk_w);
  // the token's top-k was stored by lanes of the first wavefront: it releases
  // them to the whole device, then counts the workgroup in
  if (threadIdx.x < kWave) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (threadIdx.x == 0) last = atomicAdd(counter, 1) == static_cast<int>(gridDim.x) - 1;
  }
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every other token's top-k
  if (T * k <= kWavePairs) {
    permute_wave(topk_idx, T * k, E, counts, offsets, sorted_pair, pair_row, passes);
    return;
  }
  pm::permute_chunk(topk_idx, T * k, E, 0, true, counts, offsets, sorted_pair, pair_row, offs);
  __syncthreads();
  build_tile_table<kDecRows>(offs, E, passes, s);
}

struct FrontLayout {
  size_t partial, counter, total;
};

// The front end's scratch follows the expert-FFN workspace (whose encoded-x and
// pass-table regions it fills).
FrontLayout front_layout(int T, int d, int F, int E, int k) {
  FrontLayout L;
  L.partial = ws_layout(T, d, F, E, k).total;
  L.counter = L.partial + align256((size_t)(d / 64) * T * E * sizeof(double));
  L.total = L.counter + 256;
  return L;
}

}  // namespace

bool forward_front_fits(int T, int d, int F, int k) {
  return T <= rt::kSmallT && T * k <= pm::kChunk && ffn_decode_shape(T, d, F);
}

size_t forward_front_bytes(int T, int d, int F, int E, int k) {
  return front_layout(T, d, F, E, k).total;
}

hipError_t launch_forward_front(const uint16_t* x, const float* w_router, const float* b_router,
                                int T, int d, int F, int E, int k, int32_t* topk_idx,
                                float* topk_w, int32_t* counts, int32_t* offsets,
                                int32_t* sorted_pair, int32_t* pair_row, void* ws,
                                hipStream_t stream) {
  const WsLayout W = ws_layout(T, d, F, E, k);
  const FrontLayout L = front_layout(T, d, F, E, k);
  uint8_t* base = static_cast<uint8_t*>(ws);
  double* partial = reinterpret_cast<double*>(base + L.partial);
  int* counter = reinterpret_cast<int*>(base + L.counter);
  const int nslices = d / 64;
  const int nenc = (T * (d / 32) + 7) / 8;
  hipLaunchKernelGGL(front_partials_encode, dim3(nslices + nenc), dim3(256), 0, stream, x, w_router,
                     T, d, E, partial, nslices, base + W.x, counter);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int4* passes = reinterpret_cast<int4*>(base + W.passes);
  hipLaunchKernelGGL(front_select_permute, dim3(T), dim3(256), 0, stream, partial, nslices, b_router,
                     T, E, k, topk_idx, topk_w, counts, offsets, sorted_pair, pair_row, passes,
                     counter);
  return hipGetLastError();
}

}  // namespace moe
