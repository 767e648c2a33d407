// Dispatch: per-expert histogram, exclusive scan, stable permutation and its
// inverse (Perplexity, "GPT-OSS el dia 0", section "Nuclis per a GPT-OSS / MoE":
// dispatch selects each expert's tokens).
//
// One kernel, no inter-block communication. Block b owns the pairs
// [b*kChunk, (b+1)*kChunk). Every block first histograms the whole routing table
// in LDS (the table is tiny: 4*T int32, L2-resident), counting separately the
// pairs before its chunk; from that it knows the exclusive scan of the totals
// and where its own pairs of each expert start. It then ranks its pairs 256 at a
// time: inside a wavefront, lanes holding the same expert are found with one
// ballot per expert-index bit and ranked by popcount of the lower lanes; per-
// wave counts in LDS give the offset across the block's four wavefronts. The
// result is the unique stable counting sort by expert (pairs of an expert in
// ascending pair order = ascending token order). Only integer LDS atomics are
// used, so the output is deterministic.
#include "common.hpp"
#include "ffn_dev.hpp"
#include "permute_dev.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(pm::kThreads) void permute_hist(const int32_t* __restrict__ idx, int P,
                                                             int E, int32_t* __restrict__ chist) {
  pm::chunk_histogram(idx, P, E, blockIdx.x, chist);
}

__global__ __launch_bounds__(pm::kThreads) void permute_kernel(const int32_t* __restrict__ idx, int P,
                                                               int E, int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pair,
                                                               int32_t* __restrict__ pair_row,
                                                               const int32_t* __restrict__ chist,
                                                               int4* __restrict__ tiles,
                                                               int4* __restrict__ passes) {
  __shared__ int offs[pm::kMaxE + 1];
  __shared__ int s[257];
  pm::permute_chunk(idx, P, E, blockIdx.x * pm::kChunk, blockIdx.x == 0, counts, offsets, sorted_pair,
                    pair_row, offs, chist, gridDim.x);
  // workgroup 0 also lays out the expert GEMMs' row tiles from the offsets it holds
  if (tiles && blockIdx.x == 0) {
    __syncthreads();
    build_tile_table<kBM>(offs, E, tiles, s);
  }
  if (passes && blockIdx.x == 0) {
    __syncthreads();
    build_tile_table<kDecRows>(offs, E, passes, s);
  }
}

}  // namespace

size_t permute_workspace_bytes(int T, int E, int k) {
  const size_t blocks = ((size_t)T * k + pm::kChunk - 1) / pm::kChunk;
  return blocks > 1 ? blocks * E * sizeof(int32_t) : 0;
}

hipError_t launch_permute(const int32_t* topk_idx, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* pair_row, void* ws,
                          hipStream_t stream, int4* tiles, int4* passes) {
  const int P = T * k;
  const int blocks = (P + pm::kChunk - 1) / pm::kChunk;
  int32_t* chist = nullptr;
  if (blocks > 1) {
    chist = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(permute_hist, dim3(blocks), dim3(pm::kThreads), 0, stream, topk_idx, P, E, chist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(permute_kernel, dim3(blocks), dim3(pm::kThreads), 0, stream, topk_idx, P, E,
                     counts, offsets, sorted_pair, pair_row, chist, tiles, passes);
  return hipGetLastError();
}

}  // namespace moe
