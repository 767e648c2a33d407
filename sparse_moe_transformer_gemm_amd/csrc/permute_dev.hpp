// Dispatch: per-expert histogram, exclusive scan, stable permutation and its
// inverse (Perplexity, "GPT-OSS el dia 0", section "Nuclis per a GPT-OSS / MoE":
// dispatch selects each expert's tokens).
//
// Shared by permute.hip and the fused decode front end (front.hip). Block b
// owns the pairs [b*kChunk, (b+1)*kChunk). With one chunk, the block histograms
// the routing table itself; with several, a first launch writes one histogram
// per chunk and each block of the second sums them (totals, and the counts of
// the chunks before its own). From that it knows the exclusive scan of the
// totals and where its own pairs of each expert start. It then ranks its pairs 256 at a
// time: inside a wavefront, lanes holding the same expert are found with one
// ballot per expert-index bit and ranked by popcount of the lower lanes; per-
// wave counts in LDS give the offset across the block's four wavefronts. The
// result is the unique stable counting sort by expert (pairs of an expert in
// ascending pair order = ascending token order). Only integer LDS atomics are
// used, so the output is deterministic.
#pragma once

#include "common.hpp"

namespace moe {
namespace pm {

constexpr int kThreads = 256;
constexpr int kChunk = 512;
constexpr int kMaxE = 256;

// Per-chunk expert histograms: chunk c's counts of its pairs [c*kChunk,
// (c+1)*kChunk) into chist[c][0..E), by one workgroup (one counter set per
// wavefront, so that the LDS atomics of the four wavefronts do not collide).
__device__ __forceinline__ void chunk_histogram(const int32_t* __restrict__ idx, int P, int E,
                                                int chunk, int32_t* __restrict__ chist) {
  __shared__ int wh[kThreads / kWave][kMaxE];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  for (int e = tid; e < kMaxE; e += kThreads)
    for (int w = 0; w < kThreads / kWave; ++w) wh[w][e] = 0;
  __syncthreads();
  const int start = chunk * kChunk, end = min(P, start + kChunk);
  for (int q = start + tid; q < end; q += kThreads) atomicAdd(&wh[wave][idx[q]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int c = 0;
    for (int w = 0; w < kThreads / kWave; ++w) c += wh[w][e];
    chist[(size_t)chunk * E + e] = c;
  }
}

// Pairs [start, min(P, start + kChunk)) of the stable counting sort, by one
// workgroup of kThreads; the workgroup that owns pair 0 also writes counts and
// offsets (write_totals). offsets_lds, if given, receives the offsets as well
// (visible to the workgroup when the call returns). With chist (the nchunks
// chunk histograms of chunk_histogram) the totals and the counts before this
// chunk come from there instead of from a pass over every pair.
__device__ __forceinline__ void permute_chunk(const int32_t* __restrict__ idx, int P, int E,
                                              int start, bool write_totals,
                                              int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ sorted_pair,
                                              int32_t* __restrict__ pair_row,
                                              int* offsets_lds = nullptr,
                                              const int32_t* __restrict__ chist = nullptr,
                                              int nchunks = 0) {
  __shared__ int total[kMaxE];
  __shared__ int before[kMaxE];
  __shared__ int scan[kMaxE];
  __shared__ int run[kMaxE];
  __shared__ int wcnt[kThreads / kWave][kMaxE];
  __shared__ int scantmp[kThreads / kWave];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int end = min(P, start + kChunk);

  for (int e = tid; e < kMaxE; e += kThreads) {
    total[e] = 0;
    before[e] = 0;
    run[e] = 0;
    for (int w = 0; w < kThreads / kWave; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();

  if (chist) {
    // every thread takes entries i = tid, tid + 256, ... of the nchunks x E
    // histograms, eight loads in flight at a time, and adds them into the
    // totals (and, for chunks before this one, into `before`) with LDS integer
    // atomics: integer sums do not depend on the order, so the result is exact
    // and deterministic
    const int mine = start / kChunk;
    const int n = nchunks * E;
    for (int i0 = tid; i0 < n; i0 += 8 * kThreads) {
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kThreads;
        h[u] = i < n ? chist[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kThreads;
        if (i < n && h[u]) {
          const int c = i / E, e = i - c * E;
          atomicAdd(&total[e], h[u]);
          if (c < mine) atomicAdd(&before[e], h[u]);
        }
      }
    }
  } else {
    for (int q = tid; q < P; q += kThreads) {
      const int e = idx[q];
      atomicAdd(&total[e], 1);
      if (q < start) atomicAdd(&before[e], 1);
    }
  }
  __syncthreads();

  // exclusive scan of total[0..E)
  static_assert(kThreads == 256 && kMaxE == 256, "one scan entry per thread");
  const int val = (tid < E) ? total[tid] : 0;
  const int excl = block_inclusive_scan256(val, scantmp) - val;
  scan[tid] = excl;
  if (write_totals && tid < E) {
    counts[tid] = val;
    offsets[tid] = excl;
    if (tid == E - 1) offsets[E] = excl + val;
  }
  if (offsets_lds && tid < E) {  // the offsets also to the caller's LDS [E + 1]
    offsets_lds[tid] = excl;
    if (tid == E - 1) offsets_lds[E] = excl + val;
  }
  __syncthreads();

  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

  for (int s = start; s < end; s += kThreads) {
    const int q = s + tid;
    const bool valid = q < end;
    const int e = valid ? idx[q] : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t set = __ballot(valid && bit);
      same &= bit ? set : ~set;
    }
    const int rank = __popcll(same & lower);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int pos = scan[e] + before[e] + run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      sorted_pair[pos] = q;
      pair_row[q] = pos;
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w = 0; w < kThreads / kWave; ++w) {
        add += wcnt[w][tid];
        wcnt[w][tid] = 0;
      }
      run[tid] += add;
    }
    __syncthreads();
  }
}

}  // namespace pm
}  // namespace moe
