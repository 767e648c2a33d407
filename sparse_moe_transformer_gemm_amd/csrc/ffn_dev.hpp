// Pieces of the expert-FFN call that the fused decode front end (front.hip)
// shares: the encoded-row addressing, the device-built row-tile tables, the
// decode-shape activation encoder and the workspace layout.
#pragma once

#include "layout.hpp"
#include "mx6.hpp"

namespace moe {

constexpr int kBM = 128;        // rows per prefill tile
constexpr int kDecRows = 16;    // dispatch rows per decode pass

inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

__device__ __forceinline__ uint32_t enc_pitch(int K) { return (uint32_t)nsteps_of(K) * kChunk; }

// Byte offsets of block b's codes and scales inside an encoded row.
__device__ __forceinline__ uint32_t enc_codes_at(int b) { return (b >> 2) * kChunk + (b & 3) * kEncBytes; }
__device__ __forceinline__ uint32_t enc_scale_at(int b) { return (b >> 2) * kChunk + kChunkScales + (b & 3) * 2; }

// ------------------------------------------------------------------ tile table

// Row-tile table of the grouped GEMMs, built on the device from the expert
// offsets by one workgroup (BM = 128 rows for the prefill tiles, 16 for the
// decode passes; `s` is 257 ints of LDS):
// table[0].x = number of row tiles (sum over experts of ceil(count / BM));
// table[1 + mt] = {expert, first row of the tile within the expert, offsets[e],
// count_e} for row tile mt, tiles in expert order. One 16-byte load gives a
// workgroup everything it needs to locate its rows.
template <int BM>
__device__ __forceinline__ void build_tile_table(const int32_t* __restrict__ offsets, int E,
                                                 int4* __restrict__ table, int* s) {
  __shared__ int tmp[4];
  const int t = threadIdx.x;
  const int v = t < E ? (offsets[t + 1] - offsets[t] + BM - 1) / BM : 0;
  s[t + 1] = block_inclusive_scan256(v, tmp);  // s[1 + e] = tiles of experts 0..e
  if (t == 0) s[0] = 0;
  __syncthreads();
  const int total = s[E];
  if (t == 0) table[0] = make_int4(total, 0, 0, 0);
  for (int mt = t; mt < total; mt += 256) {
    int lo = 0, hi = E;  // s[lo] <= mt < s[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s[mid] <= mt) lo = mid; else hi = mid;
    }
    const int o = offsets[lo];
    table[1 + mt] = make_int4(lo, (mt - s[lo]) * BM, o, offsets[lo + 1] - o);
  }
}

// Decode-shape activation encoder, the work of one 256-thread workgroup number
// `blk`: one (row, 32-element block) per half wavefront, lane j takes element j
// and the block is encoded cooperatively (short latency).
__device__ __forceinline__ void encode_rows_group(const uint16_t* __restrict__ x, int rows, int K,
                                                  uint8_t* __restrict__ enc, int blk) {
  __shared__ uint8_t scratch[8 * 64];
  const int nblk = K / 32;
  const int nrec = rows * nblk;
  const int g = blk * 8 + (threadIdx.x >> 5);
  const int gg = g < nrec ? g : nrec - 1;
  const int row = gg / nblk, b = gg - row * nblk;
  const float v = bf16_to_f32(x[(size_t)gg * 32 + (threadIdx.x & 31)]);
  uint8_t* r = enc + (size_t)row * enc_pitch(K);
  encode_group32(v, scratch + (threadIdx.x >> 5) * 64, r + enc_codes_at(b),
                 reinterpret_cast<uint16_t*>(r + enc_scale_at(b)), g < nrec);
}

// ------------------------------------------------------------------ workspace

struct WsLayout {
  size_t x, h, tiles, passes, total;
};

// upper bound on the number of row tiles of BM rows: sum over experts of ceil(count / BM)
inline int max_row_tiles(int T, int E, int k, int BM) {
  const int P = T * k;
  return (P + BM - 1) / BM + (E < P ? E : P);
}

inline WsLayout ws_layout(int T, int d, int F, int E, int k) {
  WsLayout L;
  const size_t P = (size_t)T * k;
  L.x = 0;
  L.h = L.x + align256((size_t)T * nsteps_of(d) * kChunk);
  L.tiles = L.h + align256(P * nsteps_of(F) * kChunk);
  L.passes = L.tiles + align256((size_t)(1 + max_row_tiles(T, E, k, kBM)) * sizeof(int4));
  L.total = L.passes + align256((size_t)(1 + max_row_tiles(T, E, k, kDecRows)) * sizeof(int4));
  return L;
}

}  // namespace moe
