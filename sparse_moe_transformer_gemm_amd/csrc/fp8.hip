// FP8-E4M3 expert weights with one float32 scale per 128x128 block: the
// pages' serving variant (Perplexity, "GPT-OSS el dia 0", section "GPT-OSS a
// Hopper": the MXFP4 experts were converted once to FP8 with 128x128 block
// scales and run on FP8 GEMMs extended with a bias term; section "Nuclis per a
// GPT-OSS / MoE": the bias is loaded into the accumulators), on gfx950.
//
//   convert_kernel  MXFP4 (OCP layout) -> FP8 codes [E][N][K] + float32 block
//                   scales [E][ceil(N/128)][ceil(K/128)]. The block scale is
//                   2^(largest E8M0 exponent of the block); every element
//                   E2M1 * 2^(s - smax) then has at most two significant bits
//                   and, while smax - s <= 8, is an E4M3 value exactly, so the
//                   FP8 layer is the MXFP4 layer. Larger spreads round to nearest
//                   even (E4M3 subnormals bottom out at 2^-9).
//   pack_fp8_kernel FP8 codes -> the B-operand order of the 32x32x64 scaled MFMA
//                   with an FP8 B: [E][N/32][ceil(K/128)][2][64 lanes][32 B].
//                   With an 8-bit B the instruction takes K in 16-element
//                   pieces (checked on gfx950 against an FP6 A and an FP4 B):
//                   lane half h holds K elements 16h..16h+15 in bytes 0..15 and
//                   32+16h..32+16h+15 in bytes 16..31 of its 64-element range,
//                   while the A operand (and a 4-bit B) hold 32h..32h+31. So
//                   entry (e, g, j, s, l), row 32g + l%32, h = l/32, is: bytes
//                   0..15 = elements 16h.. of block 4j + s, bytes 16..31 =
//                   elements 16h.. of block 4j + 2 + s (the A halves of MFMA
//                   half s being blocks 4j + s and 4j + 2 + s, as for MXFP4);
//                   zero past K.
//   grouped_fp8     the expert GEMMs for few rows (T <= 64). A workgroup is one
//                   wavefront and takes one 32-row tile of the dispatch rows of
//                   an expert (a 32-row tile table) and one column unit: 32
//                   h-columns (their gate and up rows) for gate/up, 64 output
//                   columns for down. Per 128-deep K step: four MFMAs (two K
//                   halves x the hi and lo MXFP6 terms of the activations) per
//                   32-column group into a step accumulator with unit B scale,
//                   then acc += block scale * step (the block scale is per 128
//                   rows x 128 K, one value per group and step). Accumulators
//                   start at the bias. Operands come straight from global
//                   memory, the next step's loaded while the current step's
//                   MFMAs run.
//   grouped_fp8_tile the same arithmetic for many rows: four wavefronts per
//                   128-row tile and a wider column unit (64 h-columns for
//                   gate/up; 128, 96 or 64 output columns for down), each K
//                   step's weight codes staged once per workgroup in LDS.
#include "ffn_dev.hpp"
#include "mx6.hpp"

namespace moe {
namespace {

// ------------------------------------------------------------------ convert

// float -> E4M3 code, round to nearest even, saturating at 448 (inputs here are
// finite). Subnormal E4M3 values are multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fabsf(v);
  if (!(a > 0.0f)) return sign;
  int e = static_cast<int>((__float_as_uint(a) >> 23) & 255u) - 127;  // floor(log2 a), normal a
  if (e < -6) return sign | static_cast<uint32_t>(rintf(a * 512.0f));  // 8 -> 0x08, the smallest normal
  int q = static_cast<int>(rintf(ldexpf(a, 3 - e)));                   // 8 .. 16
  if (q == 16) {
    q = 8;
    ++e;
  }
  int code = ((e + 7) << 3) | (q - 8);
  if (e + 7 > 15 || code > 0x7E) code = 0x7E;
  return sign | static_cast<uint32_t>(code);
}

__device__ __forceinline__ float e2m1_f(uint32_t c) {
  const uint32_t m = c & 7u;
  const float mag = m < 2u ? 0.5f * m : (m < 4u ? 1.0f + 0.5f * (m - 2u) : (m < 6u ? 2.0f + (m - 4u) : 4.0f + 2.0f * (m - 6u)));
  return (c & 8u) ? -mag : mag;
}

// one workgroup per (K block j, N block i, expert e) of 128 x 128
__global__ __launch_bounds__(256) void convert_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int N,
                                                      int K, uint8_t* __restrict__ out,
                                                      float* __restrict__ bscale) {
  __shared__ int smax_w[4];
  const int j = blockIdx.x, i = blockIdx.y, e = blockIdx.z;
  const int nb = (N + 127) / 128, kb = (K + 127) / 128;
  const int n0 = 128 * i, k0 = 128 * j;
  const int nrows = min(128, N - n0), nkb = min(4, K / 32 - 4 * j);
  const int tid = threadIdx.x;
  const uint8_t* sc = scales + ((size_t)e * N + n0) * (K / 32) + 4 * j;
  int m = 0;
  for (int t = tid; t < nrows * 4; t += 256) {
    const int r = t >> 2, b = t & 3;
    if (b < nkb) m = max(m, (int)sc[(size_t)r * (K / 32) + b]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) smax_w[tid >> 6] = m;
  __syncthreads();
  const int smax = max(max(smax_w[0], smax_w[1]), max(smax_w[2], smax_w[3]));
  if (tid == 0) bscale[((size_t)e * nb + i) * kb + j] = ldexpf(1.0f, smax - 127);
  // 16 elements (8 code bytes) per thread and pass: 128 rows x 8 pieces
  for (int t = tid; t < nrows * 8; t += 256) {
    const int r = t >> 3, p = t & 7;
    const int kk = k0 + 16 * p;
    if (kk >= K) continue;
    const size_t row = (size_t)e * N + n0 + r;
    const uint2 src = *reinterpret_cast<const uint2*>(codes + row * (K / 2) + kk / 2);
    const int s = scales[row * (K / 32) + kk / 32];
    const float f = ldexpf(1.0f, s - smax);
    const uint32_t w[2] = {src.x, src.y};
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t c = (w[q >> 3] >> (4 * (q & 7))) & 15u;
      o[q >> 2] |= e4m3_rne(e2m1_f(c) * f) << (8 * (q & 3));
    }
    *reinterpret_cast<uint4*>(out + row * K + kk) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ------------------------------------------------------------------ pack

// one thread per 16-byte output piece: piece i = (((e*G + g)*S + j)*2 + s)*128 + 2l + p,
// p = 0: elements 16(l/32).. of block 4j + s; p = 1: the same of block 4j + 2 + s
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint8_t* __restrict__ src, int K,
                                                       size_t pieces, int S,
                                                       uint8_t* __restrict__ dst) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int p = (int)(i & 1), l = (int)((i >> 1) & 63), s = (int)((i >> 7) & 1);
  const size_t rest = i >> 8;                  // (e*G + g)*S + j
  const int j = (int)(rest % (size_t)S);
  const size_t row = (rest / (size_t)S) * 32 + (l & 31);   // e*N + 32g + l%32
  const int blk = 4 * j + 2 * p + s;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (blk < K / 32)
    v = *reinterpret_cast<const uint4*>(src + row * (size_t)K + (size_t)blk * 32 + 16 * (l >> 5));
  reinterpret_cast<uint4*>(dst)[i] = v;
}

// ------------------------------------------------------------------ GEMM

constexpr int kF8Step = 4096;  // packed FP8 code bytes per (32-row group, 128-deep step)
constexpr int kF8Rows = 32;    // dispatch rows per GEMM tile

// D += A (FP6 E2M3, scale byte OPA of sa) x B (FP8 E4M3, unit scale).
template <int OPA>
__device__ __forceinline__ v16f mfma_f6f8(const v8i& a, const v8i& b, const v16f& c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 0, OPA, sa, 0, 0x7F7F7F7F);
}

// Few rows (T <= 64): one wavefront per (32-row tile, column unit), grid (32-row
// tiles of the tile table, column units). A column unit is two 32-row weight
// groups: gate group u and up group u (32 h-columns) for gate/up, output groups
// 2u and 2u + 1 for down. Operands come straight from global memory, the next
// step's loaded while the current step's MFMAs run.
template <bool GATEUP>
__global__ __launch_bounds__(64) void grouped_fp8(const FfnArgs a, const uint8_t* __restrict__ ain,
                                                  uint8_t* __restrict__ hout, const int4* __restrict__ tiles) {
  __shared__ __attribute__((aligned(16))) float stage[32 * 36];
  // the valid rows' chunks of one K step (the wavefront's activation window)
  __shared__ __attribute__((aligned(16))) uint8_t awin[32 * kChunk];
  const int mt = blockIdx.x, u = blockIdx.y;
  if (mt >= __builtin_amdgcn_readfirstlane(tiles[0].x)) return;
  const int4 ent = tiles[1 + mt];  // {expert, first row within the expert, offsets[e], count_e}
  const int lane = threadIdx.x & 63, lr = lane & 31, half = lane >> 5;
  const int e = __builtin_amdgcn_readfirstlane(ent.x);
  const int r0 = __builtin_amdgcn_readfirstlane(ent.y);
  const int off = __builtin_amdgcn_readfirstlane(ent.z);
  const int rows = min(32, __builtin_amdgcn_readfirstlane(ent.w) - r0);
  if (rows <= 0) return;   // (no workgroup barrier below)
  const int K = GATEUP ? a.d : a.F, N = GATEUP ? a.F : a.d;
  const int nst = nsteps_of(K), nblkK = K / 32;
  const int nbN = (N + 127) / 128;
  const int g0 = GATEUP ? u : 2 * u, g1 = GATEUP ? u : 2 * u + 1;

  const int rr = min(lr, rows - 1);
  // window piece c = lane + 64 i: row c / 13 (valid rows only), piece c % 13 of
  // the row's 208-byte chunk; each lane's source row
  constexpr int kWinPieces = (32 * kChunkPieces + 63) / 64;   // loads per lane, at most
  const int npieces = rows * kChunkPieces;
  const uint8_t* wsrc[kWinPieces];
#pragma unroll
  for (int i = 0; i < kWinPieces; ++i) {
    const int c = lane + 64 * i;
    const int wr = min(c / kChunkPieces, rows - 1), pc = c % kChunkPieces;
    const uint32_t arw = GATEUP ? (uint32_t)a.sorted_pair[off + r0 + wr] / (uint32_t)a.k : (uint32_t)(off + r0 + wr);
    wsrc[i] = ain + (size_t)arw * nst * kChunk + pc * 16;
  }
  const uint8_t* B0 = (GATEUP ? a.wg_codes : a.wd_codes) + ((size_t)e * (N / 32) + g0) * nst * kF8Step + lane * 32;
  const uint8_t* B1 = (GATEUP ? a.wu_codes : a.wd_codes) + ((size_t)e * (N / 32) + g1) * nst * kF8Step + lane * 32;
  const float* S0 = reinterpret_cast<const float*>(GATEUP ? a.wg_scales : a.wd_scales) +
                    ((size_t)e * nbN + (32 * g0) / 128) * nst;
  const float* S1 = reinterpret_cast<const float*>(GATEUP ? a.wu_scales : a.wd_scales) +
                    ((size_t)e * nbN + (32 * g1) / 128) * nst;

  // bias-initialised accumulators: lane l holds column l%32 of its group
  v16f acc0, acc1;
  {
    const uint16_t* bs0 = GATEUP ? a.b_gate : a.b_down;
    const uint16_t* bs1 = GATEUP ? a.b_up : a.b_down;
    const float b0 = bf16_to_f32(bs0[(size_t)e * N + 32 * g0 + lr]);
    const float b1 = bf16_to_f32(bs1[(size_t)e * N + 32 * g1 + lr]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc0[i] = b0;
      acc1[i] = b1;
    }
  }

  // Step j's operands: the activation window (the valid rows' 208-byte chunks,
  // 16 bytes per lane and load, staged through LDS so that each row is loaded
  // once, not once per lane that uses it); B: 32 codes per lane and K half (half
  // 1 is 2048 B on); the block scales. From the window each lane reads its two A
  // blocks (96 B: hi, lo of block 2h, then of block 2h+1) and their four E8M0 bytes.
  struct Ops {
    v4i w[kWinPieces];
    v8i b00, b01, b10, b11;
    float s0, s1;
  };
  auto load_ops = [&](int j, Ops& o) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kWinPieces; ++i)
      if (64 * i < npieces && lane + 64 * i < npieces)
        o.w[i] = *reinterpret_cast<const v4i*>(wsrc[i] + (size_t)j * kChunk);
    const v8i* p0 = reinterpret_cast<const v8i*>(B0 + (size_t)j * kF8Step);
    const v8i* p1 = reinterpret_cast<const v8i*>(B1 + (size_t)j * kF8Step);
    o.b00 = p0[0];
    o.b01 = p0[64];
    o.b10 = p1[0];
    o.b11 = p1[64];
    o.s0 = S0[j];
    o.s1 = S1[j];
  };
  Ops cur, nxt;
  load_ops(0, cur);
  for (int j = 0; j < nst; ++j) {
    // this step's window to LDS (the previous step's reads of it are complete:
    // a wavefront's LDS accesses run in order), then each lane's A operands
#pragma unroll
    for (int i = 0; i < kWinPieces; ++i) {
      const int c = lane + 64 * i;
      if (64 * i < npieces && c < npieces)
        *reinterpret_cast<v4i*>(awin + (c / kChunkPieces) * kChunk + (c % kChunkPieces) * 16) = cur.w[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (j + 1 < nst) load_ops(j + 1, nxt);
    const v4i* ap = reinterpret_cast<const v4i*>(awin + rr * kChunk + half * 96);
    const v4i a0 = ap[0], a1 = ap[1], a2 = ap[2], a3 = ap[3], a4 = ap[4], a5 = ap[5];
    int sa = *reinterpret_cast<const int*>(awin + rr * kChunk + kChunkScales + 4 * half);
    const v8i b00 = cur.b00, b01 = cur.b01, b10 = cur.b10, b11 = cur.b11;
    const float s0 = cur.s0, s1 = cur.s1;
    // in a half step at the end of K (K % 128 == 64) lane half 1 has no blocks:
    // its B codes are zero and its A codes finite (E2M3 has no NaN), so only the
    // never-written scale bytes are replaced by finite ones
    if (half && 4 * j + 2 >= nblkK) sa = 0x7F7F7F7F;
    const v8i hi0 = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, -1, -1);
    const v8i lo0 = __builtin_shufflevector(a1, a2, 2, 3, 4, 5, 6, 7, -1, -1);
    const v8i hi1 = __builtin_shufflevector(a3, a4, 0, 1, 2, 3, 4, 5, -1, -1);
    const v8i lo1 = __builtin_shufflevector(a4, a5, 2, 3, 4, 5, 6, 7, -1, -1);
    v16f t0 = mfma_f6f8<0>(hi0, b00, v16f{}, sa);
    v16f t1 = mfma_f6f8<0>(hi0, b10, v16f{}, sa);
    t0 = mfma_f6f8<1>(lo0, b00, t0, sa);
    t1 = mfma_f6f8<1>(lo0, b10, t1, sa);
    t0 = mfma_f6f8<2>(hi1, b01, t0, sa);
    t1 = mfma_f6f8<2>(hi1, b11, t1, sa);
    t0 = mfma_f6f8<3>(lo1, b01, t0, sa);
    t1 = mfma_f6f8<3>(lo1, b11, t1, sa);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc0[i] = fmaf(s0, t0[i], acc0[i]);
      acc1[i] = fmaf(s1, t1[i], acc1[i]);
    }
    cur = nxt;
  }

  if constexpr (GATEUP) {
    // h = silu(g) * u through LDS; lane r < rows encodes row r's block u
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * half + (i & 3);
      stage[row * 36 + lr] = silu_mul(acc0[i], acc1[i]);
    }
    // the wavefront's own staging area: a wavefront-level barrier
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < rows) {
      float v[32];
#pragma unroll
      for (int c = 0; c < 32; ++c) v[c] = stage[lane * 36 + c];
      uint32_t hw[6], lw[6], sc;
      encode_block(v, hw, lw, sc);
      uint8_t* hrow = hout + (size_t)(off + r0 + lane) * enc_pitch(a.F);
      store_enc(hrow + enc_codes_at(u), hw, lw);
      *reinterpret_cast<uint16_t*>(hrow + enc_scale_at(u)) = static_cast<uint16_t>(sc);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < rows) {
        float* yr = a.y_sorted + (size_t)(off + r0 + row) * N;
        yr[32 * g0 + lr] = acc0[i];
        yr[32 * g1 + lr] = acc1[i];
      }
    }
  }
}

// Many rows (T > 64): one workgroup of four wavefronts per (128-row tile,
// column unit), wave w taking rows 32w .. 32w+31 of the tile. A column unit is
// NB 32-row weight groups: for gate/up the gate groups NG u .. NG u + NG - 1
// and the up groups of the same h-columns (NG = NB / 2), for down the output
// groups NB u .. NB u + NB - 1. Each K step's weight codes (NB x 4 KB) are
// loaded once per workgroup, a step ahead, into one of two LDS buffers, and
// every wavefront reads its B operands there; the activations come straight
// from global memory, the next step's loaded while the current step's MFMAs
// run. The grid is one-dimensional: logical tiles (column unit fastest) are
// dealt to the 8 XCDs in contiguous ranges, so the column units of one row
// tile run on one XCD and read its encoded rows from that XCD's L2.
template <bool GATEUP, int NB>
__global__ __launch_bounds__(256) void grouped_fp8_tile(const FfnArgs a, const uint8_t* __restrict__ ain,
                                                        uint8_t* __restrict__ hout,
                                                        const int4* __restrict__ tiles, int ncolu) {
  constexpr int NG = GATEUP ? NB / 2 : NB;   // groups per weight matrix
  static_assert(!GATEUP || NB % 2 == 0, "gate/up units pair gate and up groups");
  static_assert(kF8Step == 256 * 16, "thread t stages the 16 bytes at 16 t of each group's step");
  __shared__ __attribute__((aligned(16))) float stage_all[4][32 * 36];
  __shared__ __attribute__((aligned(16))) uint8_t bsm[2 * NB * kF8Step];
  const int total = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = total >> 3, rem = total & 7;
  const int L = xcd * per + min(xcd, rem) + slot;   // a bijection onto [0, total)
  const int mt = L / ncolu, u = L - mt * ncolu;
  // (the whole workgroup leaves together: no barrier has been reached)
  if (mt >= __builtin_amdgcn_readfirstlane(tiles[0].x)) return;
  const int4 ent = tiles[1 + mt];  // {expert, first row within the expert, offsets[e], count_e}
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 31, half = lane >> 5;
  const int e = __builtin_amdgcn_readfirstlane(ent.x);
  const int r0 = __builtin_amdgcn_readfirstlane(ent.y) + 32 * wave;
  const int off = __builtin_amdgcn_readfirstlane(ent.z);
  const int rows = min(32, __builtin_amdgcn_readfirstlane(ent.w) - r0);
  // a wavefront without rows still stages weights and meets every barrier (it
  // reads the tile's first row and stores nothing)
  const int rbase = rows > 0 ? r0 : __builtin_amdgcn_readfirstlane(ent.y);
  float* stage = stage_all[wave];
  const int K = GATEUP ? a.d : a.F, N = GATEUP ? a.F : a.d;
  const int nst = nsteps_of(K), nblkK = K / 32;
  const int nbN = (N + 127) / 128;
  auto grp = [&](int i) { return GATEUP ? NG * u + (i % NG) : NB * u + i; };
  auto codes = [&](int i) { return GATEUP ? (i < NG ? a.wg_codes : a.wu_codes) : a.wd_codes; };
  auto bscales = [&](int i) {
    return reinterpret_cast<const float*>(GATEUP ? (i < NG ? a.wg_scales : a.wu_scales) : a.wd_scales) +
           ((size_t)e * nbN + (32 * grp(i)) / 128) * nst;
  };

  const int rr = rows > 0 ? min(lr, rows - 1) : 0;
  const uint32_t arow =
      GATEUP ? (uint32_t)a.sorted_pair[off + rbase + rr] / (uint32_t)a.k : (uint32_t)(off + rbase + rr);
  const uint8_t* A = ain + (size_t)arow * nst * kChunk;
  // staging: thread t copies bytes 16 t .. 16 t + 15 of every group's step
  const uint8_t* Bst[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) Bst[i] = codes(i) + ((size_t)e * (N / 32) + grp(i)) * nst * kF8Step + 16 * threadIdx.x;
  const float* S[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) S[i] = bscales(i);

  // bias-initialised accumulators: lane l holds column l%32 of its group
  v16f acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const uint16_t* bs = GATEUP ? (i < NG ? a.b_gate : a.b_up) : a.b_down;
    const float b = bf16_to_f32(bs[(size_t)e * N + 32 * grp(i) + lr]);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = b;
  }

  // step j's activation operands: the lane's two A blocks (96 B: hi, lo of
  // block 2h, then of block 2h+1) and their four E8M0 bytes; the block scales
  struct Ops {
    v4i a[6];
    int sa;
    float s[NB];
  };
  auto load_ops = [&](int j, Ops& o) __attribute__((always_inline)) {
    const v4i* ap = reinterpret_cast<const v4i*>(A + (size_t)j * kChunk + half * 96);
#pragma unroll
    for (int i = 0; i < 6; ++i) o.a[i] = ap[i];
    o.sa = *reinterpret_cast<const int*>(A + (size_t)j * kChunk + kChunkScales + 4 * half);
#pragma unroll
    for (int i = 0; i < NB; ++i) o.s[i] = S[i][j];
  };
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  auto stage_load = [&](int j, u4v (&r)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NB; ++i) r[i] = *reinterpret_cast<const u4v*>(Bst[i] + (size_t)j * kF8Step);
  };
  // In LDS a group's step is [K half s][16-byte piece q][lane][16 B] (in memory
  // it is [s][lane][32 B]), so that each 16-byte operand read of a wavefront
  // covers 1 KB of consecutive bytes (with lanes 32 B apart it took two passes)
  const uint32_t st_lds = (threadIdx.x >> 7) * 2048 + (threadIdx.x & 1) * 1024 + ((threadIdx.x >> 1) & 63) * 16;
  auto stage_store = [&](int buf, const u4v (&r)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<u4v*>(bsm + (buf * NB + i) * kF8Step + st_lds) = r[i];
  };
  // the lane's 32 codes of K half s of group i (the B operand of one MFMA)
  auto ldb = [&](const uint8_t* buf, int i, int hs) __attribute__((always_inline)) {
    const v4i* q = reinterpret_cast<const v4i*>(buf + i * kF8Step + hs * 2048 + lane * 16);
    return __builtin_shufflevector(q[0], q[64], 0, 1, 2, 3, 4, 5, 6, 7);
  };
  Ops cur, nxt;
  load_ops(0, cur);
  {
    u4v r[NB];
    stage_load(0, r);
    stage_store(0, r);
    __syncthreads();
  }
  for (int j = 0; j < nst; ++j) {
    u4v bnext[NB];
    if (j + 1 < nst) {
      stage_load(j + 1, bnext);
      load_ops(j + 1, nxt);
    }
    const v4i a0 = cur.a[0], a1 = cur.a[1], a2 = cur.a[2], a3 = cur.a[3], a4 = cur.a[4], a5 = cur.a[5];
    int sa = cur.sa;
    // in a half step at the end of K (K % 128 == 64) lane half 1 has no blocks:
    // its B codes are zero and its A codes finite (E2M3 has no NaN), so only the
    // never-written scale bytes are replaced by finite ones
    if (half && 4 * j + 2 >= nblkK) sa = 0x7F7F7F7F;
    const v8i hi0 = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, -1, -1);
    const v8i lo0 = __builtin_shufflevector(a1, a2, 2, 3, 4, 5, 6, 7, -1, -1);
    const v8i hi1 = __builtin_shufflevector(a3, a4, 0, 1, 2, 3, 4, 5, -1, -1);
    const v8i lo1 = __builtin_shufflevector(a4, a5, 2, 3, 4, 5, 6, 7, -1, -1);
    const uint8_t* bb = bsm + (j & 1) * NB * kF8Step;
    // groups in pairs: two independent MFMA chains of four, then their scaled
    // sums into the accumulators (an odd last group alone)
#pragma unroll
    for (int p = 0; p < NB; p += 2) {
      if (p + 1 < NB) {
        const v8i b00 = ldb(bb, p, 0), b10 = ldb(bb, p + 1, 0);
        v16f t0 = mfma_f6f8<0>(hi0, b00, v16f{}, sa);
        v16f t1 = mfma_f6f8<0>(hi0, b10, v16f{}, sa);
        t0 = mfma_f6f8<1>(lo0, b00, t0, sa);
        t1 = mfma_f6f8<1>(lo0, b10, t1, sa);
        const v8i b01 = ldb(bb, p, 1), b11 = ldb(bb, p + 1, 1);
        t0 = mfma_f6f8<2>(hi1, b01, t0, sa);
        t1 = mfma_f6f8<2>(hi1, b11, t1, sa);
        t0 = mfma_f6f8<3>(lo1, b01, t0, sa);
        t1 = mfma_f6f8<3>(lo1, b11, t1, sa);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[p][r] = fmaf(cur.s[p], t0[r], acc[p][r]);
          acc[p + 1][r] = fmaf(cur.s[p + 1], t1[r], acc[p + 1][r]);
        }
      } else {
        const v8i b00 = ldb(bb, p, 0), b01 = ldb(bb, p, 1);
        v16f t0 = mfma_f6f8<0>(hi0, b00, v16f{}, sa);
        t0 = mfma_f6f8<1>(lo0, b00, t0, sa);
        t0 = mfma_f6f8<2>(hi1, b01, t0, sa);
        t0 = mfma_f6f8<3>(lo1, b01, t0, sa);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[p][r] = fmaf(cur.s[p], t0[r], acc[p][r]);
      }
    }
    // the buffer of step j - 1, free since the last barrier
    if (j + 1 < nst) stage_store((j + 1) & 1, bnext);
    __syncthreads();
    cur = nxt;
  }

  if constexpr (GATEUP) {
    // h = silu(g) * u per h group through the wavefront's LDS staging area;
    // lane r < rows encodes row r's block
#pragma unroll
    for (int q = 0; q < NG; ++q) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * half + (i & 3);
        stage[row * 36 + lr] = silu_mul(acc[q][i], acc[NG + q][i]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < rows) {
        float v[32];
#pragma unroll
        for (int c = 0; c < 32; ++c) v[c] = stage[lane * 36 + c];
        uint32_t hw[6], lw[6], sc;
        encode_block(v, hw, lw, sc);
        uint8_t* hrow = hout + (size_t)(off + r0 + lane) * enc_pitch(a.F);
        store_enc(hrow + enc_codes_at(grp(q)), hw, lw);
        *reinterpret_cast<uint16_t*>(hrow + enc_scale_at(grp(q))) = static_cast<uint16_t>(sc);
      }
      // every lane's reads of the area come before the next group's writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < rows) {
        float* yr = a.y_sorted + (size_t)(off + r0 + row) * N;
#pragma unroll
        for (int g = 0; g < NB; ++g) yr[32 * grp(g) + lr] = acc[g][i];
      }
    }
  }
}

__global__ __launch_bounds__(256) void round_bf16_kernel(float* __restrict__ w, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) w[i] = bf16_to_f32(f32_to_bf16(w[i]));
}

// The activation encode of the FP8 call (x, once per token) with the 32-row
// tile table built by the launch's last workgroup.
template <int BM>
__global__ __launch_bounds__(256) void encode_x_tiles(const uint16_t* __restrict__ x, int rows, int K,
                                                      uint8_t* __restrict__ enc,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      int4* __restrict__ tiles) {
  if (blockIdx.x == gridDim.x - 1) {
    __shared__ int s[257];
    build_tile_table<BM>(offsets, E, tiles, s);
    return;
  }
  const int nblk = K / 32;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * nblk) return;
  const int row = idx / nblk, b = idx - row * nblk;
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)idx * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = src[q];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[q * 8 + 2 * i] = bf16_to_f32(ws[i] & 0xffffu);
      v[q * 8 + 2 * i + 1] = bf16_to_f32(ws[i] >> 16);
    }
  }
  uint32_t hi[6], lo[6], sc;
  encode_block(v, hi, lo, sc);
  uint8_t* r = enc + (size_t)row * enc_pitch(K);
  store_enc(r + enc_codes_at(b), hi, lo);
  *reinterpret_cast<uint16_t*>(r + enc_scale_at(b)) = static_cast<uint16_t>(sc);
}

}  // namespace

size_t fp8_packed_bytes(int E, int N, int K) { return (size_t)E * (N / 32) * nsteps_of(K) * kF8Step; }

hipError_t launch_convert_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                                       uint8_t* out, float* bscale, hipStream_t stream) {
  hipLaunchKernelGGL(convert_kernel, dim3((K + 127) / 128, (N + 127) / 128, E), dim3(256), 0, stream, codes,
                     scales, N, K, out, bscale);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const uint8_t* codes, int E, int N, int K, uint8_t* out, hipStream_t stream) {
  const size_t pieces = fp8_packed_bytes(E, N, K) / 16;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, codes, K,
                     pieces, nsteps_of(K), out);
  return hipGetLastError();
}

// 32-column weight groups per down workgroup with many rows
static int fp8_down_groups(int d) { return d % 128 == 0 ? 4 : (d % 96 == 0 ? 3 : 2); }

hipError_t launch_expert_ffn_fp8(const FfnArgs& a, hipStream_t stream) {
  const WsLayout L = ws_layout(a.T, a.d, a.F, a.E, a.k);
  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  uint8_t* xenc = ws + L.x;
  uint8_t* henc = ws + L.h;
  // the 32-row table fits the region sized for the 16-row decode passes
  int4* tp = reinterpret_cast<int4*>(ws + L.passes);
  const int nx = a.T * (a.d / 32);
  const bool wide = a.T > 64;
  if (wide)
    hipLaunchKernelGGL(encode_x_tiles<kF8Rows * 4>, dim3((nx + 255) / 256 + 1), dim3(256), 0, stream, a.x, a.T, a.d,
                       xenc, a.offsets, a.E, tp);
  else
    hipLaunchKernelGGL(encode_x_tiles<kF8Rows>, dim3((nx + 255) / 256 + 1), dim3(256), 0, stream, a.x, a.T, a.d,
                       xenc, a.offsets, a.E, tp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (wide) {
    // gate/up: 64 h-columns per workgroup (F is a multiple of 64); down: the
    // widest of 128, 96 and 64 output columns that divides d (six gate/up
    // groups or more than four down groups take more than half a SIMD's
    // registers)
    const unsigned mts = (unsigned)max_row_tiles(a.T, a.E, a.k, kF8Rows * 4);
    hipLaunchKernelGGL((grouped_fp8_tile<true, 4>), dim3(mts * (a.F / 64)), dim3(256), 0, stream, a, xenc, henc, tp,
                       a.F / 64);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int dg = fp8_down_groups(a.d);
    const int nu = a.d / (32 * dg);
    if (dg == 4)
      hipLaunchKernelGGL((grouped_fp8_tile<false, 4>), dim3(mts * nu), dim3(256), 0, stream, a, henc, henc, tp, nu);
    else if (dg == 3)
      hipLaunchKernelGGL((grouped_fp8_tile<false, 3>), dim3(mts * nu), dim3(256), 0, stream, a, henc, henc, tp, nu);
    else
      hipLaunchKernelGGL((grouped_fp8_tile<false, 2>), dim3(mts * nu), dim3(256), 0, stream, a, henc, henc, tp, nu);
    return hipGetLastError();
  }
  const unsigned mts = (unsigned)max_row_tiles(a.T, a.E, a.k, kF8Rows);
  hipLaunchKernelGGL((grouped_fp8<true>), dim3(mts, a.F / 32), dim3(64), 0, stream, a, xenc, henc, tp);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((grouped_fp8<false>), dim3(mts, a.d / 64), dim3(64), 0, stream, a, henc, henc, tp);
  return hipGetLastError();
}

hipError_t launch_round_bf16(float* w, int n, hipStream_t stream) {
  hipLaunchKernelGGL(round_bf16_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, w, n);
  return hipGetLastError();
}

}  // namespace moe
