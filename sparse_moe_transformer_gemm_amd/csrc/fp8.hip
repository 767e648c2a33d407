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
//   grouped_fp8     the expert GEMMs. A workgroup is one wavefront and takes
//                   one 32-row tile of the dispatch rows of an expert (a 32-row
//                   tile table) and one column unit: 32 h-columns (their gate
//                   and up rows) for gate/up, 64 output columns for down. Per
//                   128-deep K step: four MFMAs (two K halves x the hi and lo
//                   MXFP6 terms of the activations) per 32-column group into a
//                   step accumulator with unit B scale, then acc += block scale
//                   * step (the block scale is per 128 rows x 128 K, one value
//                   per group and step). Accumulators start at the bias.
//                   The next step's operands are loaded while the current
//                   step's MFMAs run. With one wavefront everything comes
//                   straight from global memory (2 wavefronts per SIMD). With
//                   many rows a workgroup of four wavefronts takes a 128-row
//                   tile; the four share each step's weight codes, loaded once
//                   per workgroup into a double-buffered LDS stage.
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

// WAVES = 1: grid (32-row tiles, column units), the tile table of 32 rows.
// WAVES = 4 (many rows): one workgroup per (128-row tile, column unit), wave w
// taking rows 32w .. 32w+31 of the tile: the four wavefronts read the same
// weights, so three of the four reads of each weight byte hit the CU's L1; a
// one-dimensional grid whose logical tiles (column unit fastest) are dealt to
// the 8 XCDs in contiguous ranges, so the column units of one row tile run on
// one XCD and read its encoded rows from that XCD's L2 (measured: 6.5 -> 5.1 ms
// for the prefill-20b FP8 call, against row tiles fastest).
template <bool GATEUP, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void grouped_fp8(const FfnArgs a, const uint8_t* __restrict__ ain,
                                                          uint8_t* __restrict__ hout,
                                                          const int4* __restrict__ tiles, int ncolu) {
  __shared__ __attribute__((aligned(16))) float stage_all[WAVES][32 * 36];
  // WAVES = 4: each K step's weight codes (both 32-row groups, 8 KB) are loaded
  // once per workgroup into one of two LDS buffers, a step ahead, and every
  // wavefront reads its operands there (instead of each wavefront loading all
  // of them: the texture addressers were the bound)
  __shared__ __attribute__((aligned(16))) uint8_t bsm[WAVES == 4 ? 4 * 4096 : 16];
  int mt, u;
  if constexpr (WAVES == 1) {
    mt = blockIdx.x;
    u = blockIdx.y;
  } else {
    const int total = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = total >> 3, rem = total & 7;
    const int L = xcd * per + min(xcd, rem) + slot;   // a bijection onto [0, total)
    mt = L / ncolu;
    u = L - mt * ncolu;
  }
  if (mt >= __builtin_amdgcn_readfirstlane(tiles[0].x)) return;
  const int4 ent = tiles[1 + mt];  // {expert, first row within the expert, offsets[e], count_e}
  const int wave = WAVES == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 31, half = lane >> 5;
  const int e = __builtin_amdgcn_readfirstlane(ent.x);
  const int r0 = __builtin_amdgcn_readfirstlane(ent.y) + 32 * wave;
  const int off = __builtin_amdgcn_readfirstlane(ent.z);
  const int rows = min(32, __builtin_amdgcn_readfirstlane(ent.w) - r0);
  // WAVES = 1 has no workgroup barrier; with WAVES = 4 a wavefront without rows
  // still takes part in the weight staging and its barriers (it reads the tile's
  // first row and stores nothing)
  if (WAVES == 1 && rows <= 0) return;
  const int rbase = rows > 0 ? r0 : __builtin_amdgcn_readfirstlane(ent.y);
  float* stage = stage_all[wave];
  const int K = GATEUP ? a.d : a.F, N = GATEUP ? a.F : a.d;
  const int nst = nsteps_of(K), nblkK = K / 32;
  const int nbN = (N + 127) / 128;
  const int g0 = GATEUP ? u : 2 * u, g1 = GATEUP ? u : 2 * u + 1;

  const int rr = rows > 0 ? min(lr, rows - 1) : 0;
  const uint32_t arow =
      GATEUP ? (uint32_t)a.sorted_pair[off + rbase + rr] / (uint32_t)a.k : (uint32_t)(off + rbase + rr);
  const uint8_t* A = ain + (size_t)arow * nst * kChunk;
  const uint8_t* Bg0 = (GATEUP ? a.wg_codes : a.wd_codes) + ((size_t)e * (N / 32) + g0) * nst * kF8Step;
  const uint8_t* Bg1 = (GATEUP ? a.wu_codes : a.wd_codes) + ((size_t)e * (N / 32) + g1) * nst * kF8Step;
  const uint8_t* B0 = Bg0 + lane * 32;
  const uint8_t* B1 = Bg1 + lane * 32;
  // WAVES = 4 staging: thread t copies bytes 32 (t % 128) .. + 31 of group t / 128
  const uint8_t* Bst = (threadIdx.x < 128 ? Bg0 : Bg1) + (threadIdx.x & 127) * 32;
  const uint32_t bst_lds = (threadIdx.x >> 7) * kF8Step + (threadIdx.x & 127) * 32;
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

  // Step j's operands: the lane's two A blocks (96 B: hi, lo of block 2h, then
  // of block 2h+1) and their four E8M0 bytes; B: 32 codes per lane and K half
  // (half 1 is 2048 B on); the block scales. Step j+1's are loaded before step
  // j's MFMAs.
  struct Ops {
    v4i a[6];
    int sa;
    v8i b00, b01, b10, b11;
    float s0, s1;
  };
  auto load_ops = [&](int j, Ops& o) __attribute__((always_inline)) {
    const v4i* ap = reinterpret_cast<const v4i*>(A + (size_t)j * kChunk + half * 96);
#pragma unroll
    for (int i = 0; i < 6; ++i) o.a[i] = ap[i];
    o.sa = *reinterpret_cast<const int*>(A + (size_t)j * kChunk + kChunkScales + 4 * half);
    if constexpr (WAVES == 1) {
      const v8i* p0 = reinterpret_cast<const v8i*>(B0 + (size_t)j * kF8Step);
      const v8i* p1 = reinterpret_cast<const v8i*>(B1 + (size_t)j * kF8Step);
      o.b00 = p0[0];
      o.b01 = p0[64];
      o.b10 = p1[0];
      o.b11 = p1[64];
    }
    o.s0 = S0[j];
    o.s1 = S1[j];
  };
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  auto stage_load = [&](int j, u4v (&r)[2]) __attribute__((always_inline)) {
    const u4v* p = reinterpret_cast<const u4v*>(Bst + (size_t)j * kF8Step);
    r[0] = p[0];
    r[1] = p[1];
  };
  auto stage_store = [&](int buf, const u4v (&r)[2]) __attribute__((always_inline)) {
    u4v* q = reinterpret_cast<u4v*>(bsm + buf * 2 * kF8Step + bst_lds);
    q[0] = r[0];
    q[1] = r[1];
  };
  Ops cur, nxt;
  load_ops(0, cur);
  if constexpr (WAVES == 4) {
    u4v r[2];
    stage_load(0, r);
    stage_store(0, r);
    __syncthreads();
  }
  for (int j = 0; j < nst; ++j) {
    u4v bnext[2];
    if constexpr (WAVES == 4) {
      if (j + 1 < nst) stage_load(j + 1, bnext);
    }
    if (j + 1 < nst) load_ops(j + 1, nxt);
    const v4i a0 = cur.a[0], a1 = cur.a[1], a2 = cur.a[2], a3 = cur.a[3], a4 = cur.a[4], a5 = cur.a[5];
    int sa = cur.sa;
    v8i b00, b01, b10, b11;
    if constexpr (WAVES == 4) {
      const v8i* l0 = reinterpret_cast<const v8i*>(bsm + (j & 1) * 2 * kF8Step + lane * 32);
      const v8i* l1 = reinterpret_cast<const v8i*>(bsm + (j & 1) * 2 * kF8Step + kF8Step + lane * 32);
      b00 = l0[0];
      b01 = l0[64];
      b10 = l1[0];
      b11 = l1[64];
    } else {
      b00 = cur.b00;
      b01 = cur.b01;
      b10 = cur.b10;
      b11 = cur.b11;
    }
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
    if constexpr (WAVES == 4) {
      // the buffer of step j - 1, free since the last barrier
      if (j + 1 < nst) stage_store((j + 1) & 1, bnext);
      __syncthreads();
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
    const int mts = max_row_tiles(a.T, a.E, a.k, kF8Rows * 4);
    hipLaunchKernelGGL((grouped_fp8<true, 4>), dim3((unsigned)(mts * (a.F / 32))), dim3(256), 0, stream, a, xenc,
                       henc, tp, a.F / 32);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((grouped_fp8<false, 4>), dim3((unsigned)(mts * (a.d / 64))), dim3(256), 0, stream, a, henc,
                       henc, tp, a.d / 64);
    return hipGetLastError();
  }
  const unsigned mts = (unsigned)max_row_tiles(a.T, a.E, a.k, kF8Rows);
  hipLaunchKernelGGL((grouped_fp8<true, 1>), dim3(mts, a.F / 32), dim3(64), 0, stream, a, xenc, henc, tp, a.F / 32);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((grouped_fp8<false, 1>), dim3(mts, a.d / 64), dim3(64), 0, stream, a, henc, henc, tp, a.d / 64);
  return hipGetLastError();
}

hipError_t launch_round_bf16(float* w, int n, hipStream_t stream) {
  hipLaunchKernelGGL(round_bf16_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, w, n);
  return hipGetLastError();
}

}  // namespace moe
