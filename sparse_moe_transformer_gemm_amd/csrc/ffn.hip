// Grouped expert FFN on gfx950 scaled matrix cores (V_MFMA_SCALE_F32_32X32X64_F8F6F4).
//
// For every expert e and dispatch row p of e (Perplexity, "GPT-OSS el dia 0",
// section "MLP": SwiGLU experts with biases; section "Nuclis per a GPT-OSS / MoE":
// the bias is loaded into the GEMM accumulators once per output tile):
//   h_p = silu(x_t Wg^T + bg) * (x_t Wu^T + bu)      gate/up GEMM, fused epilogue
//   y_p = h_p Wd^T + bd                               down GEMM
// B operands are the MXFP4 weights exactly as stored (E2M1 nibbles + E8M0 block
// scales, no dequantisation). A operands are two-term MXFP6 encodings (mx6.hpp):
// x is encoded once per token row by encode_rows, h by the gate/up epilogue.
//
// Two kernel shapes, chosen on the host from T (expert row counts stay on the
// device):
//   prefill  128 dispatch rows x 64*NF weight rows per workgroup, 2x2 wavefronts,
//            K in 128-deep stages copied from global memory straight into LDS
//            (three stages in flight), laid out in MFMA fragment order. The grid
//            is an upper bound on the number of (row tile, column tile) pairs; a
//            tile table built on the device maps a workgroup to its expert, and
//            surplus workgroups exit. Tiles are rastered in groups of a few row
//            tiles x all column tiles and each XCD (dispatch is round-robin over
//            the 8 XCDs) takes a contiguous range of them, so resident
//            workgroups share A rows and expert weights in their L2.
//   decode   weight streaming for few rows per expert: one workgroup per
//            (expert, 32 output columns), the four wavefronts split K, stream the
//            weights straight from HBM into MFMA registers, and reduce their
//            partial tiles through LDS in fixed order (deterministic).
#include "mx6.hpp"

namespace moe {
namespace {

constexpr int kBM = 128;        // rows per prefill tile
constexpr int kPrefGM = 8;      // row tiles per raster group of the prefill grid
constexpr int kDecodeMaxT = 64; // decode kernels when T <= this

struct EncIn {
  const uint8_t* codes;     // [rows][K/32][48]
  const uint16_t* scales;   // [rows][K/32]
};
struct EncOut {
  uint8_t* codes;
  uint16_t* scales;
};

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// ------------------------------------------------------------------ encode x

// Activation encoding, two shapes: few rows (decode) -- one (row, 32-element
// block) per half wavefront, lane j takes element j and the block is encoded
// cooperatively (short latency); many rows (prefill) -- one block per thread
// (no barriers, throughput).
__global__ __launch_bounds__(256) void encode_rows_thread(const uint16_t* __restrict__ x, int rows,
                                                          int K, uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ scales) {
  const int nblk = K / 32;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * nblk) return;
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
  store_enc(codes + (size_t)idx * kEncBytes, hi, lo);
  scales[idx] = static_cast<uint16_t>(sc);
}

__global__ __launch_bounds__(256) void encode_rows(const uint16_t* __restrict__ x, int rows,
                                                   int K, uint8_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scales) {
  __shared__ uint8_t scratch[8 * 64];
  const int nrec = rows * (K / 32);
  const int g = blockIdx.x * 8 + (threadIdx.x >> 5);
  const int gg = g < nrec ? g : nrec - 1;
  const float v = bf16_to_f32(x[(size_t)gg * 32 + (threadIdx.x & 31)]);
  encode_group32(v, scratch + (threadIdx.x >> 5) * 64, codes + (size_t)gg * kEncBytes,
                 scales + gg, g < nrec);
}

// ------------------------------------------------------------------ tile table

// tile_prefix[e] = sum_{e' < e} ceil(count_e' / kBM); tile_prefix[E] = total tiles.
__global__ __launch_bounds__(256) void tile_prefix_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int32_t* __restrict__ tp) {
  __shared__ int s[256];
  const int t = threadIdx.x;
  const int v = t < E ? (offsets[t + 1] - offsets[t] + kBM - 1) / kBM : 0;
  s[t] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += add;
    __syncthreads();
  }
  if (t < E) tp[t + 1] = s[t];
  if (t == 0) tp[0] = 0;
}

// Division by a runtime divisor d >= 1 as a multiply: x / d = (x * m) >> 32 with
// m = ceil(2^32 / d), exact for x < 2^32 / d (here x < 2^20).
__device__ __forceinline__ uint64_t div_magic(uint32_t d) { return ((1ull << 32) + d - 1) / d; }
__device__ __forceinline__ uint32_t div_by(uint32_t x, uint64_t m) {
  return static_cast<uint32_t>((static_cast<uint64_t>(x) * m) >> 32);
}

// Workgroup id -> logical tile such that XCD x (ids = x mod 8) owns the
// contiguous logical range [x*G/8, (x+1)*G/8) (a bijection on [0, G)).
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int per = G >> 3, rem = G & 7, x = bid & 7, i = bid >> 3;
  return x * per + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ uint2 lds64(const uint8_t* p) {
  return *reinterpret_cast<const uint2*>(p);
}

// ------------------------------------------------------------------ prefill

// One workgroup = 128 dispatch rows x 64*NF weight rows, 2x2 wavefronts; wave
// (wm, wn) owns rows 64wm..64wm+63 (two 32-row fragments) and NF 32-row weight
// fragments (for gate/up: NF/2 gate and NF/2 up fragments of the same h-columns,
// so SwiGLU can be applied to the tile).
//
// K advances in 128-deep stages (four 32-element blocks) that are copied from
// global memory straight into LDS by buffer-to-LDS loads (lane i of a copy
// writes LDS bytes [16i, 16i+16) for 16-byte copies and the dword 4i for 4- and
// 2-byte ones, zero-extended), three stages in
// flight: the copy of stage t+2 is issued when stage t is computed. Each stage
// is laid out in MFMA fragment order, so every fragment read is one contiguous
// 16-byte-per-lane LDS read: within a stage, lane half h of a 32x32x64 MFMA
// takes blocks 2h (first MFMA step) and 2h+1 (second), the same permutation of K
// for A and B, which makes every lane's share of a stage contiguous in global
// memory as well. Rows past the tile's count, blocks past K and stages past the
// end are read as zero through the resource's range check.
template <int NF, bool GATEUP>
struct Prefill {
  static constexpr int BN = 64 * NF;                   // weight rows per workgroup
  static constexpr int NFR = 2 * NF;                   // 32-row weight fragments
  static constexpr int MROWS = GATEUP ? BN / 2 : BN;   // output columns per workgroup
  static constexpr int FM = GATEUP ? NF / 2 : NF;      // fragments per matrix per wave
  // stage layout in LDS (bytes)
  static constexpr int A_OFF = 0;                          // [wm][mf][step][lane][48]
  static constexpr int AS_OFF = A_OFF + 8 * 64 * kEncBytes; // [wm][mf][lane][4]
  static constexpr int B_OFF = AS_OFF + 4 * 64 * 4;         // [frag][step][lane][16]
  static constexpr int BS_OFF = B_OFF + NFR * 2 * 64 * 16;  // [frag][lane][4] (2 bytes used)
  static constexpr int NBS = (NFR + 3) / 4 * 4;             // scale copies, padded to 4 waves
  static constexpr int STAGE = BS_OFF + NBS * 256;
  // copies per wave per stage: A codes, A scales, B codes, B scales
  static constexpr int NA = 24 / 4;
  static constexpr int NB = NFR * 2 / 4;
  static constexpr int NBSW = NBS / 4;
  static constexpr int PER_WAVE = NA + 1 + NB + NBSW;
  static constexpr int EP_PITCH = 36;                  // floats per row of the SwiGLU staging tile
  static_assert(!GATEUP || NF % 2 == 0, "gate/up tiles pair gate and up fragments");
  static_assert(PER_WAVE <= 63, "one stage of copies must fit the vector memory counter");
  static_assert(3 * STAGE <= 160 * 1024, "three stage buffers must fit the 160 KB of LDS");
  static_assert(!GATEUP || 2 * 64 * EP_PITCH * 4 <= STAGE, "SwiGLU staging of two waves must fit a stage buffer");
};

// s_waitcnt with only the vector memory counter bounded (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and lgkmcnt at max).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Buffer-to-LDS copy of SIZE bytes per lane (16, 4 or 2) into `lds` (wave-uniform).
template <int SIZE>
__device__ __forceinline__ void lds_copy(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  static_assert(SIZE == 16 || SIZE == 4 || SIZE == 2, "copy sizes used here");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds, 16, voff, soff, 0, 0);
  else if constexpr (SIZE == 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds, 4, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds, 2, voff, soff, 0, 0);
}

template <int NF, bool GATEUP>
__global__ __launch_bounds__(256) void grouped_prefill(const FfnArgs a, const EncIn ain,
                                                       const EncOut hout,
                                                       const int32_t* __restrict__ tile_prefix,
                                                       int ntn) {
  using C = Prefill<NF, GATEUP>;
  // three stage buffers as separate objects, so the compiler can tell the copy
  // into one from the reads of another
  __shared__ __attribute__((aligned(16))) uint8_t st0[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[C::STAGE];

  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const int nblkK = K / 32;
  const int nsteps = (K + 127) / 128;
  const int E = a.E;

  // ---- tile of this workgroup. Logical tiles are grouped kPrefGM row tiles x all
  // column tiles, row tile fastest, so the workgroups resident at one time share
  // a few row tiles of A and a few column tiles of B in L2; the groups are laid
  // out contiguously per XCD.
  const int total_mt = tile_prefix[E];
  const int G = total_mt * ntn;
  if ((int)blockIdx.x >= G) return;
  const int logical = xcd_remap(blockIdx.x, G);
  const int grp = logical / (kPrefGM * ntn);
  const int gm = min(kPrefGM, total_mt - grp * kPrefGM);
  const int r = logical - grp * kPrefGM * ntn;
  const int nt = r / gm;
  const int mt = grp * kPrefGM + (r - nt * gm);
  int lo = 0, hi = E;  // tile_prefix[lo] <= mt < tile_prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_prefix[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int off = a.offsets[e];
  const int cnt = a.offsets[e + 1] - off;
  const int m0 = (mt - tile_prefix[e]) * kBM;
  const int rows_valid = min(kBM, cnt - m0);
  const int col0 = nt * C::MROWS;  // first output column of each matrix in this tile

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- resources
  const uint32_t arow_bytes = (uint32_t)nblkK * kEncBytes;
  const rsrc_t ar = GATEUP ? make_rsrc(ain.codes, (uint32_t)a.T * arow_bytes)
                           : make_rsrc(ain.codes + (size_t)(off + m0) * arow_bytes,
                                       (uint32_t)rows_valid * arow_bytes);
  const rsrc_t asr = GATEUP ? make_rsrc(ain.scales, (uint32_t)a.T * nblkK * 2)
                            : make_rsrc(ain.scales + (size_t)(off + m0) * nblkK,
                                        (uint32_t)rows_valid * nblkK * 2);
  const uint64_t kmagic = div_magic((uint32_t)a.k);  // token of dispatch pair q: q / k
  const rsrc_t br0 = make_rsrc((GATEUP ? a.wg_codes : a.wd_codes) + (size_t)e * N * (K / 2),
                               (uint32_t)N * (K / 2));
  const rsrc_t bsr0 = make_rsrc((GATEUP ? a.wg_scales : a.wd_scales) + (size_t)e * N * nblkK,
                                (uint32_t)N * nblkK);
  const rsrc_t br1 = GATEUP ? make_rsrc(a.wu_codes + (size_t)e * N * (K / 2), (uint32_t)N * (K / 2)) : br0;
  const rsrc_t bsr1 = GATEUP ? make_rsrc(a.wu_scales + (size_t)e * N * nblkK, (uint32_t)N * nblkK) : bsr0;
  // weight row of lane c (0..31) of B fragment phi, and whether phi is an up fragment
  auto frag_up = [&](int phi) { return GATEUP && (phi % NF) >= NF / 2; };
  auto frag_row = [&](int phi, int c) -> int {
    if (GATEUP) {
      const int w = phi / NF, f = phi % NF;
      return col0 + w * C::FM * 32 + (f < NF / 2 ? f : f - NF / 2) * 32 + c;
    }
    return col0 + phi * 32 + c;
  };

  // ---- biases of this lane's output columns, loaded together with the dispatch
  // entries below and before the first copies (waiting for them must not wait
  // for the copies)
  float bias[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int phi = wn * NF + f;
    const uint16_t* bsrc = GATEUP ? (frag_up(phi) ? a.b_up : a.b_gate) : a.b_down;
    bias[f] = bf16_to_f32(bsrc[(size_t)e * N + frag_row(phi, lr)]);
  }

  // ---- per-lane source offsets of this wave's copies (fixed across stages; the
  // stage's K distance goes into the uniform offset). The dispatch entries of
  // the rows are all loaded first (rows past the count read the last row), so
  // their latencies overlap.
  int a_rowi[C::NA];
  uint32_t a_src[C::NA + 1];
#pragma unroll
  for (int t = 0; t < C::NA; ++t) {
    const int q = (wave + 4 * t) * 64 + lane;          // 16-byte slot in the A region
    const int g = q / 384, rem = q - g * 384;          // g = wm*2 + mf
    const int l = (rem - (rem / 192) * 192) / 3;
    a_rowi[t] = (g >> 1) * 64 + (g & 1) * 32 + (l & 31);
  }
  const int as_rowi = (wave >> 1) * 64 + (wave & 1) * 32 + lr;
  if (GATEUP) {
#pragma unroll
    for (int t = 0; t <= C::NA; ++t) {
      const int row = t < C::NA ? a_rowi[t] : as_rowi;
      a_src[t] = (uint32_t)a.sorted_pair[off + m0 + min(row, rows_valid - 1)];
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t <= C::NA; ++t) a_src[t] = div_by(a_src[t], kmagic);
  } else {
#pragma unroll
    for (int t = 0; t <= C::NA; ++t) a_src[t] = (uint32_t)(t < C::NA ? a_rowi[t] : as_rowi);
  }
  uint32_t a_off[C::NA];
  int a_blk[C::NA];
#pragma unroll
  for (int t = 0; t < C::NA; ++t) {
    const int q = (wave + 4 * t) * 64 + lane;
    const int rem = q - (q / 384) * 384;
    const int s = rem / 192, rem2 = rem - s * 192;
    const int l = rem2 / 3, j = rem2 - l * 3;
    a_blk[t] = 2 * (l >> 5) + s;
    a_off[t] = a_rowi[t] < rows_valid ? a_src[t] * arow_bytes + a_blk[t] * kEncBytes + j * 16 : kOutOfRange;
  }
  const int as_blk = 2 * half;
  const uint32_t as_off = as_rowi < rows_valid ? a_src[C::NA] * (nblkK * 2) + as_blk * 2 : kOutOfRange;
  uint32_t b_off[C::NB];
  int b_blk[C::NB];
#pragma unroll
  for (int t = 0; t < C::NB; ++t) {
    const int i = wave + 4 * t, phi = i >> 1, s = i & 1;
    b_blk[t] = 2 * half + s;
    b_off[t] = (uint32_t)frag_row(phi, lr) * (K / 2) + b_blk[t] * 16;
  }
  uint32_t bs_off[C::NBSW];
#pragma unroll
  for (int t = 0; t < C::NBSW; ++t) {
    const int phi = wave + 4 * t;
    bs_off[t] = phi < C::NFR ? (uint32_t)frag_row(phi, lr) * nblkK + 2 * half : kOutOfRange;
  }

  // Copy stage st into LDS buffer `buf`.
  auto issue = [&](int st, uint8_t* buf) {
    const int kb = __builtin_amdgcn_readfirstlane(4 * st);
#pragma unroll
    for (int t = 0; t < C::NA; ++t)
      lds_copy<16>(ar, buf + C::A_OFF + (wave + 4 * t) * 1024,
                   kb + a_blk[t] < nblkK ? a_off[t] : kOutOfRange, kb * kEncBytes);
    lds_copy<4>(asr, buf + C::AS_OFF + wave * 256, kb + as_blk < nblkK ? as_off : kOutOfRange, kb * 2);
#pragma unroll
    for (int t = 0; t < C::NB; ++t) {
      const int i = wave + 4 * t;
      lds_copy<16>(frag_up(i >> 1) ? br1 : br0, buf + C::B_OFF + i * 1024,
                   kb + b_blk[t] < nblkK ? b_off[t] : kOutOfRange, kb * 16);
    }
#pragma unroll
    for (int t = 0; t < C::NBSW; ++t) {
      const int phi = wave + 4 * t;
      lds_copy<2>(frag_up(phi) ? bsr1 : bsr0, buf + C::BS_OFF + phi * 256,
                  kb + 2 * half < nblkK ? bs_off[t] : kOutOfRange, kb);
    }
  };

  v16f acc[2][NF];

  // Compute one stage out of LDS buffer `buf`: both MFMA steps' fragments are
  // read first, then 2 x 2 x NF x 2 scaled MFMAs (hi and lo terms of A).
  auto compute = [&](const uint8_t* buf, int st) {
    // Padding stages past K compute nothing. A half stage at the end of K (K % 128
    // == 64) still takes both MFMA steps: each holds one valid block (block 2h+s
    // of lane half h) and one zero block.
    if (4 * st >= nblkK) return;
    v8i ahi[2][2], alo[2][2];
    int sa[2];
#pragma unroll
    for (int mf = 0; mf < 2; ++mf) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4* p = reinterpret_cast<const uint4*>(
            buf + C::A_OFF + ((wm * 2 + mf) * 2 + s) * 64 * kEncBytes + lane * kEncBytes);
        const uint4 q0 = p[0], q1 = p[1], q2 = p[2];
        ahi[mf][s] = v8i{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, 0, 0};
        alo[mf][s] = v8i{(int)q1.z, (int)q1.w, (int)q2.x, (int)q2.y, (int)q2.z, (int)q2.w, 0, 0};
      }
      sa[mf] = reinterpret_cast<const int*>(buf + C::AS_OFF + (wm * 2 + mf) * 256)[lane];
    }
    v8i bf[NF][2];
    int sbs[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int phi = wn * NF + f;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 q = reinterpret_cast<const uint4*>(buf + C::B_OFF + (phi * 2 + s) * 1024)[lane];
        bf[f][s] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      }
      sbs[f] = reinterpret_cast<const int*>(buf + C::BS_OFF + phi * 256)[lane];
    }
    // step 0: scale bytes 0 (A hi), 1 (A lo), 0 (B); step 1: bytes 2, 3, 1
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        acc[mf][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ahi[mf][0], bf[f][0], acc[mf][f], 2, 4,
                                                                    0, sa[mf], 0, sbs[f]);
        acc[mf][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(alo[mf][0], bf[f][0], acc[mf][f], 2, 4,
                                                                    1, sa[mf], 0, sbs[f]);
      }
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        acc[mf][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ahi[mf][1], bf[f][1], acc[mf][f], 2, 4,
                                                                    2, sa[mf], 1, sbs[f]);
        acc[mf][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(alo[mf][1], bf[f][1], acc[mf][f], 2, 4,
                                                                    3, sa[mf], 1, sbs[f]);
      }
  };

  // One step: wait for this wave's copies of stage st (the next stage's copies
  // stay in flight), barrier (everyone's copies of st have landed and everyone
  // has finished reading the buffer that the copy issued next overwrites),
  // copy stage st+2, compute stage st.
  auto step = [&](int st, const uint8_t* cur, uint8_t* nxt2) {
    MOE_WAIT_VMCNT(C::PER_WAVE);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves across the barrier
    __builtin_amdgcn_sched_barrier(0);
    issue(st + 2, nxt2);
    compute(cur, st);
  };

  // ---- accumulators start at the bias of their output column
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mf][f][i] = bias[f];
  __builtin_amdgcn_sched_barrier(0);

  issue(0, st0);
  issue(1, st1);
  // Steps go in threes (one per buffer); stages past the end copy zeros and
  // compute nothing.
  for (int t = 0; t < nsteps; t += 3) {
    step(t, st0, st2);
    step(t + 1, st1, st0);
    step(t + 2, st2, st1);
  }
  MOE_WAIT_VMCNT(0);
  __syncthreads();

  if constexpr (GATEUP) {
    // h = silu(g) * u; per gate fragment f, the wave's two 32x32 tiles go to
    // LDS as 64 rows x 32 columns and each lane encodes one row's 32-column
    // block as two-term MXFP6.
    float* ep = reinterpret_cast<float*>(wave < 2 ? st0 : st1) + (wave & 1) * 64 * C::EP_PITCH;
    const int nblkF = a.F / 32;
    const int grow = m0 + wm * 64 + lane;
#pragma unroll
    for (int f = 0; f < C::FM; ++f) {
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rr = mf * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          const float g = acc[mf][f][i], u = acc[mf][f + C::FM][i];
          ep[rr * C::EP_PITCH + lr] = g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
        }
      __builtin_amdgcn_wave_barrier();
      float v[32];
      const float4* src = reinterpret_cast<const float4*>(ep + lane * C::EP_PITCH);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 t4 = src[q];
        v[4 * q] = t4.x;
        v[4 * q + 1] = t4.y;
        v[4 * q + 2] = t4.z;
        v[4 * q + 3] = t4.w;
      }
      __builtin_amdgcn_wave_barrier();
      uint32_t hw[6], lw[6], sc;
      encode_block(v, hw, lw, sc);
      if (grow < cnt) {
        const size_t rec = (size_t)(off + grow) * nblkF + (col0 + wn * C::FM * 32 + f * 32) / 32;
        store_enc(hout.codes + rec * kEncBytes, hw, lw);
        hout.scales[rec] = static_cast<uint16_t>(sc);
      }
    }
  } else {
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = wm * 64 + mf * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (rr < rows_valid) {
          float* yr = a.y_sorted + (size_t)(off + m0 + rr) * N + col0 + wn * NF * 32 + lr;
#pragma unroll
          for (int f = 0; f < NF; ++f) yr[f * 32] = acc[mf][f][i];
        }
      }
  }
}

// ------------------------------------------------------------------ decode

// Weight streaming for few rows per expert. One workgroup per (expert, 64 output
// columns); wavefront w owns columns 16w..16w+15 over the full K and uses the
// 16x16x128 scaled MFMA (16 rows = one decode-sized row tile). K is processed in
// super-stages of kSS 128-deep steps: per super-stage every wavefront issues all
// its weight loads (straight from HBM into MFMA registers) while the workgroup
// stages the expert's activation rows for the same K window in LDS, so each
// super-stage costs one memory latency and the activations are read from L2
// once per workgroup instead of once per wavefront. Small register and LDS
// footprints keep many workgroups per CU, and with them enough bytes in flight.
//
// 16x16x128 layout (checked on gfx950): lane l supplies row/column l%16 and K
// elements 32*(l/16) .. +31 of the step; result lane l holds column l%16, rows
// 4*(l/16) + i, i = 0..3.
typedef float v4f __attribute__((ext_vector_type(4)));

template <int OPA>
__device__ __forceinline__ v4f mfma16_f6f4(const v8i& a, const v8i& b, const v4f& c, int sa,
                                           int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 2, 4, OPA, sa, 0, sb);
}

constexpr int kDecSS = 4;                  // 128-deep K steps per stage
constexpr int kDecPF = 2;                  // stages of loads in flight ahead of the one computed
constexpr int kDecMaxStages = 8;           // decode kernels cover K <= kDecMaxStages * kDecSS * 128
constexpr int kDecWB = 4 * kDecSS;         // 32-element blocks per K window
constexpr int kDecMaxBlk = kDecMaxStages * kDecWB;  // 32-element blocks of the longest K
constexpr int kDecAPitch = kDecWB * kEncBytes + 8;  // LDS bytes per activation row (padded)
constexpr int kDecAChunks = 16 * kDecWB * 3;        // 16-byte chunks of the activation window
constexpr int kDecAPerT = kDecAChunks / 256;        // ... per thread
constexpr int kDecBSPitch = kDecMaxBlk + 4;         // LDS bytes per weight-scale row (odd dword count)
constexpr int kDecASPitch = kDecMaxBlk + 2;         // LDS uint16 per activation-scale row (odd dword count)
constexpr int kDecBSLoads = 64 * kDecMaxBlk / 2 / 256;  // uint16 weight-scale loads per thread (max)
static_assert(kDecSS % 4 == 0, "the window staging splits evenly over 256 threads");
static_assert(kDecAChunks % 256 == 0, "window staging must divide evenly");

// Gate/up: waves 0,1 stream the gate rows of 32 h-columns, waves 2,3 the up rows
// of the same columns (one matrix per wave keeps the register footprint small);
// down: 4 waves x 16 output columns. The block scales of the workgroup's weight
// rows (all of K) and of its activation rows are loaded into LDS once, up front,
// in few coalesced loads. The stage loop is unrolled at compile time (NSTAGE
// stages of kDecSS steps): the weight codes and the activation window of stage
// s+kDecPF are issued while stage s is computed, held in register rings, and
// the window is copied to LDS one stage before it is read. Loads are issued in
// the order they are consumed, so waiting for one never waits for a younger one
// (the vector memory counter retires in order). All global reads are buffer
// loads: K blocks past the end (the half step when K % 128 == 64) and rows past
// the count read as zero.
template <bool GATEUP, int NSTAGE>
__global__ __launch_bounds__(256, 2) void grouped_decode(const FfnArgs a, const EncIn ain,
                                                         const EncOut hout) {
  constexpr int COLS = GATEUP ? 32 : 64;  // output columns per workgroup
  constexpr int PF = kDecPF;
  // scale loads actually needed for NSTAGE stages
  constexpr int BSL = (64 * NSTAGE * kDecWB / 2 + 255) / 256;
  static_assert(BSL <= kDecBSLoads, "scale staging bounds");
  static_assert(kDecMaxBlk / 2 <= 64, "one activation-scale row per wavefront load");
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][16 * kDecAPitch];
  // [row][blk] activation scales and [wave*16 + col][blk] weight scales, each with
  // a 4-byte dump slot at the end for lanes past the last entry
  __shared__ __attribute__((aligned(4))) uint16_t sAs[16 * kDecASPitch + 2];
  __shared__ __attribute__((aligned(4))) uint8_t sBs[64 * kDecBSPitch + 4];
  __shared__ __attribute__((aligned(16))) float gtile[GATEUP ? 2 * 16 * 36 : 4];

  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const int nblkK = K / 32;
  const int nst = (K + 127) / 128;   // 128-deep steps (the last may be half: K % 128 == 64)
  const int ncb = N / COLS;
  const int e = blockIdx.x / ncb;
  const int j = blockIdx.x - e * ncb;
  const int off = a.offsets[e];
  const int cnt = a.offsets[e + 1] - off;
  if (cnt == 0) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, q = lane >> 4;
  const int n = GATEUP ? j * 32 + (wave & 1) * 16 + l16 : j * 64 + wave * 16 + l16;
  const bool up = GATEUP && wave >= 2;
  const uint8_t* codes = GATEUP ? (up ? a.wu_codes : a.wg_codes) : a.wd_codes;
  const rsrc_t wr = make_rsrc(codes + (size_t)e * N * (K / 2), (uint32_t)((size_t)N * (K / 2)));
  const float bias = bf16_to_f32((GATEUP ? (up ? a.b_up : a.b_gate) : a.b_down)[(size_t)e * N + n]);
  const uint32_t wrow = (uint32_t)n * (K / 2);
  // activation rows: gathered tokens (gate/up) or this expert's rows of h (down)
  const rsrc_t ar = GATEUP ? make_rsrc(ain.codes, (uint32_t)((size_t)a.T * nblkK * kEncBytes))
                           : make_rsrc(ain.codes + (size_t)off * nblkK * kEncBytes,
                                       (uint32_t)((size_t)cnt * nblkK * kEncBytes));
  const rsrc_t asr = GATEUP ? make_rsrc(ain.scales, (uint32_t)((size_t)a.T * nblkK * 2))
                            : make_rsrc(ain.scales + (size_t)off * nblkK, (uint32_t)(cnt * nblkK * 2));
  const uint64_t kmagic = div_magic((uint32_t)a.k);  // token of dispatch pair q: q / k

  const rsrc_t sg = make_rsrc((GATEUP ? a.wg_scales : a.wd_scales) + (size_t)e * N * nblkK,
                              (uint32_t)(N * nblkK));
  const rsrc_t su = GATEUP ? make_rsrc(a.wu_scales + (size_t)e * N * nblkK, (uint32_t)(N * nblkK)) : sg;
  const int per_row = nblkK / 2;                        // uint16/uint32 entries per scale row
  const uint64_t prmagic = div_magic((uint32_t)per_row);

  // one stage's worth of loads for this thread
  struct Packet {
    uint4 w[kDecSS];              // weight codes (MFMA B operand, this lane)
    uint4 a[kDecAPerT];           // activation window chunks (staged to LDS)
  };
  // The stage's distance along K goes into the uniform buffer offset, so the
  // per-lane offsets are the same in every stage; only the last stage can hold
  // blocks past K, and only there are lanes redirected out of range.
  auto issue_w = [&](int st, Packet& pk) {
    const bool last = st == NSTAGE - 1;
    const uint32_t wso = (uint32_t)st * kDecSS * 64;    // weight bytes per 128-deep step: 64
#pragma unroll
    for (int u = 0; u < kDecSS; ++u) {
      const bool live = !last || (st * kDecSS + u) * 4 + q < nblkK;
      pk.w[u] = bload16(wr, live ? wrow + (u * 4 + q) * 16 : kOutOfRange, wso);
    }
  };

  for (int m0 = 0; m0 < cnt; m0 += 16) {
    const int rows = min(16, cnt - m0);
    Packet ring[PF + 1];
    __syncthreads();  // LDS of the previous row tile is no longer read

    // ---- prologue. Loads are issued in this order: the weight codes of the
    // first PF stages (they depend on nothing), the weight scales (first row
    // tile only), the row tile's dispatch entries; then, once those have
    // arrived, the activation scales and windows. So the prologue costs two
    // memory latencies, and the first weights arrive meanwhile.
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < NSTAGE) issue_w(p, ring[p]);
    // weight scales of the workgroup's 64 rows, all of K, as uint16 (two blocks)
    // row after row, so consecutive lanes read consecutive bytes; entries past
    // the end read zero and go to a dump slot
    uint32_t bsv[BSL];
    if (m0 == 0) {
#pragma unroll
      for (int i = 0; i < BSL; ++i) {
        const int idx = tid + 256 * i;
        const int row = min((int)div_by((uint32_t)idx, prmagic), 63), h = idx - row * per_row;
        const int w = row >> 4, r = row & 15;
        const int nn = GATEUP ? j * 32 + (w & 1) * 16 + r : j * 64 + w * 16 + r;
        const uint32_t o = idx < 64 * per_row ? (uint32_t)nn * nblkK + 2 * h : kOutOfRange;
        bsv[i] = (GATEUP && w >= 2) ? bload2(su, o) : bload2(sg, o);
      }
    }
    // activation rows: tokens of the row tile's dispatch pairs (gate/up) or the
    // expert's rows of h (down); rows past the count repeat the last one
    uint32_t src_row[16];
    if (GATEUP) {
#pragma unroll
      for (int r = 0; r < 16; ++r) src_row[r] = (uint32_t)a.sorted_pair[off + m0 + min(r, rows - 1)];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < 16; ++r) src_row[r] = div_by(src_row[r], kmagic);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) src_row[r] = (uint32_t)(m0 + min(r, rows - 1));
    }
    // activation scales of the row tile, all of K, as uint32 (two blocks): wave w
    // loads rows w, w+4, w+8, w+12, lane h the entry h of the row
    uint32_t asv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wave + 4 * i;
      asv[i] = bload4(asr, row < rows && lane < per_row ? src_row[row] * nblkK * 2 + 4 * lane : kOutOfRange);
    }
    uint32_t arow[kDecAPerT];
    int alds[kDecAPerT], ablk[kDecAPerT];
#pragma unroll
    for (int i = 0; i < kDecAPerT; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (kDecWB * 3), rem = c - row * (kDecWB * 3);
      const int blk = rem / 3, part = rem - blk * 3;
      alds[i] = row * kDecAPitch + blk * kEncBytes + part * 16;
      ablk[i] = blk;
      arow[i] = row < rows ? src_row[row] * nblkK * kEncBytes + part * 16 : kOutOfRange;
    }
    auto issue_a = [&](int st, Packet& pk) {
      const bool last = st == NSTAGE - 1;
      const int kb0 = st * kDecWB;
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i) {
        const bool live = !last || kb0 + ablk[i] < nblkK;
        pk.a[i] = bload16(ar, live ? arow[i] + ablk[i] * kEncBytes : kOutOfRange,
                          (uint32_t)kb0 * kEncBytes);
      }
    };
    auto stage_to_lds = [&](const Packet& pk, int buf) {
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i) {
        uint2* d = reinterpret_cast<uint2*>(sA[buf] + alds[i]);
        d[0] = make_uint2(pk.a[i].x, pk.a[i].y);
        d[1] = make_uint2(pk.a[i].z, pk.a[i].w);
      }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < NSTAGE) issue_a(p, ring[p]);

    // ---- scales to LDS (their loads are older than the windows': storing them
    // does not wait for the windows)
    if (m0 == 0) {
#pragma unroll
      for (int i = 0; i < BSL; ++i) {
        const int idx = tid + 256 * i;
        const int row = min((int)div_by((uint32_t)idx, prmagic), 63), h = idx - row * per_row;
        const int o = idx < 64 * per_row ? row * kDecBSPitch + 2 * h : 64 * kDecBSPitch;
        *reinterpret_cast<uint16_t*>(sBs + o) = static_cast<uint16_t>(bsv[i]);
      }
      // blocks nblkK, nblkK+1 are read (with zero codes) by the half step at the
      // end of K when K % 128 == 64: their scales must be finite, so they are
      // zeroed (2^-127); they lie in the row padding when K % 128 == 0
      if (tid < 64) *reinterpret_cast<uint16_t*>(sBs + tid * kDecBSPitch + nblkK) = 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wave + 4 * i;
      const int o = lane < per_row ? row * kDecASPitch + 2 * lane : 16 * kDecASPitch;
      *reinterpret_cast<uint32_t*>(sAs + o) = asv[i];
    }
    if (tid < 16)  // zero scales for the two blocks past K, as for the weights
      *reinterpret_cast<uint32_t*>(sAs + tid * kDecASPitch + nblkK) = 0u;

    v4f acc = v4f{bias, bias, bias, bias};
    auto issue = [&](int st, Packet& pk) {
      issue_w(st, pk);
      issue_a(st, pk);
    };
    stage_to_lds(ring[0], 0);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st) {
      if (st + PF < NSTAGE) issue(st + PF, ring[(st + PF) % (PF + 1)]);
      const Packet& cur = ring[st % (PF + 1)];
      const int buf = st & 1;
#pragma unroll
      for (int u = 0; u < kDecSS; ++u) {
        if (st * kDecSS + u < nst) {
          const int blk = st * kDecWB + 4 * u + q;
          const uint8_t* pa = sA[buf] + l16 * kDecAPitch + (4 * u + q) * kEncBytes;
          const uint2 h0 = lds64(pa), h1 = lds64(pa + 8), h2 = lds64(pa + 16);
          const uint2 g0 = lds64(pa + 24), g1 = lds64(pa + 32), g2 = lds64(pa + 40);
          const v8i ahi = {(int)h0.x, (int)h0.y, (int)h1.x, (int)h1.y, (int)h2.x, (int)h2.y, 0, 0};
          const v8i alo = {(int)g0.x, (int)g0.y, (int)g1.x, (int)g1.y, (int)g2.x, (int)g2.y, 0, 0};
          const int as = sAs[l16 * kDecASPitch + blk];
          const int bs = sBs[(wave * 16 + l16) * kDecBSPitch + blk];
          const v8i b = {(int)cur.w[u].x, (int)cur.w[u].y, (int)cur.w[u].z, (int)cur.w[u].w, 0, 0, 0, 0};
          acc = mfma16_f6f4<0>(ahi, b, acc, as, bs);
          acc = mfma16_f6f4<1>(alo, b, acc, as, bs);
        }
      }
      if (st + 1 < NSTAGE) stage_to_lds(ring[(st + 1) % (PF + 1)], (st + 1) & 1);
      __syncthreads();
    }

    if constexpr (GATEUP) {
      // waves 0,1 hold g, waves 2,3 hold u for the same 16 rows x 32 columns;
      // then one lane per row encodes the row's 32-column block of h
      float* t = gtile + (wave >> 1) * 16 * 36;
#pragma unroll
      for (int i = 0; i < 4; ++i) t[(4 * q + i) * 36 + (wave & 1) * 16 + l16] = acc[i];
      __syncthreads();
      if (tid < rows) {
        float v[32];
        const float4* g4 = reinterpret_cast<const float4*>(gtile + tid * 36);
        const float4* u4 = reinterpret_cast<const float4*>(gtile + 16 * 36 + tid * 36);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4 g = g4[c], u = u4[c];
          v[4 * c] = silu_mul(g.x, u.x);
          v[4 * c + 1] = silu_mul(g.y, u.y);
          v[4 * c + 2] = silu_mul(g.z, u.z);
          v[4 * c + 3] = silu_mul(g.w, u.w);
        }
        uint32_t hw[6], lw[6], sc;
        encode_block(v, hw, lw, sc);
        const size_t rec = (size_t)(off + m0 + tid) * (a.F / 32) + j;
        store_enc(hout.codes + rec * kEncBytes, hw, lw);
        hout.scales[rec] = static_cast<uint16_t>(sc);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < rows) a.y_sorted[(size_t)(off + m0 + 4 * q + i) * N + n] = acc[i];
    }
  }
}

// ------------------------------------------------------------------ host side

struct WsLayout {
  size_t xc, xs, hc, hs, tp, total;
};

WsLayout ws_layout(int T, int d, int F, int E, int k) {
  WsLayout L;
  const size_t P = (size_t)T * k;
  L.xc = 0;
  L.xs = L.xc + align256((size_t)T * (d / 32) * kEncBytes);
  L.hc = L.xs + align256((size_t)T * (d / 32) * 2);
  L.hs = L.hc + align256(P * (F / 32) * kEncBytes);
  L.tp = L.hs + align256(P * (F / 32) * 2);
  L.total = L.tp + align256((size_t)(E + 1) * 4);
  return L;
}

template <int NF, bool GATEUP>
hipError_t launch_prefill(const FfnArgs& a, EncIn ain, EncOut hout, const int32_t* tp,
                          hipStream_t stream) {
  const int N = GATEUP ? a.F : a.d;
  const int ntn = N / Prefill<NF, GATEUP>::MROWS;
  const int P = a.T * a.k;
  const int mt_max = (P + kBM - 1) / kBM + (a.E < P ? a.E : P);
  const long long grid = (long long)mt_max * ntn;
  hipLaunchKernelGGL((grouped_prefill<NF, GATEUP>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                     ain, hout, tp, ntn);
  return hipGetLastError();
}

template <bool GATEUP>
hipError_t launch_decode(const FfnArgs& a, EncIn ain, EncOut hout, hipStream_t stream) {
  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const dim3 grid(a.E * (N / (GATEUP ? 32 : 64)));
  const int nstage = ((K + 127) / 128 + kDecSS - 1) / kDecSS;
#define MOE_DECODE_CASE(S) \
  case S: hipLaunchKernelGGL((grouped_decode<GATEUP, S>), grid, dim3(256), 0, stream, a, ain, hout); break;
  switch (nstage) {
    MOE_DECODE_CASE(1) MOE_DECODE_CASE(2) MOE_DECODE_CASE(3) MOE_DECODE_CASE(4)
    MOE_DECODE_CASE(5) MOE_DECODE_CASE(6) MOE_DECODE_CASE(7) MOE_DECODE_CASE(8)
    default: return hipErrorInvalidValue;  // callers route K beyond this to the prefill kernel
  }
#undef MOE_DECODE_CASE
  static_assert(kDecMaxStages == 8, "keep the cases above in step with kDecMaxStages");
  return hipGetLastError();
}

bool decode_fits(int K) { return ((K + 127) / 128 + kDecSS - 1) / kDecSS <= kDecMaxStages; }

}  // namespace

size_t ffn_workspace_bytes(int T, int d, int F, int E, int k) {
  return ws_layout(T, d, F, E, k).total;
}

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream) {
  const WsLayout L = ws_layout(a.T, a.d, a.F, a.E, a.k);
  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  EncOut xout{ws + L.xc, reinterpret_cast<uint16_t*>(ws + L.xs)};
  EncIn xin{ws + L.xc, reinterpret_cast<const uint16_t*>(ws + L.xs)};
  EncOut hout{ws + L.hc, reinterpret_cast<uint16_t*>(ws + L.hs)};
  EncIn hin{ws + L.hc, reinterpret_cast<const uint16_t*>(ws + L.hs)};
  int32_t* tp = reinterpret_cast<int32_t*>(ws + L.tp);

  const int nx = a.T * (a.d / 32);
  if (nx <= 16384)
    hipLaunchKernelGGL(encode_rows, dim3((nx + 7) / 8), dim3(256), 0, stream, a.x, a.T, a.d,
                       xout.codes, xout.scales);
  else
    hipLaunchKernelGGL(encode_rows_thread, dim3((nx + 255) / 256), dim3(256), 0, stream, a.x, a.T,
                       a.d, xout.codes, xout.scales);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // Per GEMM: the weight-streaming decode kernel for few rows per expert and K
  // it can unroll, the LDS-tiled kernel otherwise (both read/write the same
  // encoded layouts, so they can be mixed).
  const bool dec_gu = a.T <= kDecodeMaxT && decode_fits(a.d);
  const bool dec_dn = a.T <= kDecodeMaxT && decode_fits(a.F);
  if (!dec_gu || !dec_dn) {
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(256), 0, stream, a.offsets, a.E, tp);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // Column tiles: the widest that divides N (gate/up: 32*NF h-columns, down:
  // 64*NF output columns per workgroup).
  if (dec_gu) {
    err = launch_decode<true>(a, xin, hout, stream);
  } else if (a.F % 192 == 0) {
    err = launch_prefill<6, true>(a, xin, hout, tp, stream);
  } else if (a.F % 128 == 0) {
    err = launch_prefill<4, true>(a, xin, hout, tp, stream);
  } else {
    err = launch_prefill<2, true>(a, xin, hout, tp, stream);
  }
  if (err != hipSuccess) return err;
  if (dec_dn) return launch_decode<false>(a, hin, hout, stream);
  if (a.d % 320 == 0) return launch_prefill<5, false>(a, hin, hout, tp, stream);
  if (a.d % 192 == 0) return launch_prefill<3, false>(a, hin, hout, tp, stream);
  if (a.d % 128 == 0) return launch_prefill<2, false>(a, hin, hout, tp, stream);
  return launch_prefill<1, false>(a, hin, hout, tp, stream);
}


}  // namespace moe
