// Grouped expert FFN on gfx950 scaled matrix cores (V_MFMA_SCALE_F32_*_F8F6F4).
//
// For every expert e and dispatch row p of e (Perplexity, "GPT-OSS el dia 0",
// section "MLP": SwiGLU experts with biases; section "Nuclis per a GPT-OSS / MoE":
// the bias is loaded into the GEMM accumulators once per output tile):
//   h_p = silu(x_t Wg^T + bg) * (x_t Wu^T + bu)      gate/up GEMM, fused epilogue
//   y_p = h_p Wd^T + bd                               down GEMM
// B operands are the MXFP4 weights in the packed fragment layout (layout.hpp):
// E2M1 nibbles and E8M0 block scales unchanged, never dequantised. A operands are
// two-term MXFP6 encodings (mx6.hpp) in 208-byte step chunks: x is encoded once
// per token row, h by the gate/up epilogue.
//
// Two kernel shapes, chosen on the host from T (expert row counts stay on the
// device):
//   prefill  128 dispatch rows x 64*NF weight rows per workgroup, 2x2 wavefronts,
//            K in 128-deep steps copied from global memory straight into LDS
//            (three steps in flight). Every copy instruction moves 1 KB: a packed
//            B fragment is one contiguous kilobyte, and A rows are copied as
//            whole 208-byte chunks. The grid is an upper bound on the number of
//            (row tile, column tile) pairs; a tile table built on the device maps
//            a workgroup to its expert, and surplus workgroups exit. Tiles are
//            rastered in groups of a few row tiles x all column tiles and each
//            XCD (dispatch is round-robin over the 8 XCDs) takes a contiguous
//            range of them, so resident workgroups share A rows and expert
//            weights in their L2.
//   decode   weight streaming for few rows per expert: one workgroup per
//            (expert, 32 h-columns) or (expert, 64 output columns); each
//            wavefront streams one 16-row half of a packed 32-row group straight
//            from HBM into MFMA registers (16x16x128 MFMA, 16 rows per pass).
#include "mx6.hpp"

namespace moe {
namespace {

constexpr int kBM = 128;        // rows per prefill tile
constexpr int kPrefGM = 8;      // row tiles per raster group of the prefill grid
constexpr int kDecodeMaxT = 64; // decode kernels when T <= this

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

__device__ __forceinline__ uint32_t enc_pitch(int K) { return (uint32_t)nsteps_of(K) * kChunk; }

// Byte offsets of block b's codes and scales inside an encoded row.
__device__ __forceinline__ uint32_t enc_codes_at(int b) { return (b >> 2) * kChunk + (b & 3) * kEncBytes; }
__device__ __forceinline__ uint32_t enc_scale_at(int b) { return (b >> 2) * kChunk + kChunkScales + (b & 3) * 2; }

// ------------------------------------------------------------------ encode x

// Activation encoding, two shapes: few rows (decode) -- one (row, 32-element
// block) per half wavefront, lane j takes element j and the block is encoded
// cooperatively (short latency); many rows (prefill) -- one block per thread
// (no barriers, throughput).
__global__ __launch_bounds__(256) void encode_rows_thread(const uint16_t* __restrict__ x, int rows,
                                                          int K, uint8_t* __restrict__ enc) {
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

__global__ __launch_bounds__(256) void encode_rows(const uint16_t* __restrict__ x, int rows,
                                                   int K, uint8_t* __restrict__ enc) {
  __shared__ uint8_t scratch[8 * 64];
  const int nblk = K / 32;
  const int nrec = rows * nblk;
  const int g = blockIdx.x * 8 + (threadIdx.x >> 5);
  const int gg = g < nrec ? g : nrec - 1;
  const int row = gg / nblk, b = gg - row * nblk;
  const float v = bf16_to_f32(x[(size_t)gg * 32 + (threadIdx.x & 31)]);
  uint8_t* r = enc + (size_t)row * enc_pitch(K);
  encode_group32(v, scratch + (threadIdx.x >> 5) * 64, r + enc_codes_at(b),
                 reinterpret_cast<uint16_t*>(r + enc_scale_at(b)), g < nrec);
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

// ------------------------------------------------------------------ prefill

// One workgroup = 128 dispatch rows x 64*NF weight rows, 2x2 wavefronts; wave
// (wm, wn) owns rows 64wm..64wm+63 (two 32-row fragments) and NF 32-row weight
// groups (for gate/up: NF/2 gate and NF/2 up groups of the same h-columns, so
// SwiGLU can be applied to the tile).
//
// Each K step is copied from global memory straight into LDS by buffer-to-LDS
// loads (lane i of a copy writes LDS bytes [16i, 16i+16) for 16-byte copies and
// the dword 4i, zero-extended, for 2-byte ones), three steps in flight: the copy
// of step t+2 is issued when step t is computed. LDS layout of one step:
//   A   [128 rows][208 B]  the rows' encoded chunks as stored (copy q of 16 B:
//                          row q/13, piece q%13; lanes of one row read one run)
//   B   [group][half][lane][16 B]  packed fragments, 1 KB per copy
//   BS  [group][lane][4 B]         packed scales (2 bytes used)
// MFMA half s of a step takes, in lane half h, block 2h + s of A and of B. Rows
// past the tile's count, blocks past K and steps past the end are read as zero
// through the resource's range check.
template <int NF, bool GATEUP>
struct Prefill {
  static constexpr int BN = 64 * NF;                   // weight rows per workgroup
  static constexpr int NFR = 2 * NF;                   // 32-row weight groups per workgroup
  static constexpr int MROWS = GATEUP ? BN / 2 : BN;   // output columns per workgroup
  static constexpr int FM = GATEUP ? NF / 2 : NF;      // groups per matrix per wave
  static constexpr int A_COPIES = kBM * kChunkPieces / 64;
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = A_OFF + kBM * kChunk;
  static constexpr int BS_OFF = B_OFF + NFR * 2 * 1024;
  static constexpr int STAGE = BS_OFF + NFR * 256;
  static constexpr int NA = (A_COPIES + 3) / 4;        // A copies per wave (at most)
  static constexpr int NB = NFR * 2 / 4;               // B copies per wave
  static constexpr int NBSW = (NFR + 3) / 4;           // scale copies per wave (at most)
  // copies wave w issues per step
  static constexpr int copies(int w) { return (A_COPIES - w + 3) / 4 + NB + (NFR - w + 3) / 4; }
  static constexpr int EP_PITCH = 36;                  // floats per row of the SwiGLU staging tile
  static_assert(kBM * kChunkPieces % 64 == 0, "A copies are whole instructions");
  static_assert(!GATEUP || NF % 2 == 0, "gate/up tiles pair gate and up groups");
  static_assert(copies(0) <= 63, "one step of copies must fit the vector memory counter");
  static_assert(3 * STAGE <= 160 * 1024, "three step buffers must fit the 160 KB of LDS");
  static_assert(!GATEUP || 2 * 64 * EP_PITCH * 4 <= STAGE, "SwiGLU staging of two waves must fit a step buffer");
};

// s_waitcnt with only the vector memory counter bounded (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and lgkmcnt at max).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Buffer-to-LDS copy of SIZE bytes per lane (16 or 2) into `lds` (wave-uniform).
template <int SIZE>
__device__ __forceinline__ void lds_copy(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  static_assert(SIZE == 16 || SIZE == 2, "copy sizes used here");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds, 2, voff, soff, 0, 0);
}

template <int NF, bool GATEUP>
__global__ __launch_bounds__(256) void grouped_prefill(const FfnArgs a, const uint8_t* __restrict__ ain,
                                                       uint8_t* __restrict__ hout,
                                                       const int32_t* __restrict__ tile_prefix,
                                                       int ntn) {
  using C = Prefill<NF, GATEUP>;
  // three step buffers as separate objects, so the compiler can tell the copy
  // into one from the reads of another
  __shared__ __attribute__((aligned(16))) uint8_t st0[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[C::STAGE];
  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const int nblkK = K / 32;
  const int nst = nsteps_of(K);
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
  const uint32_t apitch = (uint32_t)nst * kChunk;
  const rsrc_t ar = GATEUP ? make_rsrc(ain, (uint32_t)a.T * apitch)
                           : make_rsrc(ain + (size_t)(off + m0) * apitch, (uint32_t)rows_valid * apitch);
  const uint64_t kmagic = div_magic((uint32_t)a.k);  // token of dispatch pair q: q / k
  const size_t gstride = (size_t)nst * kWStep;        // packed code bytes per 32-row group
  const size_t sstride = (size_t)nst * kWSStep;       // packed scale bytes per 32-row group
  const size_t egroups = (size_t)e * (N / 32);
  const rsrc_t br0 = make_rsrc((GATEUP ? a.wg_codes : a.wd_codes) + egroups * gstride,
                               (uint32_t)((N / 32) * gstride));
  const rsrc_t bsr0 = make_rsrc((GATEUP ? a.wg_scales : a.wd_scales) + egroups * sstride,
                                (uint32_t)((N / 32) * sstride));
  const rsrc_t br1 = GATEUP ? make_rsrc(a.wu_codes + egroups * gstride, (uint32_t)((N / 32) * gstride)) : br0;
  const rsrc_t bsr1 = GATEUP ? make_rsrc(a.wu_scales + egroups * sstride, (uint32_t)((N / 32) * sstride)) : bsr0;
  // first weight row of group phi, and whether phi is an up group
  auto frag_up = [&](int phi) { return GATEUP && (phi % NF) >= NF / 2; };
  auto frag_row = [&](int phi) -> int {
    if (GATEUP) {
      const int w = phi / NF, f = phi % NF;
      return col0 + w * C::FM * 32 + (f < NF / 2 ? f : f - NF / 2) * 32;
    }
    return col0 + phi * 32;
  };

  // ---- biases of this lane's output columns, loaded together with the dispatch
  // entries below and before the first copies (waiting for them must not wait
  // for the copies)
  float bias[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int phi = wn * NF + f;
    const uint16_t* bsrc = GATEUP ? (frag_up(phi) ? a.b_up : a.b_gate) : a.b_down;
    bias[f] = bf16_to_f32(bsrc[(size_t)e * N + frag_row(phi) + lr]);
  }

  // ---- per-lane source offsets of this wave's A copies (fixed across steps; the
  // step's K distance goes into the uniform offset). Copy i = wave + 4t covers
  // 16-byte pieces 64i + lane: row (64i + lane) / 13, piece (64i + lane) % 13.
  int a_piece[C::NA];
  uint32_t a_src[C::NA];
#pragma unroll
  for (int t = 0; t < C::NA; ++t) {
    const int q = (wave + 4 * t) * 64 + lane;
    const int row = q / kChunkPieces;
    a_piece[t] = q - row * kChunkPieces;
    a_src[t] = (uint32_t)min(row, rows_valid - 1);
  }
  if (GATEUP) {
#pragma unroll
    for (int t = 0; t < C::NA; ++t) a_src[t] = (uint32_t)a.sorted_pair[off + m0 + a_src[t]];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < C::NA; ++t) a_src[t] = div_by(a_src[t], kmagic);
  }
  uint32_t a_off[C::NA];
#pragma unroll
  for (int t = 0; t < C::NA; ++t) {
    const int q = (wave + 4 * t) * 64 + lane;
    const bool ok = wave + 4 * t < C::A_COPIES && q / kChunkPieces < rows_valid;
    a_off[t] = ok ? a_src[t] * apitch + a_piece[t] * 16 : kOutOfRange;
  }
  // B copies: copy i = wave + 4t is half i & 1 of group i >> 1; scale copy t is
  // group wave + 4t. Only the lane offset varies across lanes.
  uint32_t b_off[C::NB];
#pragma unroll
  for (int t = 0; t < C::NB; ++t) {
    const int i = wave + 4 * t;
    b_off[t] = (uint32_t)(frag_row(i >> 1) / 32) * (uint32_t)gstride + (i & 1) * 1024 + lane * 16;
  }
  uint32_t bs_off[C::NBSW];
#pragma unroll
  for (int t = 0; t < C::NBSW; ++t) {
    const int phi = wave + 4 * t;
    bs_off[t] = phi < C::NFR ? (uint32_t)(frag_row(phi) / 32) * (uint32_t)sstride + lane * 2 : kOutOfRange;
  }

  // Copy step st into LDS buffer `buf`.
  auto issue = [&](int st, uint8_t* buf) {
    const bool live = st < nst;
    const bool halfst = 4 * st + 2 >= nblkK;  // blocks 2, 3 of this step are past K
#pragma unroll
    for (int t = 0; t < C::NA; ++t) {
      const int i = wave + 4 * t;
      if (i < C::A_COPIES) {
        const bool pad = halfst && a_piece[t] >= 6 && a_piece[t] < 12;
        lds_copy<16>(ar, buf + C::A_OFF + i * 1024, live && !pad ? a_off[t] : kOutOfRange,
                     (uint32_t)st * kChunk);
      }
    }
#pragma unroll
    for (int t = 0; t < C::NB; ++t) {
      const int i = wave + 4 * t;
      lds_copy<16>(frag_up(i >> 1) ? br1 : br0, buf + C::B_OFF + i * 1024,
                   live ? b_off[t] : kOutOfRange, (uint32_t)st * kWStep);
    }
#pragma unroll
    for (int t = 0; t < C::NBSW; ++t) {
      const int phi = wave + 4 * t;
      if (phi < C::NFR)
        lds_copy<2>(frag_up(phi) ? bsr1 : bsr0, buf + C::BS_OFF + phi * 256,
                    live ? bs_off[t] : kOutOfRange, (uint32_t)st * kWSStep);
    }
  };

  // Wait until this wave's copies of the step about to be computed have landed;
  // the next step's copies (issued after it) stay in flight.
  auto wait_step = [&]() {
    if (wave == 0) MOE_WAIT_VMCNT(C::copies(0));
    else if (wave == 1) MOE_WAIT_VMCNT(C::copies(1));
    else if (wave == 2) MOE_WAIT_VMCNT(C::copies(2));
    else MOE_WAIT_VMCNT(C::copies(3));
  };

  v16f acc[2][NF];

  // Compute one step out of LDS buffer `buf`: both MFMA halves' fragments are
  // read first, then 2 x 2 x NF x 2 scaled MFMAs (hi and lo terms of A).
  auto compute = [&](const uint8_t* buf, int st) {
    // Steps past K compute nothing. A half step at the end of K (K % 128 == 64)
    // still takes both MFMA halves: lane half 0 holds blocks 0, 1 (valid), lane
    // half 1 zero codes with their scale bytes forced finite.
    if (st >= nst) return;
    const bool halfst = 4 * st + 2 >= nblkK;
    v8i ahi[2][2], alo[2][2];
    int sa[2];
#pragma unroll
    for (int mf = 0; mf < 2; ++mf) {
      const uint8_t* rowp = buf + C::A_OFF + (wm * 64 + mf * 32 + lr) * kChunk;
      const uint4* p = reinterpret_cast<const uint4*>(rowp + half * 96);
      const uint4 q0 = p[0], q1 = p[1], q2 = p[2], q3 = p[3], q4 = p[4], q5 = p[5];
      ahi[mf][0] = v8i{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, 0, 0};
      alo[mf][0] = v8i{(int)q1.z, (int)q1.w, (int)q2.x, (int)q2.y, (int)q2.z, (int)q2.w, 0, 0};
      ahi[mf][1] = v8i{(int)q3.x, (int)q3.y, (int)q3.z, (int)q3.w, (int)q4.x, (int)q4.y, 0, 0};
      alo[mf][1] = v8i{(int)q4.z, (int)q4.w, (int)q5.x, (int)q5.y, (int)q5.z, (int)q5.w, 0, 0};
      const int s = *reinterpret_cast<const int*>(rowp + kChunkScales + 4 * half);
      sa[mf] = halfst && half ? 0 : s;
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
    // half 0: scale bytes 0 (A hi), 1 (A lo), 0 (B); half 1: bytes 2, 3, 1
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

  // One step: wait for this wave's copies of step st, barrier (everyone's copies
  // of st have landed and everyone has finished reading the buffer that the copy
  // issued next overwrites), copy step st+2, compute step st.
  auto step = [&](int st, const uint8_t* cur, uint8_t* nxt2) {
    wait_step();
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
  // Steps go in threes (one per buffer); steps past the end copy zeros and
  // compute nothing.
  for (int t = 0; t < nst; t += 3) {
    step(t, st0, st2);
    step(t + 1, st1, st0);
    step(t + 2, st2, st1);
  }
  MOE_WAIT_VMCNT(0);
  __syncthreads();

  if constexpr (GATEUP) {
    // h = silu(g) * u; per gate group f, the wave's two 32x32 tiles go to LDS as
    // 64 rows x 32 columns and each lane encodes one row's 32-column block as
    // two-term MXFP6 into the row's step chunk.
    float* ep = reinterpret_cast<float*>(wave < 2 ? st0 : st1) + (wave & 1) * 64 * C::EP_PITCH;
    const uint32_t hpitch = (uint32_t)nsteps_of(a.F) * kChunk;
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
        const int b = (col0 + wn * C::FM * 32 + f * 32) / 32;
        uint8_t* hrow = hout + (size_t)(off + grow) * hpitch;
        store_enc(hrow + enc_codes_at(b), hw, lw);
        *reinterpret_cast<uint16_t*>(hrow + enc_scale_at(b)) = static_cast<uint16_t>(sc);
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

// Weight streaming for few rows per expert. One workgroup per (expert, 32
// h-columns) for gate/up -- waves 0,1 stream the two 16-row halves of the gate
// group, waves 2,3 those of the up group -- or per (expert, 64 output columns)
// for down -- wave w streams the 16-row half w&1 of group 2j + w/2. Each
// wavefront uses the 16x16x128 scaled MFMA (16 rows = one decode-sized row
// tile) over the whole of K. K is processed in stages of kDecSS steps, fully
// unrolled at compile time (NSTAGE stages): the weight codes and the activation
// window of stage s+kDecPF are issued while stage s is computed, held in
// register rings, and the window is copied to LDS one stage before it is read,
// so the activations are read from L2 once per workgroup rather than once per
// wavefront. Loads are issued in the order they are consumed, so waiting for one
// never waits for a younger one (the vector memory counter retires in order).
// All global reads are buffer loads: blocks past K and rows past the count read
// as zero. The packed weight scales of the workgroup's two groups (all of K) are
// staged in LDS once.
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

constexpr int kDecSS = 4;                            // 128-deep steps per stage
constexpr int kDecPF = 2;                            // stages of loads in flight ahead of the one computed
constexpr int kDecMaxStages = 8;                     // decode kernels cover K <= kDecMaxStages * kDecSS * 128
constexpr int kDecMaxSteps = kDecMaxStages * kDecSS;
constexpr int kDecAPitch = kDecSS * kChunk + 16;     // LDS bytes per activation row (padded: no bank conflicts)
constexpr int kDecAPieces = 16 * kDecSS * kChunkPieces;  // 16-byte pieces of one stage's window
constexpr int kDecAPerT = (kDecAPieces + 255) / 256;     // ... per thread (at most)
static_assert(kDecMaxSteps * kWSStep / 16 <= 256, "one scale piece per thread and group");

template <bool GATEUP, int NSTAGE>
__global__ __launch_bounds__(256, 2) void grouped_decode(const FfnArgs a, const uint8_t* __restrict__ ain,
                                                         uint8_t* __restrict__ hout) {
  constexpr int COLS = GATEUP ? 32 : 64;  // output columns per workgroup
  constexpr int PF = kDecPF;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][16 * kDecAPitch];
  // packed weight scales of the two groups: [group][step][lane] uint16
  __shared__ __attribute__((aligned(16))) uint16_t sBs[2 * kDecMaxSteps * 64];
  __shared__ __attribute__((aligned(16))) float gtile[GATEUP ? 2 * 16 * 36 : 4];

  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const int nblkK = K / 32;
  const int nst = nsteps_of(K);      // 128-deep steps (the last may be half: K % 128 == 64)
  const int ncb = N / COLS;
  const int e = blockIdx.x / ncb;
  const int j = blockIdx.x - e * ncb;
  const int off = a.offsets[e];
  const int cnt = a.offsets[e + 1] - off;
  if (cnt == 0) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, q = lane >> 4;
  const int sub = wave & 1;                          // 16-row half of the group
  const int g = GATEUP ? j : 2 * j + (wave >> 1);    // this wave's 32-row weight group
  const bool up = GATEUP && wave >= 2;
  const int n = 32 * g + 16 * sub + l16;             // output column of this lane
  const uint8_t* codes = GATEUP ? (up ? a.wu_codes : a.wg_codes) : a.wd_codes;
  const size_t gstride = (size_t)nst * kWStep;
  const rsrc_t wr = make_rsrc(codes + ((size_t)e * (N / 32) + g) * gstride, (uint32_t)gstride);
  // lane (column l16, K sub-block q): half q&1, lane 32*(q/2) + 16*sub + l16 of the packed step
  const uint32_t wl = (uint32_t)(q & 1) * 1024 + (uint32_t)((q >> 1) * 32 + 16 * sub + l16) * 16;
  const float bias = bf16_to_f32((GATEUP ? (up ? a.b_up : a.b_gate) : a.b_down)[(size_t)e * N + n]);
  const uint32_t apitch = (uint32_t)nst * kChunk;
  // activation rows: gathered tokens (gate/up) or this expert's rows of h (down)
  const rsrc_t ar = GATEUP ? make_rsrc(ain, (uint32_t)a.T * apitch)
                           : make_rsrc(ain + (size_t)off * apitch, (uint32_t)cnt * apitch);
  const uint64_t kmagic = div_magic((uint32_t)a.k);  // token of dispatch pair q: q / k

  const size_t sstride = (size_t)nst * kWSStep;
  const uint8_t* s0 = (GATEUP ? a.wg_scales : a.wd_scales) + ((size_t)e * (N / 32) + (GATEUP ? j : 2 * j)) * sstride;
  const uint8_t* s1 = GATEUP ? a.wu_scales + ((size_t)e * (N / 32) + j) * sstride : s0 + sstride;
  const rsrc_t rs0 = make_rsrc(s0, (uint32_t)sstride), rs1 = make_rsrc(s1, (uint32_t)sstride);

  // one stage's worth of loads for this thread
  struct Packet {
    uint4 w[kDecSS];              // weight codes (MFMA B operand, this lane)
    uint4 a[kDecAPerT];           // activation window pieces (staged to LDS)
  };
  // The step's distance along K goes into the uniform buffer offset, so the
  // per-lane offsets are the same in every stage. In a half step at the end of K
  // the lanes of sub-blocks 2, 3 read nothing.
  auto issue_w = [&](int st, Packet& pk) {
#pragma unroll
    for (int u = 0; u < kDecSS; ++u) {
      const int jj = st * kDecSS + u;
      const bool live = jj < nst && (4 * jj + 2 < nblkK || q < 2);
      pk.w[u] = bload16(wr, live ? wl : kOutOfRange, (uint32_t)jj * kWStep);
    }
  };

  for (int m0 = 0; m0 < cnt; m0 += 16) {
    const int rows = min(16, cnt - m0);
    Packet ring[PF + 1];
    __syncthreads();  // LDS of the previous row tile is no longer read

    // ---- prologue. Loads are issued in this order: the weight codes of the
    // first PF stages (they depend on nothing), the weight scales (first row
    // tile only), the window pieces' dispatch entries; then, once those have
    // arrived, the activation windows. So the prologue costs two memory
    // latencies, and the first weights arrive meanwhile.
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < NSTAGE) issue_w(p, ring[p]);
    uint4 bsv0, bsv1;
    if (m0 == 0) {
      const uint32_t o = tid < nst * (kWSStep / 16) ? (uint32_t)tid * 16 : kOutOfRange;
      bsv0 = bload16(rs0, o);
      bsv1 = bload16(rs1, o);
    }
    // window piece c = tid + 256i: row c / 52, step u = (c % 52) / 13, piece c % 13
    uint32_t arow[kDecAPerT];
    int alds[kDecAPerT], au[kDecAPerT], ap[kDecAPerT];
#pragma unroll
    for (int i = 0; i < kDecAPerT; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (kDecSS * kChunkPieces), rem = c - row * (kDecSS * kChunkPieces);
      au[i] = rem / kChunkPieces;
      ap[i] = rem - au[i] * kChunkPieces;
      alds[i] = row * kDecAPitch + au[i] * kChunk + ap[i] * 16;
      arow[i] = (uint32_t)min(row, rows - 1);
    }
    if (GATEUP) {
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i) arow[i] = (uint32_t)a.sorted_pair[off + m0 + arow[i]];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i) arow[i] = div_by(arow[i], kmagic);
    } else {
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i) arow[i] += (uint32_t)m0;
    }
#pragma unroll
    for (int i = 0; i < kDecAPerT; ++i) {
      const int c = tid + 256 * i;
      const bool ok = c < kDecAPieces && c / (kDecSS * kChunkPieces) < rows;
      arow[i] = ok ? arow[i] * apitch + (uint32_t)(au[i] * kChunk + ap[i] * 16) : kOutOfRange;
    }
    auto issue_a = [&](int st, Packet& pk) {
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i) {
        const int jj = st * kDecSS + au[i];
        const bool pad = 4 * jj + 2 >= nblkK && ap[i] >= 6 && ap[i] < 12;
        pk.a[i] = bload16(ar, jj < nst && !pad ? arow[i] : kOutOfRange,
                          (uint32_t)(st * kDecSS) * kChunk);
      }
    };
    auto stage_to_lds = [&](const Packet& pk, int buf) {
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i)
        if (tid + 256 * i < kDecAPieces) *reinterpret_cast<uint4*>(sA[buf] + alds[i]) = pk.a[i];
    };
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < NSTAGE) issue_a(p, ring[p]);

    // ---- weight scales to LDS (their loads are older than the windows': storing
    // them does not wait for the windows)
    if (m0 == 0 && tid < nst * (kWSStep / 16)) {
      *reinterpret_cast<uint4*>(sBs + tid * 8) = bsv0;
      *reinterpret_cast<uint4*>(sBs + kDecMaxSteps * 64 + tid * 8) = bsv1;
    }

    v4f acc = v4f{bias, bias, bias, bias};
    auto issue = [&](int st, Packet& pk) {
      issue_w(st, pk);
      issue_a(st, pk);
    };
    const uint16_t* bsrow = sBs + (wave >> 1) * kDecMaxSteps * 64 + (q >> 1) * 32 + 16 * sub + l16;
    stage_to_lds(ring[0], 0);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st) {
      if (st + PF < NSTAGE) issue(st + PF, ring[(st + PF) % (PF + 1)]);
      const Packet& cur = ring[st % (PF + 1)];
      const int buf = st & 1;
#pragma unroll
      for (int u = 0; u < kDecSS; ++u) {
        const int jj = st * kDecSS + u;
        if (jj < nst) {
          const uint8_t* rowp = sA[buf] + l16 * kDecAPitch + u * kChunk;
          const uint4* pa = reinterpret_cast<const uint4*>(rowp + q * kEncBytes);
          const uint4 x0 = pa[0], x1 = pa[1], x2 = pa[2];
          const v8i ahi = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, 0, 0};
          const v8i alo = {(int)x1.z, (int)x1.w, (int)x2.x, (int)x2.y, (int)x2.z, (int)x2.w, 0, 0};
          int as = *reinterpret_cast<const uint16_t*>(rowp + kChunkScales + 2 * q);
          if (4 * jj + 2 >= nblkK && q >= 2) as = 0;  // blocks past K: zero codes, finite scales
          const int bs = bsrow[jj * 64] >> (8 * (q & 1));
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
      for (int i = 0; i < 4; ++i) t[(4 * q + i) * 36 + sub * 16 + l16] = acc[i];
      __syncthreads();
      if (tid < rows) {
        float v[32];
        const float4* g4 = reinterpret_cast<const float4*>(gtile + tid * 36);
        const float4* u4 = reinterpret_cast<const float4*>(gtile + 16 * 36 + tid * 36);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4 gg = g4[c], uu = u4[c];
          v[4 * c] = silu_mul(gg.x, uu.x);
          v[4 * c + 1] = silu_mul(gg.y, uu.y);
          v[4 * c + 2] = silu_mul(gg.z, uu.z);
          v[4 * c + 3] = silu_mul(gg.w, uu.w);
        }
        uint32_t hw[6], lw[6], sc;
        encode_block(v, hw, lw, sc);
        uint8_t* hrow = hout + (size_t)(off + m0 + tid) * enc_pitch(a.F);
        store_enc(hrow + enc_codes_at(j), hw, lw);
        *reinterpret_cast<uint16_t*>(hrow + enc_scale_at(j)) = static_cast<uint16_t>(sc);
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
  size_t x, h, tp, total;
};

WsLayout ws_layout(int T, int d, int F, int E, int k) {
  WsLayout L;
  const size_t P = (size_t)T * k;
  L.x = 0;
  L.h = L.x + align256((size_t)T * nsteps_of(d) * kChunk);
  L.tp = L.h + align256(P * nsteps_of(F) * kChunk);
  L.total = L.tp + align256((size_t)(E + 1) * 4);
  return L;
}

template <int NF, bool GATEUP>
hipError_t launch_prefill(const FfnArgs& a, const uint8_t* ain, uint8_t* hout, const int32_t* tp,
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
hipError_t launch_decode(const FfnArgs& a, const uint8_t* ain, uint8_t* hout, hipStream_t stream) {
  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const dim3 grid(a.E * (N / (GATEUP ? 32 : 64)));
  const int nstage = (nsteps_of(K) + kDecSS - 1) / kDecSS;
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

bool decode_fits(int K) { return (nsteps_of(K) + kDecSS - 1) / kDecSS <= kDecMaxStages; }

}  // namespace

size_t ffn_workspace_bytes(int T, int d, int F, int E, int k) {
  return ws_layout(T, d, F, E, k).total;
}

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream) {
  const WsLayout L = ws_layout(a.T, a.d, a.F, a.E, a.k);
  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  uint8_t* xenc = ws + L.x;
  uint8_t* henc = ws + L.h;
  int32_t* tp = reinterpret_cast<int32_t*>(ws + L.tp);

  const int nx = a.T * (a.d / 32);
  if (nx <= 16384)
    hipLaunchKernelGGL(encode_rows, dim3((nx + 7) / 8), dim3(256), 0, stream, a.x, a.T, a.d, xenc);
  else
    hipLaunchKernelGGL(encode_rows_thread, dim3((nx + 255) / 256), dim3(256), 0, stream, a.x, a.T,
                       a.d, xenc);
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
    err = launch_decode<true>(a, xenc, henc, stream);
  } else if (a.F % 192 == 0) {
    err = launch_prefill<6, true>(a, xenc, henc, tp, stream);
  } else if (a.F % 128 == 0) {
    err = launch_prefill<4, true>(a, xenc, henc, tp, stream);
  } else {
    err = launch_prefill<2, true>(a, xenc, henc, tp, stream);
  }
  if (err != hipSuccess) return err;
  if (dec_dn) return launch_decode<false>(a, henc, henc, stream);
  if (a.d % 320 == 0) return launch_prefill<5, false>(a, henc, henc, tp, stream);
  if (a.d % 192 == 0) return launch_prefill<3, false>(a, henc, henc, tp, stream);
  if (a.d % 128 == 0) return launch_prefill<2, false>(a, henc, henc, tp, stream);
  return launch_prefill<1, false>(a, henc, henc, tp, stream);
}

}  // namespace moe
