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
//   prefill  128 dispatch rows x 64*NF weight rows per workgroup, 4x2 wavefronts
//            (two per SIMD), K in 128-deep steps copied from global memory straight into LDS
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
#include "ffn_dev.hpp"
#include "mx6.hpp"

namespace moe {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// row tiles per raster group of the prefill grid (gate/up, down): chosen by
// measurement; the 32 workgroups of an XCD then share GM row tiles of A and
// 32/GM column tiles of the weights
template <bool GATEUP>
constexpr int kPrefGM = GATEUP ? 8 : 4;
constexpr int kDecodeMaxT = 64; // decode kernels when T <= this

// The tables the GEMMs of this call need, built by one extra workgroup of the
// activation encoder (same launch); either pointer may be null.
struct TableJob {
  const int32_t* offsets;
  int E;
  int4* tiles;   // 128-row prefill tiles
  int4* passes;  // 16-row decode passes
};
__device__ __forceinline__ void build_tables(const TableJob& tj) {
  __shared__ int s[257];
  if (tj.tiles) build_tile_table<kBM>(tj.offsets, tj.E, tj.tiles, s);
  __syncthreads();
  if (tj.passes) build_tile_table<kDecRows>(tj.offsets, tj.E, tj.passes, s);
}

// ------------------------------------------------------------------ encode x

// Activation encoding, two shapes: few rows (decode) -- one (row, 32-element
// block) per half wavefront, lane j takes element j and the block is encoded
// cooperatively (short latency); many rows (prefill) -- one block per thread
// (no barriers, throughput).
__global__ __launch_bounds__(256) void encode_rows_thread(const uint16_t* __restrict__ x, int rows,
                                                          int K, uint8_t* __restrict__ enc,
                                                          const TableJob tj) {
  if (blockIdx.x == gridDim.x - 1) {
    build_tables(tj);
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

__global__ __launch_bounds__(256) void encode_rows(const uint16_t* __restrict__ x, int rows,
                                                   int K, uint8_t* __restrict__ enc, const TableJob tj) {
  if (blockIdx.x == gridDim.x - 1) {
    build_tables(tj);
    return;
  }
  encode_rows_group(x, rows, K, enc, blockIdx.x);
}

// Division by a runtime divisor d >= 1 as a multiply: x / d = (x * m) >> 32 with
// m = ceil(2^32 / d), exact for x < 2^32 / d (here x < 2^20).
__device__ __forceinline__ uint64_t div_magic(uint32_t d) { return ((1ull << 32) + d - 1) / d; }
__device__ __forceinline__ uint32_t div_by(uint32_t x, uint64_t m) {
  return static_cast<uint32_t>((static_cast<uint64_t>(x) * m) >> 32);
}

// ------------------------------------------------------------------ prefill

// One workgroup = 128 dispatch rows x 64*NF weight rows, eight wavefronts, two
// per SIMD: while one waits (for its LDS reads, its copies, the barrier) the
// other's MFMAs keep the matrix unit busy. Wave (wm, wn), wm = 0..3, wn = 0..1,
// owns rows 32wm..32wm+31 (one 32-row fragment) and NF 32-row weight groups (for
// gate/up: NF/2 gate and NF/2 up groups of the same h-columns, so SwiGLU can be
// applied to the tile).
//
// Each K step is copied from global memory straight into LDS by buffer-to-LDS
// loads (lane i of a copy writes LDS bytes [16i, 16i+16) for 16-byte copies and
// [4i, 4i+4) for 4-byte ones) into three step buffers that rotate from step to
// step and from tile to tile: step st+2 is copied while step st is computed.
// LDS layout of one step:
//   A   [128 rows][208 B]  the rows' encoded chunks as stored (copy q of 16 B:
//                          row q/13, piece q%13; lanes of one row read one run)
//   B   [group][half][lane][16 B]  packed fragments, 1 KB per copy
//   BS  [matrix][group of the matrix][lane][2 B]  packed scales; one 4-byte copy
//                          covers two groups of one matrix (lanes 0-31, 32-63)
// The copies of a step are dealt out over the eight waves in equal numbers (a
// wave whose share is short issues the rest into a junk area, reading nothing;
// the weight copies of one matrix go to the same waves, gate/up: 0-3 and 4-7),
// and each wave spreads its copies among its MFMAs: the texture addresser takes
// about 16 cycles per 64-lane copy, so copies issued back to back would hold the
// wave. MFMA half s of a step takes, in lane half h, block 2h + s of A and of B.
// Rows past the tile's count, blocks past K and steps past the end are read as
// zero through the resource's range check.
constexpr int kPrefWaves = 8;

template <int NF, bool GATEUP>
struct Prefill {
  static constexpr int W = kPrefWaves;
  static constexpr int BN = 64 * NF;                   // weight rows per workgroup
  static constexpr int NFR = 2 * NF;                   // 32-row weight groups per workgroup
  static constexpr int MROWS = GATEUP ? BN / 2 : BN;   // output columns per workgroup
  static constexpr int FM = GATEUP ? NF / 2 : NF;      // groups per matrix per wave
  static constexpr int NMAT = GATEUP ? 2 : 1;
  static constexpr int GPM = NFR / NMAT;               // groups per matrix
  static constexpr int A_COPIES = kBM * kChunkPieces / 64;
  static constexpr int WPM = W / NMAT;                 // waves copying the weights of one matrix
  static constexpr int B_COPIES = 2 * GPM;             // code copies per matrix
  static constexpr int S_COPIES = GPM / 2;             // scale copies per matrix
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = A_OFF + kBM * kChunk;
  static constexpr int BS_OFF = B_OFF + NFR * 2 * 1024;
  static constexpr int EP_PITCH = 36;                  // floats per row of the SwiGLU staging tile
  static constexpr int EP_BYTES = W * 32 * EP_PITCH * 4;  // epilogue staging of all eight waves
  static constexpr int STAGE_DATA = BS_OFF + NFR * 128;
  // one step's copies, or the epilogue's staging, which reuses a step buffer
  static constexpr int STAGE = EP_BYTES > STAGE_DATA ? EP_BYTES : STAGE_DATA;
  // copy slots per wave: A copies i = wave + 8t, then, for the matrix of the
  // wave (gate/up: waves 0-3 gate, 4-7 up), code copies c = r + WPM t and scale
  // copies p = r + WPM t, r the wave's rank among that matrix's waves (t = 0, 1,
  // ...); slot k numbers them A, code, scale
  static constexpr int NA = (A_COPIES + W - 1) / W;
  static constexpr int NB = (B_COPIES + WPM - 1) / WPM;
  static constexpr int NS = (S_COPIES + WPM - 1) / WPM;
  static constexpr int KB0 = NA, KS0 = NA + NB, KMAX = NA + NB + NS;  // copies per wave per step
  // slots k < KSPLIT go among the 2 NF MFMAs that follow a step barrier (half 1
  // of the step before), the rest among the next 2 NF (half 0 of the step)
  static constexpr int KSPLIT = (KMAX + 1) / 2;
  static_assert(kBM * kChunkPieces % 64 == 0, "A copies are whole instructions");
  static_assert(kBM == 4 * 32, "one 32-row fragment per wave row");
  static_assert(!GATEUP || NF % 2 == 0, "gate/up tiles pair gate and up groups");
  static_assert(GPM % 2 == 0, "scale copies take two groups of one matrix");
  static_assert(2 * KMAX <= 63, "two steps of copies must fit the vector memory counter");
  static_assert(KSPLIT > 0 && KSPLIT < KMAX, "each half step carries copies");
  static_assert(3 * STAGE + 1024 <= 160 * 1024, "three step buffers and the junk area must fit the 160 KB of LDS");
  static_assert(EP_BYTES <= STAGE, "epilogue staging of the eight waves must fit one step buffer");
};

// s_waitcnt with only the vector memory counter bounded (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and lgkmcnt at max),
// and with only the LDS/scalar counter at zero.
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define MOE_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14))

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Buffer resource as four SGPRs (base, stride 0, size in bytes, raw 32-bit
// data): the form the inline-asm copies below take.
__device__ __forceinline__ v4i rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_void_ptr)p);
}
// Buffer-to-LDS copy of SIZE bytes per lane (16 or 4) to the LDS address `lds`
// (wave-uniform); out-of-range lanes write zeros. Written as inline asm so that
// the compiler does not guard every LDS read with a wait for all copies in flight
// (it cannot tell which buffer a copy writes); the kernel bounds the vector
// memory counter itself before each barrier. The LDS address reaches M0 through
// the operand constraint (the compiler sets M0), and the asm has no register outputs.
template <int SIZE>
__device__ __forceinline__ void lds_copy(v4i r, uint32_t lds, uint32_t voff, uint32_t soff) {
  static_assert(SIZE == 16 || SIZE == 4, "copy sizes used here");
  // the resource, M0 and the uniform offset live in SGPRs (no-ops when the
  // compiler already knows the values are uniform)
  r = v4i{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
          __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
  lds = __builtin_amdgcn_readfirstlane(lds);
  soff = __builtin_amdgcn_readfirstlane(soff);
  if constexpr (SIZE == 16)
    asm volatile("buffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "{m0}"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
  else
    asm volatile("buffer_load_dword %1, %2, %3 offen lds"
                 :: "{m0}"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
}

template <int V>
struct IC {
  static constexpr int v = V;
};

// f(IC<I>{}) for I = B .. E-1, in order
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}

template <int NF, bool GATEUP>
__global__ __launch_bounds__(kPrefWaves * 64) void grouped_prefill(const FfnArgs a, const uint8_t* __restrict__ ain,
                                                                   uint8_t* __restrict__ hout,
                                                                   const int4* __restrict__ tiles, int ntn) {
  using C = Prefill<NF, GATEUP>;
  constexpr int W = C::W;
  // the three step buffers (rotated through pointers below)
  __shared__ __attribute__((aligned(16))) uint8_t st0[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[C::STAGE];
  // destination of the copy slots a wave has no copy for (they read nothing)
  __shared__ __attribute__((aligned(16))) uint8_t junk[1024];
  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const int nblkK = K / 32;
  const int nst = nsteps_of(K);

  // ---- persistent schedule. Logical tiles are grouped kPrefGM row tiles x all
  // column tiles, row tile fastest, and each XCD (workgroups are dispatched
  // round-robin over the 8 XCDs) owns a contiguous range of logical tiles, which
  // its workgroups take in turn: the tiles in flight on one XCD at any time are
  // consecutive, so they share a few row tiles of A and a few column tiles of B
  // in that XCD's L2.
  const int total_mt = __builtin_amdgcn_readfirstlane(tiles[0].x);
  const int G = total_mt * ntn;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const int per = G >> 3, rem = G & 7;
  const int xbeg = xcd * per + min(xcd, rem);
  const int xend = xbeg + per + (xcd < rem ? 1 : 0);
  int logical = xbeg + slot;
  if (logical >= xend) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (W - 1);
  const int lane = tid & 63, lr = lane & 31, half = lane >> 5;
  const int wm = wave & 3, wn = wave >> 2;
  const int mw = wave / C::WPM, rw = wave % C::WPM;  // matrix this wave copies, its rank among the copiers
  const uint32_t apitch = (uint32_t)nst * kChunk;
  const uint64_t kmagic = div_magic((uint32_t)a.k);  // token of dispatch pair q: q / k
  const uint32_t gstride = (uint32_t)nst * kWStep;    // packed code bytes per 32-row group
  const uint32_t sstride = (uint32_t)nst * kWSStep;   // packed scale bytes per 32-row group
  const uint32_t lane16 = lane * 16;

  // A copy t of this wave is copy i = wave + 8t: 16-byte pieces 64i + lane, i.e.
  // row (64i + lane) / 13, piece (64i + lane) % 13, the same for every tile and
  // step (recomputed where used). Pieces 6..11 hold blocks 2, 3 of the step.
  auto a_row = [&](int t) -> int { return ((wave + W * t) * 64 + lane) / kChunkPieces; };
  auto a_piece = [&](int t) -> int { return ((wave + W * t) * 64 + lane) % kChunkPieces; };
  // Group gg of matrix m is workgroup group phi (gate/up: wave column w holds
  // NF/2 gate groups, then the NF/2 up groups of the same columns).
  auto group_of = [&](int m, int gg) -> int {
    if (GATEUP) return (gg / (NF / 2)) * NF + m * (NF / 2) + gg % (NF / 2);
    return gg;
  };
  // first weight row of group phi within its matrix, relative to the tile's col0
  auto group_row = [&](int phi) -> int {
    if (GATEUP) {
      const int w = phi / NF, f = phi % NF;
      return w * C::FM * 32 + (f < NF / 2 ? f : f - NF / 2) * 32;
    }
    return phi * 32;
  };
  // Scale copy p of matrix mw covers its groups 2p, 2p+1: lane half h takes
  // group 2p + h; its LDS bytes sit at BS_OFF + 128 (mw GPM + gg).
  auto scale_voff = [&](int p) -> uint32_t {
    return (uint32_t)(group_row(group_of(mw, 2 * p + half)) / 32) * sstride + lr * 4;
  };

  const uint32_t junk_lds = lds_addr(junk);

  // ---- per-tile state (all wave-uniform)
  int e, m0, off, cnt, rows_valid, col0;
  v4i ar, br, bsr;  // A rows; this wave's matrix: codes, scales
  uint32_t a_off[C::NA];  // per-lane A source offsets (step 0)
  float bias[NF], nbias[NF];  // of the tile being computed; of the tile set up last

  // A tile's table entry, column tile, dispatch entries (gate/up: the token of
  // each A copy's row) and raw bf16 biases are fetched ahead of time: the entry
  // two tiles ahead, the rest one tile ahead, each only after the loads it
  // depends on have completed, so fetching never makes this wave wait. R holds
  // everything for the next tile, E the entry of the one after; each is refilled
  // in place right after it has been consumed, so no loaded value is ever copied
  // (a copy would wait for its load).
  struct Pre {
    int4 ent;
    int nt;
    uint32_t src[C::NA];
    uint32_t bias[NF];  // raw bf16 (never combined before use: that would wait for the loads)
  };
  auto fetch_entry = [&](int lg, Pre& P) __attribute__((always_inline)) {
    const int grp = lg / (kPrefGM<GATEUP> * ntn);
    const int gm = min(kPrefGM<GATEUP>, total_mt - grp * kPrefGM<GATEUP>);
    const int r = lg - grp * kPrefGM<GATEUP> * ntn;
    P.nt = r / gm;
    // through the constant address space: scalar loads into SGPRs
    const __attribute__((address_space(4))) int* ct = (const __attribute__((address_space(4))) int*)tiles;
    const int q = 4 * (1 + grp * kPrefGM<GATEUP> + (r - P.nt * gm));
    P.ent = make_int4(ct[q], ct[q + 1], ct[q + 2], ct[q + 3]);
  };
  auto fetch_rest = [&](const Pre& Ein, Pre& P) __attribute__((always_inline)) {
    P.ent = Ein.ent;
    P.nt = Ein.nt;
    const int pe = __builtin_amdgcn_readfirstlane(P.ent.x);
    const int pm0 = __builtin_amdgcn_readfirstlane(P.ent.y), poff = __builtin_amdgcn_readfirstlane(P.ent.z);
    const int rv = min(kBM, __builtin_amdgcn_readfirstlane(P.ent.w) - pm0);
#pragma unroll
    for (int t = 0; t < C::NA; ++t) {
      const int row = min(a_row(t), rv - 1);
      P.src[t] = GATEUP ? (uint32_t)a.sorted_pair[poff + pm0 + row] : (uint32_t)row;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int phi = wn * NF + f;
      const bool upg = GATEUP && f >= NF / 2;
      const uint16_t* bsrc = GATEUP ? (upg ? a.b_up : a.b_gate) : a.b_down;
      P.bias[f] = bsrc[(size_t)pe * N + P.nt * C::MROWS + group_row(phi) + lr];
    }
  };
  auto setup = [&](const Pre& P) __attribute__((always_inline)) {
    e = __builtin_amdgcn_readfirstlane(P.ent.x);
    m0 = __builtin_amdgcn_readfirstlane(P.ent.y);
    off = __builtin_amdgcn_readfirstlane(P.ent.z);
    cnt = __builtin_amdgcn_readfirstlane(P.ent.w);
    rows_valid = min(kBM, cnt - m0);
    col0 = __builtin_amdgcn_readfirstlane(P.nt) * C::MROWS;
    ar = GATEUP ? rsrc4(ain, (uint32_t)a.T * apitch)
                : rsrc4(ain + (size_t)(off + m0) * apitch, (uint32_t)rows_valid * apitch);
    const size_t eb = (size_t)e * (N / 32) * gstride, es = (size_t)e * (N / 32) * sstride;
    br = rsrc4((GATEUP ? (mw ? a.wu_codes : a.wg_codes) : a.wd_codes) + eb, (uint32_t)(N / 32) * gstride);
    bsr = rsrc4((GATEUP ? (mw ? a.wu_scales : a.wg_scales) : a.wd_scales) + es, (uint32_t)(N / 32) * sstride);
#pragma unroll
    for (int t = 0; t < C::NA; ++t) {
      const uint32_t tok = GATEUP ? div_by(P.src[t], kmagic) : P.src[t];
      const bool ok = wave + W * t < C::A_COPIES && a_row(t) < rows_valid;
      a_off[t] = ok ? tok * apitch + a_piece(t) * 16 : kOutOfRange;
    }
  };
  // the biases of the tile P describes (taken with its setup, so P can be
  // refilled right after), added to its accumulators at its end
  auto take_bias = [&](const Pre& P) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < NF; ++f) nbias[f] = bf16_to_f32((uint16_t)P.bias[f]);
  };

  // Copy slot k (see Prefill) of step st of the tile set up last into the LDS
  // buffer at `base`. Weight copies read one contiguous kilobyte: the lane offset
  // is lane*16, the group and step go into the uniform offset. A slot this wave
  // has no copy for, and every copy of a dead step (past K, or after the last
  // tile), read nothing; the former write (zeros) to the junk area.
  auto issue_copy = [&](auto Kc, int st, bool dead, uint32_t base) __attribute__((always_inline)) {
    constexpr int k = decltype(Kc)::v;
    if constexpr (k < C::KB0) {
      constexpr int t = k;
      const bool have = wave + W * t < C::A_COPIES;  // otherwise a_off[t] is out of range
      // the step is past K, or this piece holds its blocks 2, 3 and they are
      const bool pad = dead || (4 * st + 2 >= nblkK && a_piece(t) >= 6 && a_piece(t) < 12);
      lds_copy<16>(ar, have ? base + C::A_OFF + (wave + W * t) * 1024 : junk_lds,
                   pad ? kOutOfRange : a_off[t], (uint32_t)st * kChunk);
    } else if constexpr (k < C::KS0) {
      constexpr int t = k - C::KB0;
      const int c = rw + C::WPM * t;  // code copy: half c & 1 of group c >> 1 of matrix mw
      const bool have = c < C::B_COPIES;
      const int phi = group_of(mw, have ? c >> 1 : 0), sh = c & 1;
      const uint32_t so = (uint32_t)((col0 + group_row(phi)) / 32) * gstride + sh * 1024 + (uint32_t)st * kWStep;
      lds_copy<16>(br, have ? base + C::B_OFF + (phi * 2 + sh) * 1024 : junk_lds,
                   have && !dead ? lane16 : kOutOfRange, so);
    } else {
      constexpr int t = k - C::KS0;
      const int p = rw + C::WPM * t;
      const bool have = p < C::S_COPIES;
      const uint32_t so = (uint32_t)(col0 / 32) * sstride + (uint32_t)st * kWSStep;
      lds_copy<4>(bsr, have ? base + C::BS_OFF + (mw * C::GPM + 2 * p) * 128 : junk_lds,
                  have && !dead ? scale_voff(have ? p : 0) : kOutOfRange, so);
    }
  };
  // Copy slots K0 <= k < K1 of step st into `buf`, back to back. Every wave
  // issues every slot of every step (those past K read nothing), so the number
  // of copies in flight behind a step is the same at every wait.
  auto issue = [&](int st, uint8_t* buf, auto K0c, auto K1c) __attribute__((always_inline)) {
    const uint32_t base = lds_addr(buf);
    static_for<decltype(K0c)::v, decltype(K1c)::v>(
        [&](auto Kc) __attribute__((always_inline)) { issue_copy(Kc, st, st >= nst, base); });
  };

  v16f acc[NF];

  // The fragments of one MFMA half of a step: in lane half h, block 2h + s of A
  // (both terms) and of B; the scale dwords, read with half 0, serve both halves.
  // While one half is computed the other is read: the A terms and the last NSP
  // B groups into the set of registers the half being computed does not use
  // (read first), the other B groups (and with half 0 all B scales) each right
  // after the last MFMA of the running half that reads the registers it
  // overwrites. So the last read of a half is issued a few MFMAs before its end.
  constexpr int NSP = NF < 2 ? NF : 2;  // B groups with a register set per half
  constexpr int FR = NF - NSP;          // B groups read in place
  v8i ah[2], al[2], bf[NF > NSP ? NF - NSP : 1], bsp[2][NSP];
  int sa, sb[NF];
  bool halfst;  // the step's blocks 2, 3 are past K
  auto arow = [&](const uint8_t* buf, int s) __attribute__((always_inline)) {
    return buf + C::A_OFF + (wm * 32 + lr) * kChunk + half * 96 + s * kEncBytes;
  };
  auto ld_b = [&](const uint8_t* buf, int s, int f) __attribute__((always_inline)) {
    return fp4_operand(reinterpret_cast<const v4i*>(buf + C::B_OFF + ((wn * NF + f) * 2 + s) * 1024)[lane]);
  };
  auto ld_sb = [&](const uint8_t* buf, int f) __attribute__((always_inline)) {
    const int m = GATEUP && f >= NF / 2 ? 1 : 0;
    const int gg = GATEUP ? wn * (NF / 2) + f % (NF / 2) : wn * NF + f;
    return (int)reinterpret_cast<const uint16_t*>(buf + C::BS_OFF + (m * C::GPM + gg) * 128)[lane];
  };
  auto rd_sa = [&](const uint8_t* buf, int st) __attribute__((always_inline)) {
    halfst = 4 * st + 2 >= nblkK;
    sa = *reinterpret_cast<const int*>(buf + C::A_OFF + (wm * 32 + lr) * kChunk + kChunkScales + 4 * half);
  };
  // everything of half 0 of step st
  auto read_all = [&](const uint8_t* buf, int st) __attribute__((always_inline)) {
    ah[0] = load_term_hi(arow(buf, 0));
    al[0] = load_term_lo(arow(buf, 0));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f < FR) bf[f] = ld_b(buf, 0, f);
      else bsp[0][f - FR] = ld_b(buf, 0, f);
      sb[f] = ld_sb(buf, f);
    }
    rd_sa(buf, st);
  };
  // 2 x NF scaled MFMAs of half S of a step: the hi terms of all tiles, then the
  // lo terms, so that no MFMA waits on the accumulator of the one just before it.
  // With Z (the tile's first half) the hi MFMAs start from zero.
  // Scale bytes: A hi 2s, A lo 2s+1, B s. A half step at the end of K
  // (K % 128 == 64) still takes both MFMA halves: lane half 0 holds blocks 0, 1
  // (valid), lane half 1 zero codes whose scale bytes (never written) are forced
  // finite. Copy slots K0 <= k < K1 of step cst (into the buffer at cbase; dead
  // with cdead) go evenly among them. With RD, half RS (the other one) of step
  // rst is read from rbuf meanwhile, as described above.
  auto mma_half = [&](auto S, auto K0c, auto K1c, int cst, bool cdead, uint32_t cbase, auto RD, const uint8_t* rbuf,
                      int rst, auto RS, auto Z) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::v, rs = decltype(RS)::v;
    constexpr bool zero = decltype(Z)::v != 0;
    constexpr bool rd = decltype(RD)::v != 0;
    constexpr int k0 = decltype(K0c)::v, k1 = decltype(K1c)::v, nk = k1 - k0;
    constexpr int NM = 2 * NF;
    static_assert(!rd || rs != s, "the other half is read");
    const int sav = halfst && half ? 0 : sa;
    static_for<0, NM>([&](auto Jc) __attribute__((always_inline)) {
      constexpr int j = decltype(Jc)::v;
      constexpr int term = j / NF, f = j % NF;
      const v8i& bop = [&]() -> const v8i& {
        if constexpr (f < FR) return bf[f < FR ? f : 0];
        else return bsp[s][f - FR];
      }();
      acc[f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(term ? al[s] : ah[s], bop, zero && !term ? v16f{} : acc[f],
                                                              2, 4, 2 * s + term, sav, s, sb[f]);
      if constexpr (rd) {
        if constexpr (j == 0) {
          ah[rs] = load_term_hi(arow(rbuf, rs));
          if constexpr (rs == 0) rd_sa(rbuf, rst);
        }
        if constexpr (j == (NM > 1 ? 1 : 0)) al[rs] = load_term_lo(arow(rbuf, rs));
        static_for<0, NSP>([&](auto Ic) __attribute__((always_inline)) {
          constexpr int i = decltype(Ic)::v;
          if constexpr (j == (2 + i < NM ? 2 + i : NM - 1)) bsp[rs][i] = ld_b(rbuf, rs, FR + i);
        });
        if constexpr (term == 1 && f < FR) bf[f < FR ? f : 0] = ld_b(rbuf, rs, f);
        if constexpr (term == 1 && rs == 0) sb[f] = ld_sb(rbuf, f);
      }
      static_for<k0, k1>([&](auto Kc) __attribute__((always_inline)) {
        constexpr int k = decltype(Kc)::v;
        if constexpr (nk > 0 && (k - k0) * NM / nk == j) issue_copy(Kc, cst, cdead, cbase);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- first tile (its fetches wait; later tiles' do not)
  Pre R, E;
  bool more = logical + nslot < xend, more2 = logical + 2 * nslot < xend;
  {
    Pre e0, p0, e1;
    fetch_entry(logical, e0);
    if (more) fetch_entry(logical + nslot, e1);
    if (more2) fetch_entry(logical + 2 * nslot, E);
    fetch_rest(e0, p0);
    if (more) fetch_rest(e1, R);
    setup(p0);
    take_bias(p0);
#pragma unroll
    for (int f = 0; f < NF; ++f) bias[f] = nbias[f];
  }
  issue(0, st0, IC<0>{}, IC<C::KMAX>{});
  issue(1, st1, IC<0>{}, IC<C::KMAX>{});

  // Wait until step st+1 has landed (step st+2 may be in flight) and every wave
  // has completed its reads of step st (barrier).
  auto step_barrier = [&]() __attribute__((always_inline)) {
    MOE_WAIT_VMCNT(C::KMAX);
    MOE_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves across the barrier
    __builtin_amdgcn_sched_barrier(0);
  };
  // X_{st-1} to X_st (straight-line code: a branch inside would let the
  // compiler move MFMAs across a barrier), copying step cst (dead with cdead)
  // into c2
  auto period = [&](int st, uint8_t* c0, uint8_t* c2, int cst, bool cdead) __attribute__((always_inline)) {
    const uint32_t cb = lds_addr(c2);
    mma_half(IC<1>{}, IC<0>{}, IC<C::KSPLIT>{}, cst, cdead, cb, IC<1>{}, c0, st, IC<0>{}, IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
    mma_half(IC<0>{}, IC<C::KSPLIT>{}, IC<C::KMAX>{}, cst, cdead, cb, IC<1>{}, c0, st, IC<1>{}, IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
    step_barrier();
  };

  // The three step buffers rotate: at a tile's start bx, by, bz hold its steps
  // 0, 1, 2, and each step moves them on by one, so after the tile they hold
  // steps nst, nst+1, nst+2, i.e. the next tile's 0, 1, 2.
  uint8_t *bx = st0, *by = st1, *bz = st2;
  auto rot = [&]() __attribute__((always_inline)) {
    uint8_t* const tmp = bx;
    bx = by;
    by = bz;
    bz = tmp;
  };
  // With three or more steps per tile the next tile's first two steps are
  // copied among the MFMAs of this tile's last two (hand-over), so their first
  // round trip is hidden; otherwise they are copied after the tile.
  const bool handover = nst >= 3;
  int c_off, c_m0, c_cnt, c_rows, c_col0;  // the output coordinates of the tile being computed
  auto save_coords = [&]() __attribute__((always_inline)) {
    c_off = off;
    c_m0 = m0;
    c_cnt = cnt;
    c_rows = rows_valid;
    c_col0 = col0;
  };

  for (;;) {
    // ---- main loop. Step st lives in buffer st % 3 of the rotation. Barrier
    // X_st comes between the two MFMA halves of step st: before it, the MFMAs of
    // half 0 of step st read half 1 of st; after it, those of half 1 read half 0
    // of step st+1, which X_st certifies has landed. Step st+2 is copied into the
    // buffer of step st-1 (free since X_{st-1}) among the MFMAs between X_{st-1}
    // and X_st. The wavefront that reaches a barrier first has its next operands
    // in registers, so the matrix unit idles only while the barrier collects the
    // waves.
    save_coords();
    // step 0 has landed (step 1 may be in flight); every wave is done with the
    // previous tile's epilogue staging in bz
    MOE_WAIT_VMCNT(C::KMAX);
    MOE_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    read_all(bx, 0);
    __builtin_amdgcn_sched_barrier(0);
    // up to X_0: half 0 of step 0, all copies of step 2
    mma_half(IC<0>{}, IC<0>{}, IC<C::KMAX>{}, 2, nst <= 2, lds_addr(bz), IC<1>{}, bx, 0, IC<1>{}, IC<1>{});
    // (the empty asm keeps these MFMAs ahead of the barrier)
#pragma unroll
    for (int f = 0; f < NF; ++f) asm volatile("" : "+v"(acc[f]));
    __builtin_amdgcn_sched_barrier(0);
    step_barrier();
    rot();
    // steps 1 .. nst-3, copying steps 3 .. nst-1; then steps nst-2, nst-1,
    // which with the hand-over copy the next tile's steps 0 and 1 (set up
    // first), otherwise nothing. Loops, so that the operands carried from one
    // step to the next keep their registers.
    for (int t = 1; t + 2 < nst; ++t) {
      period(t, bx, bz, t + 2, false);
      rot();
    }
    if (handover && more) {
      setup(R);
      take_bias(R);
    }
    for (int t = max(1, nst - 2); t < nst; ++t) {
      period(t, bx, bz, t + 2 - nst, !(handover && more));
      rot();
    }
    // half 1 of the last step; the empty asm keeps its MFMAs here (left alone,
    // the compiler sinks them past the next tile's copies, where their operands
    // would take registers the copies' setup needs)
    mma_half(IC<1>{}, IC<0>{}, IC<0>{}, 0, true, 0u, IC<0>{}, bx, 0, IC<0>{}, IC<0>{});
#pragma unroll
    for (int f = 0; f < NF; ++f) asm volatile("" : "+v"(acc[f]));
    __builtin_amdgcn_sched_barrier(0);

    // ---- without the hand-over, the next tile's first two steps are copied
    // now, while this tile's epilogue runs. The epilogue stages through bz, the
    // buffer of this tile's last step, which no copy targets before the next
    // tile's barrier. The fetches for the tiles after the next are issued after
    // the epilogue and complete while the next tile is computed.
    if (!handover) {
      MOE_WAIT_VMCNT(0);
      __syncthreads();
      if (more) {
        setup(R);
        take_bias(R);
        issue(0, bx, IC<0>{}, IC<C::KMAX>{});
        issue(1, by, IC<0>{}, IC<C::KMAX>{});
      }
    }
    const bool more3 = logical + 3 * nslot < xend;

    if constexpr (GATEUP) {
      // h = silu(g) * u; per gate group f, the wave's 32x32 tile goes to LDS as
      // 32 rows x 32 columns, the even columns of a row first and then the odd
      // ones (the conversions' operand order), and lanes 0..31 each encode one
      // row's 32-column block as two-term MXFP6 into the row's step chunk.
      float* ep = reinterpret_cast<float*>(bz) + wave * 32 * C::EP_PITCH;
      const uint32_t hpitch = (uint32_t)nsteps_of(a.F) * kChunk;
      const int grow = c_m0 + wm * 32 + lane;
#pragma unroll
      for (int f = 0; f < C::FM; ++f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rr = 8 * (i >> 2) + 4 * half + (i & 3);
          const float g = acc[f][i] + bias[f], u = acc[f + C::FM][i] + bias[f + C::FM];
          ep[rr * C::EP_PITCH + (lr & 1) * 16 + (lr >> 1)] = g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < 32) {
          const v16f* src = reinterpret_cast<const v16f*>(ep + lane * C::EP_PITCH);
          uint32_t hw[6], lw[6], sc;
          encode_block_eo(src[0], src[1], hw, lw, sc);
          if (grow < c_cnt) {
            const int b = (c_col0 + wn * C::FM * 32 + f * 32) / 32;
            uint8_t* hrow = hout + (size_t)(c_off + grow) * hpitch;
            store_enc(hrow + enc_codes_at(b), hw, lw);
            *reinterpret_cast<uint16_t*>(hrow + enc_scale_at(b)) = static_cast<uint16_t>(sc);
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    } else {
      // y = the fp32 accumulators plus bias, staged per 32-column group through
      // LDS (bz) so that each lane
      // stores 16 contiguous bytes: store q of a wave writes 8 whole rows of the
      // group (8 lanes x 16 B per row) instead of 64 single floats.
      float* ep = reinterpret_cast<float*>(bz) + wave * 32 * C::EP_PITCH;
      const int srow = lane >> 3, scol = (lane & 7) * 4;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rr = 8 * (i >> 2) + 4 * half + (i & 3);
          ep[rr * C::EP_PITCH + lr] = acc[f][i] + bias[f];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 8 * q + srow;  // row within the wave's 32
          const float4 v = *reinterpret_cast<const float4*>(ep + r * C::EP_PITCH + scol);
          // non-temporal: y is read once, by the combine, after the GEMM
          if (wm * 32 + r < c_rows)
            __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w},
                                        reinterpret_cast<v4f*>(a.y_sorted + (size_t)(c_off + c_m0 + wm * 32 + r) * N +
                                                               c_col0 + wn * NF * 32 + f * 32 + scol));
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    if (!more) break;
#pragma unroll
    for (int f = 0; f < NF; ++f) bias[f] = nbias[f];
    if (more2) fetch_rest(E, R);
    if (more3) fetch_entry(logical + 3 * nslot, E);
    logical += nslot;
    more = more2;
    more2 = more3;
  }
}

// ------------------------------------------------------------------ decode

// Weight streaming for few rows per expert, persistent. The work is a list of
// items (expert pass, column group): a pass is up to 16 dispatch rows of one
// expert (the decode tile table), a column group is 32 h-columns for gate/up
// -- waves 0,1 stream the two 16-row halves of the gate group, waves 2,3 those
// of the up group -- or 64 output columns for down -- wave w streams the 16-row
// half w&1 of group 2j + w/2. Each workgroup takes every G-th item of the list.
// Each wavefront uses the 16x16x128 scaled MFMA (16 rows = one pass) over the
// whole of K, in stages of kDecSS steps, fully unrolled (NSTAGE stages, a
// multiple of the ring depth so the ring continues from one item to the next):
// the weight codes and the activation window of stage s+kDecPF are issued while
// stage s is computed, held in a register ring, and the window is copied to LDS
// one stage before it is read, so the activations are read from L2 once per
// workgroup. The last kDecPF stages of an item issue the first stages of the
// workgroup's next item, whose table entry, dispatch entries, bias and packed
// weight scales were fetched one item ahead (the entry two items ahead): the
// weight stream never drains between items. Loads are issued in the order they
// are consumed, so waiting for one never waits for a younger one. All global
// reads are buffer loads: blocks past K and rows past the count read as zero.
// The weights, read once, are loaded non-temporal (nt), which measured 5.7% (gate/up)
// and 10% (down) faster on decode-20b than cached loads.
//
// 16x16x128 layout (checked on gfx950): lane l supplies row/column l%16 and K
// elements 32*(l/16) .. +31 of the step; result lane l holds column l%16, rows
// 4*(l/16) + i, i = 0..3.

template <int OPA>
__device__ __forceinline__ v4f mfma16_f6f4(const v8i& a, const v8i& b, const v4f& c, int sa,
                                           int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 2, 4, OPA, sa, 0, sb);
}

constexpr int kDecSS = 4;                            // 128-deep steps per stage
constexpr int kDecPF = 2;                            // stages of loads in flight ahead of the one computed
constexpr int kDecMaxSteps = 32;                     // decode kernels cover K <= 32 * 128
constexpr int kDecAPitch = kDecSS * kChunk + 16;     // LDS bytes per activation row (padded: no bank conflicts)
constexpr int kDecAPieces = kDecRows * kDecSS * kChunkPieces;  // 16-byte pieces of one stage's window
constexpr int kDecAPerT = (kDecAPieces + 255) / 256;     // ... per thread (at most)
static_assert(kDecMaxSteps * kWSStep / 16 <= 256, "one scale piece per thread and group");

template <bool GATEUP, int NSTAGE>
__global__ __launch_bounds__(256, 2) void grouped_decode(const FfnArgs a, const uint8_t* __restrict__ ain,
                                                         uint8_t* __restrict__ hout,
                                                         const int4* __restrict__ passes) {
  constexpr int COLS = GATEUP ? 32 : 64;  // output columns per item
  constexpr int PF = kDecPF;
  static_assert(NSTAGE % (PF + 1) == 0, "the ring continues across items");
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kDecRows * kDecAPitch];
  // packed weight scales of an item's two groups, by item parity: [item&1][group][step][lane] uint16
  __shared__ __attribute__((aligned(16))) uint16_t sBs[2][2 * kDecMaxSteps * 64];
  __shared__ __attribute__((aligned(16))) float gtile[GATEUP ? 2 * kDecRows * 36 : 4];

  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const int nblkK = K / 32;
  const int nst = nsteps_of(K);      // 128-deep steps (the last may be half: K % 128 == 64)
  const int ncol = N / COLS;
  const int nitems = __builtin_amdgcn_readfirstlane(passes[0].x) * ncol;
  const int G = gridDim.x;
  int item = blockIdx.x;
  if (item >= nitems) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int lane = tid & 63, l16 = lane & 15, q = lane >> 4;
  const int sub = wave & 1;                          // 16-row half of the group
  const bool up = GATEUP && wave >= 2;
  const uint32_t apitch = (uint32_t)nst * kChunk;
  const uint32_t gstride = (uint32_t)nst * kWStep, sstride = (uint32_t)nst * kWSStep;
  const uint64_t kmagic = div_magic((uint32_t)a.k);  // token of dispatch pair q: q / k
  // lane (column l16, K sub-block q): half q&1, lane 32*(q/2) + 16*sub + l16 of the packed step
  const uint32_t wl = (uint32_t)(q & 1) * 1024 + (uint32_t)((q >> 1) * 32 + 16 * sub + l16) * 16;
  const uint8_t* codes = GATEUP ? (up ? a.wu_codes : a.wg_codes) : a.wd_codes;
  const uint16_t* bias_src = GATEUP ? (up ? a.b_up : a.b_gate) : a.b_down;
  const rsrc_t ar_x = make_rsrc(ain, (uint32_t)a.T * apitch);

  // window piece c = tid + 256i: row c / 52, step u = (c % 52) / 13, piece c % 13
  int alds[kDecAPerT], au[kDecAPerT], ap[kDecAPerT], arw[kDecAPerT];
#pragma unroll
  for (int i = 0; i < kDecAPerT; ++i) {
    const int c = tid + 256 * i;
    arw[i] = c / (kDecSS * kChunkPieces);
    const int rem = c - arw[i] * (kDecSS * kChunkPieces);
    au[i] = rem / kChunkPieces;
    ap[i] = rem - au[i] * kChunkPieces;
    alds[i] = arw[i] * kDecAPitch + au[i] * kChunk + ap[i] * 16;
  }

  // ---- what an item needs, fetched ahead: the table entry (two items ahead),
  // then (one item ahead) the dispatch entries of the window rows, the bias of
  // this lane's column and the packed scales of the item's two groups
  struct Ahead {
    int4 ent;          // {expert, first row within the expert, offsets[e], count_e}
    int j;             // column group
    uint32_t src[kDecAPerT];
    uint32_t bias;
    uint4 bs0, bs1;
  };
  auto fetch_entry = [&](int it, Ahead& A) {
    A.j = it % ncol;
    A.ent = passes[1 + it / ncol];
  };
  auto fetch_rest = [&](Ahead& A) {
    const int e = __builtin_amdgcn_readfirstlane(A.ent.x);
    const int m0 = __builtin_amdgcn_readfirstlane(A.ent.y), off = __builtin_amdgcn_readfirstlane(A.ent.z);
    const int rows = min(kDecRows, __builtin_amdgcn_readfirstlane(A.ent.w) - m0);
    const int j = A.j;
#pragma unroll
    for (int i = 0; i < kDecAPerT; ++i) {
      const int r = min(arw[i], rows - 1);
      A.src[i] = GATEUP ? (uint32_t)a.sorted_pair[off + m0 + r] : (uint32_t)(off + m0 + r);
    }
    const int g = GATEUP ? j : 2 * j + (wave >> 1);
    A.bias = bias_src[(size_t)e * N + 32 * g + 16 * sub + l16];
    const uint8_t* s0 = (GATEUP ? a.wg_scales : a.wd_scales) + ((size_t)e * (N / 32) + (GATEUP ? j : 2 * j)) * sstride;
    const uint8_t* s1 = GATEUP ? a.wu_scales + ((size_t)e * (N / 32) + j) * sstride : s0 + sstride;
    const uint32_t o = tid < nst * (kWSStep / 16) ? (uint32_t)tid * 16 : kOutOfRange;
    A.bs0 = bload16(make_rsrc(s0, sstride), o);
    A.bs1 = bload16(make_rsrc(s1, sstride), o);
  };

  // ---- the item being issued (its weight resource and window offsets)
  struct Issue {
    rsrc_t wr, ar;
    uint32_t arow[kDecAPerT];
  };
  auto make_issue = [&](const Ahead& A, Issue& I) {
    const int e = __builtin_amdgcn_readfirstlane(A.ent.x);
    const int m0 = __builtin_amdgcn_readfirstlane(A.ent.y);
    const int rows = min(kDecRows, __builtin_amdgcn_readfirstlane(A.ent.w) - m0);
    const int g = GATEUP ? A.j : 2 * A.j + (wave >> 1);
    I.wr = make_rsrc(codes + ((size_t)e * (N / 32) + g) * gstride, gstride);
    I.ar = GATEUP ? ar_x : make_rsrc(ain, (uint32_t)(a.T * a.k) * apitch);
#pragma unroll
    for (int i = 0; i < kDecAPerT; ++i) {
      const int c = tid + 256 * i;
      const bool ok = c < kDecAPieces && arw[i] < rows;
      const uint32_t row = GATEUP ? div_by(A.src[i], kmagic) : A.src[i];
      I.arow[i] = ok ? row * apitch + (uint32_t)(au[i] * kChunk + ap[i] * 16) : kOutOfRange;
    }
  };

  // One ring slot: the weights of a stage and the activation window of the
  // stage after it. The window is copied to LDS at the end of the stage before
  // the one that reads it, so it travels in the batch of loads of that earlier
  // stage: copying it then never waits for loads younger than the ones the
  // stage just computed already needed (the vector memory counter retires in
  // order).
  struct Packet {
    uint4 w[kDecSS];              // weight codes (MFMA B operand, this lane)
    uint4 a[kDecAPerT];           // activation window pieces of the next stage (staged to LDS)
  };
  // Stage st of an item: the step's distance along K goes into the uniform
  // buffer offset, so the per-lane offsets are the same in every stage. In a
  // half step at the end of K the lanes of sub-blocks 2, 3 read nothing.
  auto issue_w = [&](const Issue& I, int st, Packet& pk) {
#pragma unroll
    for (int u = 0; u < kDecSS; ++u) {
      const int jj = st * kDecSS + u;
      const bool live = jj < nst && (4 * jj + 2 < nblkK || q < 2);
      pk.w[u] = bload16nt(I.wr, live ? wl : kOutOfRange, (uint32_t)jj * kWStep);
    }
  };
  auto issue_a = [&](const Issue& I, int st, uint4 (&dst)[kDecAPerT]) {
#pragma unroll
    for (int i = 0; i < kDecAPerT; ++i) {
      const int jj = st * kDecSS + au[i];
      const bool pad = 4 * jj + 2 >= nblkK && ap[i] >= 6 && ap[i] < 12;
      dst[i] = bload16(I.ar, jj < nst && !pad ? I.arow[i] : kOutOfRange, (uint32_t)(st * kDecSS) * kChunk);
    }
  };
  auto stage_to_lds = [&](const uint4 (&win)[kDecAPerT], int buf) {
#pragma unroll
    for (int i = 0; i < kDecAPerT; ++i)
      if (tid + 256 * i < kDecAPieces) *reinterpret_cast<uint4*>(sA[buf] + alds[i]) = win[i];
  };
  auto scales_to_lds = [&](const Ahead& A, int par) {
    if (tid < nst * (kWSStep / 16)) {
      *reinterpret_cast<uint4*>(sBs[par] + tid * 8) = A.bs0;
      *reinterpret_cast<uint4*>(sBs[par] + kDecMaxSteps * 64 + tid * 8) = A.bs1;
    }
  };

  // ---- prologue: the first item's data (these fetches wait), the next item's
  // rest and the entry of the one after
  Ahead cur, nxt, nn;
  bool has1 = item + G < nitems, has2 = item + 2 * G < nitems;
  fetch_entry(item, cur);
  if (has1) fetch_entry(item + G, nxt);
  if (has2) fetch_entry(item + 2 * G, nn);
  fetch_rest(cur);
  if (has1) fetch_rest(nxt);
  Issue ic, in;
  make_issue(cur, ic);
  Packet ring[PF + 1];
  {
    uint4 win0[kDecAPerT];
    issue_a(ic, 0, win0);
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      issue_w(ic, p, ring[p]);
      if (p + 1 < NSTAGE) issue_a(ic, p + 1, ring[p].a);
    }
    scales_to_lds(cur, 0);
    stage_to_lds(win0, 0);
  }
  __syncthreads();

  for (int n = 0;; ++n) {
    const int par = n & 1;
    const int m0 = __builtin_amdgcn_readfirstlane(cur.ent.y);
    const int off = __builtin_amdgcn_readfirstlane(cur.ent.z);
    const int rows = min(kDecRows, __builtin_amdgcn_readfirstlane(cur.ent.w) - m0);
    const int j = cur.j;
    const int pb = (n * NSTAGE) & 1;  // window buffer of this item's stage 0
    // two accumulators (hi and lo terms), so consecutive MFMAs do not depend on
    // each other; summed once at the end of the item
    v4f acc, acc2 = v4f{0.f, 0.f, 0.f, 0.f};
    {
      const float b = bf16_to_f32((uint16_t)cur.bias);
      acc = v4f{b, b, b, b};
    }
    const uint16_t* bsrow = sBs[par] + (wave >> 1) * kDecMaxSteps * 64 + (q >> 1) * 32 + 16 * sub + l16;
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st) {
      // slot of stage st + PF: its weights and the window of the stage after it,
      // of this item or of the next
      if (st == NSTAGE - PF - 1 && has1) make_issue(nxt, in);
      Packet& pn = ring[(st + PF) % (PF + 1)];
      if (st + PF < NSTAGE) issue_w(ic, st + PF, pn);
      else if (has1) issue_w(in, st + PF - NSTAGE, pn);
      if (st + PF + 1 < NSTAGE) issue_a(ic, st + PF + 1, pn.a);
      else if (has1) issue_a(in, st + PF + 1 - NSTAGE, pn.a);
      const Packet& pc = ring[st % (PF + 1)];
      const uint8_t* wbuf = sA[(pb + st) & 1];
#pragma unroll
      for (int u = 0; u < kDecSS; ++u) {
        const int jj = st * kDecSS + u;
        if (jj < nst) {
          const uint8_t* rowp = wbuf + l16 * kDecAPitch + u * kChunk;
          v8i ahi, alo;
          load_block_terms3(rowp + q * kEncBytes, ahi, alo);
          int as = *reinterpret_cast<const uint16_t*>(rowp + kChunkScales + 2 * q);
          if (4 * jj + 2 >= nblkK && q >= 2) as = 0;  // blocks past K: zero codes, finite scales
          const int bs = bsrow[jj * 64] >> (8 * (q & 1));
          const v8i b = fp4_operand(v4i{(int)pc.w[u].x, (int)pc.w[u].y, (int)pc.w[u].z, (int)pc.w[u].w});
          acc = mfma16_f6f4<0>(ahi, b, acc, as, bs);
          acc2 = mfma16_f6f4<1>(alo, b, acc2, as, bs);
        }
      }
      if (st == NSTAGE - 1 && has1) scales_to_lds(nxt, par ^ 1);
      if (st + 1 < NSTAGE || has1) stage_to_lds(pc.a, (pb + st + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue of this item (the next item's first stages are in flight)
    acc += acc2;
    if constexpr (GATEUP) {
      // waves 0,1 hold g, waves 2,3 hold u for the same 16 rows x 32 columns;
      // all 256 threads form h = silu(g) * u in place of g, two elements each
      // (one lane per row doing all 32 took ~3,000 cycles with the matrix
      // work of the next item waiting on it: decode-20b's gate/up launch went
      // from 48.0 to 45.3-46.2 us), then one lane per row encodes the row's
      // 32-column block of h
      float* t = gtile + (wave >> 1) * kDecRows * 36;
#pragma unroll
      for (int i = 0; i < 4; ++i) t[(4 * q + i) * 36 + sub * 16 + l16] = acc[i];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kDecRows * 32 / 256; ++i) {
        const int el = tid + 256 * i, r = el >> 5, c = el & 31;
        gtile[r * 36 + c] = silu_mul(gtile[r * 36 + c], gtile[kDecRows * 36 + r * 36 + c]);
      }
      __syncthreads();
      if (tid < rows) {
        float v[32];
        const float4* g4 = reinterpret_cast<const float4*>(gtile + tid * 36);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float4 gg = g4[c];
          v[4 * c] = gg.x;
          v[4 * c + 1] = gg.y;
          v[4 * c + 2] = gg.z;
          v[4 * c + 3] = gg.w;
        }
        uint32_t hw[6], lw[6], sc;
        encode_block(v, hw, lw, sc);
        uint8_t* hrow = hout + (size_t)(off + m0 + tid) * enc_pitch(a.F);
        store_enc(hrow + enc_codes_at(j), hw, lw);
        *reinterpret_cast<uint16_t*>(hrow + enc_scale_at(j)) = static_cast<uint16_t>(sc);
      }
    } else {
      const int nout = 32 * (2 * j + (wave >> 1)) + 16 * sub + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < rows) a.y_sorted[(size_t)(off + m0 + 4 * q + i) * N + nout] = acc[i];
    }
    if (!has1) break;
    // advance: nxt becomes current; its rest was fetched one item ago, the
    // entry after it two items ago
    const bool has3 = item + 3 * G < nitems;
    item += G;
    cur = nxt;
    ic = in;
    if (has2) {
      nxt = nn;
      fetch_rest(nxt);
    }
    if (has3) fetch_entry(item + 2 * G, nn);
    has1 = has2;
    has2 = has3;
  }
}

// ------------------------------------------------------------------ host side

template <int NF, bool GATEUP>
hipError_t launch_prefill(const FfnArgs& a, const uint8_t* ain, uint8_t* hout, const int4* tp,
                          int ncu, hipStream_t stream) {
  const int N = GATEUP ? a.F : a.d;
  const int ntn = N / Prefill<NF, GATEUP>::MROWS;
  // persistent: one workgroup of eight waves per CU (the LDS holds one), 8 per XCD at least
  const long long tiles_max = (long long)max_row_tiles(a.T, a.E, a.k, kBM) * ntn;
  long long grid = ncu < tiles_max ? ncu : tiles_max;
  grid = grid < 8 ? 8 : grid & ~7LL;
  hipLaunchKernelGGL((grouped_prefill<NF, GATEUP>), dim3((unsigned)grid), dim3(kPrefWaves * 64), 0, stream, a,
                     ain, hout, tp, ntn);
  return hipGetLastError();
}

template <bool GATEUP, int NSTAGE>
hipError_t launch_decode_n(const FfnArgs& a, const uint8_t* ain, uint8_t* hout, const int4* passes,
                           int ncu, hipStream_t stream) {
  const int N = GATEUP ? a.F : a.d;
  const long long items_max = (long long)max_row_tiles(a.T, a.E, a.k, kDecRows) * (N / (GATEUP ? 32 : 64));
  int occ = 0;
  hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, grouped_decode<GATEUP, NSTAGE>, 256, 0);
  if (err != hipSuccess) return err;
  long long grid = (long long)ncu * (occ > 0 ? occ : 1);
  if (grid > items_max) grid = items_max;
  hipLaunchKernelGGL((grouped_decode<GATEUP, NSTAGE>), dim3((unsigned)grid), dim3(256), 0, stream, a, ain,
                     hout, passes);
  return hipGetLastError();
}

// Stages of kDecSS steps, rounded up to a multiple of the ring depth.
int decode_stages(int K) {
  const int s = (nsteps_of(K) + kDecSS - 1) / kDecSS;
  return (s + kDecPF) / (kDecPF + 1) * (kDecPF + 1);
}

// Stage counts M * (kDecPF + 1) for M = 1 .. (enough for kDecMaxSteps).
constexpr int kDecMaxM = ((kDecMaxSteps + kDecSS - 1) / kDecSS + kDecPF) / (kDecPF + 1);
template <bool GATEUP, int M>
hipError_t launch_decode_m(int nstage, const FfnArgs& a, const uint8_t* ain, uint8_t* hout,
                           const int4* passes, int ncu, hipStream_t stream) {
  if constexpr (M == 0) {
    return hipErrorInvalidValue;  // callers route K beyond this to the prefill kernel
  } else {
    if (nstage == M * (kDecPF + 1))
      return launch_decode_n<GATEUP, M * (kDecPF + 1)>(a, ain, hout, passes, ncu, stream);
    return launch_decode_m<GATEUP, M - 1>(nstage, a, ain, hout, passes, ncu, stream);
  }
}

template <bool GATEUP>
hipError_t launch_decode(const FfnArgs& a, const uint8_t* ain, uint8_t* hout, const int4* passes, int ncu,
                         hipStream_t stream) {
  return launch_decode_m<GATEUP, kDecMaxM>(decode_stages(GATEUP ? a.d : a.F), a, ain, hout, passes, ncu,
                                            stream);
}

bool decode_fits(int K) { return nsteps_of(K) <= kDecMaxSteps; }

}  // namespace

size_t ffn_workspace_bytes(int T, int d, int F, int E, int k) {
  return ws_layout(T, d, F, E, k).total;
}

bool ffn_decode_shape(int T, int d, int F) {
  return T <= kDecodeMaxT && decode_fits(d) && decode_fits(F);
}

// The prefill down GEMM tiles the output columns by 320, 192 or 128; a width
// that none of them divides (d = 64 mod 128 and a multiple of neither 192 nor
// 320) takes the weight-streaming kernel at any T.
bool ffn_down_decode(int T, int d, int F) {
  const bool no_tile = d % 320 != 0 && d % 192 != 0 && d % 128 != 0;
  return decode_fits(F) && (T <= kDecodeMaxT || no_tile);
}

bool ffn_supported(int T, int d, int F) {
  const bool no_tile = d % 320 != 0 && d % 192 != 0 && d % 128 != 0;
  return !(T > kDecodeMaxT && no_tile && !decode_fits(F));
}

hipError_t launch_expert_ffn_stage(const FfnArgs& a, hipStream_t stream, int stage, bool front_done) {
  const WsLayout L = ws_layout(a.T, a.d, a.F, a.E, a.k);
  int dev = 0, ncu = 0;
  hipError_t qerr = hipGetDevice(&dev);
  if (qerr == hipSuccess) qerr = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (qerr != hipSuccess) return qerr;
  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  uint8_t* xenc = ws + L.x;
  uint8_t* henc = ws + L.h;
  int4* tp = reinterpret_cast<int4*>(ws + L.tiles);

  // Per GEMM: the weight-streaming decode kernel for few rows per expert and K
  // it can unroll, the LDS-tiled kernel otherwise (both read/write the same
  // encoded layouts, so they can be mixed).
  const bool dec_gu = a.T <= kDecodeMaxT && decode_fits(a.d);
  const bool dec_dn = ffn_down_decode(a.T, a.d, a.F);
  int4* pp = reinterpret_cast<int4*>(ws + L.passes);
  const TableJob tj{a.offsets, a.E, (!dec_gu || !dec_dn) ? tp : nullptr, (dec_gu || dec_dn) ? pp : nullptr};

  if (stage == 0) {
    // x is encoded once; one extra workgroup of the same launch builds the tables
    // (or the whole-block call's front end has done both)
    if (front_done) return hipSuccess;
    // the decode-sized encoder (cooperative, short latency) for T <= 64, the
    // one-block-per-thread encoder (the many-token router's) otherwise
    const int nx = a.T * (a.d / 32);
    if (a.T <= kDecodeMaxT)
      hipLaunchKernelGGL(encode_rows, dim3((nx + 7) / 8 + 1), dim3(256), 0, stream, a.x, a.T, a.d, xenc, tj);
    else
      hipLaunchKernelGGL(encode_rows_thread, dim3((nx + 255) / 256 + 1), dim3(256), 0, stream, a.x, a.T,
                         a.d, xenc, tj);
    return hipGetLastError();
  }
  if (stage == 1) {
    // Column tiles: the widest that divides N (gate/up: 32*NF h-columns, down:
    // 64*NF output columns per workgroup) -- for gate/up only while that many
    // tiles, at the most the row tiles can be, still give every CU one;
    // otherwise the 64-column tile, so that few rows spread over more CUs
    // (measured at T = 128, d = F = 512: 33.0 -> 31.5 us per layer). The tile
    // width does not change any output's summation order.
    if (dec_gu) return launch_decode<true>(a, xenc, henc, pp, ncu, stream);
    const long long mts = max_row_tiles(a.T, a.E, a.k, kBM);
    if (a.F % 192 == 0 && mts * (a.F / 192) >= ncu) return launch_prefill<6, true>(a, xenc, henc, tp, ncu, stream);
    if (a.F % 128 == 0 && mts * (a.F / 128) >= ncu) return launch_prefill<4, true>(a, xenc, henc, tp, ncu, stream);
    return launch_prefill<2, true>(a, xenc, henc, tp, ncu, stream);
  }
  if (stage == 2) {
    if (dec_dn) return launch_decode<false>(a, henc, henc, pp, ncu, stream);
    if (a.d % 320 == 0) return launch_prefill<5, false>(a, henc, henc, tp, ncu, stream);
    if (a.d % 192 == 0) return launch_prefill<3, false>(a, henc, henc, tp, ncu, stream);
    if (a.d % 128 == 0) return launch_prefill<2, false>(a, henc, henc, tp, ncu, stream);
    return hipErrorInvalidValue;   // rejected by ffn_supported
  }
  return hipErrorInvalidValue;
}

uint8_t* ffn_xenc(const FfnArgs& a) {
  return static_cast<uint8_t*>(a.ws) + ws_layout(a.T, a.d, a.F, a.E, a.k).x;
}

int4* ffn_tiles(const FfnArgs& a) {
  return reinterpret_cast<int4*>(static_cast<uint8_t*>(a.ws) + ws_layout(a.T, a.d, a.F, a.E, a.k).tiles);
}

int4* ffn_passes(const FfnArgs& a) {
  return reinterpret_cast<int4*>(static_cast<uint8_t*>(a.ws) + ws_layout(a.T, a.d, a.F, a.E, a.k).passes);
}

void* ffn_ws_end(const FfnArgs& a) {
  return static_cast<uint8_t*>(a.ws) + ws_layout(a.T, a.d, a.F, a.E, a.k).total;
}

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream, bool front_done) {
  for (int stage = 0; stage < 3; ++stage) {
    const hipError_t err = launch_expert_ffn_stage(a, stream, stage, front_done);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
