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
//   prefill  128-row x (64*NF)-column output tiles per workgroup, 2x2 wavefronts,
//            A and B staged through LDS in 64-deep K steps (double buffered, rows
//            padded so the fragment reads are bank-conflict free). The grid is an
//            upper bound on the number of (row tile, column tile) pairs; a tile
//            table built on the device maps a workgroup to its expert, and
//            surplus workgroups exit. Workgroup ids are remapped so each XCD
//            (dispatch is round-robin over the 8 XCDs) works on a contiguous
//            range of tiles, sharing A rows and expert weights in its own L2.
//   decode   weight streaming for few rows per expert: one workgroup per
//            (expert, 32 output columns), the four wavefronts split K, stream the
//            weights straight from HBM into MFMA registers, and reduce their
//            partial tiles through LDS in fixed order (deterministic).
#include "mx6.hpp"

namespace moe {
namespace {

constexpr int kBM = 128;        // rows per prefill tile
constexpr int kAPitch = 104;    // LDS bytes per A row per K step: 2 blocks x 48 B + 8 pad
constexpr int kBPitch = 40;     // LDS bytes per B row per K step: 2 blocks x 16 B + 8 pad
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

template <int NF, bool GATEUP>
struct Prefill {
  static constexpr int BNB = 2 * NF * 32;  // B rows (weight rows) per workgroup
  static constexpr int A_BYTES = kBM * kAPitch;
  static constexpr int AS_BYTES = kBM * 4;
  static constexpr int B_BYTES = BNB * kBPitch;
  static constexpr int BS_BYTES = BNB * 2;
  static constexpr int STAGE = A_BYTES + AS_BYTES + B_BYTES + BS_BYTES;
  static constexpr int NW = GATEUP ? NF / 2 : NF;      // output column frags per wave
  static constexpr int EP_PITCH = NW * 32 + 4;        // floats
  static constexpr int EPI = GATEUP ? 4 * 64 * EP_PITCH * 4 : 0;
  static constexpr int SINK = (2 * STAGE > EPI ? 2 * STAGE : EPI);  // 16-byte dump slot
  static constexpr int SMEM = SINK + 16;
  static constexpr int A_CHUNKS = kBM * 6;             // 16-byte chunks per stage
  static constexpr int A_PER_T = (A_CHUNKS + 255) / 256;
  static constexpr int B_CHUNKS = BNB * 2;
  static constexpr int B_PER_T = (B_CHUNKS + 255) / 256;
  static constexpr int BS_PER_T = (BNB + 255) / 256;
};

template <int NF, bool GATEUP>
__global__ __launch_bounds__(256) void grouped_prefill(const FfnArgs a, const EncIn ain,
                                                       const EncOut hout,
                                                       const int32_t* __restrict__ tile_prefix,
                                                       int ntn) {
  using C = Prefill<NF, GATEUP>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::SMEM];

  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const int nblkK = K / 32;
  const int nsteps = K / 64;
  const int E = a.E;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = logical / ntn;
  const int nt = logical - mt * ntn;
  if (mt >= tile_prefix[E]) return;
  int lo = 0, hi = E;  // tile_prefix[lo] <= mt < tile_prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_prefix[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int off = a.offsets[e];
  const int cnt = a.offsets[e + 1] - off;
  const int m0 = (mt - tile_prefix[e]) * kBM;
  const int ncol0 = nt * (C::NW * 64);  // first output column (h column for gate/up)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- per-thread global sources (fixed across K steps). Every load is
  // unconditional: rows past the expert's count read its last row (results
  // discarded), chunk indices past the tile are clamped and their LDS stores go
  // to a sink slot, so the compiler can keep the prefetch in flight.
  const int rows_valid = min(kBM, cnt - m0);
  const uint8_t* a_src[C::A_PER_T];
  int a_lds[C::A_PER_T];
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = min(tid + 256 * i, C::A_CHUNKS - 1);
    const int row = c / 6, part = c - row * 6;
    a_lds[i] = tid + 256 * i < C::A_CHUNKS ? row * kAPitch + part * 16 : C::SINK;
    const int p = off + m0 + min(row, rows_valid - 1);
    const int src = GATEUP ? a.sorted_pair[p] / a.k : p;
    a_src[i] = ain.codes + (size_t)src * nblkK * kEncBytes + part * 16;
  }
  const uint16_t* as_src;
  {
    const int p = off + m0 + min(tid & (kBM - 1), rows_valid - 1);
    const int src = GATEUP ? a.sorted_pair[p] / a.k : p;
    as_src = ain.scales + (size_t)src * nblkK;
  }
  auto b_row = [&](int brow, const uint8_t*& codes, const uint8_t*& scales) {
    int n;
    if (GATEUP) {
      const int w = brow / (NF * 32), f = (brow / 32) % NF, cc = brow & 31;
      const bool up = f >= C::NW;
      n = ncol0 + w * C::NW * 32 + (up ? f - C::NW : f) * 32 + cc;
      codes = up ? a.wu_codes : a.wg_codes;
      scales = up ? a.wu_scales : a.wg_scales;
    } else {
      n = ncol0 + brow;
      codes = a.wd_codes;
      scales = a.wd_scales;
    }
    codes += ((size_t)e * N + n) * (K / 2);
    scales += ((size_t)e * N + n) * nblkK;
  };
  const uint8_t* b_src[C::B_PER_T];
  int b_lds[C::B_PER_T];
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = min(tid + 256 * i, C::B_CHUNKS - 1);
    const uint8_t* sc;
    b_row(c >> 1, b_src[i], sc);
    b_src[i] += (c & 1) * 16;
    b_lds[i] = tid + 256 * i < C::B_CHUNKS ? C::A_BYTES + C::AS_BYTES + (c >> 1) * kBPitch + (c & 1) * 16
                                           : C::SINK;
  }
  const uint8_t* bs_src[C::BS_PER_T];
  int bs_lds[C::BS_PER_T];
#pragma unroll
  for (int i = 0; i < C::BS_PER_T; ++i) {
    const int brow = min(tid + 256 * i, C::BNB - 1);
    const uint8_t* co;
    b_row(brow, co, bs_src[i]);
    bs_lds[i] = tid + 256 * i < C::BNB ? C::A_BYTES + C::AS_BYTES + C::B_BYTES + brow * 2 : C::SINK;
  }

  uint4 ra[C::A_PER_T], rb[C::B_PER_T];
  uint32_t ras = 0;
  uint16_t rbs[C::BS_PER_T];

  auto load_stage = [&](int s) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + s * 96);
    ras = *reinterpret_cast<const uint32_t*>(as_src + 2 * s);
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + s * 32);
#pragma unroll
    for (int i = 0; i < C::BS_PER_T; ++i) rbs[i] = *reinterpret_cast<const uint16_t*>(bs_src[i] + 2 * s);
  };
  auto store_stage = [&](int buf) {
    uint8_t* st = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      uint2* d = reinterpret_cast<uint2*>(a_lds[i] == C::SINK ? smem + C::SINK : st + a_lds[i]);
      d[0] = make_uint2(ra[i].x, ra[i].y);
      d[1] = make_uint2(ra[i].z, ra[i].w);
    }
    if (tid < kBM) reinterpret_cast<uint32_t*>(st + C::A_BYTES)[tid] = ras;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      uint2* d = reinterpret_cast<uint2*>(b_lds[i] == C::SINK ? smem + C::SINK : st + b_lds[i]);
      d[0] = make_uint2(rb[i].x, rb[i].y);
      d[1] = make_uint2(rb[i].z, rb[i].w);
    }
#pragma unroll
    for (int i = 0; i < C::BS_PER_T; ++i)
      *reinterpret_cast<uint16_t*>(bs_lds[i] == C::SINK ? smem + C::SINK : st + bs_lds[i]) = rbs[i];
  };

  // ---- accumulators start at the bias of their output column
  v16f acc[2][NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    float b;
    if (GATEUP) {
      const bool up = f >= C::NW;
      const int col = ncol0 + wn * C::NW * 32 + (up ? f - C::NW : f) * 32 + lr;
      b = bf16_to_f32((up ? a.b_up : a.b_gate)[(size_t)e * N + col]);
    } else {
      b = bf16_to_f32(a.b_down[(size_t)e * N + ncol0 + wn * NF * 32 + f * 32 + lr]);
    }
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mf][f][i] = b;
  }

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) load_stage(s + 1);
    const uint8_t* st = smem + (s & 1) * C::STAGE;
    v8i ahi[2], alo[2];
    int sa[2];
#pragma unroll
    for (int mf = 0; mf < 2; ++mf) {
      const int row = wm * 64 + mf * 32 + lr;
      const uint8_t* p = st + row * kAPitch + half * 48;
      const uint2 h0 = lds64(p), h1 = lds64(p + 8), h2 = lds64(p + 16);
      const uint2 l0 = lds64(p + 24), l1 = lds64(p + 32), l2 = lds64(p + 40);
      ahi[mf] = v8i{(int)h0.x, (int)h0.y, (int)h1.x, (int)h1.y, (int)h2.x, (int)h2.y, 0, 0};
      alo[mf] = v8i{(int)l0.x, (int)l0.y, (int)l1.x, (int)l1.y, (int)l2.x, (int)l2.y, 0, 0};
      sa[mf] = *reinterpret_cast<const uint16_t*>(st + C::A_BYTES + row * 4 + half * 2);
    }
    const uint8_t* bst = st + C::A_BYTES + C::AS_BYTES;
    v8i b[NF];
    int sb[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int brow = wn * NF * 32 + f * 32 + lr;
      const uint8_t* q = bst + brow * kBPitch + half * 16;
      const uint2 b0 = lds64(q), b1 = lds64(q + 8);
      b[f] = v8i{(int)b0.x, (int)b0.y, (int)b1.x, (int)b1.y, 0, 0, 0, 0};
      sb[f] = bst[C::B_BYTES + brow * 2 + half];
    }
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[mf][f] = mfma_f6f4<0>(ahi[mf], b[f], acc[mf][f], sa[mf], sb[f]);
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[mf][f] = mfma_f6f4<1>(alo[mf], b[f], acc[mf][f], sa[mf], sb[f]);
    if (s + 1 < nsteps) store_stage((s + 1) & 1);
    __syncthreads();
  }

  if constexpr (GATEUP) {
    // h = silu(g) * u into LDS (the staging buffers are free after the last sync),
    // then one lane per row encodes its 32-column blocks as two-term MXFP6.
    float* ep = reinterpret_cast<float*>(smem) + wave * 64 * C::EP_PITCH;
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int f = 0; f < C::NW; ++f)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = mf * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          ep[r * C::EP_PITCH + f * 32 + lr] = silu_mul(acc[mf][f][i], acc[mf][f + C::NW][i]);
        }
    __syncthreads();
    const int grow = m0 + wm * 64 + lane;
    if (grow < cnt) {
      const int p = off + grow;
      const int nblkF = a.F / 32;
#pragma unroll
      for (int f = 0; f < C::NW; ++f) {
        float v[32];
        const float4* src = reinterpret_cast<const float4*>(ep + lane * C::EP_PITCH + f * 32);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 t = src[q];
          v[4 * q] = t.x;
          v[4 * q + 1] = t.y;
          v[4 * q + 2] = t.z;
          v[4 * q + 3] = t.w;
        }
        uint32_t hw[6], lw[6], sc;
        encode_block(v, hw, lw, sc);
        const int blk = (ncol0 + wn * C::NW * 32 + f * 32) / 32;
        uint4* dst = reinterpret_cast<uint4*>(hout.codes + ((size_t)p * nblkF + blk) * kEncBytes);
        dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        dst[1] = make_uint4(hw[4], hw[5], lw[0], lw[1]);
        dst[2] = make_uint4(lw[2], lw[3], lw[4], lw[5]);
        hout.scales[(size_t)p * nblkF + blk] = static_cast<uint16_t>(sc);
      }
    }
  } else {
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m0 + wm * 64 + mf * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (r < cnt) {
          float* yr = a.y_sorted + (size_t)(off + r) * N + ncol0 + wn * NF * 32 + lr;
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
constexpr int kDecAPitch = kDecWB * kEncBytes + 8;  // LDS bytes per activation row (padded)
constexpr int kDecAChunks = 16 * kDecWB * 3;        // 16-byte chunks of the activation window
constexpr int kDecAPerT = kDecAChunks / 256;        // ... per thread
constexpr int kDecASPerT = 16 * kDecWB / 256;       // activation scale entries per thread
constexpr int kDecBSPerT = 64 * kDecWB / 256;       // weight scale bytes per thread
static_assert(kDecSS % 4 == 0, "the window staging splits evenly over 256 threads");
static_assert(kDecAChunks % 256 == 0 && (16 * kDecWB) % 256 == 0 && (64 * kDecWB) % 256 == 0,
              "window staging must divide evenly");

// Gate/up: waves 0,1 stream the gate rows of 32 h-columns, waves 2,3 the up rows
// of the same columns (one matrix per wave keeps the register footprint small);
// down: 4 waves x 16 output columns. The stage loop is unrolled at compile time
// (NSTAGE stages of kDecSS steps): the weight codes of stage s+kDecPF and the
// activation window (+ both kinds of scales) of stage s+kDecPF are issued while
// stage s is computed, held in register rings, and the window is copied to LDS
// one stage before it is read. Loads are issued in the order they are consumed,
// so waiting for one never waits for a younger one (the vector memory counter
// retires in order). All global reads are buffer loads: K blocks past the end
// (the half step when K % 128 == 64) and rows past the count read as zero.
template <bool GATEUP, int NSTAGE>
__global__ __launch_bounds__(256, 2) void grouped_decode(const FfnArgs a, const EncIn ain,
                                                         const EncOut hout) {
  constexpr int COLS = GATEUP ? 32 : 64;  // output columns per workgroup
  constexpr int PF = kDecPF;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][16 * kDecAPitch];
  __shared__ uint16_t sAs[2][16 * kDecWB];
  __shared__ uint8_t sBs[2][64 * kDecWB];   // weight scales of the window: [wave*16 + col][blk]
  __shared__ __attribute__((aligned(16))) float gtile[GATEUP ? 2 * 16 * 36 : 4];
  __shared__ uint8_t escratch[GATEUP ? 8 * 64 : 4];

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
  const uint8_t* scales = GATEUP ? (up ? a.wu_scales : a.wg_scales) : a.wd_scales;
  const rsrc_t wr = make_rsrc(codes + (size_t)e * N * (K / 2), (uint32_t)((size_t)N * (K / 2)));
  const rsrc_t sr = make_rsrc(scales + (size_t)e * N * nblkK, (uint32_t)(N * nblkK));
  const float bias = bf16_to_f32((GATEUP ? (up ? a.b_up : a.b_gate) : a.b_down)[(size_t)e * N + n]);
  const uint32_t wrow = (uint32_t)n * (K / 2);
  // the weight-scale row this thread stages: column (wave, tid % 16) of the workgroup
  const uint32_t srow_t = (uint32_t)(GATEUP ? j * 32 + (wave & 1) * 16 + (tid & 15)
                                            : j * 64 + wave * 16 + (tid & 15)) * nblkK;
  // activation rows: gathered tokens (gate/up) or this expert's rows of h (down)
  const rsrc_t ar = GATEUP ? make_rsrc(ain.codes, (uint32_t)((size_t)a.T * nblkK * kEncBytes))
                           : make_rsrc(ain.codes + (size_t)off * nblkK * kEncBytes,
                                       (uint32_t)((size_t)cnt * nblkK * kEncBytes));
  const rsrc_t asr = GATEUP ? make_rsrc(ain.scales, (uint32_t)((size_t)a.T * nblkK * 2))
                            : make_rsrc(ain.scales + (size_t)off * nblkK, (uint32_t)(cnt * nblkK * 2));

  for (int m0 = 0; m0 < cnt; m0 += 16) {
    const int rows = min(16, cnt - m0);
    uint32_t arow[kDecAPerT];
    int alds[kDecAPerT], ablk[kDecAPerT];
#pragma unroll
    for (int i = 0; i < kDecAPerT; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (kDecWB * 3), rem = c - row * (kDecWB * 3);
      const int blk = rem / 3, part = rem - blk * 3;
      alds[i] = row * kDecAPitch + blk * kEncBytes + part * 16;
      ablk[i] = blk;
      const int src = GATEUP ? a.sorted_pair[off + m0 + min(row, rows - 1)] / a.k : m0 + row;
      arow[i] = row < rows ? (uint32_t)(src * nblkK * kEncBytes + part * 16) : kOutOfRange;
    }
    uint32_t asrow[kDecASPerT];
    int asblk[kDecASPerT];
#pragma unroll
    for (int i = 0; i < kDecASPerT; ++i) {
      const int ent = tid + 256 * i;
      const int row = ent / kDecWB;
      asblk[i] = ent - row * kDecWB;
      const int src = GATEUP ? a.sorted_pair[off + m0 + min(row, rows - 1)] / a.k : m0 + row;
      asrow[i] = row < rows ? (uint32_t)(src * nblkK * 2) : kOutOfRange;
    }

    // one stage's worth of loads for this thread
    struct Packet {
      uint4 w[kDecSS];              // weight codes (MFMA B operand, this lane)
      uint4 a[kDecAPerT];           // activation window chunks (staged to LDS)
      uint32_t as[kDecASPerT];      // activation scales (staged)
      uint32_t bs[kDecBSPerT];      // weight scales (staged)
    };
    // The stage's distance along K goes into the uniform buffer offset, so the
    // per-lane offsets are the same in every stage; only the last stage can hold
    // blocks past K, and only there are lanes redirected out of range.
    auto issue = [&](int st, Packet& pk) {
      const bool last = st == NSTAGE - 1;
      const uint32_t wso = (uint32_t)st * kDecSS * 64;    // weight bytes per 128-deep step: 64
#pragma unroll
      for (int u = 0; u < kDecSS; ++u) {
        const bool live = !last || (st * kDecSS + u) * 4 + q < nblkK;
        pk.w[u] = bload16(wr, live ? wrow + (u * 4 + q) * 16 : kOutOfRange, wso);
      }
      const int kb0 = st * kDecWB;
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i) {
        const bool live = !last || kb0 + ablk[i] < nblkK;
        pk.a[i] = bload16(ar, live ? arow[i] + ablk[i] * kEncBytes : kOutOfRange,
                          (uint32_t)kb0 * kEncBytes);
      }
#pragma unroll
      for (int i = 0; i < kDecASPerT; ++i) {
        const bool live = !last || kb0 + asblk[i] < nblkK;
        pk.as[i] = bload2(asr, live ? asrow[i] + asblk[i] * 2 : kOutOfRange, (uint32_t)kb0 * 2);
      }
#pragma unroll
      for (int i = 0; i < kDecBSPerT; ++i) {
        const int bl = ((tid >> 4) & 3) * kDecBSPerT + i;
        const bool live = !last || kb0 + bl < nblkK;
        pk.bs[i] = bload1(sr, live ? srow_t + bl : kOutOfRange, (uint32_t)kb0);
      }
    };
    auto stage_to_lds = [&](const Packet& pk, int buf) {
#pragma unroll
      for (int i = 0; i < kDecAPerT; ++i) {
        uint2* d = reinterpret_cast<uint2*>(sA[buf] + alds[i]);
        d[0] = make_uint2(pk.a[i].x, pk.a[i].y);
        d[1] = make_uint2(pk.a[i].z, pk.a[i].w);
      }
#pragma unroll
      for (int i = 0; i < kDecASPerT; ++i) sAs[buf][tid + 256 * i] = static_cast<uint16_t>(pk.as[i]);
#pragma unroll
      for (int i = 0; i < kDecBSPerT; ++i)
        sBs[buf][(wave * 16 + (tid & 15)) * kDecWB + ((tid >> 4) & 3) * kDecBSPerT + i] =
            static_cast<uint8_t>(pk.bs[i]);
    };

    v4f acc = v4f{bias, bias, bias, bias};
    Packet ring[PF + 1];
    __syncthreads();  // LDS of the previous row tile is no longer read
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < NSTAGE) issue(p, ring[p]);
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
          const uint8_t* pa = sA[buf] + l16 * kDecAPitch + (4 * u + q) * kEncBytes;
          const uint2 h0 = lds64(pa), h1 = lds64(pa + 8), h2 = lds64(pa + 16);
          const uint2 g0 = lds64(pa + 24), g1 = lds64(pa + 32), g2 = lds64(pa + 40);
          const v8i ahi = {(int)h0.x, (int)h0.y, (int)h1.x, (int)h1.y, (int)h2.x, (int)h2.y, 0, 0};
          const v8i alo = {(int)g0.x, (int)g0.y, (int)g1.x, (int)g1.y, (int)g2.x, (int)g2.y, 0, 0};
          const int as = sAs[buf][l16 * kDecWB + 4 * u + q];
          const int bs = sBs[buf][(wave * 16 + l16) * kDecWB + 4 * u + q];
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
      // then each half wavefront encodes one row's 32-column block of h
      float* t = gtile + (wave >> 1) * 16 * 36;
#pragma unroll
      for (int i = 0; i < 4; ++i) t[(4 * q + i) * 36 + (wave & 1) * 16 + l16] = acc[i];
      __syncthreads();
      const int nblkF = a.F / 32;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int row = pass * 8 + (tid >> 5), col = tid & 31;
        const float h = silu_mul(gtile[row * 36 + col], gtile[16 * 36 + row * 36 + col]);
        const size_t rec = (size_t)(off + m0 + min(row, rows - 1)) * nblkF + j;
        encode_group32(h, escratch + (tid >> 5) * 64, hout.codes + rec * kEncBytes,
                       hout.scales + rec, row < rows);
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
  const int ntn = N / (Prefill<NF, GATEUP>::NW * 64);
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

// Largest column-fragment count per wave that tiles N exactly (64*q columns per
// workgroup, q in {3, 2, 1}).
int pick_q(int N) { return N % 192 == 0 ? 3 : (N % 128 == 0 ? 2 : 1); }

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
  if (dec_gu) {
    err = launch_decode<true>(a, xin, hout, stream);
  } else {
    switch (pick_q(a.F)) {
      case 3: err = launch_prefill<6, true>(a, xin, hout, tp, stream); break;
      case 2: err = launch_prefill<4, true>(a, xin, hout, tp, stream); break;
      default: err = launch_prefill<2, true>(a, xin, hout, tp, stream); break;
    }
  }
  if (err != hipSuccess) return err;
  if (dec_dn) return launch_decode<false>(a, hin, hout, stream);
  switch (pick_q(a.d)) {
    case 3: return launch_prefill<3, false>(a, hin, hout, tp, stream);
    case 2: return launch_prefill<2, false>(a, hin, hout, tp, stream);
    default: return launch_prefill<1, false>(a, hin, hout, tp, stream);
  }
}


}  // namespace moe
