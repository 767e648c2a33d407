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

__global__ __launch_bounds__(256) void encode_rows(const uint16_t* __restrict__ x, int rows,
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
  uint4* dst = reinterpret_cast<uint4*>(codes + (size_t)idx * kEncBytes);
  dst[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  dst[1] = make_uint4(hi[4], hi[5], lo[0], lo[1]);
  dst[2] = make_uint4(lo[2], lo[3], lo[4], lo[5]);
  scales[idx] = static_cast<uint16_t>(sc);
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
  static constexpr int SMEM = 2 * STAGE > EPI ? 2 * STAGE : EPI;
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

  // ---- per-thread global sources (fixed across K steps)
  const uint8_t* a_src[C::A_PER_T];
  int a_lds[C::A_PER_T];
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + 256 * i;
    const int row = c / 6, part = c - row * 6;
    a_src[i] = nullptr;
    a_lds[i] = row * kAPitch + part * 16;
    if (c < C::A_CHUNKS && row < cnt - m0) {
      const int p = off + m0 + row;
      const int src = GATEUP ? a.sorted_pair[p] / a.k : p;
      a_src[i] = ain.codes + (size_t)src * nblkK * kEncBytes + part * 16;
    }
  }
  const uint16_t* as_src = nullptr;
  if (tid < kBM && tid < cnt - m0) {
    const int p = off + m0 + tid;
    const int src = GATEUP ? a.sorted_pair[p] / a.k : p;
    as_src = ain.scales + (size_t)src * nblkK;
  }
  const uint8_t* b_src[C::B_PER_T];
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + 256 * i;
    b_src[i] = nullptr;
    if (c < C::B_CHUNKS) {
      const int brow = c >> 1, part = c & 1;
      const uint8_t* base;
      int n;
      if (GATEUP) {
        const int w = brow / (NF * 32), f = (brow / 32) % NF, cc = brow & 31;
        const bool up = f >= C::NW;
        n = ncol0 + w * C::NW * 32 + (up ? f - C::NW : f) * 32 + cc;
        base = up ? a.wu_codes : a.wg_codes;
      } else {
        n = ncol0 + brow;
        base = a.wd_codes;
      }
      b_src[i] = base + ((size_t)e * N + n) * (K / 2) + part * 16;
    }
  }
  const uint8_t* bs_src[C::BS_PER_T];
#pragma unroll
  for (int i = 0; i < C::BS_PER_T; ++i) {
    const int brow = tid + 256 * i;
    bs_src[i] = nullptr;
    if (brow < C::BNB) {
      const uint8_t* base;
      int n;
      if (GATEUP) {
        const int w = brow / (NF * 32), f = (brow / 32) % NF, cc = brow & 31;
        const bool up = f >= C::NW;
        n = ncol0 + w * C::NW * 32 + (up ? f - C::NW : f) * 32 + cc;
        base = up ? a.wu_scales : a.wg_scales;
      } else {
        n = ncol0 + brow;
        base = a.wd_scales;
      }
      bs_src[i] = base + ((size_t)e * N + n) * nblkK;
    }
  }

  uint4 ra[C::A_PER_T], rb[C::B_PER_T];
  uint32_t ras = 0;
  uint16_t rbs[C::BS_PER_T];

  auto load_stage = [&](int s) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i)
      ra[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + s * 96) : make_uint4(0, 0, 0, 0);
    ras = as_src ? *reinterpret_cast<const uint32_t*>(as_src + 2 * s) : 0u;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i)
      if (b_src[i]) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + s * 32);
#pragma unroll
    for (int i = 0; i < C::BS_PER_T; ++i)
      if (bs_src[i]) rbs[i] = *reinterpret_cast<const uint16_t*>(bs_src[i] + 2 * s);
  };
  auto store_stage = [&](int buf) {
    uint8_t* st = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      if (tid + 256 * i < C::A_CHUNKS) {
        uint2* d = reinterpret_cast<uint2*>(st + a_lds[i]);
        d[0] = make_uint2(ra[i].x, ra[i].y);
        d[1] = make_uint2(ra[i].z, ra[i].w);
      }
    }
    if (tid < kBM) reinterpret_cast<uint32_t*>(st + C::A_BYTES)[tid] = ras;
    uint8_t* bst = st + C::A_BYTES + C::AS_BYTES;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int c = tid + 256 * i;
      if (c < C::B_CHUNKS) {
        uint2* d = reinterpret_cast<uint2*>(bst + (c >> 1) * kBPitch + (c & 1) * 16);
        d[0] = make_uint2(rb[i].x, rb[i].y);
        d[1] = make_uint2(rb[i].z, rb[i].w);
      }
    }
    uint16_t* bss = reinterpret_cast<uint16_t*>(bst + C::B_BYTES);
#pragma unroll
    for (int i = 0; i < C::BS_PER_T; ++i)
      if (tid + 256 * i < C::BNB) bss[tid + 256 * i] = rbs[i];
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

template <bool GATEUP>
__global__ __launch_bounds__(256) void grouped_decode(const FfnArgs a, const EncIn ain,
                                                      const EncOut hout) {
  constexpr int NM = GATEUP ? 2 : 1;  // weight matrices streamed (gate+up, or down)
  __shared__ __attribute__((aligned(16))) float red[3 * 64 * 16 * NM];
  __shared__ __attribute__((aligned(16))) float htile[32 * 33];

  const int K = GATEUP ? a.d : a.F;
  const int N = GATEUP ? a.F : a.d;
  const int nblkK = K / 32;
  const int nsteps = K / 64;
  const int ncb = N / 32;
  const int e = blockIdx.x / ncb;
  const int j = blockIdx.x - e * ncb;
  const int off = a.offsets[e];
  const int cnt = a.offsets[e + 1] - off;
  if (cnt == 0) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, half = lane >> 5;
  const int s_begin = wave * nsteps / 4, s_end = (wave + 1) * nsteps / 4;
  const int n = j * 32 + lr;
  const uint8_t* wc[NM];
  const uint8_t* wsc[NM];
  float bias[NM];
  if (GATEUP) {
    wc[0] = a.wg_codes + ((size_t)e * N + n) * (K / 2) + half * 16;
    wsc[0] = a.wg_scales + ((size_t)e * N + n) * nblkK + half;
    bias[0] = bf16_to_f32(a.b_gate[(size_t)e * N + n]);
    wc[NM - 1] = a.wu_codes + ((size_t)e * N + n) * (K / 2) + half * 16;
    wsc[NM - 1] = a.wu_scales + ((size_t)e * N + n) * nblkK + half;
    bias[NM - 1] = bf16_to_f32(a.b_up[(size_t)e * N + n]);
  } else {
    wc[0] = a.wd_codes + ((size_t)e * N + n) * (K / 2) + half * 16;
    wsc[0] = a.wd_scales + ((size_t)e * N + n) * nblkK + half;
    bias[0] = bf16_to_f32(a.b_down[(size_t)e * N + n]);
  }

  for (int m0 = 0; m0 < cnt; m0 += 32) {
    const int row = m0 + lr;
    const bool valid = row < cnt;
    int src = 0;
    if (valid) src = GATEUP ? a.sorted_pair[off + row] / a.k : off + row;
    const uint8_t* ap = ain.codes + ((size_t)src * nblkK + half) * kEncBytes;
    const uint16_t* asp = ain.scales + (size_t)src * nblkK + half;

    v16f acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][i] = wave == 0 ? bias[m] : 0.f;

    for (int s0 = s_begin; s0 < s_end; s0 += 4) {
      uint4 w[4][NM];
      int ws[4][NM];
      uint4 x0[4], x1[4], x2[4];
      int xs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + u;
        if (s < s_end) {
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            w[u][m] = *reinterpret_cast<const uint4*>(wc[m] + s * 32);
            ws[u][m] = wsc[m][2 * s];
          }
          if (valid) {
            const uint4* xp = reinterpret_cast<const uint4*>(ap + s * 2 * kEncBytes);
            x0[u] = xp[0];
            x1[u] = xp[1];
            x2[u] = xp[2];
            xs[u] = asp[2 * s];
          } else {
            x0[u] = x1[u] = x2[u] = make_uint4(0, 0, 0, 0);
            xs[u] = 0;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (s0 + u < s_end) {
          const v8i ahi = {(int)x0[u].x, (int)x0[u].y, (int)x0[u].z, (int)x0[u].w,
                           (int)x1[u].x, (int)x1[u].y, 0, 0};
          const v8i alo = {(int)x1[u].z, (int)x1[u].w, (int)x2[u].x, (int)x2[u].y,
                           (int)x2[u].z, (int)x2[u].w, 0, 0};
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const v8i b = {(int)w[u][m].x, (int)w[u][m].y, (int)w[u][m].z, (int)w[u][m].w, 0, 0, 0, 0};
            acc[m] = mfma_f6f4<0>(ahi, b, acc[m], xs[u], ws[u][m]);
            acc[m] = mfma_f6f4<1>(alo, b, acc[m], xs[u], ws[u][m]);
          }
        }
      }
    }

    // fixed-order reduction of the four K-quarters through LDS
    __syncthreads();
    if (wave > 0) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[(((wave - 1) * NM + m) * 16 + i) * 64 + lane] = acc[m][i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w2 = 0; w2 < 3; ++w2)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[m][i] += red[((w2 * NM + m) * 16 + i) * 64 + lane];
      if constexpr (GATEUP) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * half + (i & 3);
          htile[r * 33 + lr] = silu_mul(acc[0][i], acc[1][i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = m0 + 8 * (i >> 2) + 4 * half + (i & 3);
          if (r < cnt) a.y_sorted[(size_t)(off + r) * N + n] = acc[0][i];
        }
      }
    }
    if constexpr (GATEUP) {
      __syncthreads();
      if (wave == 0 && lane < 32 && m0 + lane < cnt) {
        float v[32];
#pragma unroll
        for (int c = 0; c < 32; ++c) v[c] = htile[lane * 33 + c];
        uint32_t hw[6], lw[6], sc;
        encode_block(v, hw, lw, sc);
        const int p = off + m0 + lane;
        const int nblkF = a.F / 32;
        uint4* dst = reinterpret_cast<uint4*>(hout.codes + ((size_t)p * nblkF + j) * kEncBytes);
        dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        dst[1] = make_uint4(hw[4], hw[5], lw[0], lw[1]);
        dst[2] = make_uint4(lw[2], lw[3], lw[4], lw[5]);
        hout.scales[(size_t)p * nblkF + j] = static_cast<uint16_t>(sc);
      }
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
  hipLaunchKernelGGL(encode_rows, dim3((nx + 255) / 256), dim3(256), 0, stream, a.x, a.T, a.d,
                     xout.codes, xout.scales);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (a.T <= kDecodeMaxT) {
    hipLaunchKernelGGL(grouped_decode<true>, dim3(a.E * (a.F / 32)), dim3(256), 0, stream, a, xin,
                       hout);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_decode<false>, dim3(a.E * (a.d / 32)), dim3(256), 0, stream, a, hin,
                       hout);
    return hipGetLastError();
  }

  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(256), 0, stream, a.offsets, a.E, tp);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  switch (pick_q(a.F)) {
    case 3: err = launch_prefill<6, true>(a, xin, hout, tp, stream); break;
    case 2: err = launch_prefill<4, true>(a, xin, hout, tp, stream); break;
    default: err = launch_prefill<2, true>(a, xin, hout, tp, stream); break;
  }
  if (err != hipSuccess) return err;
  switch (pick_q(a.d)) {
    case 3: return launch_prefill<3, false>(a, hin, hout, tp, stream);
    case 2: return launch_prefill<2, false>(a, hin, hout, tp, stream);
    default: return launch_prefill<1, false>(a, hin, hout, tp, stream);
  }
}

}  // namespace moe
