// Attention with per-head sinks (Perplexity, "GPT-OSS el dia 0", section
// "Atenció: GQA amb Attention Sinks": every head has a pretrained sink that
// takes part in the softmax; section "Nuclis per a GPT-OSS / Atenció de
// buidatge": an online softmax takes the sink in by starting its running
// maximum at the head's sink value and its running denominator at 1, in the
// first KV chunk only when the keys are split into chunks). The sink is a
// softmax entry without a value vector:
//   out = sum_j exp(z_j) v_j / (exp(s_h) + sum_j exp(z_j)),  z_j = scale <q, k_j>,
// over the keys the query sees (causal; optionally a sliding window), with
// grouped KV heads (query head h reads KV head h / (Hq / Hkv)).
//
// Both kernels work on 32-key tiles with gfx950's bf16 matrix cores. A
// wavefront holds 32 query slots; per tile it computes S^T = K Q^T (32 keys x
// 32 slots, four 32x32x16 bf16 MFMAs over the head size 64), so each lane holds
// one slot's 16 keys and a slot's running max and sum need one cross-half
// shuffle; then the online softmax update (base 2, log2(e) folded into the
// scale) and O^T += V^T P^T with P^T taken from the S^T accumulators as bf16.
// In the accumulator a lane l holds slot l%32 and keys 8(i/4) + 4(l/32) + i%4
// (i = 0..15); the matrix instruction pairs element t of A's lane half with
// element t of B's, so the V^T operand of MFMA c (keys 16c .. 16c+15) lists,
// for lane half h, the keys its P^T registers 8c .. 8c+7 hold:
// 16c + 8(t/4) + 4h + t%4.
//
// The running maximum is raised only when a tile's maximum exceeds it by more
// than 8 (base 2): probabilities then stay below 2^8, and the 32 output
// rescales per lane and tile are skipped on most tiles. The result is the same
// quantity (numerator and denominator share the stale maximum), rounded
// differently.
//
// attn_fwd (many queries, FlashAttention-2 style): a workgroup takes 32
// consecutive queries of one batch entry and KV head, one wavefront per query
// head of the group (up to 8), all sharing each K/V tile staged once in LDS
// (double-buffered, one barrier per tile); slot = query.
// attn_dec (few queries: G * Tq <= 32 for G = Hq / Hkv): one wavefront packs
// the G heads x Tq queries of a KV head into its 32 slots; a workgroup holds
// one wavefront per KV head (up to 4) of one batch entry, all on the same chunk
// of keys, so together they stream whole contiguous KV rows; each wavefront
// loads whole 128-byte rows of its head, passes K through LDS to the MFMA
// operand layout and V through an LDS transpose, with two tiles in flight.
// A single chunk of keys normalises and stores bf16 output; several chunks
// store partials (running max, denominator, unnormalised output) that
// attn_merge adds in chunk order.
#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f_a __attribute__((ext_vector_type(16)));
// 16 bytes as a native vector (copies of HIP's uint4 struct between address
// spaces can leave the array behind in scratch memory)
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

constexpr int kHD = 64;             // head size
constexpr int kQB = 32;             // query slots per wavefront
constexpr int kKT = 32;             // keys per tile
constexpr int kKS = 72;             // K tile row stride in LDS (halves): 144 B, conflict-free 16 B reads
constexpr int kVS = 36;             // V^T tile row stride in LDS (halves): 72 B
constexpr int kKTile = kKT * kKS;   // halves
constexpr int kVTile = kHD * kVS;   // halves
constexpr int kBuf = kKTile + kVTile;
constexpr int kDecW = 4;            // wavefronts (KV heads) per attn_dec workgroup, at most
constexpr int kPS = 68;             // partial record (floats): m, l, 2 unused, o[64]
constexpr int kPO = 4;              // offset of o in the record
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;        // lazy-rescale threshold (base 2)

struct AttnArgs {
  const uint16_t *q, *k, *v;
  const float* sinks;
  uint16_t* out;
  float* part;          // [B][Tq][Hq][nchunks][kPS] when nchunks > 1
  int B, Tq, S, Hq, Hkv, window, nchunks, chunk, kofs;   // chunk c: keys kofs + [c chunk, (c+1) chunk)
  float scale;
};

__device__ __forceinline__ v8bf as_bf(u4v u) {
  union {
    u4v u;
    v8bf b;
  } c;
  c.u = u;
  return c.b;
}

__device__ __forceinline__ v8bf as_bf(uint4 u) {
  union {
    uint4 u;
    v8bf b;
  } c;
  c.u = u;
  return c.b;
}

// orders LDS accesses of different lanes of one wavefront (no workgroup barrier)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// One tile of the online softmax for a lane's slot. s: this lane's 16 raw
// scores, -inf where the key is invisible. On return pf holds the bf16 P^T
// operands 2^(sc2 s - m) (0 where invisible); m, l, o0, o1 are updated.
__device__ __forceinline__ void softmax_tile(v16f_a& s, float& m, float& l, v16f_a& o0, v16f_a& o1,
                                             float sc2, v8bf (&pf)[2]) {
  float tmax = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * sc2;   // sc2 > 0: the max of the scaled scores
  if (__builtin_amdgcn_ballot_w64(tmax > m + kTau)) {
    const float mn = fmaxf(m, tmax);
    const float alpha = m == mn ? 1.0f : ex2(m - mn);   // m = -inf: 0
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o0[i] *= alpha;
      o1[i] *= alpha;
    }
    m = mn;
  }
  // m = -inf here: no visible key so far, every s is -inf and every p 0
  const float nb = m == -INFINITY ? 0.0f : -m;
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i] = ex2(fmaf(s[i], sc2, nb));
    psum += s[i];
  }
  l += psum + __shfl_xor(psum, 32);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[c2][e] = (__bf16)s[8 * c2 + e];
}

// O^T += V^T P^T over one tile; vt: the tile's V^T [dim][key] (row stride kVS)
__device__ __forceinline__ void pv_tile(const uint16_t* vt, int lr, int hf, const v8bf (&pf)[2],
                                        v16f_a& o0, v16f_a& o1) {
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const int key0 = 16 * c2 + 4 * hf;   // V^T element t: key key0 + 8 (t / 4) + t % 4
    const uint2 v0a = *reinterpret_cast<const uint2*>(&vt[lr * kVS + key0]);
    const uint2 v0b = *reinterpret_cast<const uint2*>(&vt[lr * kVS + key0 + 8]);
    const uint2 v1a = *reinterpret_cast<const uint2*>(&vt[(32 + lr) * kVS + key0]);
    const uint2 v1b = *reinterpret_cast<const uint2*>(&vt[(32 + lr) * kVS + key0 + 8]);
    o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(make_uint4(v0a.x, v0a.y, v0b.x, v0b.y)), pf[c2], o0, 0, 0, 0);
    o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(make_uint4(v1a.x, v1a.y, v1b.x, v1b.y)), pf[c2], o1, 0, 0, 0);
  }
}

// a slot's partial (m, l, o) into a 16-byte-aligned record of kPS floats; lane
// half hf holds dims 8 j + 4 hf .. +3 (j = 0..3) of each 32-dim half
__device__ __forceinline__ void store_partial(float* p, int hf, float m, float l, const v16f_a& o0,
                                              const v16f_a& o1) {
  if (hf == 0) {
    p[0] = m;
    p[1] = l;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = 8 * j + 4 * hf;
    *reinterpret_cast<float4*>(p + kPO + d) = make_float4(o0[4 * j], o0[4 * j + 1], o0[4 * j + 2], o0[4 * j + 3]);
    *reinterpret_cast<float4*>(p + kPO + 32 + d) = make_float4(o1[4 * j], o1[4 * j + 1], o1[4 * j + 2], o1[4 * j + 3]);
  }
}

// normalised bf16 output of a lane's slot into row lr of st (32 x 64 halves)
__device__ __forceinline__ void stage_out(uint16_t* st, int lr, int hf, float l, const v16f_a& o0,
                                          const v16f_a& o1) {
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int d = 8 * (i >> 2) + 4 * hf + (i & 3);
    st[lr * kHD + d] = f32_to_bf16(o0[i] * inv);
    st[lr * kHD + 32 + d] = f32_to_bf16(o1[i] * inv);
  }
}

// NP: K/V pair pieces per thread and tile (256 pieces / threads, rounded up)
template <int NP>
__global__ __launch_bounds__(512) void attn_fwd(const AttnArgs a) {
  const int G = a.Hq / a.Hkv;
  // two K/V tile buffers; after the loop, the per-wavefront output staging
  __shared__ __attribute__((aligned(16))) uint16_t sm[8 * kQB * kHD > 2 * kBuf ? 8 * kQB * kHD : 2 * kBuf];
  const int bg = blockIdx.x, c = blockIdx.z;
  const int qb = gridDim.y - 1 - blockIdx.y;    // the longest causal rows first
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int tid = threadIdx.x, nthr = G * 64;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, hf = lane >> 5;
  const int h = g * G + wave;
  const int q0 = qb * kQB;
  const int qi = q0 + lr;                       // this lane's query
  const bool qvalid = qi < a.Tq;
  const int qpos = a.S - a.Tq + qi;             // its position
  // keys this workgroup covers: its chunk, cut to what any of its queries sees
  const int qpos_lo = a.S - a.Tq + q0, qpos_hi = a.S - a.Tq + min(q0 + kQB, a.Tq) - 1;
  int k0 = a.kofs + c * a.chunk, k1 = min(a.S, k0 + a.chunk);
  k1 = min(k1, qpos_hi + 1);
  if (a.window > 0) k0 = max(k0, qpos_lo - a.window + 1);
  const int ntile = k1 > k0 ? (k1 - k0 + kKT - 1) / kKT : 0;

  // Q^T fragments (B operand): lane l = query l%32, dims 16 ks + 8 hf .. +7
  v8bf qf[4];
  {
    const uint16_t* qr = a.q + (((size_t)b * a.Tq + min(qi, a.Tq - 1)) * a.Hq + h) * kHD;
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) qf[ks2] = as_bf(*reinterpret_cast<const uint4*>(qr + 16 * ks2 + 8 * hf));
  }
  const float sc2 = a.scale * kLog2e;
  float m = c == 0 ? a.sinks[h] * kLog2e : -INFINITY;   // running max (base 2)
  float l = c == 0 ? 1.0f : 0.0f;                       // running denominator
  v16f_a o0 = {}, o1 = {};                              // O^T: dims 0..31, 32..63 x queries

  // Tile loads: piece p < 128 holds keys 2 (p%16) and +1 of K at dims 8 (p/16) .. +7;
  // p in [128, 256) the same of V. Thread tid takes pieces tid + j nthr.
  uint4 pre[NP][2];
  auto gload = [&](int t) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int p = tid + j * nthr;
      if (p < 256) {
        const int pp = p & 127, dg = pp >> 4, kk = k0 + t * kKT + 2 * (pp & 15);
        const uint16_t* base = (p < 128 ? a.k : a.v) + (size_t)b * a.S * a.Hkv * kHD + g * kHD + 8 * dg;
        pre[j][0] = *reinterpret_cast<const uint4*>(base + (size_t)min(kk, a.S - 1) * a.Hkv * kHD);
        pre[j][1] = *reinterpret_cast<const uint4*>(base + (size_t)min(kk + 1, a.S - 1) * a.Hkv * kHD);
      }
    }
  };
  // K rows as they are; V as V^T with the key pair in one 32-bit word
  auto lstore = [&](int buf) {
    uint16_t* kt = sm + buf * kBuf;
    uint16_t* vt = kt + kKTile;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int p = tid + j * nthr;
      if (p < 256) {
        const int pp = p & 127, dg = pp >> 4, mm = pp & 15;
        if (p < 128) {
          *reinterpret_cast<uint4*>(&kt[(2 * mm) * kKS + 8 * dg]) = pre[j][0];
          *reinterpret_cast<uint4*>(&kt[(2 * mm + 1) * kKS + 8 * dg]) = pre[j][1];
        } else {
          const uint32_t x[4] = {pre[j][0].x, pre[j][0].y, pre[j][0].z, pre[j][0].w};
          const uint32_t y[4] = {pre[j][1].x, pre[j][1].y, pre[j][1].z, pre[j][1].w};
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint32_t lo = (x[t >> 1] >> (16 * (t & 1))) & 0xffffu;
            const uint32_t hi = (y[t >> 1] >> (16 * (t & 1))) & 0xffffu;
            *reinterpret_cast<uint32_t*>(&vt[(8 * dg + t) * kVS + 2 * mm]) = lo | (hi << 16);
          }
        }
      }
    }
  };
  if (ntile > 0) {
    gload(0);
    lstore(0);
  }
  if (ntile > 1) gload(1);
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const uint16_t* kt = sm + (t & 1) * kBuf;
    // S^T = K Q^T over the head size
    v16f_a s = {};
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const v8bf kf = as_bf(*reinterpret_cast<const uint4*>(&kt[lr * kKS + 16 * ks2 + 8 * hf]));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks2], s, 0, 0, 0);
    }
    const int kb = k0 + t * kKT;
    v8bf pf[2];
    // every key of the tile visible to every query of the workgroup
    const bool full = kb + kKT <= k1 && kb + kKT - 1 <= qpos_lo && (a.window <= 0 || kb > qpos_hi - a.window);
    if (!full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = kb + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (!(qvalid && kj < k1 && kj <= qpos && (a.window <= 0 || kj > qpos - a.window))) s[i] = -INFINITY;
      }
    }
    softmax_tile(s, m, l, o0, o1, sc2, pf);
    pv_tile(kt + kKTile, lr, hf, pf, o0, o1);
    // buffer (t+1)&1 was last read for tile t-1, which every wavefront finished
    // before the barrier that ended it
    if (t + 1 < ntile) lstore((t + 1) & 1);
    if (t + 2 < ntile) gload(t + 2);
    __syncthreads();
  }

  // lane l holds query l%32, dims 8(i/4) + 4 hf + i%4 (+32 in o1)
  if (a.nchunks == 1) {
    uint16_t* st = sm + wave * kQB * kHD;
    stage_out(st, lr, hf, l, o0, o1);
    wave_sync();
    // 32 queries x 128 B: 4 passes of 16 bytes per lane
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) {
      const int idx = p2 * 64 + lane, row = idx >> 3, col = (idx & 7) * 8;
      if (q0 + row < a.Tq)
        *reinterpret_cast<uint4*>(a.out + (((size_t)b * a.Tq + q0 + row) * a.Hq + h) * kHD + col) =
            *reinterpret_cast<const uint4*>(&st[row * kHD + col]);
    }
  } else if (qvalid) {
    store_partial(a.part + ((((size_t)b * a.Tq + qi) * a.Hq + h) * a.nchunks + c) * kPS, hf, m, l, o0, o1);
  }
}

// rows key0 + 8 i (i = 0..3, clamped to the last key) of K and V, 16 bytes each,
// non-temporal: the caches are read once
__device__ __forceinline__ void dec_rows(const uint16_t* kbase, const uint16_t* vbase, size_t rs, int key0,
                                         int S, u4v (&kc)[4], u4v (&vc)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t row = (size_t)min(key0 + 8 * i, S - 1) * rs;
    kc[i] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(kbase + row));
    vc[i] = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(vbase + row));
  }
}

__global__ __launch_bounds__(kDecW * 64) __attribute__((amdgpu_waves_per_eu(3))) void attn_dec(const AttnArgs a) {
  // per wavefront: a tile's K rows [key][dim] (row stride kKS), then the same
  // tile's V^T [dim][key] (row stride kVS) in the same place; finally the output
  // per wavefront: [0, kKTile) the tile area, [kKTile, 2 kKTile) its 32 slots'
  // queries [slot][dim] (row stride kKS)
  __shared__ __attribute__((aligned(16))) uint16_t kv[kDecW][2 * kKTile];
  static_assert(kVTile <= kKTile && kQB * kHD <= kKTile, "one area per wavefront");
  const int G = a.Hq / a.Hkv;
  const int nw = blockDim.x >> 6, ngr = (a.Hkv + nw - 1) / nw;
  const int b = blockIdx.x / ngr, c = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hf = lane >> 5;
  const int g = (blockIdx.x - b * ngr) * nw + wave;   // this wavefront's KV head
  if (g >= a.Hkv) return;                             // (no workgroup barrier below)
  // slot lr = (query tq, head hq of the group), tq = lr / G
  const int tq = lr / G, hq = lr - tq * G;
  const bool sval = tq < a.Tq;
  const int tqc = min(tq, a.Tq - 1), h = g * G + hq;
  const int qpos = a.S - a.Tq + tqc;
  const int qpos_lo = a.S - a.Tq, qpos_hi = a.S - 1;
  int k0 = a.kofs + c * a.chunk;
  const int k1 = min(a.S, k0 + a.chunk);
  if (a.window > 0) k0 = max(k0, qpos_lo - a.window + 1);
  const int ntile = k1 > k0 ? (k1 - k0 + kKT - 1) / kKT : 0;

  uint16_t* buf = kv[wave];
  uint16_t* qs = buf + kKTile;
  {
    // lane (slot lr, half hf): 64 bytes of its slot's query
    const uint16_t* qr = a.q + (((size_t)b * a.Tq + tqc) * a.Hq + h) * kHD + 32 * hf;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u4v*>(&qs[lr * kKS + 32 * hf + 8 * j]) = *reinterpret_cast<const u4v*>(qr + 8 * j);
  }
  const float sc2 = a.scale * kLog2e;
  float m = c == 0 ? a.sinks[h] * kLog2e : -INFINITY;
  float l = c == 0 ? 1.0f : 0.0f;
  v16f_a o0 = {}, o1 = {};

  // Tile loads, whole rows: instruction i gives lane l 16 bytes (dims 8 (l%8) ..
  // +7) of key 8 i + l/8, so each instruction reads 8 full 128-byte rows of this
  // KV head, and the workgroup's wavefronts (its consecutive KV heads) read
  // contiguous stretches of each position's KV row.
  const size_t rs = (size_t)a.Hkv * kHD;
  const int rk = lane >> 3, cd = (lane & 7) * 8;
  const uint16_t* kbase = a.k + (size_t)b * a.S * rs + g * kHD + cd;
  const uint16_t* vbase = a.v + (size_t)b * a.S * rs + g * kHD + cd;
  // two register slots: tile t in slot t % 2; a slot is refilled with tile t + 2
  // as soon as tile t's K and V have left it, so two tiles are in flight
  // while one is computed
  auto tile = [&](int t, u4v (&kc)[4], u4v (&vc)[4]) __attribute__((always_inline)) {
    // K rows -> LDS -> A operand (key lr, dims 16 j + 8 hf .. +7)
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u4v*>(&buf[(8 * i + rk) * kKS + cd]) = kc[i];
    wave_sync();
    v16f_a s = {};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v8bf kf = as_bf(*reinterpret_cast<const u4v*>(&buf[lr * kKS + 16 * j + 8 * hf]));
      const v8bf qf = as_bf(*reinterpret_cast<const u4v*>(&qs[lr * kKS + 16 * j + 8 * hf]));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, s, 0, 0, 0);
    }
    wave_sync();   // the K reads are done before V^T overwrites them
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) buf[(cd + e) * kVS + 8 * i + rk] = (uint16_t)(vc[i][e >> 1] >> (16 * (e & 1)));
    }
    if (t + 2 < ntile) dec_rows(kbase, vbase, rs, k0 + (t + 2) * kKT + rk, a.S, kc, vc);
    const int kb = k0 + t * kKT;
    v8bf pf[2];
    const bool full = kb + kKT <= k1 && kb + kKT - 1 <= qpos_lo && (a.window <= 0 || kb > qpos_hi - a.window);
    if (!full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = kb + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (!(sval && kj < k1 && kj <= qpos && (a.window <= 0 || kj > qpos - a.window))) s[i] = -INFINITY;
      }
    }
    softmax_tile(s, m, l, o0, o1, sc2, pf);
    wave_sync();   // the V^T tile written by every lane
    pv_tile(buf, lr, hf, pf, o0, o1);
    wave_sync();   // and read before the next tile's K overwrites it
  };
  u4v ka[4], va[4], kb2[4], vb2[4];
  if (ntile > 0) dec_rows(kbase, vbase, rs, k0 + rk, a.S, ka, va);
  if (ntile > 1) dec_rows(kbase, vbase, rs, k0 + kKT + rk, a.S, kb2, vb2);
  for (int t = 0; t < ntile; t += 2) {
    tile(t, ka, va);
    if (t + 1 < ntile) tile(t + 1, kb2, vb2);
  }

  if (a.nchunks == 1) {
    stage_out(buf, lr, hf, l, o0, o1);
    wave_sync();
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) {
      const int idx = p2 * 64 + lane, r = idx >> 3, col = (idx & 7) * 8, rq = r / G;
      if (rq < a.Tq)
        *reinterpret_cast<uint4*>(a.out + (((size_t)b * a.Tq + rq) * a.Hq + g * G + (r - rq * G)) * kHD + col) =
            *reinterpret_cast<const uint4*>(&buf[r * kHD + col]);
    }
  } else if (sval) {
    store_partial(a.part + ((((size_t)b * a.Tq + tq) * a.Hq + h) * a.nchunks + c) * kPS, hf, m, l, o0, o1);
  }
}

// out = (sum_c O_c 2^(m_c - M)) / (sum_c l_c 2^(m_c - M)), M = max_c m_c, chunks in
// order. One wavefront per output row (batch entry, query, head): lane c < nchunks
// reads chunk c's m and l, the row maximum is a wavefront reduction, and lane d
// sums dimension d over the chunks in order, the weights broadcast from their
// lanes and the loads of eight chunks issued together. Chunk 0 carries the sink,
// so M is finite. At most 64 chunks.
__global__ __launch_bounds__(256) void attn_merge(const AttnArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.B * a.Tq * a.Hq) return;
  const float* p = a.part + (size_t)row * a.nchunks * kPS;
  const float mc = lane < a.nchunks ? p[lane * kPS] : -INFINITY;
  const float lc = lane < a.nchunks ? p[lane * kPS + 1] : 0.0f;
  float M = mc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float w = mc == -INFINITY ? 0.0f : exp2f(mc - M);
  float L = 0.0f, O = 0.0f;
  int c = 0;
  for (; c + 8 <= a.nchunks; c += 8) {
    float ov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ov[j] = p[(c + j) * kPS + kPO + lane];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wj = __shfl(w, c + j), lj = __shfl(lc, c + j);
      L += lj * wj;
      O += ov[j] * wj;
    }
  }
  for (; c < a.nchunks; ++c) {
    const float wj = __shfl(w, c), lj = __shfl(lc, c);
    L += lj * wj;
    O += p[c * kPS + kPO + lane] * wj;
  }
  a.out[(size_t)row * kHD + lane] = f32_to_bf16(O / L);
}

struct AttnPlan {
  bool dec;          // attn_dec (G * Tq <= 32) or attn_fwd
  int nchunks, chunk, kofs;
};

AttnPlan attn_plan(int B, int Tq, int S, int Hq, int Hkv, int window) {
  const int G = Hq / Hkv;
  const bool dec = G * Tq <= kQB;
  // the keys any query sees start at kofs
  const int kofs = window > 0 ? max(0, S - Tq - window + 1) : 0;
  const int span = S - kofs, nt = (span + kKT - 1) / kKT;
  int n, maxn;
  if (dec) {
    n = (3072 + B * Hkv - 1) / (B * Hkv);            // 3072 wavefronts: 12 per CU, all resident
    maxn = (nt + 1) / 2;                              // >= 2 tiles per wavefront
  } else {
    const int blocks = B * Hkv * ((Tq + kQB - 1) / kQB);
    n = (1024 + blocks - 1) / blocks;
    maxn = (span + 255) / 256;                        // chunks of at least 256 keys
  }
  n = n > maxn ? maxn : n;
  n = n > 64 ? 64 : n;                                // attn_merge takes at most 64
  n = n < 1 ? 1 : n;
  const int chunk = ((nt + n - 1) / n) * kKT;
  return {dec, (span + chunk - 1) / chunk, chunk, kofs};
}

}  // namespace

size_t attention_workspace_bytes(int B, int Tq, int S, int Hq, int Hkv, int window) {
  const AttnPlan p = attn_plan(B, Tq, S, Hq, Hkv, window);
  return p.nchunks > 1 ? (size_t)B * Tq * Hq * p.nchunks * kPS * sizeof(float) : 0;
}

hipError_t launch_attention_sink(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* sinks, int B, int Tq, int S, int Hq, int Hkv,
                                 int window, float scale, uint16_t* out, void* ws,
                                 hipStream_t stream) {
  const AttnPlan p = attn_plan(B, Tq, S, Hq, Hkv, window);
  AttnArgs a{q, k, v, sinks, out, static_cast<float*>(ws), B, Tq, S, Hq, Hkv, window,
             p.nchunks, p.chunk, p.kofs, scale};
  const int G = Hq / Hkv;
  if (p.dec) {
    const int nw = Hkv < kDecW ? Hkv : kDecW;
    hipLaunchKernelGGL(attn_dec, dim3(B * ((Hkv + nw - 1) / nw), p.nchunks), dim3(nw * 64), 0, stream, a);
  } else {
    // x: batch entry and KV head, so consecutive workgroups (dealt out over the
    // chip's 8 L2 slices in turn) keep one KV head per slice when Hkv = 8
    const dim3 grid(B * Hkv, (Tq + kQB - 1) / kQB, p.nchunks);
    if (G >= 4)
      hipLaunchKernelGGL(attn_fwd<1>, grid, dim3(G * 64), 0, stream, a);
    else if (G >= 2)
      hipLaunchKernelGGL(attn_fwd<2>, grid, dim3(G * 64), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_fwd<4>, grid, dim3(G * 64), 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.nchunks == 1) return err;
  const int rows = B * Tq * Hq;
  hipLaunchKernelGGL(attn_merge, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
