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
// attn_fwd, in the style of FlashAttention-2 on gfx950's bf16 matrix cores. A
// workgroup takes 32 consecutive queries of one batch entry and one KV head,
// with one wavefront per query head of the group (up to 8; they share every K/V tile,
// which is staged once in LDS), and one chunk of the keys. Per 32-key tile a
// wavefront computes S^T = K Q^T (32 keys x 32 queries, four 32x32x16 bf16
// MFMAs over the head size 64), so each lane holds one query's 16 keys and a
// query's running max and sum need one cross-half shuffle; then the online
// softmax update (in base 2, log2(e) folded into the scale) and O^T += V^T P^T,
// P^T taken from the S^T accumulators as bf16. In the accumulator a lane l
// holds query l%32 and keys 8(i/4) + 4(l/32) + i%4 (i = 0..15); the matrix
// instruction pairs element t of A's lane half with element t of B's, so the
// V^T operand of MFMA c (keys 16c .. 16c+15) lists, for lane half h, the keys
// its P^T registers 8c .. 8c+7 hold: 16c + 8(t/4) + 4h + t%4.
// A single chunk normalises and stores bf16 output; several chunks store the
// partial (running max, denominator, unnormalised output) and attn_merge adds
// them in chunk order.
#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f_a __attribute__((ext_vector_type(16)));

constexpr int kHD = 64;      // head size
constexpr int kQB = 32;      // queries per workgroup
constexpr int kKT = 32;      // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const uint16_t *q, *k, *v;
  const float* sinks;
  uint16_t* out;
  float* part;          // [B][Tq][Hq][nchunks][2 + 64] when nchunks > 1
  int B, Tq, S, Hq, Hkv, window, nchunks, chunk;
  float scale;
};

__device__ __forceinline__ v8bf as_bf(uint4 u) {
  union {
    uint4 u;
    v8bf b;
  } c;
  c.u = u;
  return c.b;
}

__global__ __launch_bounds__(512) void attn_fwd(const AttnArgs a) {
  const int G = a.Hq / a.Hkv;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kKT * kHD];   // [key][dim]
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kHD * kKT];   // [dim][key]
  __shared__ __attribute__((aligned(16))) uint16_t ost[8][kQB * kHD];  // output staging per wave
  const int qb = blockIdx.x, bg = blockIdx.y, c = blockIdx.z;
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
  int k0 = c * a.chunk, k1 = min(a.S, k0 + a.chunk);
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

  // K/V tile loads: threads [0, 256) one 16-byte piece of K each, [256, 512) of V
  const bool loader = tid < 512;
  const int piece = tid & 255, pkey = piece >> 3, pdim = (piece & 7) * 8;
  auto gload = [&](int t) -> uint4 {
    const int key = min(k0 + t * kKT + pkey, a.S - 1);
    const uint16_t* src = (tid < 256 ? a.k : a.v) + (((size_t)b * a.S + key) * a.Hkv + g) * kHD + pdim;
    return *reinterpret_cast<const uint4*>(src);
  };
  auto lstore = [&](int buf, uint4 u) {
    if (tid < 256) {
      *reinterpret_cast<uint4*>(&ks[buf][pkey * kHD + pdim]) = u;
    } else {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) vt[buf][(pdim + t) * kKT + pkey] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
    }
  };
  uint4 pre = make_uint4(0u, 0u, 0u, 0u);
  if (ntile > 0 && loader && nthr >= 512) lstore(0, gload(0));
  // fewer than 512 threads (G < 8): the tile is loaded in several rounds
  if (ntile > 0 && nthr < 512) {
    for (int p2 = tid; p2 < 512; p2 += nthr) {
      const int pc = p2 & 255, key = min(k0 + (pc >> 3), a.S - 1), dim = (pc & 7) * 8;
      const uint4 u = *reinterpret_cast<const uint4*>((p2 < 256 ? a.k : a.v) +
                                                      (((size_t)b * a.S + key) * a.Hkv + g) * kHD + dim);
      if (p2 < 256) *reinterpret_cast<uint4*>(&ks[0][(pc >> 3) * kHD + dim]) = u;
      else {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        for (int t = 0; t < 8; ++t) vt[0][(dim + t) * kKT + (pc >> 3)] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
      }
    }
  }
  __syncthreads();

  for (int t = 0; t < ntile; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntile;
    if (more && loader && nthr >= 512) pre = gload(t + 1);
    // S^T = K Q^T over the head size
    v16f_a s = {};
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const v8bf kf = as_bf(*reinterpret_cast<const uint4*>(&ks[buf][lr * kHD + 16 * ks2 + 8 * hf]));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks2], s, 0, 0, 0);
    }
    // mask, tile max, online update
    const int kb = k0 + t * kKT;
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kj = kb + 8 * (i >> 2) + 4 * hf + (i & 3);
      const bool vis = qvalid && kj < k1 && kj <= qpos && (a.window <= 0 || kj > qpos - a.window);
      s[i] = vis ? s[i] * sc2 : -INFINITY;
      tmax = fmaxf(tmax, s[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);
    const float base = mn == -INFINITY ? 0.0f : mn;
    const float alpha = exp2f(m - base);
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = exp2f(s[i] - base);
      psum += s[i];
    }
    psum += __shfl_xor(psum, 32);
    l = l * alpha + psum;
    m = mn;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o0[i] *= alpha;
      o1[i] *= alpha;
    }
    // O^T += V^T P^T: two 16-key MFMAs per 32-dim half
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      v8bf pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (__bf16)s[8 * c2 + e];
      // keys of V^T's element t: 16 c2 + 8 (t / 4) + 4 hf + t % 4 -> two runs of 4
      const int key0 = 16 * c2 + 4 * hf;
      const uint2 v0a = *reinterpret_cast<const uint2*>(&vt[buf][lr * kKT + key0]);
      const uint2 v0b = *reinterpret_cast<const uint2*>(&vt[buf][lr * kKT + key0 + 8]);
      const uint2 v1a = *reinterpret_cast<const uint2*>(&vt[buf][(32 + lr) * kKT + key0]);
      const uint2 v1b = *reinterpret_cast<const uint2*>(&vt[buf][(32 + lr) * kKT + key0 + 8]);
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(make_uint4(v0a.x, v0a.y, v0b.x, v0b.y)), pf, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(make_uint4(v1a.x, v1a.y, v1b.x, v1b.y)), pf, o1, 0, 0, 0);
    }
    __syncthreads();   // every wave is done with buffer buf^1 (read in tile t-1)
    if (more) {
      if (nthr >= 512) {
        if (loader) lstore(buf ^ 1, pre);
      } else {
        for (int p2 = tid; p2 < 512; p2 += nthr) {
          const int pc = p2 & 255, key = min(k0 + (t + 1) * kKT + (pc >> 3), a.S - 1), dim = (pc & 7) * 8;
          const uint4 u = *reinterpret_cast<const uint4*>((p2 < 256 ? a.k : a.v) +
                                                          (((size_t)b * a.S + key) * a.Hkv + g) * kHD + dim);
          if (p2 < 256) *reinterpret_cast<uint4*>(&ks[buf ^ 1][(pc >> 3) * kHD + dim]) = u;
          else {
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
            for (int t2 = 0; t2 < 8; ++t2)
              vt[buf ^ 1][(dim + t2) * kKT + (pc >> 3)] = (uint16_t)(w[t2 >> 1] >> (16 * (t2 & 1)));
          }
        }
      }
    }
    __syncthreads();
  }

  // lane l holds query l%32, dims 8(i/4) + 4 hf + i%4 (+32 in o1)
  if (a.nchunks == 1) {
    const float inv = 1.0f / l;
    uint16_t* st = ost[wave];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 8 * (i >> 2) + 4 * hf + (i & 3);
      st[lr * kHD + d] = f32_to_bf16(o0[i] * inv);
      st[lr * kHD + 32 + d] = f32_to_bf16(o1[i] * inv);
    }
    __builtin_amdgcn_wave_barrier();
    // 32 queries x 128 B: 4 passes of 16 bytes per lane
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) {
      const int idx = p2 * 64 + lane, row = idx >> 3, col = (idx & 7) * 8;
      if (q0 + row < a.Tq)
        *reinterpret_cast<uint4*>(a.out + (((size_t)b * a.Tq + q0 + row) * a.Hq + h) * kHD + col) =
            *reinterpret_cast<const uint4*>(&st[row * kHD + col]);
    }
  } else if (qvalid) {
    float* p = a.part + ((((size_t)b * a.Tq + qi) * a.Hq + h) * a.nchunks + c) * (2 + kHD);
    if (hf == 0) {
      p[0] = m;
      p[1] = l;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 8 * (i >> 2) + 4 * hf + (i & 3);
      p[2 + d] = o0[i];
      p[2 + 32 + d] = o1[i];
    }
  }
}

// out = (sum_c O_c 2^(m_c - M)) / (sum_c l_c 2^(m_c - M)), M = max_c m_c, chunks in
// order; one thread per output element. Chunk 0 carries the sink, so M is finite.
__global__ __launch_bounds__(256) void attn_merge(const AttnArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n = (size_t)a.B * a.Tq * a.Hq * kHD;
  if (i >= n) return;
  const size_t row = i / kHD;
  const int d = (int)(i - row * kHD);
  const float* p = a.part + row * a.nchunks * (2 + kHD);
  float M = -INFINITY;
  for (int c = 0; c < a.nchunks; ++c) M = fmaxf(M, p[c * (2 + kHD)]);
  float L = 0.0f, O = 0.0f;
  for (int c = 0; c < a.nchunks; ++c) {
    const float* pc = p + c * (2 + kHD);
    const float w = pc[0] == -INFINITY ? 0.0f : exp2f(pc[0] - M);
    L += pc[1] * w;
    O += pc[2 + d] * w;
  }
  a.out[i] = f32_to_bf16(O / L);
}

struct AttnPlan {
  int nchunks, chunk;
};

AttnPlan attn_plan(int B, int Tq, int S, int Hkv) {
  const int blocks = B * Hkv * ((Tq + kQB - 1) / kQB);
  int n = (1024 + blocks - 1) / blocks;             // aim at >= 1024 workgroups
  const int maxn = (S + 255) / 256;                  // chunks of at least 256 keys
  n = n < 1 ? 1 : (n > maxn ? maxn : n);
  const int chunk = ((S + n - 1) / n + kKT - 1) / kKT * kKT;
  return {(S + chunk - 1) / chunk, chunk};
}

}  // namespace

size_t attention_workspace_bytes(int B, int Tq, int S, int Hq, int Hkv) {
  const AttnPlan p = attn_plan(B, Tq, S, Hkv);
  return p.nchunks > 1 ? (size_t)B * Tq * Hq * p.nchunks * (2 + kHD) * sizeof(float) : 0;
}

hipError_t launch_attention_sink(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* sinks, int B, int Tq, int S, int Hq, int Hkv,
                                 int window, float scale, uint16_t* out, void* ws,
                                 hipStream_t stream) {
  const AttnPlan p = attn_plan(B, Tq, S, Hkv);
  AttnArgs a{q, k, v, sinks, out, static_cast<float*>(ws), B, Tq, S, Hq, Hkv, window,
             p.nchunks, p.chunk, scale};
  const int G = Hq / Hkv;
  hipLaunchKernelGGL(attn_fwd, dim3((Tq + kQB - 1) / kQB, B * Hkv, p.nchunks), dim3(G * 64), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.nchunks == 1) return err;
  const size_t n = (size_t)B * Tq * Hq * kHD;
  hipLaunchKernelGGL(attn_merge, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
