// MX helpers for gfx950's scaled matrix cores.
//
// The expert weights are MXFP4 (E2M1 codes, one E8M0 scale per 32 K-elements) and
// feed V_MFMA_SCALE_F32_32X32X64_F8F6F4 directly as the B operand. The A operand
// (activations) must be FP8/FP6/FP4 too; a single 6-bit term loses too much, so
// each 32-element block is stored as two MXFP6-E2M3 terms, hi + lo, each with its
// own E8M0 scale, and both terms go through the same MFMA accumulator:
//   hi = RNE_E2M3(v / 2^s1) with s1 = floor(log2 max|v|) - 2   (|hi| <= 7.5, saturated)
//   r  = v - hi * 2^s1          (exact in fp32)
//   lo = RNE_E2M3(r / 2^s2) with s2 = floor(log2 max|r|) - 2
// The pair carries about 8 significant bits relative to the block's largest
// element, like bf16 does per element.
//
// Register layout of the 32x32x64 scaled MFMA (checked on gfx950 with random
// operands): lane l supplies row (A) / column (B) l%32 and K elements
// 32*(l/32) .. 32*(l/32)+31; element j sits at bits [w*j, w*j+w) of the
// little-endian concatenation of the operand VGPRs (w = 6 for FP6 in 6 VGPRs,
// w = 4 for FP4 in 4 VGPRs); the lane's scale VGPR supplies the E8M0 byte picked
// by op_sel (value 2^(s-127)) for its 32 elements. The 16 fp32 results of lane l
// are column l%32, rows 8*(i/4) + 4*(l/32) + (i%4) for i = 0..15.
#pragma once

#include "common.hpp"
#include "layout.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

// MFMA operands built from loads without register copies: the FP6 operand uses
// 6 of its 8 registers and the FP4 operand 4; the unused ones are left undefined
// (shuffle index -1) rather than zeroed, so every load can land directly in the
// operand's registers.
__device__ __forceinline__ v8i fp6_operand(v4i w03, v2i w45) {
  const v4i t = __builtin_shufflevector(w45, w45, 0, 1, -1, -1);
  return __builtin_shufflevector(w03, t, 0, 1, 2, 3, 4, 5, -1, -1);
}
__device__ __forceinline__ v8i fp6_operand(v2i w01, v4i w25) {
  const v4i t = __builtin_shufflevector(w01, w01, 0, 1, -1, -1);
  return __builtin_shufflevector(t, w25, 0, 1, 4, 5, 6, 7, -1, -1);
}
__device__ __forceinline__ v8i fp4_operand(v4i w) {
  return __builtin_shufflevector(w, w, 0, 1, 2, 3, -1, -1, -1, -1);
}
// One encoded 32-element block in LDS (48 bytes at p, 16-byte aligned): hi term
// in bytes 0..23, lo term in bytes 24..47. The lo term is read through an LDS
// address the compiler cannot relate to p, so that it does not fuse the hi
// term's last 8 bytes and the lo term's first 8 into one 16-byte read (which
// would then need register copies to assemble the operands, and those copies
// wait for the read).
typedef __attribute__((address_space(3))) const v4i lds_v4i;
typedef __attribute__((address_space(3))) const v2i lds_v2i;
__device__ __forceinline__ void load_block_terms(const uint8_t* p, v8i& hi, v8i& lo) {
  const uint32_t a = (uint32_t)(size_t)(__attribute__((address_space(3))) const uint8_t*)p;
  uint32_t b = a + 24;
  asm volatile("" : "+v"(b));
  hi = fp6_operand(*(lds_v4i*)(size_t)a, *(lds_v2i*)(size_t)(a + 16));
  lo = fp6_operand(*(lds_v2i*)(size_t)b, *(lds_v4i*)(size_t)(b + 8));
}

// The hi and the lo term of that block separately (for reads spread among MFMAs).
__device__ __forceinline__ v8i load_term_hi(const uint8_t* p) {
  const uint32_t a = (uint32_t)(size_t)(__attribute__((address_space(3))) const uint8_t*)p;
  return fp6_operand(*(lds_v4i*)(size_t)a, *(lds_v2i*)(size_t)(a + 16));
}
__device__ __forceinline__ v8i load_term_lo(const uint8_t* p) {
  uint32_t b = (uint32_t)(size_t)(__attribute__((address_space(3))) const uint8_t*)p + 24;
  asm volatile("" : "+v"(b));
  return fp6_operand(*(lds_v2i*)(size_t)b, *(lds_v4i*)(size_t)(b + 8));
}

// The same two terms from three 16-byte LDS reads of the block's 48 bytes (no
// 8-byte reads: with the decode window's row pitch, 16-byte reads by 16 lanes of
// different rows and one K sub-block cover distinct banks, while 8-byte reads of
// two sub-blocks at once collide).
__device__ __forceinline__ void load_block_terms3(const uint8_t* p, v8i& hi, v8i& lo) {
  const uint32_t a = (uint32_t)(size_t)(__attribute__((address_space(3))) const uint8_t*)p;
  const v4i r0 = *(lds_v4i*)(size_t)a;
  const v4i r1 = *(lds_v4i*)(size_t)(a + 16);
  const v4i r2 = *(lds_v4i*)(size_t)(a + 32);
  hi = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, -1, -1);
  lo = __builtin_shufflevector(r1, r2, 2, 3, 4, 5, 6, 7, -1, -1);
}

// 2^n for n in [-127, 127] as an fp32 (2^-127 is subnormal).
__device__ __forceinline__ float pow2i(int n) {
  return n >= -126 ? __uint_as_float(static_cast<uint32_t>(n + 127) << 23)
                   : __uint_as_float(0x00400000u);
}

// floor(log2 a) for a normal positive float; -127 for zero/subnormal input.
__device__ __forceinline__ int ilog2f(float a) {
  return static_cast<int>((__float_as_uint(a) >> 23) & 255u) - 127;
}

// E2M3 magnitude code of |q| (already divided by the block scale), round to
// nearest even, saturating at 7.5. Magnitudes: code/8 below 2, 2 + (code-16)/4
// in [2, 4), 4 + (code-24)/2 in [4, 7.5]; all divisions here are exact.
__device__ __forceinline__ uint32_t e2m3_code(float a) {
  int c;
  if (a < 2.0f) {
    c = static_cast<int>(rintf(a * 8.0f));
  } else if (a < 4.0f) {
    c = 16 + static_cast<int>(rintf((a - 2.0f) * 4.0f));
  } else {
    c = 24 + static_cast<int>(rintf((a - 4.0f) * 2.0f));
    c = c > 31 ? 31 : c;
  }
  return static_cast<uint32_t>(c);
}

__device__ __forceinline__ float e2m3_value(uint32_t c) {
  const float f = static_cast<float>(c);
  return c < 16u ? f * 0.125f : (c < 24u ? 2.0f + (f - 16.0f) * 0.25f : 4.0f + (f - 24.0f) * 0.5f);
}

__device__ __forceinline__ void pack6(const uint32_t (&c)[32], uint32_t (&w)[6]) {
#pragma unroll
  for (int i = 0; i < 6; ++i) w[i] = 0u;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int bit = 6 * j, word = bit >> 5, off = bit & 31;
    w[word] |= c[j] << off;
    if (off > 26) w[word + 1] |= c[j] >> (32 - off);
  }
}

// Block exponent of a two-term block: floor(log2 amax) - 2 puts the largest
// magnitude in [4, 8) of the E2M3 range; blocks whose maximum is below 2^-124
// (zero blocks included) get the smallest normal scale 2^-126.
__device__ __forceinline__ int block_exp(float amax) {
  const int s = ilog2f(amax) - 2;
  return s < -126 ? -126 : s;
}

typedef uint32_t v6u __attribute__((ext_vector_type(6)));
typedef float v32f __attribute__((ext_vector_type(32)));

// Encode one block of 32 floats into two E2M3 terms (codes) and their scales,
// with the gfx950 scaled conversions: V_CVT_SCALEF32_2XPK16_FP6_F32 divides by
// the scale, rounds to nearest even and saturates at 7.5, packing its first
// operand into the even and its second into the odd element positions;
// V_CVT_SCALEF32_PK32_F32_FP6 decodes the 32 codes back (times the scale), so
// the residual v - hi is exact.
__device__ __forceinline__ void encode_block(const float (&v)[32], uint32_t (&hi)[6],
                                             uint32_t (&lo)[6], uint32_t& scales) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int s1 = block_exp(amax);
  const float sc1 = pow2i(s1);
  v16f ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = v[2 * i];
    od[i] = v[2 * i + 1];
  }
  const v6u h = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, sc1);
  const v32f back = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(h, sc1);
  float ramax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = v[2 * i] - back[2 * i];
    od[i] = v[2 * i + 1] - back[2 * i + 1];
    ramax = fmaxf(ramax, fmaxf(fabsf(ev[i]), fabsf(od[i])));
  }
  const int s2 = block_exp(ramax);
  const v6u l = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, pow2i(s2));
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    hi[i] = h[i];
    lo[i] = l[i];
  }
  scales = static_cast<uint32_t>(s1 + 127) | (static_cast<uint32_t>(s2 + 127) << 8);
}

// The same encoding from the block's even-indexed elements (ev[i] = element 2i)
// and odd-indexed ones (od[i] = element 2i+1), the operand order of the
// conversions, so that no register copies are needed to form them.
__device__ __forceinline__ void encode_block_eo(const v16f& ev, const v16f& od, uint32_t (&hi)[6],
                                                uint32_t (&lo)[6], uint32_t& scales) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = fmaxf(amax, fabsf(ev[i]));
    amax = fmaxf(amax, fabsf(od[i]));
  }
  const int s1 = block_exp(amax);
  const float sc1 = pow2i(s1);
  const v6u h = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, sc1);
  const v32f back = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(h, sc1);
  v16f re, ro;
  float ramax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    re[i] = ev[i] - back[2 * i];
    ro[i] = od[i] - back[2 * i + 1];
    ramax = fmaxf(ramax, fabsf(re[i]));
    ramax = fmaxf(ramax, fabsf(ro[i]));
  }
  const int s2 = block_exp(ramax);
  const v6u l = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(re, ro, pow2i(s2));
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    hi[i] = h[i];
    lo[i] = l[i];
  }
  scales = static_cast<uint32_t>(s1 + 127) | (static_cast<uint32_t>(s2 + 127) << 8);
}

// The same encoding done by a group of 32 lanes (a half wavefront), one element
// per lane: j = lane & 31 holds element j of the block. The block maxima are
// shuffle reductions inside the half wavefront; the 6-bit codes are packed
// through `scratch` (64 bytes of LDS per group) and 12 lanes store the 48-byte
// record (lane j < 6: hi word j, 6 <= j < 12: lo word j-6) plus lane 0 the scales.
// Every thread of the workgroup must call it (it contains a barrier); `store`
// false computes without writing (rows past the count).
__device__ __forceinline__ void encode_group32(float v, uint8_t* scratch, uint8_t* dst_codes,
                                               uint16_t* dst_scales, bool store) {
  const int j = threadIdx.x & 31;
  float amax = fabsf(v);
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const int s1 = block_exp(amax);
  const uint32_t m1 = e2m3_code(fabsf(v) * pow2i(-s1));
  const uint32_t sign1 = __float_as_uint(v) >> 31;
  const float back = e2m3_value(m1) * pow2i(s1);
  const float r = v - (sign1 ? -back : back);
  float ramax = fabsf(r);
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) ramax = fmaxf(ramax, __shfl_xor(ramax, o));
  const int s2 = block_exp(ramax);
  const uint32_t m2 = e2m3_code(fabsf(r) * pow2i(-s2));
  scratch[j] = static_cast<uint8_t>((sign1 << 5) | m1);
  scratch[32 + j] = static_cast<uint8_t>(((__float_as_uint(r) >> 31) << 5) | m2);
  __syncthreads();
  if (store && j < 12) {
    const uint8_t* c = scratch + (j < 6 ? 0 : 32);
    const int w = j < 6 ? j : j - 6;   // word w holds bits [32w, 32w+32) of the 192-bit field
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 7; ++t) {
      const int code = (32 * w) / 6 + t;       // codes overlapping this word
      if (code < 32) {
        const int bit = 6 * code - 32 * w;     // position of the code's bit 0 in the word
        const uint32_t cv = c[code];
        if (bit >= 0 && bit < 32) word |= cv << bit;
        else if (bit < 0 && bit > -6) word |= cv >> (-bit);
      }
    }
    reinterpret_cast<uint32_t*>(dst_codes)[j] = word;
    if (j == 0)
      *dst_scales = static_cast<uint16_t>((s1 + 127) | ((s2 + 127) << 8));
  }
  __syncthreads();
}

__device__ __forceinline__ void store_enc(uint8_t* dst_codes, const uint32_t (&hw)[6],
                                          const uint32_t (&lw)[6]) {
  uint4* dst = reinterpret_cast<uint4*>(dst_codes);
  dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  dst[1] = make_uint4(hw[4], hw[5], lw[0], lw[1]);
  dst[2] = make_uint4(lw[2], lw[3], lw[4], lw[5]);
}

// ------------------------------------------------------------------ buffer loads
// Raw buffer loads: a 128-bit resource (base, size in bytes) held in SGPRs plus a
// 32-bit per-lane byte offset. Offsets at or past the size read as zero without
// touching memory, which is how out-of-range K blocks and rows are padded.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword3 0x00020000: raw (untyped) 32-bit data, the usual value on CDNA
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// `off` is the per-lane byte offset (VGPR), `soff` an optional wave-uniform one
// (SGPR); a lane whose `off` is kOutOfRange reads zero.
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  return make_uint4(t[0], t[1], t[2], t[3]);
}
// The same with the non-temporal cache policy (nt): for data read once, so that
// it does not displace reusable lines.
__device__ __forceinline__ uint4 bload16nt(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 2);
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}
__device__ __forceinline__ uint32_t bload2(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}
__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, soff, 0);
}
// Every resource here is < 1 GiB and every uniform offset < 1 GiB, so a lane
// offset of 2^31 stays out of range whatever uniform offset is added to it.
constexpr uint32_t kOutOfRange = 0x80000000u;

// D += A(FP6 E2M3, scale byte OPA of sa) x B(FP4 E2M1, scale byte 0 of sb).
template <int OPA>
__device__ __forceinline__ v16f mfma_f6f4(const v8i& a, const v8i& b, const v16f& c, int sa,
                                          int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 4, OPA, sa, 0, sb);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

}  // namespace moe
