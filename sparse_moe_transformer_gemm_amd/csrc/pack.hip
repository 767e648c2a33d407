// One-time repacking of MXFP4 expert weights from the OCP layout ([E][N][K/2]
// codes, [E][N][K/32] scales, K contiguous) into the MFMA-fragment layout the
// GEMMs stream (layout.hpp). A pure byte permutation: every code nibble and scale
// byte is copied unchanged; blocks past K are zero. Run at weight-load time, not
// per layer call.
#include "common.hpp"
#include "layout.hpp"

namespace moe {
namespace {

// One thread per 16-byte output piece: piece i = ((e*G + g)*S + j)*128 + s*64 + l
// holds row 32g + l%32, block 4j + 2*(l/32) + s of expert e (G = N/32 groups, S steps).
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ src, int K,
                                                         size_t pieces, int S,
                                                         uint8_t* __restrict__ dst) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int l = (int)(i & 63), s = (int)((i >> 6) & 1);
  const size_t rest = i >> 7;                  // (e*G + g)*S + j
  const int j = (int)(rest % (size_t)S);
  const size_t row = (rest / (size_t)S) * 32 + (l & 31);   // e*N + 32g + l%32
  const int blk = 4 * j + 2 * (l >> 5) + s;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (blk < K / 32) v = *reinterpret_cast<const uint4*>(src + row * (size_t)(K / 2) + (size_t)blk * 16);
  reinterpret_cast<uint4*>(dst)[i] = v;
}

// One thread per 2-byte output entry: entry i = ((e*G + g)*S + j)*64 + l holds the
// scales of row 32g + l%32, blocks 4j + 2*(l/32) and 4j + 2*(l/32) + 1.
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src, int K,
                                                          size_t entries, int S,
                                                          uint16_t* __restrict__ dst) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= entries) return;
  const int l = (int)(i & 63);
  const size_t rest = i >> 6;
  const int j = (int)(rest % (size_t)S);
  const size_t row = (rest / (size_t)S) * 32 + (l & 31);
  const int nblk = K / 32;
  const int b0 = 4 * j + 2 * (l >> 5);
  const uint8_t* r = src + row * (size_t)nblk;
  const uint32_t s0 = b0 < nblk ? r[b0] : 0u;
  const uint32_t s1 = b0 + 1 < nblk ? r[b0 + 1] : 0u;
  dst[i] = static_cast<uint16_t>(s0 | (s1 << 8));
}

}  // namespace

hipError_t launch_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                             uint8_t* codes_out, uint8_t* scales_out, hipStream_t stream) {
  const int S = nsteps_of(K);
  const size_t pieces = packed_codes_bytes(E, N, K) / 16;
  const size_t entries = packed_scales_bytes(E, N, K) / 2;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                     stream, codes, K, pieces, S, codes_out);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0,
                     stream, scales, K, entries, S, reinterpret_cast<uint16_t*>(scales_out));
  return hipGetLastError();
}

}  // namespace moe
