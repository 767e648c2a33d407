// Shared device helpers and kernel launcher declarations (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Inclusive prefix sum of one int per thread over a workgroup of 256 threads:
// a shuffle scan inside each wavefront, then the totals of the wavefronts before
// it (two barriers instead of the sixteen of a Hillis-Steele scan through LDS).
// `tmp` is 4 ints of LDS; every thread of the workgroup must call it.
__device__ __forceinline__ int block_inclusive_scan256(int v, int* tmp) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) tmp[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += tmp[w];
  __syncthreads();  // tmp is free again for the caller's next scan
  return v + add;
}

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; arguments are validated by the caller.

size_t route_workspace_bytes(int T, int d, int E);
hipError_t launch_route(const uint16_t* x, const float* w_router, const float* b_router,
                        int T, int d, int E, int k, int32_t* topk_idx, float* topk_w,
                        void* ws, hipStream_t stream);

// The many-token routing (T > 64) that also writes x encoded for the expert
// GEMMs into xenc (rows of nsteps(d) * 208 bytes), as the FFN's own encode would;
// ws: route_workspace_bytes(T, d, E) of scratch (its partial logits).
hipError_t launch_route_encode(const uint16_t* x, const float* w_router, const float* b_router,
                               int T, int d, int E, int k, int32_t* topk_idx, float* topk_w,
                               uint8_t* xenc, void* ws, hipStream_t stream);

// Several chunks of pairs (T * k > 512): per-chunk histograms in the workspace
// (permute_workspace_bytes), then the ranks.
size_t permute_workspace_bytes(int T, int E, int k);
// With tiles (passes) non-null, the workgroup that writes the offsets also
// builds the expert GEMMs' 128-row tile table (16-row pass table) there, as the
// FFN's encode launch would.
hipError_t launch_permute(const int32_t* topk_idx, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* pair_row, void* ws,
                          hipStream_t stream, int4* tiles = nullptr, int4* passes = nullptr);

// Repack one [E][N][K] MXFP4 tensor from the OCP layout into the packed
// fragment layout (layout.hpp).
hipError_t launch_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                             uint8_t* codes_out, uint8_t* scales_out, hipStream_t stream);

struct FfnArgs {
  int T, d, F, E, k;
  const uint16_t* x;
  const int32_t* sorted_pair;
  const int32_t* offsets;
  // weights in the packed fragment layout
  const uint8_t *wg_codes, *wg_scales, *wu_codes, *wu_scales, *wd_codes, *wd_scales;
  const uint16_t *b_gate, *b_up, *b_down;
  float* y_sorted;
  void* ws;
};
size_t ffn_workspace_bytes(int T, int d, int F, int E, int k);
// Both expert GEMMs take the weight-streaming decode kernels at this shape.
bool ffn_decode_shape(int T, int d, int F);
// The down GEMM takes the weight-streaming kernel (T <= 64, or an output width
// that no prefill column tile divides); such widths then need F <= 4096, which
// ffn_supported checks.
bool ffn_down_decode(int T, int d, int F);
bool ffn_supported(int T, int d, int F);
// front_done: x is already encoded and the tile tables the GEMMs need are
// built in the workspace (by launch_forward_front at decode sizes, by
// launch_route_encode and launch_permute with the tile table otherwise).
hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream, bool front_done = false);
// Where launch_expert_ffn keeps the encoded x and the 128-row tile table in the
// workspace (for callers that fill them themselves).
uint8_t* ffn_xenc(const FfnArgs& a);
int4* ffn_tiles(const FfnArgs& a);
int4* ffn_passes(const FfnArgs& a);  // the 16-row pass table of the decode kernels
// The workspace past the FFN's regions (ffn_workspace_bytes from the start):
// where the whole-block call keeps the permutation's chunk histograms while the
// encoded x already sits in the FFN's region.
void* ffn_ws_end(const FfnArgs& a);
// One stage of it: 0 encodes x and builds the tile tables (nothing when
// front_done), 1 runs the gate/up GEMM with SwiGLU into the encoded h, 2 the
// down GEMM into y_sorted; the three in order are launch_expert_ffn.
hipError_t launch_expert_ffn_stage(const FfnArgs& a, hipStream_t stream, int stage, bool front_done = false);

// Fused route + permute + activation encode of the whole-block call, for the
// shapes where forward_front_fits; its scratch follows the FFN workspace and
// forward_front_bytes is the total.
bool forward_front_fits(int T, int d, int F, int k);
size_t forward_front_bytes(int T, int d, int F, int E, int k);
hipError_t launch_forward_front(const uint16_t* x, const float* w_router, const float* b_router,
                                int T, int d, int F, int E, int k, int32_t* topk_idx,
                                float* topk_w, int32_t* counts, int32_t* offsets,
                                int32_t* sorted_pair, int32_t* pair_row, void* ws,
                                hipStream_t stream);

// FP8-E4M3 expert weights with float32 128x128 block scales (fp8.hip). In FfnArgs
// the w*_codes point at packed FP8 codes and the w*_scales at the float32 block
// scales [E][ceil(N/128)][ceil(K/128)].
size_t fp8_packed_bytes(int E, int N, int K);
hipError_t launch_convert_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                                       uint8_t* out, float* bscale, hipStream_t stream);
hipError_t launch_pack_fp8(const uint8_t* codes, int E, int N, int K, uint8_t* out, hipStream_t stream);
hipError_t launch_expert_ffn_fp8(const FfnArgs& a, hipStream_t stream);
// Round n float32 values to the nearest bf16 (ties to even), in place.
hipError_t launch_round_bf16(float* w, int n, hipStream_t stream);

// Attention with per-head sinks (attention.hip): head size 64, Hq / Hkv <= 8.
size_t attention_workspace_bytes(int B, int Tq, int S, int Hq, int Hkv, int window);
hipError_t launch_attention_sink(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* sinks, int B, int Tq, int S, int Hq, int Hkv,
                                 int window, float scale, uint16_t* out, void* ws,
                                 hipStream_t stream);

// The allocation-free whole-block call's scratch: a device array of this many
// bytes per GPU (noalloc.hip); *ptr receives its address on the current device.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_combine(const float* y_sorted, const int32_t* pair_row, const float* topk_w,
                          int T, int d, int k, uint16_t* out, hipStream_t stream);

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gain, int T, int d, float eps,
                          uint16_t* out, hipStream_t stream);
hipError_t launch_residual_add(const uint16_t* x, const uint16_t* m, int T, int d,
                               uint16_t* out, hipStream_t stream);
// xout = bf16(x + m), then nout = RMSNorm(xout) with `gain`: the bytes of
// launch_residual_add followed by launch_rmsnorm, in one pass.
hipError_t launch_residual_rmsnorm(const uint16_t* x, const uint16_t* m, const uint16_t* gain, int T,
                                   int d, float eps, uint16_t* xout, uint16_t* nout,
                                   hipStream_t stream);

}  // namespace moe
