// Device-side data layouts shared by the weight packer, the activation encoders
// and the grouped GEMMs.
//
// K (the contraction dimension) is walked in steps of 128 elements, i.e. four
// 32-element MX blocks. A step of a 32x32x64 scaled MFMA pair (or of one
// 16x16x128 MFMA) consumes exactly one such step of A and of B.
//
// Packed MXFP4 weights (written once by moe_pack_mxfp4, read by every GEMM).
// A matrix W[N][K] of one expert is cut into 32-row groups g and K steps j; the
// (g, j) tile is stored as two 1 KB halves s = 0, 1, each being one B operand of
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 as the 64 lanes hold it:
//     codes[e][g][j][s][lane][16 B]  = the 32 E2M1 codes of row 32g + lane%32,
//                                      block 4j + 2*(lane/32) + s (nibble order as
//                                      in the raw layout: element 2i in the low
//                                      nibble of byte i)
//     scales[e][g][j][lane][2 B]     = E8M0 scales of that row's blocks
//                                      4j + 2*(lane/32) and 4j + 2*(lane/32) + 1
// Blocks past K (the second half of the last step when K % 128 == 64) hold zero
// codes and zero scale bytes (2^-127, finite), so they contribute nothing. One
// step of a 32-row group is then 2 KB of codes and 128 B of scales, each
// contiguous: a wavefront copies an operand with one fully coalesced 1 KB load.
// A 16x16x128 MFMA lane (column c, K sub-block kb) takes half s = kb % 2, lane
// 32*(kb/2) + c (+16 for the upper 16 rows of the group): four 256-byte runs.
//
// Encoded activations (x once per token, h once per dispatch row): per row, one
// 208-byte chunk per K step:
//     [4 blocks x 48 B codes: hi term 24 B, lo term 24 B, 6 bits per element]
//     [4 x uint16 scales: byte 0 hi E8M0, byte 1 lo E8M0][8 B unused]
// so a row's step is contiguous (13 pieces of 16 B) and a fragment lane's two
// blocks are one 96-byte run. Row pitch: nsteps(K) * 208 bytes. The second half
// of the last step when K % 128 == 64 is never written; readers mask it.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kStepK = 128;        // K elements per step
constexpr int kStepBlocks = 4;     // 32-element MX blocks per step
constexpr int kEncBytes = 48;      // encoded codes of one 32-element block (hi + lo)
constexpr int kChunk = 208;        // bytes of one row's step of encoded activations
constexpr int kChunkScales = 192;  // offset of the four uint16 scales in a chunk
constexpr int kChunkPieces = 13;   // 16-byte pieces per chunk
constexpr int kWStep = 2048;       // packed code bytes per (32-row group, step)
constexpr int kWSStep = 128;       // packed scale bytes per (32-row group, step)

__host__ __device__ inline int nsteps_of(int K) { return (K + kStepK - 1) / kStepK; }

// Bytes of the packed form of a [E][N][K] MXFP4 tensor.
inline size_t packed_codes_bytes(int E, int N, int K) {
  return (size_t)E * (N / 32) * nsteps_of(K) * kWStep;
}
inline size_t packed_scales_bytes(int E, int N, int K) {
  return (size_t)E * (N / 32) * nsteps_of(K) * kWSStep;
}

}  // namespace moe
