// MFMA / LDS helpers shared by the prefill kernels (gfx950, wave64).
#pragma once

#include "zg_common.hpp"

namespace zg {

constexpr int kWaves = 8;                  // waves per prefill workgroup
constexpr int kThreads = kWaves * 64;

// v_mfma_f32_32x32x16_bf16. Lane l supplies A[l % 32][8 (l / 32) + j] and B[8 (l / 32) + j][l % 32]
// (j = 0..7); accumulator register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8 a, const bf16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i % 4) of the 8-byte
// rows addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ i16x4 lds_read_tr(const unsigned char* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Work item of workgroup `block` in a grid of n_tiles tiles x per_pair (sequence, KV head) pairs,
// tile index 0 being the heaviest. Workgroup i runs on XCD i mod 8; when the pairs split evenly
// over the 8 XCDs, each XCD walks its pairs one at a time (all tiles of a pair, heaviest first), so
// the workgroups resident on an XCD stream the same rows through its L2. Otherwise tile-major.
__device__ __forceinline__ void xcd_pair_major(int block, int per_pair, int n_tiles, int& tile,
                                               int& pair) {
  if (per_pair % 8 == 0) {
    const int j = block >> 3;
    const int pl = j / n_tiles;
    tile = j - pl * n_tiles;
    pair = (block & 7) + 8 * pl;
  } else {
    tile = block / per_pair;
    pair = block - tile * per_pair;
  }
}

}  // namespace zg
