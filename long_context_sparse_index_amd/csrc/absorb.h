// Weight absorption of the query (q_lat = W_UK[h] q_nope per head), as one
// wave's share of the work; used by the absorb kernel and, for decode
// batches, by spare workgroups of the top-k finish kernel.
#pragma once

#include "dsa_common.h"

namespace dsa {

constexpr int kAbsorbStage = 32 * 40;  // bf16 per wave: a 32 x 32 output block, rows padded to 40

// One wave: latent columns c0 .. c0+31 of head h, for the 32-query tiles
// [tb0, tb1).  The wave keeps its W_UK fragments resident (B[k=d][n=c] =
// W_UK[h][c][d], contiguous 16-byte loads) and takes q_nope rows as A.  Each
// 32 x 32 output block is rounded to bf16 (nearest even), staged in the
// wave's LDS area `stage` (kAbsorbStage elements) and written as 16-byte
// pieces of q_lat rows.  q_lat [T, 64, 512] bf16.
__device__ __forceinline__ void absorb_wave(const uint16_t* __restrict__ q_nope,
                                            const uint16_t* __restrict__ w_uk,
                                            uint16_t* __restrict__ q_lat, int T, int h, int c0,
                                            int tb0, int tb1, uint16_t* stage) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, n = lane & 31;
  const int c = c0 + n;
  bf16x8 bw[kNope / 16];
  const uint16_t* bp = w_uk + ((int64_t)h * kLat + c) * kNope + 8 * g;
#pragma unroll
  for (int j = 0; j < kNope / 16; ++j) bw[j] = as_bf16x8(ld16(bp + 16 * j));
  for (int tb = tb0; tb < tb1; ++tb) {
    const int t = min(tb * 32 + n, T - 1);
    const uint16_t* ap = q_nope + ((int64_t)t * kHeads + h) * kNope + 8 * g;
    bf16x8 a[kNope / 16];
#pragma unroll
    for (int j = 0; j < kNope / 16; ++j) a[j] = as_bf16x8(ld16(ap + 16 * j));
    f32x16 acc = {};
#pragma unroll
    for (int j = 0; j < kNope / 16; ++j) acc = mfma32(a[j], bw[j], acc);
    // element r of lane (g, n): query row 8(r/4) + 4g + r%4 of the tile, column n
#pragma unroll
    for (int r = 0; r < 16; ++r)
      stage[(8 * (r >> 2) + 4 * g + (r & 3)) * 40 + n] = (uint16_t)f32_to_bf16_bits(acc[r]);
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // lane L writes 16 columns (half L & 1) of tile row L >> 1
    const int row = lane >> 1, half = lane & 1;
    const int tr = tb * 32 + row;
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(&stage[row * 40 + 16 * half]);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(&stage[row * 40 + 16 * half + 8]);
    if (tr < T) {
      uint16_t* dst = q_lat + ((int64_t)tr * kHeads + h) * kLat + c0 + 16 * half;
      st16(dst, v0);
      st16(dst + 8, v1);
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next tile's writes
  }
}

}  // namespace dsa
