// INT4 latent cache: quantisation of bf16 cache rows.
//
// Page "GLM-5 7440亿参数，202K长上下文突破极限", section 六, recommends INT4 KV-cache
// quantisation for 202K contexts (a saving of more than 60%); it fixes no
// format.  Row format (400 bytes, 35% of a 1152-byte bf16 row): the 512 latent
// values in 8 groups of 64 with one bf16 scale per group, 4-bit two's
// complement codes (element 2i in the low nibble of byte i); the 64 rope
// values stay bf16.  Per group: s = bf16(absmax / 7), q = clamp(rint(x / s),
// -7, 7) (divisions correctly rounded in fp32, ties to even; s = 0 gives
// q = 0).  The MLA core dequantises q * s while gathering.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

// One wave per row: lane l holds latent elements 8l .. 8l+7 (group l / 8).
// Grid-stride over rows (a grid of at most kQuantMaxWgs workgroups of 4 waves).
constexpr int64_t kQuantMaxWgs = 1 << 20;

__device__ __forceinline__ void quantize_row(const uint16_t* __restrict__ kv, int64_t row,
                                             uint8_t* __restrict__ out, int lane) {
  const uint16_t* src = kv + row * kRow;
  uint8_t* dst = out + row * kQ4Row;
  const u32x4 v = ld16(src + 8 * lane);
  float x[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    x[2 * m] = bf16_to_f32((uint16_t)(v[m] & 0xFFFFu));
    x[2 * m + 1] = bf16_to_f32((uint16_t)(v[m] >> 16));
  }
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[e]));
  am = fmaxf(am, xor_lane(am, 1));  // the 8 lanes of a group
  am = fmaxf(am, xor_lane(am, 2));
  am = fmaxf(am, xor_lane(am, 4));
  const uint32_t sbits = f32_to_bf16_bits(__fdiv_rn(am, 7.0f));
  const float sc = bf16_to_f32((uint16_t)sbits);
  uint32_t code = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float q = sc > 0.f ? rintf(__fdiv_rn(x[e], sc)) : 0.f;
    q = fminf(fmaxf(q, -7.f), 7.f);
    code |= ((uint32_t)(int)q & 0xFu) << (4 * e);
  }
  *reinterpret_cast<uint32_t*>(dst + 4 * lane) = code;
  if ((lane & 7) == 0) *reinterpret_cast<uint16_t*>(dst + kQ4ScaleOff + 2 * (lane >> 3)) = (uint16_t)sbits;
  if (lane < 8) *reinterpret_cast<u32x4*>(dst + kQ4RopeOff + 16 * lane) = ld16(src + kLat + 8 * lane);
}

__global__ __launch_bounds__(256) void quantize_kv_int4_kernel(const uint16_t* __restrict__ kv, int64_t rows,
                                                               uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += stride)
    quantize_row(kv, row, out, lane);
}

hipError_t launch_quantize_kv_int4(const uint16_t* kv, int64_t rows, uint8_t* out, hipStream_t st) {
  const int64_t wgs = (rows + 3) / 4 < kQuantMaxWgs ? (rows + 3) / 4 : kQuantMaxWgs;
  quantize_kv_int4_kernel<<<(unsigned)wgs, 256, 0, st>>>(kv, rows, out);
  return hipGetLastError();
}

}  // namespace dsa
