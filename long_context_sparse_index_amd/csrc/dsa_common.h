// Device helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kIdxHeads = 32;
constexpr int kIdxDim = 128;
constexpr int kHeads = 64;
constexpr int kNope = 192;
constexpr int kRope = 64;
constexpr int kQk = kNope + kRope;    // 256
constexpr int kV = 256;
constexpr int kLat = 512;
constexpr int kRow = kLat + kRope;    // 576 bf16 per latent-cache row
// INT4 latent-cache row: 256 B of codes (element 2i in the low nibble of byte
// i, two's complement), 8 bf16 group scales (groups of 64), 64 bf16 rope.
constexpr int kQ4Group = 64;
constexpr int kQ4ScaleOff = kLat / 2;                       // 256
constexpr int kQ4RopeOff = kQ4ScaleOff + 2 * kLat / kQ4Group;  // 272
constexpr int kQ4Row = kQ4RopeOff + 2 * kRope;              // 400 bytes
constexpr int kMaxTopk = 8192;    // largest index_topk accepted
constexpr int kTopkSmall = 2048;  // index_topk of the configuration tables; kernels specialise up to it

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16x2 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two fp32 -> packed bf16 (lo in bits 0..15), one hardware conversion
// (round to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource word 3 (gfx9: 32-bit data, no swizzle)

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// D = A(32x16) * B(16x32) + C.  Lane l supplies A row l%32 and B column l%32,
// each with 8 K-elements for K-group l/32.  Output element j of lane l is
// C[8*(j/4) + 4*(l/32) + j%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D = A(16x32) * B(32x16) + C.  Lane l supplies A row l%16 and B column l%16,
// each with 8 K-elements for K-group l/16.  Output element j of lane l is
// C[4*(l/16) + j][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max(x, 0) for fp32 in one integer instruction: negative values (and -0.0)
// have negative int images, +0.0 is int 0.  (fmaxf costs a canonicalize plus
// a max in IEEE mode.)  Inputs are finite.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Lane exchange within a wave (ds_bpermute based).
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ int xor_lane(int v, int mask) { return __shfl_xor(v, mask, 64); }

// Monotone unsigned image of an fp32 score: larger float <-> larger key, and
// -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // +-0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Float threshold of a key bound: for every non-NaN f, score_key(f) >= K
// exactly when f >= key_floor(K) (float order, -0 == +0).  K above the key of
// +inf gives NaN, which no compare satisfies.
__device__ __forceinline__ float key_floor(uint32_t K) {
  if (K & 0x80000000u) {
    const uint32_t b = K & 0x7FFFFFFFu;
    return b > 0x7F800000u ? __uint_as_float(0x7FC00000u) : __uint_as_float(b);
  }
  return K <= 0x007FFFFFu ? -INFINITY : __uint_as_float(~K);
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers (DPP):
// Hillis-Steele shifts of 1, 2, 4, 8 lanes inside each 16-lane row (sources
// outside the row read 0), then row 0's total is added to row 1 and row 2's
// to row 3 (row_bcast:15), and the total of rows 0-1 to rows 2 and 3
// (row_bcast:31).  A lane that a step does not write keeps `old` = 0.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its global loads and stores (__syncthreads also drains those, which
// would cancel any load issued ahead of the barrier).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan(v), 63);
}

}  // namespace dsa
