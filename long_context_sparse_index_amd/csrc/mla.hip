// Sparse MLA over the selected positions on gfx950 (weight-absorbed form).
//
// For query t, head h and kept cache rows (c_j | r_j):
//   z_j = scale * (q_nope[t,h] . (c_j W_UK[h]) + q_rope[t,h] . r_j)
//   out[t,h] = sum_j softmax(z)_j (c_j W_UV[h])
// (page "（五）一万亿次点积砍到两千次：DSA 怎么破 N²", DSA flow: full Q.K.V over the kept
// tokens, softmax, weighted V; page "2026大模型架构概览（二）：GLM 5 DSV3.2 的 DSA 与 MoE
// 配置拆解", §2.1 dims and §2.2: DSA is a filter in front of MLA.)
// Computed as
//   absorb   q_lat[t,h] = W_UK[h] q_nope[t,h]                (bf16 out)
//   core     logits against the 512-d latent + 64-d rope key, online softmax,
//            o_lat[t,h] = sum_j p_j c_j                       (split over keys)
//   merge    combine key splits (log-sum-exp)                 (bf16 out)
//   upproj   out[t,h] = o_lat[t,h] W_UV[h]
#include <type_traits>

#include "absorb.h"
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

// ---------------------------------------------------------------- absorb
// Few queries (up to 2 tiles of 32): grid (64 heads, query groups of
// kAbsorbTilesPerWg 32-query tiles, 16 / NW column groups); NW waves per
// workgroup cover 32 latent columns each (absorb_wave), so that W_UK is read
// by many CUs.  More queries use head_gemm_kernel<192, 512> (below).
constexpr int kAbsorbTilesPerWg = 8;

template <int NW>
__global__ __launch_bounds__(NW * 64) void absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                         const uint16_t* __restrict__ w_uk,
                                                         uint16_t* __restrict__ q_lat, int T) {
  __shared__ __attribute__((aligned(16))) uint16_t stage[NW][kAbsorbStage];
  const int ntb = (T + 31) / 32;
  const int tb0 = blockIdx.y * kAbsorbTilesPerWg;
  const int wave = threadIdx.x >> 6;
  absorb_wave(q_nope, w_uk, q_lat, T, blockIdx.x, (blockIdx.z * NW + wave) * 32, tb0,
              min(ntb, tb0 + kAbsorbTilesPerWg), stage[wave]);
}

// ---------------------------------------------------------------- core
// grid (T, key splits); 8 waves.  Tiles of 32 gathered rows land in a
// 3-deep LDS ring through direct-to-LDS loads (two tiles in flight while one
// is computed).  Per tile:
//   QK   wave (hg, hf) computes logits^T[16 keys of half hf][16 heads of group
//        hg] = c_tile . q^T with the group's q (576 = 512 latent + 64 rope)
//        resident as the B operand of 16x16x32 MFMAs;
//   softmax  both halves' maxima meet in LDS; the reference max of a head only
//        moves when a tile exceeds it by 2^8 (so P <= 256 and the running
//        output is rescaled rarely); P^T goes to LDS as bf16;
//   PV   wave w accumulates o^T[64 latent dims of slice w][64 heads] =
//        c_tile^T . P^T; the latent operand (8 consecutive keys of one dim per
//        lane) comes from the row-major tile by gfx950's transposing LDS read
//        (ds_read_b64_tr_b16: within 16 lanes, source lane s reads 4
//        consecutive dims of one key, and lane i receives element i % 4 of
//        source lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4).
// LDS tile layout: row r (one gathered key) = 72 slots of 16 bytes; logical
// slot c of row r sits at r*72 + ((c & ~7) | ((c ^ r) & 7)), which keeps the
// row reads of QK and the column reads of PV free of bank conflicts.
constexpr int kKT = 32;
constexpr int kSlots = kRow / 8;                  // 72 slots of 16 B per row
constexpr int kTileSlots = kKT * kSlots;          // 2304
constexpr int kCoreThreads = 512;
constexpr int kRing = 3;
constexpr int kPLds = kKT + 8;       // bf16 per P^T row (one head)
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold, log2 units
constexpr int kPartSlab = kHeads * kLat;  // bf16 values of one split partial
constexpr int kAbsent = 1 << 30;          // flag of an absent position in the contiguous core's index list

__device__ __forceinline__ int swz(int r, int c) { return r * kSlots + ((c & ~7) | ((c ^ r) & 7)); }

// INT4 cache (Q4): wave w gathers the whole raw 400-byte rows 4w .. 4w+3 of a
// tile (100 chunks of 16 B: 2 loads, the second's lanes 36-63 refetching
// chunk 99 into padding) into its own 2 KB region of a 2-slot raw ring, and
// expands those rows into the bf16 tile layout above at the end of the
// previous step: no wave reads another wave's raw rows, and the next step's
// barrier publishes the bf16 tile.
constexpr int kQ4RowsPerWave = kKT / 8;                        // 4
constexpr int kQ4WaveChunks = kQ4RowsPerWave * kQ4Row / 16;    // 100
constexpr int kQ4WaveBytes = 128 * 16;                         // 2 loads x 64 lanes x 16 B
constexpr int kQ4RawBytes = 8 * kQ4WaveBytes;                  // 16 KB per slot

// Lane l of wave w expands latent elements 32j .. 32j+31 (j = l % 16) of row
// 4w + l / 16, and lanes < 32 rope slot l % 8 of row 4w + l / 8.
__device__ __forceinline__ void dequant_rows(const uint8_t* region, uint16_t* tb, int wave, int lane) {
  const int rl = lane >> 4, j = lane & 15;
  const uint8_t* rb = region + rl * kQ4Row;
  const u32x4 c = *reinterpret_cast<const u32x4*>(rb + 16 * j);
  const float sc = bf16_to_f32(*reinterpret_cast<const uint16_t*>(rb + kQ4ScaleOff + 2 * (j >> 1)));
  const int r = kQ4RowsPerWave * wave + rl;
#pragma unroll
  for (int w = 0; w < 4; ++w) {  // dword w: elements 32j + 8w + e in nibble e
    const uint32_t d = c[w];
    u32x4 v;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float x0 = (float)((int32_t)(d << (28 - 8 * m)) >> 28) * sc;
      const float x1 = (float)((int32_t)(d << (24 - 8 * m)) >> 28) * sc;
      v[m] = cvt_pk_bf16(x0, x1);
    }
    *reinterpret_cast<u32x4*>(tb + swz(r, 4 * j + w) * 8) = v;
  }
  if (lane < kQ4RowsPerWave * 8) {
    const int rr = lane >> 3, i = lane & 7;
    *reinterpret_cast<u32x4*>(tb + swz(kQ4RowsPerWave * wave + rr, kLat / 8 + i) * 8) =
        *reinterpret_cast<const u32x4*>(region + rr * kQ4Row + kQ4RopeOff + 16 * i);
  }
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Maximum and sum of v over lanes l, l ^ 16, l ^ 32 and l ^ 48, in every lane.
// v_permlane16_swap exchanges 16-lane rows 1 and 3 of its first operand with
// rows 0 and 2 of its second, v_permlane32_swap the upper half of the first
// with the lower half of the second; with v in both operands the two results
// hold, in each lane, v of the lane and of its partner row (half).  Plain VALU
// work, unlike a shuffle through the LDS crossbar.
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// s_waitcnt vmcnt(n) (n < 16), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// s_waitcnt vmcnt(n) for n < 64 (the count's upper two bits sit in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vm_wide() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <bool PAGED, bool Q4>
__global__ __launch_bounds__(kCoreThreads) void mla_core_kernel(
    const int32_t* __restrict__ q_seq, CacheRows cr,
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q_rope,
    const void* __restrict__ kv_v, const int32_t* __restrict__ idx, int k, float scale_log2,
    int kps, int S, uint16_t* __restrict__ o_lat, uint16_t* __restrict__ o_part,
    float* __restrict__ ml_part) {
  // Three distinct arrays (not one indexed array): the compiler then waits
  // only for the direct-to-LDS loads that target the array being read.
  __shared__ __attribute__((aligned(16))) uint16_t tile0[kTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t tile1[kTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t tile2[kTileSlots * 8];  // (not used by Q4)
  __shared__ __attribute__((aligned(16))) uint8_t raw0[kQ4RawBytes];       // (Q4 only)
  __shared__ __attribute__((aligned(16))) uint8_t raw1[kQ4RawBytes];
  __shared__ __attribute__((aligned(16))) uint16_t pT[kHeads * kPLds];
  __shared__ float s_max[2][kHeads];
  __shared__ float s_alpha[kHeads];
  __shared__ float s_l[2][kHeads];
  __shared__ float s_m[kHeads];
  __shared__ float s_bias[kRing][kKT];  // 0 for a present key, -inf for an absent one
  __shared__ int s_idx[kMaxTopk + 4 * kKT];  // the split's positions (<= k), -1 padded
  const int t = blockIdx.x, sp = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS bases of the loads stay in SGPRs
  const int l16 = lane & 15, g = lane >> 4;
  const int hg = wave & 3, hf = wave >> 2;
  const int j0 = sp * kps;
  const int j1 = min(k, j0 + kps);
  // Contiguous: s_idx holds positions, rows of the query's sequence start at
  // kv_seq, and positions < 2^21 keep 32-bit byte offsets in range; an absent
  // entry is position 0 with bit 30 set (kAbsent), which the gather's 24-bit
  // offset multiply ignores.  Paged: s_idx holds pool rows (< 2^31) and
  // offsets are 64-bit; an absent entry holds ~r for the row r of position 0.
  // Either way an absent entry gathers finite data that is masked later.
  const int seq = q_seq[t];
  // row stride in elements of the gather's unit: bf16 (576) or bytes (Q4: 400)
  using Unit = typename std::conditional<Q4, uint8_t, uint16_t>::type;
  constexpr int kStride = Q4 ? kQ4Row : kRow;
  const Unit* const kv = static_cast<const Unit*>(kv_v);
  const Unit* const kv_seq = PAGED ? kv : kv + cr.seq_row0[seq] * kStride;
  const int32_t* bt = PAGED ? cr.table + (int64_t)seq * cr.max_pages : nullptr;
  const int32_t* irow = idx + (int64_t)t * k;
  const int hq = hg * 16 + l16;  // head of this lane in QK / softmax

  // o[e][j]: latent dim 64*wave + 16e + 4g + jj, head 16j + l16 (element jj)
  f32x4 o[4][4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[e][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -1e30f, l_part = 0.f;

  const int ntiles = j1 > j0 ? (j1 - j0 + kKT - 1) / kKT : 0;
  // The split's positions go to LDS first, so that no row gather waits on a
  // dependent global load of its index; the query operand loads are issued
  // just ahead of the first gathers.  Entries past the split are -1: the loop
  // (unrolled by 3) gathers up to four tiles past its last one.
  {
    // batches of kPer loads per thread (one batch covers splits of up to
    // kTopkSmall positions); all loads of a batch go out before its stores
    constexpr int kPer = (kTopkSmall + 4 * kKT + kCoreThreads - 1) / kCoreThreads;
    const int nfill = (ntiles + 4) * kKT;  // <= kMaxTopk + 4 * kKT
    for (int b0 = 0; b0 < nfill; b0 += kPer * kCoreThreads) {
      int v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int j = b0 + tid + u * kCoreThreads;
        const int e = irow[min(j0 + j, k - 1)];  // in-row read, replaced past the split
        v[u] = j0 + j < j1 ? e : -1;
        if (!PAGED) v[u] = v[u] >= 0 ? v[u] : kAbsent;
      }
      if (PAGED) {  // position -> pool row (all page loads, then the rows)
        int pg[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) pg[u] = bt[max(v[u], 0) >> cr.page_shift];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int row = (pg[u] << cr.page_shift) | (max(v[u], 0) & ((1 << cr.page_shift) - 1));
          v[u] = v[u] >= 0 ? row : ~row;
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int j = b0 + tid + u * kCoreThreads;
        if (j < nfill) s_idx[j] = v[u];
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Gather of a tile into a ring slot: wave instruction i covers the 64
  // physical slots [(8i + w) * 64, +64).  2304 slots = 4.5 instructions per
  // wave; every wave issues exactly 5 (waves 4-7 repeat the last chunk of
  // waves 0-3: same source, same destination) so that the number of
  // outstanding loads per tile is the same constant for every wave.  The DMA
  // writes lane L of an instruction to physical slot base + L; that slot holds
  // logical column (pc & ~7) | ((pc ^ row) & 7) of its row (the swizzle is an
  // involution within groups of 8), so the lane fetches that chunk.  Row and
  // column of each lane's five chunks are the same for every tile.
  // Q4: 2 loads per wave; load i covers chunks [64i, 64i + 64) of the wave's
  // rows (chunks past 99 refetch chunk 99 into the region's padding).
  constexpr int kNL = Q4 ? 2 : 5;  // gather loads per wave per tile
  int g_row[kNL];
  uint32_t g_col[kNL], g_colb[kNL];
  auto blk_of = [&](int i) {  // bf16: 64-slot block of the tile written by load i
    return i < 4 ? 8 * i + wave : 32 + (wave & 3);
  };
#pragma unroll
  for (int i = 0; i < kNL; ++i) {
    if (Q4) {
      const int c = min(64 * i + lane, kQ4WaveChunks - 1);
      const int rl = c / (kQ4Row / 16);
      g_row[i] = kQ4RowsPerWave * wave + rl;
      g_col[i] = (uint32_t)(c - rl * (kQ4Row / 16)) * 16u;  // bytes
    } else {  // physical slot lin < 2304 holds logical column (pc & ~7) | ((pc ^ row) & 7)
      const int lin = blk_of(i) * 64 + lane;
      const int r = lin / kSlots, pc = lin - r * kSlots;
      g_row[i] = r;
      g_col[i] = (uint32_t)((pc & ~7) | ((pc ^ r) & 7)) * 8u;
    }
    g_colb[i] = g_col[i] * (uint32_t)sizeof(Unit);
  }
  // Contiguous caches: a raw buffer resource over the sequence's rows (byte
  // offsets below 2^32), made wave-uniform so that it stays in SGPRs.
  const uint64_t kv_a = reinterpret_cast<uint64_t>(kv_seq);
  const uint32_t kv_lo = __builtin_amdgcn_readfirstlane((uint32_t)kv_a);
  const uint32_t kv_hi = __builtin_amdgcn_readfirstlane((uint32_t)(kv_a >> 32));
  const __amdgpu_buffer_rsrc_t kv_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)kv_hi << 32) | kv_lo), (short)0, (int)0xFFFFFFFF, kBufferWord3);
  auto gather_idx = [&](int tt, int sidx[kNL], int& valid) {
#pragma unroll
    for (int i = 0; i < kNL; ++i) sidx[i] = s_idx[tt * kKT + g_row[i]];
    valid = tid < kKT ? s_idx[tt * kKT + tid] : -1;
  };
  auto gather_issue = [&](const int sidx[kNL], int valid, void* dstt, int buf) {
#pragma unroll
    for (int i = 0; i < kNL; ++i) {
      // (named pointers: the host pass rejects cast expressions as this builtin's operands)
      uint16_t* const dst = static_cast<uint16_t*>(dstt) +
                            (Q4 ? (wave * kQ4WaveBytes + i * 64 * 16) / 2 : blk_of(i) * 64 * 8);
      if (PAGED) {
        // absent keys (and tiles past the end) fetch the row of position 0: finite data, masked later
        const int r = sidx[i] >= 0 ? sidx[i] : ~sidx[i];
        const uint16_t* const gsrc = reinterpret_cast<const uint16_t*>(kv_seq + (int64_t)r * kStride + g_col[i]);
        __builtin_amdgcn_global_load_lds(gsrc, dst, 16, 0, 0);
      } else {
        // one 24-bit multiply-add per load (bit 30 of an absent entry drops out)
        const uint32_t off = (uint32_t)(sidx[i] & 0xFFFFFF) * (uint32_t)(kStride * sizeof(Unit)) + g_colb[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, dst, 16, off, 0, 0, 0);
      }
    }
    if (tid < kKT) s_bias[buf][tid] = (PAGED ? valid >= 0 : (valid & kAbsent) == 0) ? 0.f : -INFINITY;
  };
  bf16x8 qb[18];
  {
    const uint16_t* ql = q_lat + ((int64_t)t * kHeads + hq) * kLat + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qb[ks] = as_bf16x8(ld16(ql + 32 * ks));
    const uint16_t* qr = q_rope + ((int64_t)t * kHeads + hq) * kRope + 8 * g;
    qb[16] = as_bf16x8(ld16(qr));
    qb[17] = as_bf16x8(ld16(qr + 32));
  }
  // Ring slots of the bf16 tiles (three distinct arrays).
  auto slot = [&](int b) -> void* {
    return b == 0 ? (void*)tile0 : (b == 1 ? (void*)tile1 : (void*)tile2);
  };
  // QK, softmax and PV of one tile: bf16 tile tb, key biases s_bias[vs].
  // Two barriers: after QK (the tile maxima of both key halves meet), and
  // before PV (P^T and the rescale factors are published).  `mid()` runs
  // after the first (every wave is past the previous tile's PV), `pre_pv()`
  // before the second.
  auto compute = [&](const uint16_t* tb, int vs, auto&& mid, auto&& pre_pv) {
    float bias[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) bias[jj] = s_bias[vs][hf * 16 + 4 * g + jj];
    // ---- QK: keys hf*16 + 4g + jj of head hq; three independent MFMA chains
    // (one chain of 18 would serialise on its accumulator)
    f32x4 sc;
    {
      const int r = hf * 16 + l16;
      f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        acc[ks % 3] = mfma16(as_bf16x8(*reinterpret_cast<const u32x4*>(tb + swz(r, 4 * ks + g) * 8)), qb[ks],
                             acc[ks % 3]);
      sc = acc[0] + acc[1] + acc[2];
    }
    float z[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float v = fmaf(sc[jj], scale_log2, bias[jj]);  // (rounds like the plain product)
      z[jj] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = rows_max(tmax);
    if (g == 0) s_max[hf][hq] = tmax;
    lds_barrier();
    mid();
    const float tile_max = fmaxf(s_max[0][hq], s_max[1][hq]);
    const float m_new = tile_max > m_ref + kRescaleLog2 ? tile_max : m_ref;
    // v_exp_f32 directly: results below 2^-126 flush to zero (weights that
    // small vanish against the reference maximum's weight 1 anyway)
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    m_ref = m_new;
    float p[4];
    float ps = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      p[jj] = __builtin_amdgcn_exp2f(z[jj] - m_new);
      ps += p[jj];
    }
    l_part = l_part * alpha + ps;
    *reinterpret_cast<u32x2*>(&pT[hq * kPLds + hf * 16 + 4 * g]) =
        u32x2{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])};
    if (hf == 0 && g == 0) s_alpha[hq] = alpha;
    pre_pv();
    lds_barrier();
    // ---- PV
    {
      float al[4];
      bool need = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        al[j] = s_alpha[16 * j + l16];
        need |= al[j] != 1.f;
      }
      if (__any(need)) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < 4; ++j) o[e][j] *= al[j];
      }
      bf16x8 pb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pb[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(&pT[(16 * j + l16) * kPLds + 8 * g]));
      // A of MFMA e: keys 8g .. 8g+7 of dim 64*wave + 16e + l16.  Read h of a
      // lane (source s = l16) covers key 8g + 4h + s/4, dims 16e + 4(s%4) ..+3
      // of the wave's slice: logical slot 8*wave + 2e + (s%4)/2, half (s%4)&1.
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 8 * wave + 2 * e + ((l16 & 3) >> 1);
        const uint16_t* const a0 = tb + swz(8 * g + (l16 >> 2), c) * 8 + 4 * (l16 & 1);
        const uint16_t* const a1 = tb + swz(8 * g + 4 + (l16 >> 2), c) * 8 + 4 * (l16 & 1);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a0));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a1));
        const bf16x8 fa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < 4; ++j) o[e][j] = mfma16(fa, pb[j], o[e][j]);
      }
    }
  };
  if constexpr (!Q4) {
    {
      int sidx[kNL], valid;
      gather_idx(0, sidx, valid);
      gather_issue(sidx, valid, slot(0), 0);
      gather_idx(1, sidx, valid);
      gather_issue(sidx, valid, slot(1), 1);
    }
    // Vector loads complete in issue order: vmcnt <= 5 means the query
    // operands and this wave's loads of tile 0 are in place.
    wait_vm<kNL>();
    lds_barrier();
    // Step tt issues the gather of tile tt + 2, right after its first barrier,
    // into the slot of tile tt - 1 (every wave has finished that tile's PV),
    // and before its second barrier waits for this wave's loads of tile
    // tt + 1, which that barrier then publishes for step tt + 1.
    auto step = [&](int tt, auto BUFC) {
      constexpr int buf = decltype(BUFC)::value;
      constexpr int nbuf = (buf + 2) % kRing;  // slot of tile tt + 2 (that of tile tt - 1)
      compute(static_cast<const uint16_t*>(slot(buf)), buf,
              [&]() {
                int sidx[kNL], valid;
                gather_idx(tt + 2, sidx, valid);
                gather_issue(sidx, valid, slot(nbuf), nbuf);
              },
              [&]() { wait_vm<kNL>(); });
    };
    for (int tt = 0; tt < ntiles; tt += kRing) {
      step(tt, std::integral_constant<int, 0>{});
      if (tt + 1 < ntiles) step(tt + 1, std::integral_constant<int, 1>{});
      if (tt + 2 < ntiles) step(tt + 2, std::integral_constant<int, 2>{});
    }
  } else {
    // INT4: raw tile j sits in raw slot j % 2, its bf16 expansion in tile
    // j % 2, its key biases in s_bias[j % 3].  A wave expands its own
    // rows of tile tt + 1 at the end of step tt (its loads of that tile are
    // then the older of its two tiles in flight); step tt + 1's barrier
    // publishes them.  Tile tt + 2 is gathered into the raw slot of tile tt,
    // which this wave has already expanded.
    uint8_t* const raw_w0 = raw0 + wave * kQ4WaveBytes;
    uint8_t* const raw_w1 = raw1 + wave * kQ4WaveBytes;
    {
      int sidx[kNL], valid;
      gather_idx(0, sidx, valid);
      gather_issue(sidx, valid, raw0, 0);
      gather_idx(1, sidx, valid);
      gather_issue(sidx, valid, raw1, 1);
    }
    wait_vm<kNL>();  // query operands and this wave's rows of tile 0
    if (ntiles > 0) dequant_rows(raw_w0, tile0, wave, lane);
    auto step = [&](int tt, auto BUFC) {
      constexpr int buf = decltype(BUFC)::value;  // tt % 2
      int sidx[kNL], valid;
      gather_idx(tt + 2, sidx, valid);
      lds_barrier();
      gather_issue(sidx, valid, buf == 0 ? (void*)raw0 : (void*)raw1, (tt + 2) % 3);
      if (tt < ntiles) compute(buf == 0 ? tile0 : tile1, tt % 3, [] {}, [] {});
      if (tt + 1 < ntiles) {
        wait_vm<kNL>();
        dequant_rows(buf == 0 ? raw_w1 : raw_w0, buf == 0 ? tile1 : tile0, wave, lane);
      }
    };
    for (int tt = 0; tt < ntiles; tt += 2) {
      step(tt, std::integral_constant<int, 0>{});
      step(tt + 1, std::integral_constant<int, 1>{});
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may still target this workgroup's LDS at exit

  // ---- finish: l of a head = its lanes' partial sums over both key halves
  const float l_sum = rows_sum(l_part);
  if (g == 0) {
    s_l[hf][hq] = l_sum;
    if (hf == 0) s_m[hq] = m_ref;
  }
  __syncthreads();
  const int dim0 = 64 * wave + 4 * g;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 16 * j + l16;
    const float L = s_l[0][h] + s_l[1][h];
    if (S == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* dst = o_lat + ((int64_t)t * kHeads + h) * kLat + dim0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<u32x2*>(dst + 16 * e) =
            u32x2{pack_bf16x2(o[e][j][0] * inv, o[e][j][1] * inv),
                  pack_bf16x2(o[e][j][2] * inv, o[e][j][3] * inv)};
    } else {
      // Partials are normalised by the split's own sum (a convex combination of
      // cache rows, held in bf16: the latent's own type and range, rounded to
      // nearest even) and keep the accumulator order (see mla_merge_kernel):
      // each store instruction writes 512 B of consecutive memory.
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* dst = o_part + ((int64_t)t * S + sp) * kPartSlab + ((wave * 4 + j) * 4) * 256 + lane * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<u32x2*>(dst + e * 256) =
            u32x2{cvt_pk_bf16(o[e][j][0] * inv, o[e][j][1] * inv), cvt_pk_bf16(o[e][j][2] * inv, o[e][j][3] * inv)};
      if (wave == 0 && g == 0) {
        const int64_t base = ((int64_t)t * S + sp) * kHeads + h;
        ml_part[base * 2] = s_m[h];
        ml_part[base * 2 + 1] = L;
      }
    }
  }
}

// ---------------------------------------------------------------- decode core
// Few queries (decode, up to 16): workgroups of (query, key split, 32 heads),
// 4 waves, one per SIMD; wave (hs, st) = (wave % 2, wave / 2) computes head
// group 2hh + hs (16 heads) over the 16-key tiles st, st + 2, ... of the
// split, so each tile serves two waves (32 heads), and those two waves each
// gather half of it by direct-to-LDS loads (rows 8hs .. 8hs+7 and one of its
// two rope loads); a barrier per step publishes the other wave's half.
//   QK   logits^T[16 keys][16 heads] = c_tile . q^T, 18 16x16x32 MFMAs with the
//        group's q (576 = 512 latent + 64 rope) resident as the B operand; lane
//        (g, l16) gets keys 4g .. 4g+3 of head l16, which is the B operand
//        layout of a 16x16x16 MFMA over those keys, so P stays in registers;
//   PV   o^T[512 dims][16 heads] += c_tile^T . P^T, 32 16x16x16 MFMAs whose
//        latent operand (4 keys of one dim per lane) comes from the row-major
//        tile by the transposing LDS read.
// The two waves of a head group meet in LDS at the end (max, sum, o) and
// write the split's partial.  The two workgroups of a (query, split) get
// block ids equal modulo 8, which places them on one XCD and its L2, so a row
// gathered for both head halves is read from HBM about once.
constexpr int kDecHeads = 16;
constexpr int kDecWaves = 4;
constexpr int kDecKT = 16;                          // keys per tile
constexpr int kDecMaxKps = 1024;                    // keys per split
constexpr int kDecTMax = 16;                        // batches up to this size
constexpr int kDecLatStride = kLat / 8 + 2;          // 66 slots per latent row (2 of padding)
constexpr int kDecRopeSlot0 = kDecKT * kDecLatStride;  // 1056: the rope area after 16 latent rows
constexpr int kDecTileSlots = kDecRopeSlot0 + kDecKT * (kRope / 8);  // 1184 slots of 16 B

// Tile layout (16 rows): the latent parts of the rows first, one 66-slot
// row each (logical chunk c of row r at r*66 + (c ^ (r / 8)): the XOR only
// swaps neighbouring chunks, so a lane's successive chunks stay at constant
// distances and its LDS reads share one address register), then the rope
// parts, 8 slots each (chunk c of row r at 1056 + r*8 + (c ^ (r / 2))).  The
// QK row reads (16 rows, one chunk) and the PV transposing reads (8 rows, two
// chunks per half wave) are both free of bank conflicts.
__device__ __forceinline__ int dec_lat_slot(int r, int c) { return r * kDecLatStride + (c ^ (r >> 3)); }
__device__ __forceinline__ int dec_rope_slot(int r, int c) { return kDecRopeSlot0 + r * 8 + (c ^ (r >> 1)); }

__device__ __forceinline__ f32x4 mfma16k16(v4i16 a, v4i16 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <bool PAGED, int NS>
__global__ __launch_bounds__(kDecWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_decode_kernel(
    const int32_t* __restrict__ q_seq, CacheRows cr, const uint16_t* __restrict__ q_lat,
    const uint16_t* __restrict__ q_rope, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    int T, int k, float scale_log2, int kps, int S, uint16_t* __restrict__ o_lat,
    uint16_t* __restrict__ o_part, float* __restrict__ ml_part) {
  // NS = 1..4: splits of 32*NS keys, whose 2*NS tiles are all gathered at
  // once; NS = 8: splits of 8, 12, ... 32 steps (kps / 32, a multiple of 4),
  // the four tile arrays of a stream forming a ring: tile v + 3 is gathered
  // at step v (after its barrier) into the array of tile v - 1.
  constexpr bool kRing = NS == 8;
  static_assert((NS >= 1 && NS <= 4) || NS == 8, "1-4 steps, or 8 for the ring");
  // Four distinct tile arrays (not one indexed array): the compiler then waits
  // only for the direct-to-LDS loads that target the array being read.
  // slotN[st] holds step N's tile of stream st (step N mod 4 for the ring).
  __shared__ __attribute__((aligned(16))) uint16_t slot0[2][kDecTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t slot1[2][kDecTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t slot2[2][kDecTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t slot3[2][kDecTileSlots * 8];
  __shared__ __attribute__((aligned(16))) int s_idx[kRing ? kDecMaxKps : 32 * NS];
  __shared__ float s_ml[kDecWaves][kDecHeads][2];
  // block id -> (query, split) pair P and head half hh: ids 16a + 8hh + r
  // hold pair 8a + r, head groups 2hh and 2hh + 1
  const int id = blockIdx.x;
  const int P = (id >> 4) * 8 + (id & 7);
  if (P >= T * S) return;  // (whole workgroup)
  const int t = P / S, sp = P - t * S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = wave & 1, st = wave >> 1;
  const int hg = 2 * ((id >> 3) & 1) + hs;
  const int l16 = lane & 15, g = lane >> 4;
  const int j0 = sp * kps;
  const int j1 = min(k, j0 + kps);
  const int seq = q_seq[t];
  const uint16_t* const kv_seq = PAGED ? kv : kv + cr.seq_row0[seq] * kRow;
  const int32_t* bt = PAGED ? cr.table + (int64_t)seq * cr.max_pages : nullptr;
  const int32_t* irow = idx + (int64_t)t * k;
  // The split's positions (as in mla_core_kernel: contiguous entries are
  // positions, an absent one position 0 with kAbsent set; paged entries are
  // pool rows, an absent one ~row of position 0), padded to the split's tiles.
  {
    constexpr int kFill = kRing ? kDecMaxKps : 32 * NS;
    constexpr int kPer = (kFill + kDecWaves * 64 - 1) / (kDecWaves * 64);
    const int nfill = kRing ? kps : kFill;
    int v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = tid + u * kDecWaves * 64;
      const int e = irow[min(j0 + j, k - 1)];
      v[u] = j0 + j < j1 ? e : -1;
      if (!PAGED) v[u] = v[u] >= 0 ? v[u] : kAbsent;
    }
    if (PAGED) {
      int pg[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) pg[u] = bt[max(v[u], 0) >> cr.page_shift];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int row = (pg[u] << cr.page_shift) | (max(v[u], 0) & ((1 << cr.page_shift) - 1));
        v[u] = v[u] >= 0 ? row : ~row;
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = tid + u * kDecWaves * 64;
      if (j < nfill) s_idx[j] = v[u];
    }
  }
  // q operand of QK: lane (g, l16) holds dims 32ks + 8g .. +7 of head 16hg + l16
  const int hq = kDecHeads * hg + l16;
  bf16x8 qb[18];
  {
    const uint16_t* ql = q_lat + ((int64_t)t * kHeads + hq) * kLat + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qb[ks] = as_bf16x8(ld16(ql + 32 * ks));
    const uint16_t* qr = q_rope + ((int64_t)t * kHeads + hq) * kRope + 8 * g;
    qb[16] = as_bf16x8(ld16(qr));
    qb[17] = as_bf16x8(ld16(qr + 32));
  }
  __syncthreads();

  // Half hs of tile u of the split: loads 0-7 bring the 1 KB latent parts of
  // rows 8hs .. 8hs+7 (lane L fetches logical chunk L ^ (row / 8) into
  // physical slot L of the row; the row's position is wave-uniform, so the
  // only per-lane operand is that chunk offset), load 8 rope load hs, the rope
  // parts of those 8 rows (physical slot p of rope area hs: row 8hs + p / 8,
  // logical chunk (p % 8) ^ (row / 2)).
  const uint64_t kv_a = reinterpret_cast<uint64_t>(kv_seq);
  const uint32_t kv_lo = __builtin_amdgcn_readfirstlane((uint32_t)kv_a);
  const uint32_t kv_hi = __builtin_amdgcn_readfirstlane((uint32_t)(kv_a >> 32));
  const uint16_t* const kv_u = reinterpret_cast<const uint16_t*>(((uint64_t)kv_hi << 32) | kv_lo);
  const __amdgpu_buffer_rsrc_t kv_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kv_u), (short)0, (int)0xFFFFFFFF, kBufferWord3);
  const uint32_t voff_lo = (uint32_t)lane * 16u, voff_hi = (uint32_t)(lane ^ 1) * 16u;  // rows 0-7, 8-15
  const int rope_r0 = lane >> 3;  // row of this lane's chunk in rope load 16 (load 17: + 8)
  const uint32_t rope_colb = (uint32_t)(kLat * 2) + (uint32_t)(((lane & 7) ^ (rope_r0 >> 1)) * 16);
  const uint32_t rope_colb1 = (uint32_t)(kLat * 2) + (uint32_t)(((lane & 7) ^ ((rope_r0 + 8) >> 1)) * 16);
  // Returns the mask of the tile's present rows (bit r for row r).  (The
  // entries are read in asm with its own wait: the compiler cannot tell s_idx
  // from the gathers' LDS targets and would wait for every gather in flight
  // before a plain read.)
  auto gather_half = [&](int u, uint16_t* dstt) __attribute__((always_inline)) -> uint32_t {
    int pv;
    {
      const __attribute__((address_space(3))) int* const a =
          (const __attribute__((address_space(3))) int*)(&s_idx[u * kDecKT + l16]);
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(pv) : "v"(a) : "memory");
    }
    const bool present = PAGED ? pv >= 0 : (pv & kAbsent) == 0;
    const uint32_t pmask = (uint32_t)__ballot(present) & 0xFFFFu;
    const int rb = 8 * hs;  // (wave-uniform)
    const int prh = __shfl(pv, rope_r0 + rb, 64);
    const uint32_t voff = hs ? voff_hi : voff_lo;
#pragma unroll
    for (int i = 0; i < kDecKT / 2; ++i) {
      uint16_t* const dst = dstt + (rb + i) * kDecLatStride * 8;
      const int e = __builtin_amdgcn_readlane(pv, rb + i);
      if (PAGED) {
        const int r = e >= 0 ? e : ~e;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(kv_u + (int64_t)r * kRow), (short)0, (int)0xFFFFFFFF, kBufferWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
      } else {
        const int soff = (e & 0xFFFFFF) * (kRow * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, dst, 16, voff, soff, 0, 0);
      }
    }
    uint16_t* const drh = dstt + (kDecRopeSlot0 + 64 * hs) * 8;
    const uint32_t colb = hs ? rope_colb1 : rope_colb;
    if (PAGED) {
      const int r = prh >= 0 ? prh : ~prh;
      __builtin_amdgcn_global_load_lds(kv_u + (int64_t)r * kRow + colb / 2, drh, 16, 0, 0);
    } else {
      const uint32_t o = (uint32_t)(prh & 0xFFFFFF) * (uint32_t)(kRow * 2) + colb;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, drh, 16, o, 0, 0, 0);
    }
    return pmask;
  };

  // per-lane LDS offsets (bf16 elements) of chunk g of row l16 (QK) and of
  // chunk (l16 % 4) / 2, half l16 % 2 of row 4g + l16 / 4 (PV)
  const int qk_base = dec_lat_slot(l16, g) * 8;
  const int pv_base = dec_lat_slot(4 * g + (l16 >> 2), (l16 & 3) >> 1) * 8 + 4 * (l16 & 1);

  f32x4 o[32];  // o[b]: dims 16b + 4g .. +3 of head hq
#pragma unroll
  for (int b = 0; b < 32; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -1e30f, l_part = 0.f;

  auto compute = [&](const uint16_t* tb, uint32_t pmask) __attribute__((always_inline)) {
    // ---- QK: keys 4g .. 4g+3 of head hq (three chains); the latent chunks
    // 4ks + g of row l16 lie 64 bytes apart
    const uint16_t* const tb_qk = tb + qk_base;
    f32x4 sc;
    {
      f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        acc[ks % 3] = mfma16(
            as_bf16x8(*reinterpret_cast<const u32x4*>(
                ks < 16 ? tb_qk + 32 * ks : tb + dec_rope_slot(l16, 4 * (ks - 16) + g) * 8)),
            qb[ks], acc[ks % 3]);
      sc = acc[0] + acc[1] + acc[2];
    }
    const uint32_t pm = pmask >> (4 * g);  // keys 4g .. 4g+3
    float z[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = fmaf(sc[i], scale_log2, (pm >> i) & 1u ? 0.f : -INFINITY);
      tmax = fmaxf(tmax, z[i]);
    }
    tmax = rows_max(tmax);
    // lazy reference maximum (see mla_core_kernel); v_exp_f32 directly
    const float m_new = tmax > m_ref + kRescaleLog2 ? tmax : m_ref;
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    m_ref = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < 32; ++b) o[b] *= alpha;
    }
    float p[4];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(z[i] - m_new);
      ps += p[i];
    }
    l_part = l_part * alpha + ps;
    const v4i16 pb = __builtin_bit_cast(v4i16, u32x2{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])});
    // ---- PV: source lane s of group g reads key 4g + s/4, dims 16b + 4(s%4) .. +3
    const uint16_t* const tb_pv = tb + pv_base;
#pragma unroll
    for (int b = 0; b < 32; ++b) {
      const uint16_t* const a = tb_pv + 16 * b;  // (chunks 2b + j lie 32 bytes apart)
      const v4i16 fa = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a));
      o[b] = mfma16k16(fa, pb, o[b]);
    }
  };

  // Half of each of this stream's first (NS, at most 4) tiles goes out at
  // once (9 loads per half tile); before step v the wave waits for its
  // halves of tiles up to v, and the barrier makes the other wave's halves
  // visible too.
  auto arr = [&](int v) __attribute__((always_inline)) -> uint16_t* {
    return v == 0 ? slot0[st] : v == 1 ? slot1[st] : v == 2 ? slot2[st] : slot3[st];
  };
  constexpr int kNS = kRing ? 4 : NS;  // tiles gathered before the first step
  constexpr int kHalf = kDecKT / 2 + 1;  // loads per half tile
  uint32_t pmv[kNS];
#pragma unroll
  for (int v = 0; v < kNS; ++v) pmv[v] = gather_half(st + 2 * v, arr(v));
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) asm volatile("" : "+v"(qb[ks]));
  if constexpr (!kRing) {
    auto pstep = [&](auto VC) __attribute__((always_inline)) {
      constexpr int v = decltype(VC)::value;
      if constexpr (v < NS) {
        wait_vm_wide<(NS - 1 - v) * kHalf>();
        lds_barrier();
        compute(arr(v), pmv[v]);
      }
    };
    pstep(std::integral_constant<int, 0>{});
    pstep(std::integral_constant<int, 1>{});
    pstep(std::integral_constant<int, 2>{});
    pstep(std::integral_constant<int, 3>{});
  } else {
    // Step v of array b = v % 4: wait for this wave's halves of tile v (the
    // halves of tiles v + 1, v + 2 stay in flight; step 0 also leaves tile
    // 3's, the last two steps fewer), barrier, gather tile v + 3 into the
    // array of tile v - 1 (both waves are past its step), compute tile v.
    // Rounds of four steps: the first does not refill at step 0, the last
    // refills only at its step 0; R = kps / 128 >= 2 rounds.
    const int R = kps / (8 * kDecKT);
    auto rstep = [&](int v, auto BC, auto WC, auto FC) __attribute__((always_inline)) {
      constexpr int b = decltype(BC)::value;
      wait_vm_wide<decltype(WC)::value>();
      lds_barrier();
      if constexpr (decltype(FC)::value) pmv[(b + 3) & 3] = gather_half(st + 2 * (v + 3), arr((b + 3) & 3));
      compute(arr(b), pmv[b]);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using W3 = std::integral_constant<int, 3 * kHalf>;
    using W2 = std::integral_constant<int, 2 * kHalf>;
    using W1 = std::integral_constant<int, kHalf>;
    using W0 = std::integral_constant<int, 0>;
    using Y = std::true_type;
    using N = std::false_type;
    rstep(0, I0{}, W3{}, N{});
    rstep(1, I1{}, W2{}, Y{});
    rstep(2, I2{}, W2{}, Y{});
    rstep(3, I3{}, W2{}, Y{});
    for (int r = 1; r < R - 1; ++r) {
      const int v = 4 * r;
      rstep(v, I0{}, W2{}, Y{});
      rstep(v + 1, I1{}, W2{}, Y{});
      rstep(v + 2, I2{}, W2{}, Y{});
      rstep(v + 3, I3{}, W2{}, Y{});
    }
    const int v = 4 * (R - 1);
    rstep(v, I0{}, W2{}, Y{});
    rstep(v + 1, I1{}, W2{}, N{});
    rstep(v + 2, I2{}, W1{}, N{});
    rstep(v + 3, I3{}, W0{}, N{});
  }

  // ---- the two waves of head group 2hh + hs (the streams st = 0, 1):
  // reference maxima and sums meet in LDS, then each wave adds up 16 of the
  // 32 latent blocks of 16 dims over both
  auto cw = [&](int c) __attribute__((always_inline)) { return hs + 2 * c; };  // c-th wave of the group
  const float l_sum = rows_sum(l_part);
  if (g == 0) {
    s_ml[wave][l16][0] = m_ref;
    s_ml[wave][l16][1] = l_sum;
  }
  __syncthreads();  // (also: every wave is done with its slots)
  const float mstar = fmaxf(s_ml[cw(0)][l16][0], s_ml[cw(1)][l16][0]);
  const float L = __builtin_amdgcn_exp2f(s_ml[cw(0)][l16][0] - mstar) * s_ml[cw(0)][l16][1] +
                  __builtin_amdgcn_exp2f(s_ml[cw(1)][l16][0] - mstar) * s_ml[cw(1)][l16][1];
  const float wgt = __builtin_amdgcn_exp2f(m_ref - mstar);
  // wave w's scaled o goes to [32 blocks][64 lanes] of f32x4 (32 KB) in slot w
  static_assert(sizeof(slot0) >= 32 * 64 * sizeof(f32x4), "reduction area");
  auto red = [&](int w) __attribute__((always_inline)) -> f32x4* {
    return reinterpret_cast<f32x4*>(w == 0 ? &slot0[0][0] : w == 1 ? &slot1[0][0] : w == 2 ? &slot2[0][0]
                                                                                          : &slot3[0][0]);
  };
  {
    f32x4* const mine = red(wave);
#pragma unroll
    for (int b = 0; b < 32; ++b) mine[b * 64 + lane] = o[b] * wgt;
  }
  __syncthreads();
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int bb = 0; bb < 16; ++bb) {
    const int b = 16 * st + bb;
    f32x4 sum = red(cw(0))[b * 64 + lane] + red(cw(1))[b * 64 + lane];
    sum *= inv;
    if (S == 1) {
      *reinterpret_cast<u32x2*>(o_lat + ((int64_t)t * kHeads + hq) * kLat + 16 * b + 4 * g) =
          u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
    } else {
      // head-major, as merge_upproj_kernel reads them: o_part[t][sp][h][512]
      *reinterpret_cast<u32x2*>(o_part + ((int64_t)t * S + sp) * kPartSlab + (int64_t)hq * kLat + 16 * b + 4 * g) =
          u32x2{cvt_pk_bf16(sum[0], sum[1]), cvt_pk_bf16(sum[2], sum[3])};
    }
  }
  if (S > 1 && st == 0 && g == 0) {
    const int64_t base = ((int64_t)t * S + sp) * kHeads + hq;
    ml_part[base * 2] = mstar;
    ml_part[base * 2 + 1] = L;
  }
}

// ---------------------------------------------------------------- core, one split per query
// Batches whose queries each take one key split (prefill chunks): one
// workgroup per query, 8 waves in two roles, one per SIMD each:
//   waves 0-3 (QK)  wave hg computes logits^T[32 keys][16 heads of group hg]
//                   of tile i (36 16x16x32 MFMAs against its resident q), its
//                   online softmax (a head's 32 keys are all in the wave: no
//                   exchange), and writes P^T and the rescale factors of tile i;
//   waves 4-7 (PV)  wave w accumulates o^T[128 latent dims of slice w][64
//                   heads] for tile i - 1 (32 MFMAs), reading tile i - 1's P^T.
// So every SIMD runs one wave's QK and softmax next to another's PV, and a
// tile costs one barrier.  Tiles of 32 gathered rows use a 4-slot ring: tile
// i + 2 is gathered during step i into the slot of tile i - 2 (QK'd two steps
// ago, PV'd in the last one); each row is one direct-to-LDS load (its
// position wave-uniform), the rope parts four more.  The positions come from
// the index row in global memory one step before their gather.
// Tile layout (36,864 B, slots of 16 B): latent row r at slots r*64 .. r*64+63,
// logical chunk c at r*64 + (c ^ swz(r)) with swz(r) = (r ^ 2r) mod 16; rope
// area at slot 2048, chunk c of row r at 2048 + r*8 + (c ^ ((r >> 1) & 7)).
// With these swizzles (chosen by measuring SQ_LDS_BANK_CONFLICT over candidate
// layouts on gfx950) the QK row reads, the QK rope reads and the PV
// transposing reads are all free of bank conflicts.  swz is linear over XOR and
// depends on r mod 16 only, so a lane's QK reads need 4 base addresses (one per
// chunk step mod 4; rows r + 16 add a constant) and its PV reads 8 (rows r + 4
// reuse them with the dim block index XOR 6).  P^T of the tiles of parity b is
// s_pt[b]: chunk q (keys 8q .. 8q+7) of head h at slot h*4 + (q ^ ((h >> 1) & 3))
// (conflict-free PV reads).  P^T and the rescale factors are read and written,
// and the key biases written, with inline LDS instructions that wait for
// themselves, because the compiler would otherwise order them after the
// pending gathers.
constexpr int kWsLat = kLat / 8;                       // 64 slots per latent row
constexpr int kWsRope0 = kKT * kWsLat;                 // 2048
constexpr int kWsTileSlots = kWsRope0 + kKT * (kRope / 8);  // 2304 slots = 36,864 B
constexpr int kWsNL = 5;                               // gather loads per tile of a QK wave (PV waves: 4)

__device__ __forceinline__ int ws_swz(int r) { return (r ^ (r << 1)) & 15; }
__device__ __forceinline__ int ws_lat_slot(int r, int c) { return r * kWsLat + (c ^ ws_swz(r)); }
__device__ __forceinline__ int ws_rope_slot(int r, int c) { return kWsRope0 + r * 8 + (c ^ ((r >> 1) & 7)); }
// byte offset of P^T chunk q (keys 8q .. 8q+7) of head h within s_pt[b]
__device__ __forceinline__ int ws_pt_off(int h, int q) { return 16 * (h * 4 + (q ^ ((h >> 1) & 3))); }

// Paged caches, one split per query: the index row of query t turned into pool
// rows, entries[t*stride + j] = the pool row of idx[t*k + j] (complemented when
// the entry is -1: then the row of position 0, finite data that the core masks),
// and entries[t*stride + k] = the complemented row of position 0 (what the core
// reads for rows past k).  The entries live in the first k + 1 words of the
// query's own o_lat row (64 KB), which the core writes only after its last read.
constexpr int kWsEntryStride = kHeads * kLat / 2;  // int32 words per o_lat row
static_assert(kMaxTopk + 1 <= kWsEntryStride, "a query's entries fit its o_lat row");
__global__ __launch_bounds__(256) void ws_paged_entries_kernel(const int32_t* __restrict__ q_seq, CacheRows cr,
                                                               const int32_t* __restrict__ idx, int k,
                                                               int32_t* __restrict__ entries) {
  const int t = blockIdx.x;
  const int32_t* bt = cr.table + (int64_t)q_seq[t] * cr.max_pages;
  const int32_t* irow = idx + (int64_t)t * k;
  int32_t* erow = entries + (int64_t)t * kWsEntryStride;
  const int mask = (1 << cr.page_shift) - 1;
  const int row0 = bt[0] << cr.page_shift;
  for (int j = threadIdx.x; j <= k; j += 256) {
    const int pos = j < k ? irow[j] : -1;
    erow[j] = pos >= 0 ? (bt[pos >> cr.page_shift] << cr.page_shift) | (pos & mask) : ~row0;
  }
}

template <bool PAGED>
__global__ __launch_bounds__(kCoreThreads) void mla_ws_kernel(
    const int32_t* __restrict__ q_seq, CacheRows cr, const uint16_t* __restrict__ q_lat,
    const uint16_t* __restrict__ q_rope, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    int k, float scale_log2, uint16_t* __restrict__ o_lat) {
  // Four distinct arrays: the compiler then waits only for the gathers that
  // target the array being read.
  __shared__ __attribute__((aligned(16))) uint16_t tile0[kWsTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t tile1[kWsTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t tile2[kWsTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t tile3[kWsTileSlots * 8];
  __shared__ __attribute__((aligned(16))) uint16_t s_pt[2][kHeads * kKT];
  __shared__ __attribute__((aligned(16))) float s_alpha[2][kHeads];
  __shared__ __attribute__((aligned(16))) float s_bias[4][kKT];
  __shared__ float s_l[kHeads];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool qk = wave < 4;
  const int wr = wave & 3;  // QK: head group; PV: latent slice
  const int l16 = lane & 15, g = lane >> 4;
  const int seq = q_seq[t];
  // paged: kv is the pool and idx the pool-row entries (ws_paged_entries_kernel)
  const uint16_t* const kv_seq = PAGED ? kv : kv + cr.seq_row0[seq] * kRow;
  const int32_t* irow = idx + (int64_t)t * (PAGED ? kWsEntryStride : k);
  const int ntiles = (k + kKT - 1) / kKT;

  auto slot = [&](int b) __attribute__((always_inline)) -> uint16_t* {
    return b == 0 ? tile0 : (b == 1 ? tile1 : (b == 2 ? tile2 : tile3));
  };
  auto lds_addr = [](const void* p) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
  };

  // ---- positions: lane l holds the entry of row l % 32 of a tile: the
  // position, or position 0 with kAbsent set for an absent one (-1 in the
  // index row, or past k), which the gather's 24-bit offset multiply ignores
  // Paged: an entry is a pool row, complemented when absent; rows past k read
  // the entry at k (the complemented row of position 0).
  // Every step issues the same number of loads (the step's waits count them):
  // the index words are loaded unconditionally, at a clamped index, and the
  // test for rows past k is applied where an entry is used (entry()), so the
  // loaded words travel raw (a loop-carried value computed from a load makes
  // the compiler wait for it at the loop edge).
  // Contiguous: the index row read as a buffer of k words, whose loads past
  // the end return 0 (rows that entry() makes absent), at a lane offset made
  // afresh at each load: a lane number kept live across the step loop has
  // been spilled there, and its reload at the loop edge waited for every
  // gather in flight.
  const __amdgpu_buffer_rsrc_t irow_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(irow), (short)0, PAGED ? 0 : k * 4, kBufferWord3);
  auto pos_load = [&](int u) __attribute__((always_inline)) -> int {
    if constexpr (PAGED) {
      const int j = u * kKT + (lane & 31);
      return irow[min(j, k)];
    } else {
      uint32_t l;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
      return (int)__builtin_amdgcn_raw_buffer_load_b32(irow_rsrc, (l & 31) * 4, u * kKT * 4, 0);
    }
  };
  // the entry of tile u's row `row` from its raw index word
  auto entry = [&](int raw, int u, int row) __attribute__((always_inline)) -> int {
    if constexpr (PAGED) return raw;  // (rows past k read the entry at k)
    return u * kKT + row < k && raw >= 0 ? raw : kAbsent;
  };
  // QK waves: lane l also loads the index word of the rope row it gathers, 8 wr + l / 8
  const int rope_row = 8 * wr + (lane >> 3);
  auto rope_pos_load = [&](int u) __attribute__((always_inline)) -> int {
    const int j = u * kKT + rope_row;
    return irow[PAGED ? min(j, k) : max(min(j, k - 1), 0)];
  };
  const uint64_t kv_a = reinterpret_cast<uint64_t>(kv_seq);
  const uint32_t kv_lo = __builtin_amdgcn_readfirstlane((uint32_t)kv_a);
  const uint32_t kv_hi = __builtin_amdgcn_readfirstlane((uint32_t)(kv_a >> 32));
  const uint16_t* const kv_u = reinterpret_cast<const uint16_t*>(((uint64_t)kv_hi << 32) | kv_lo);
  const __amdgpu_buffer_rsrc_t kv_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kv_u), (short)0, (int)0xFFFFFFFF, kBufferWord3);
  // latent rows wave, wave + 8, +16, +24 of a tile; QK waves also rope load wave
  uint32_t voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) voff[q] = (uint32_t)((lane ^ ws_swz(wave + 8 * q)) * 16);
  const uint32_t rope_colb = (uint32_t)(kLat * 2) + (uint32_t)(((lane & 7) ^ ((rope_row >> 1) & 7)) * 16);
  // gather of tile u into ring slot dst from the raw index words of its rows
  // (pw, and rw for the rope rows of a QK wave); a latent row's entry is made
  // in scalar registers after the readlane
  auto gather = [&](int pw, int rw, int u, uint16_t* dst, int bslot) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wave + 8 * q;
      const int e = entry(__builtin_amdgcn_readlane(pw, r), u, r);
      uint16_t* const d = dst + r * kWsLat * 8;
      if constexpr (PAGED) {
        // a resource based at the row: a pool may pass 2^32 bytes
        const uint16_t* const rowp = kv_u + (int64_t)(e ^ (e >> 31)) * kRow;
        const __amdgpu_buffer_rsrc_t rr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(rowp), (short)0, (int)0xFFFFFFFF, kBufferWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, d, 16, voff[q], 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, d, 16, voff[q], (e & 0xFFFFFF) * (kRow * 2), 0, 0);
      }
    }
    if (qk) {
      if constexpr (!PAGED) {  // (paged: rope_fetch / rope_store)
        uint16_t* const d = dst + (kWsRope0 + 64 * wr) * 8;
        const int pr = entry(rw, u, rope_row);
        const uint32_t off = (uint32_t)(pr & 0xFFFFFF) * (uint32_t)(kRow * 2) + rope_colb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kv_rsrc, d, 16, off, 0, 0, 0);
      }
      // key biases of the tile (0 present, -inf absent), wave 0
      if (wave == 0 && lane < kKT) {
        const int pe = entry(pw, u, lane);
        const float bias = (PAGED ? pe >= 0 : (pe & kAbsent) == 0) ? 0.f : -INFINITY;
        asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(&s_bias[bslot][lane])), "v"(bias) : "memory");
      }
    }
  };

  // Paged caches, QK waves: the rope parts travel through registers (a per-lane
  // 64-bit address; a direct-to-LDS global load here would make the compiler
  // wait for every load in flight wherever it waits for one).  Lane l holds the
  // 16 B that the rope DMA would put in slot l of the wave's 1 KB rope block:
  // row 8 wr + l / 8, logical chunk (l & 7) ^ ((row >> 1) & 7).  The load goes
  // out two steps before the tile is computed and is stored to LDS (an inline
  // store: a compiled one into the ring array would wait for its gathers) in
  // the step before.
  auto rope_fetch = [&](int pr) __attribute__((always_inline)) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(kv_u + (int64_t)(pr ^ (pr >> 31)) * kRow + rope_colb / 2);
  };
  auto rope_store = [&](uint16_t* dst, const u32x4& v) __attribute__((always_inline)) {
    asm volatile("ds_write_b128 %0, %1" ::"v"(lds_addr(dst + (kWsRope0 + 64 * wr + lane) * 8)), "v"(v) : "memory");
  };

  const int hq = 16 * wr + l16;

  // per-lane LDS offsets (bf16 elements) of the reads from a tile: QK chunks
  // 4j + g of row l16 (j = ks mod 4); PV dim block e (chunk 16 wr + 2e +
  // (l16 % 4) / 2, half l16 % 2) of row 8g + l16 / 4
  int qkb[4], pvb[8];
  const int pv_r0 = 8 * g + (l16 >> 2), pv_jj = (l16 & 3) >> 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) qkb[j] = ws_lat_slot(l16, 4 * j + g) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) pvb[e] = ws_lat_slot(pv_r0, 16 * wr + 2 * e + pv_jj) * 8 + 4 * (l16 & 1);

  // QK + softmax of the tile in ring slot b (parity par): writes P^T and alpha
  auto qk_step = [&](const uint16_t* tb, int b, int par, const bf16x8 (&qb)[18], float& m_ref,
                     float& l_part) __attribute__((always_inline)) {
    // chunk ks of row 16 kb + l16: latent chunk 4 ks + g at base (ks mod 4) + 16
    // chunks per 4 steps + 16 rows per kb; ks 16, 17: rope chunks
    auto qk_a = [&](int kb, int ks) __attribute__((always_inline)) -> u32x4 {
      const uint16_t* const a = ks < 16 ? tb + qkb[ks & 3] + 128 * (ks >> 2) + 16 * kWsLat * 8 * kb
                                        : tb + ws_rope_slot(16 * kb + l16, 4 * (ks - 16) + g) * 8;
      return *reinterpret_cast<const u32x4*>(a);
    };
    // The 36 operands (block kb = n / 18, step ks = n % 18) are read kQkDepth
    // ahead of their MFMA, so the MFMA chain does not wait on LDS latency read
    // by read (the interleave is pinned; the compiler would keep fewer in flight).
    const f32x4 bias[2] = {*reinterpret_cast<const f32x4*>(&s_bias[b][4 * g]),
                           *reinterpret_cast<const f32x4*>(&s_bias[b][16 + 4 * g])};
    constexpr int kQkDepth = 8;
    u32x4 A[36];
#pragma unroll
    for (int n = 0; n < kQkDepth; ++n) A[n] = qk_a(n / 18, n % 18);
    f32x4 acc[2][3] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}},
                       {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
    for (int n = 0; n < 36; ++n) {
      const int kb = n / 18, ks = n % 18;
      acc[kb][ks % 3] = mfma16(as_bf16x8(A[n]), qb[ks], acc[kb][ks % 3]);
      if (n + kQkDepth < 36) A[n + kQkDepth] = qk_a((n + kQkDepth) / 18, (n + kQkDepth) % 18);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kQkDepth + 2, 0);  // the biases and the first operands
#pragma unroll
    for (int n = 0; n < 36; ++n) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (n + kQkDepth < 36) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    const f32x4 sc[2] = {acc[0][0] + acc[0][1] + acc[0][2], acc[1][0] + acc[1][1] + acc[1][2]};
    float z[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[4 * kb + i] = fmaf(sc[kb][i], scale_log2, bias[kb][i]);
        tmax = fmaxf(tmax, z[4 * kb + i]);
      }
    tmax = rows_max(tmax);
    const float m_new = tmax > m_ref + kRescaleLog2 ? tmax : m_ref;
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    m_ref = m_new;
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(z[i] - m_new);
      ps += p[i];
    }
    l_part = l_part * alpha + ps;
    // P^T of head hq, keys 16kb + 4g .. +3: half (g & 1) of chunk 2kb + g/2
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint32_t a = lds_addr(&s_pt[par][0]) + ws_pt_off(hq, 2 * kb + (g >> 1)) + 8 * (g & 1);
      const u32x2 v = {cvt_pk_bf16(p[4 * kb], p[4 * kb + 1]), cvt_pk_bf16(p[4 * kb + 2], p[4 * kb + 3])};
      asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
    }
    if (g == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(&s_alpha[par][hq])), "v"(alpha) : "memory");
  };
  // PV of the tile in ring slot b (parity par)
  auto pv_step = [&](const uint16_t* tb, int par, f32x4 (&o)[8][4]) __attribute__((always_inline)) {
    float al[4];
    u32x4 pb[4];
    {
      // heads l16 + 16j: alpha 64 B apart, P^T rows 1 KB apart (the chunk swizzle
      // depends on (h >> 1) & 3, the same for every j)
      const uint32_t a0 = lds_addr(&s_alpha[par][l16]);
      const uint32_t p0 = lds_addr(&s_pt[par][0]) + ws_pt_off(l16, g);
      asm volatile(
          "ds_read_b32 %0, %8\n\tds_read_b32 %1, %8 offset:64\n\tds_read_b32 %2, %8 offset:128\n\t"
          "ds_read_b32 %3, %8 offset:192\n\tds_read_b128 %4, %9\n\tds_read_b128 %5, %9 offset:1024\n\t"
          "ds_read_b128 %6, %9 offset:2048\n\tds_read_b128 %7, %9 offset:3072\n\ts_waitcnt lgkmcnt(0)"
          : "=v"(al[0]), "=v"(al[1]), "=v"(al[2]), "=v"(al[3]), "=v"(pb[0]), "=v"(pb[1]), "=v"(pb[2]), "=v"(pb[3])
          : "v"(a0), "v"(p0)
          : "memory");
    }
    bool need = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) need |= al[j] != 1.f;
    if (__any(need)) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[e][j] *= al[j];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // rows pv_r0 and pv_r0 + 4 (= pv_r0 ^ 4, swizzled by swz ^ 12: dim block e ^ 6)
      const uint16_t* const a0 = tb + pvb[e];
      const uint16_t* const a1 = tb + pvb[e ^ 6] + 4 * kWsLat * 8;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a0));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(a1));
      const bf16x8 fa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int j = 0; j < 4; ++j) o[e][j] = mfma16(fa, as_bf16x8(pb[j]), o[e][j]);
    }
  };

  // The two roles run the same schedule of gathers and barriers in separate
  // code paths (so that neither holds the other's registers: q and the
  // softmax state in QK waves, the 128 accumulators in PV waves).
  // Prologue: gathers of tiles 0 and 1, positions of tile 2 (rope: 2, 3).  Step i (slot
  // b = i % 4): tile i + 2 is gathered into the slot of tile i - 2 and the
  // positions of tile i + 3 are requested; QK waves take tile i (past the
  // last tile: absent rows, no effect), PV waves tile i - 1 (from step 1 on);
  // then each wave waits for its own loads of tile i + 1 (issued one step
  // earlier: only this step's position loads and gather are younger) and the
  // barrier publishes them together with tile i's P^T and alpha.
  auto run = [&](auto QKC, auto&& work) __attribute__((always_inline)) {
    constexpr bool kQk = decltype(QKC)::value;
    // rope entries (QK waves) run one step further ahead than the latent ones:
    // loaded two steps before their gather, they have arrived by the wait that
    // ends the step before it, so using them waits for no younger gather
    int pe_next, pr_next = 0, pr_next2 = 0;
    u32x4 rope_cur = {0u, 0u, 0u, 0u};  // paged QK waves: rope of the tile after the next
    {
      const int e0 = pos_load(0), e1 = pos_load(1);  // (raw words)
      int r0 = 0, r1 = 0;
      u32x4 rope0 = {0u, 0u, 0u, 0u};
      if constexpr (kQk) {
        r0 = rope_pos_load(0);
        r1 = rope_pos_load(1);
        pr_next = rope_pos_load(2);
        pr_next2 = rope_pos_load(3);
        if constexpr (PAGED) {
          rope0 = rope_fetch(entry(r0, 0, rope_row));
          rope_cur = rope_fetch(entry(r1, 1, rope_row));
        }
      }
      pe_next = pos_load(2);
      gather(e0, r0, 0, tile0, 0);
      gather(e1, r1, 1, tile1, 1);
      __builtin_amdgcn_s_waitcnt(0);  // (both tiles, the query operands and the next positions)
      if constexpr (PAGED && kQk) rope_store(tile0, rope0);
    }
    lds_barrier();
    auto step = [&](int i, auto BC, auto PVC) __attribute__((always_inline)) {
      constexpr int b = decltype(BC)::value;
      const int pw = pe_next, rw = pr_next;  // (raw words of tile i + 2)
      pe_next = pos_load(i + 3);
      u32x4 rope_next = {0u, 0u, 0u, 0u};
      if constexpr (kQk) {
        pr_next = pr_next2;
        pr_next2 = rope_pos_load(i + 4);
        if constexpr (PAGED) rope_next = rope_fetch(entry(rw, i + 2, rope_row));  // (in place of its rope DMA)
      }
      // the position loads go out before the gathers: the waits for them count
      // only older loads
      __builtin_amdgcn_sched_barrier(0);
      gather(pw, rw, i + 2, slot((b + 2) % 4), (b + 2) % 4);
      work(i, BC, PVC);
      if constexpr (PAGED && kQk) {
        rope_store(slot((b + 1) % 4), rope_cur);  // tile i + 1, published by this step's barrier
        rope_cur = rope_next;
      }
      if constexpr (kQk) wait_vm_wide<kWsNL + 2>();
      else wait_vm_wide<kWsNL>();
      lds_barrier();
    };
    using Yes = std::integral_constant<bool, true>;
    step(0, std::integral_constant<int, 0>{}, std::integral_constant<bool, false>{});
    // (k >= 1, so there is a tile 1 to take; a loop with an entry test had the
    // compiler sink step 0's position load past its gathers into that test,
    // and the loop head then waited for the gathers of the step before it)
    int i = 1;
    do {
      step(i, std::integral_constant<int, 1>{}, Yes{});
      step(i + 1, std::integral_constant<int, 2>{}, Yes{});
      step(i + 2, std::integral_constant<int, 3>{}, Yes{});
      step(i + 3, std::integral_constant<int, 0>{}, Yes{});
      i += 4;
    } while (i <= ntiles);
    __builtin_amdgcn_s_waitcnt(0);  // no gather may still target this workgroup's LDS at exit
  };

  if (qk) {
    bf16x8 qb[18];
    {
      const uint16_t* ql = q_lat + ((int64_t)t * kHeads + hq) * kLat + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qb[ks] = as_bf16x8(ld16(ql + 32 * ks));
      const uint16_t* qr = q_rope + ((int64_t)t * kHeads + hq) * kRope + 8 * g;
      qb[16] = as_bf16x8(ld16(qr));
      qb[17] = as_bf16x8(ld16(qr + 32));
    }
    float m_ref = -1e30f, l_part = 0.f;
    run(std::integral_constant<bool, true>{}, [&](int, auto BC, auto) __attribute__((always_inline)) {
      constexpr int b = decltype(BC)::value;
      qk_step(slot(b), b, b & 1, qb, m_ref, l_part);
    });
    // 1 / (sum of a head's weights) for the PV waves
    const float l_sum = rows_sum(l_part);
    if (g == 0) s_l[hq] = l_sum;
    __syncthreads();
  } else {
    f32x4 o[8][4];  // o[e][j]: dims 128 wr + 16e + 4g .. +3 of head 16j + l16
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) o[e][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    run(std::integral_constant<bool, false>{}, [&](int, auto BC, auto PVC) __attribute__((always_inline)) {
      constexpr int b = decltype(BC)::value;
      if constexpr (decltype(PVC)::value) pv_step(slot((b + 3) % 4), (b + 1) & 1, o);
    });
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 16 * j + l16;
      const float L = s_l[h];
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* dst = o_lat + ((int64_t)t * kHeads + h) * kLat + 128 * wr + 4 * g;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<u32x2*>(dst + 16 * e) =
            u32x2{pack_bf16x2(o[e][j][0] * inv, o[e][j][1] * inv), pack_bf16x2(o[e][j][2] * inv, o[e][j][3] * inv)};
    }
  }
}

// ---------------------------------------------------------------- merge
// Split partials of (query t, split s) form one slab of kHeads * kLat bf16
// values, each normalised by its split's sum l, in the core's accumulator
// order: element i of the 4-value group number ((w * 4 + j) * 4 + e) * 64 +
// lane is latent dim 64w + 16e + 4(lane / 16) + i of head 16j + lane % 16.
// ml_part[t][s][h] = (reference max m, sum l).  grid (T, 32): workgroup
// (t, 4w + j) combines latent dims 64w .. 64w+63 of heads 16j .. 16j+15, one
// group of every split per thread, weighting split s by 2^(m_s - max m) l_s.
// CH: splits whose (m, l) pairs and partials are all requested before any is
// used (one memory latency per chunk; the launch takes the smallest of 8, 16,
// 32 that holds the splits, or 32-split chunks).  A later chunk with a larger
// maximum rescales what is summed so far (with one chunk this is the plain
// two-pass sum).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

template <int CH>
__global__ __launch_bounds__(256) void mla_merge_kernel(const uint16_t* __restrict__ o_part,
                                                        const float* __restrict__ ml_part, int S,
                                                        uint16_t* __restrict__ o_lat) {
  const int t = blockIdx.x, w = blockIdx.y >> 2, j = blockIdx.y & 3, tid = threadIdx.x;
  const int lane = tid & 63, jj = tid >> 6;
  const int h = 16 * j + (lane & 15), g = lane >> 4;
  const float* ml = ml_part + ((int64_t)t * S * kHeads + h) * 2;
  const uint16_t* src = o_part + (int64_t)t * S * kPartSlab + (((w * 4 + j) * 4 + jj) * 64 + lane) * 4;
  float mstar = -1e30f, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += CH) {
    f32x2 m_l[CH];
    u32x2 v[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int s = min(s0 + u, S - 1);  // past S: split S - 1 again, weight 0
      m_l[u] = *reinterpret_cast<const f32x2*>(ml + (int64_t)s * kHeads * 2);
      v[u] = *reinterpret_cast<const u32x2*>(src + (int64_t)s * kPartSlab);
    }
    float cm = mstar;
#pragma unroll
    for (int u = 0; u < CH; ++u) cm = s0 + u < S ? fmaxf(cm, m_l[u][0]) : cm;
    if (cm > mstar) {
      const float sc = exp2f(mstar - cm);
      L *= sc;
      acc *= sc;
      mstar = cm;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float wgt = s0 + u < S ? exp2f(m_l[u][0] - mstar) * m_l[u][1] : 0.f;
      L += wgt;
      acc += wgt * f32x4{bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y)};
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<u32x2*>(o_lat + ((int64_t)t * kHeads + h) * kLat + 64 * w + 16 * jj + 4 * g) =
      u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
}

// ---------------------------------------------------------------- upproj
// grid (64 heads, 4 blocks of 64 output dims, ceil(T / (32*kUpMT))).
// W_UV[h][:, block] is staged in LDS transposed ([e][c]) so that the B operand
// (8 consecutive c for one e) is one 16-byte LDS read.  Waves: (N-tile of 32
// dims) x (half of the 512-long K); the two K halves are summed through LDS.
constexpr int kUpEB = 64;
constexpr int kUpMT = 16;  // 32-query tiles per workgroup
constexpr int kWvLds = kLat + 8;

__global__ __launch_bounds__(256) void upproj_kernel(const uint16_t* __restrict__ o_lat,
                                                     const uint16_t* __restrict__ w_uv,
                                                     void* __restrict__ out, int out_f32, int T) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kUpEB * kWvLds];
  __shared__ float red[2][64 * 16];
  const int h = blockIdx.x, eb = blockIdx.y, mb = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int nt = wave & 1, kh = wave >> 1;
  // All of the thread's W_UV pieces (4 units of 4 rows x 8 e) and the first
  // tile's A operand are requested before any is used: the 64 KB slice of a
  // workgroup is in flight at once rather than a unit at a time.
  constexpr int kUnits = (kLat / 4) * (kUpEB / 8) / 256;
  u32x4 rows[kUnits][4];
#pragma unroll
  for (int it = 0; it < kUnits; ++it) {
    const int u = tid + 256 * it;
    const int q = u >> 3, r = u & 7;  // c = 4q..4q+3, e = 8r..8r+7
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rows[it][i] = ld16(w_uv + ((int64_t)h * kLat + 4 * q + i) * kV + eb * kUpEB + 8 * r);
  }
  auto a_load = [&](int mt, u32x4 a[16]) {
    const int trow = min((mb * kUpMT + mt) * 32 + n, T - 1);
    const uint16_t* ap = o_lat + ((int64_t)trow * kHeads + h) * kLat + kh * 256 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) a[ks] = ld16(ap + 16 * ks);
  };
  u32x4 a[16];
  a_load(0, a);
  // keep the first tile's A loads here, in flight with the W_UV loads (the
  // compiler would otherwise sink them past the barrier, one latency each)
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+v"(a[ks]));
#pragma unroll
  for (int it = 0; it < kUnits; ++it) {
    const int u = tid + 256 * it;
    const int q = u >> 3, r = u & 7;
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const uint32_t sel = (e8 & 1) ? 0x07060302u : 0x05040100u;
      const int dw = e8 >> 1;
      const u32x2 v = {__builtin_amdgcn_perm(rows[it][1][dw], rows[it][0][dw], sel),
                       __builtin_amdgcn_perm(rows[it][3][dw], rows[it][2][dw], sel)};
      *reinterpret_cast<u32x2*>(&wt[(8 * r + e8) * kWvLds + 4 * q]) = v;
    }
  }
  __syncthreads();
  const uint16_t* bp = &wt[(nt * 32 + n) * kWvLds + kh * 256 + 8 * g];
  for (int mt = 0; mt < kUpMT; ++mt) {
    const int tbase = (mb * kUpMT + mt) * 32;
    if (tbase >= T) break;
    if (mt > 0) a_load(mt, a);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      acc = mfma32(as_bf16x8(a[ks]), as_bf16x8(*reinterpret_cast<const u32x4*>(bp + 16 * ks)), acc);
    if (kh == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[nt][lane * 16 + r] = acc[r];
    }
    __syncthreads();
    if (kh == 0) {
      const int e = eb * kUpEB + nt * 32 + n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = tbase + 8 * (r >> 2) + 4 * g + (r & 3);
        const float v = acc[r] + red[nt][lane * 16 + r];
        if (tr < T) {
          const int64_t o = ((int64_t)tr * kHeads + h) * kV + e;
          if (out_f32) reinterpret_cast<float*>(out)[o] = v;
          else reinterpret_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- merge + upproj, decode
// After the decode core (batches of up to 16 queries) with key splits: the
// split merge and the V up-projection of one head as one launch.  grid (64
// heads, 4 blocks of 64 output dims, groups of tq <= 16 queries), 512
// threads.  The decode core writes its partials head-major (o_part[t][s][h]
// [512], normalised by the split's own sum) so that a head's are contiguous
// 1 KB rows.  Every load goes out before
// any is used: the W_UV slice (64 KB), and per thread the rows of one
// (query, 8-dim chunk) pair for the first 16 splits with their (m, l).  The
// merged o_lat rows (bf16, as the separate merge stores them) form the A tile
// [16 queries][512] in LDS; out[t][h][64 dims] = A . W_UV[h][:, block] by
// 16x16x32 MFMAs, wave w taking dims 16(w % 4) .. +15 over half w / 4 of K.
constexpr int kMuThreads = 512;
static_assert(kDecTMax <= 16, "the A tile holds up to 16 queries");
constexpr int kMuCh = 16;                  // splits requested at once
constexpr int kMuQueries = 16;             // queries per workgroup (at most 16: the A tile's rows)
constexpr int kMuARow = kLat + 8;          // A tile row (bf16, 16 B pad)

__global__ __launch_bounds__(kMuThreads) void merge_upproj_kernel(const uint16_t* __restrict__ o_part,
                                                                  const float* __restrict__ ml_part, int S,
                                                                  const uint16_t* __restrict__ w_uv,
                                                                  void* __restrict__ out, int out_f32, int T,
                                                                  int tq) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kUpEB * kWvLds];
  __shared__ __attribute__((aligned(16))) uint16_t sa[16 * kMuARow];
  __shared__ f32x4 red[4][64];
  const int h = blockIdx.x, eb = blockIdx.y;
  const int t0 = blockIdx.z * tq, nq = min(tq, T - t0);  // this workgroup's queries
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // W_UV[h][c][64 eb .. +63]: unit u covers c = 4q .. 4q+3, e = 8r .. 8r+7
  constexpr int kUnits = (kLat / 4) * (kUpEB / 8) / kMuThreads;
  u32x4 rows[kUnits][4];
#pragma unroll
  for (int it = 0; it < kUnits; ++it) {
    const int u = tid + kMuThreads * it;
    const int q = u >> 3, r = u & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rows[it][i] = ld16(w_uv + ((int64_t)h * kLat + 4 * q + i) * kV + eb * kUpEB + 8 * r);
  }
  // W_UV slice transposed into wt[e][c] (B operand: 8 consecutive c per
  // lane); done once the first merge loads are out, while they are in flight
  auto transpose_w = [&]() __attribute__((always_inline)) {
    // (the W_UV registers pass through an empty asm that also orders memory:
    // the compiler otherwise hoists the transposition, and its wait for the
    // W_UV loads, above the merge loads)
#pragma unroll
    for (int it = 0; it < kUnits; ++it)
      asm volatile("" : "+v"(rows[it][0]), "+v"(rows[it][1]), "+v"(rows[it][2]), "+v"(rows[it][3]) : : "memory");
#pragma unroll
    for (int it = 0; it < kUnits; ++it) {
      const int u = tid + kMuThreads * it;
      const int q = u >> 3, r = u & 7;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const uint32_t sel = (e8 & 1) ? 0x07060302u : 0x05040100u;
        const int dw = e8 >> 1;
        const u32x2 v = {__builtin_amdgcn_perm(rows[it][1][dw], rows[it][0][dw], sel),
                         __builtin_amdgcn_perm(rows[it][3][dw], rows[it][2][dw], sel)};
        *reinterpret_cast<u32x2*>(&wt[(8 * r + e8) * kWvLds + 4 * q]) = v;
      }
    }
  };
  // merge: thread pairs (query t0 + tl, chunk of 8 dims), tid + 512 i, i < 2
  const int npairs = nq * (kLat / 8);
  for (int p0 = 0; p0 < npairs; p0 += kMuThreads) {
    const int pr = p0 + tid;
    const bool live = pr < npairs;
    const int tl = live ? pr >> 6 : 0, c8 = pr & 63;
    const int t = t0 + tl;
    const uint16_t* src = o_part + ((int64_t)t * S * kHeads + h) * kLat + 8 * c8;
    const float* ml = ml_part + ((int64_t)t * S * kHeads + h) * 2;
    float mstar = -1e30f, L = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += kMuCh) {
      f32x2 m_l[kMuCh];
      u32x4 v[kMuCh];
#pragma unroll
      for (int u = 0; u < kMuCh; ++u) {
        const int sp = min(s0 + u, S - 1);  // past S: split S - 1 again, weight 0
        m_l[u] = *reinterpret_cast<const f32x2*>(ml + (int64_t)sp * kHeads * 2);
        v[u] = ld16(src + (int64_t)sp * kPartSlab);
      }
      if (p0 == 0 && s0 == 0) transpose_w();  // (every workgroup has a first round)
      float cm = mstar;
#pragma unroll
      for (int u = 0; u < kMuCh; ++u) cm = s0 + u < S ? fmaxf(cm, m_l[u][0]) : cm;
      if (cm > mstar) {
        const float sc = exp2f(mstar - cm);
        L *= sc;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= sc;
        mstar = cm;
      }
#pragma unroll
      for (int u = 0; u < kMuCh; ++u) {
        const float wgt = s0 + u < S ? exp2f(m_l[u][0] - mstar) * m_l[u][1] : 0.f;
        L += wgt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += wgt * __uint_as_float(v[u][i] << 16);
          acc[2 * i + 1] += wgt * __uint_as_float(v[u][i] & 0xFFFF0000u);
        }
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (live)
      *reinterpret_cast<u32x4*>(&sa[tl * kMuARow + 8 * c8]) =
          u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  }
  __syncthreads();
  // out rows 4g + i (queries), column l16 of dim block eblk
  const int l16 = lane & 15, g = lane >> 4;
  const int eblk = wave & 3, kh = wave >> 2;
  const uint16_t* ap = &sa[l16 * kMuARow + kh * 256 + 8 * g];
  const uint16_t* bp = &wt[(eblk * 16 + l16) * kWvLds + kh * 256 + 8 * g];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    acc = mfma16(as_bf16x8(*reinterpret_cast<const u32x4*>(ap + 32 * ks)),
                 as_bf16x8(*reinterpret_cast<const u32x4*>(bp + 32 * ks)), acc);
  if (kh == 1) red[eblk][lane] = acc;
  __syncthreads();
  if (kh == 0) {
    acc += red[eblk][lane];
    const int e = eb * kUpEB + eblk * 16 + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = 4 * g + i;
      if (tl < nq) {
        const int64_t o = ((int64_t)(t0 + tl) * kHeads + h) * kV + e;
        if (out_f32) reinterpret_cast<float*>(out)[o] = acc[i];
        else reinterpret_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16_bits(acc[i]);
      }
    }
  }
}

// ---------------------------------------------------------------- upproj, many queries
// W_UV[h] is [c][e] with e contiguous, while MFMA operands take 8 consecutive
// c per lane.  For large batches the weights are transposed once per call into
// the workspace (W_UVt [64][256 e][512 c], 16.8 MB) and the product runs as
// head_gemm_kernel<512, 256> (below).
constexpr int kUpTMin = 256;        // batches from this size use the transposed path
// 32-query tiles per head_gemm_kernel workgroup: at least 4 groups per head
// (256 workgroups), at most 32 tiles
inline int head_gemm_tiles(int ntb) { return ntb / 4 < 1 ? 1 : (ntb / 4 > 32 ? 32 : ntb / 4); }
constexpr int kUpStageRow = 36;     // fp32 per staged row (32 + pad)

__global__ __launch_bounds__(256) void wuv_transpose_kernel(const uint16_t* __restrict__ w_uv,
                                                            uint16_t* __restrict__ w_uvt) {
  // grid (64 heads, 8 blocks of 64 c, 4 blocks of 64 e): one 64 x 64 tile via LDS
  __shared__ uint16_t tile[64][66];
  const int h = blockIdx.x, c0 = blockIdx.y * 64, e0 = blockIdx.z * 64, tid = threadIdx.x;
  const int r = tid >> 2, q = tid & 3;  // row of the tile, 16-element quarter
  {
    const uint16_t* src = w_uv + ((int64_t)h * kLat + c0 + r) * kV + e0 + 16 * q;
    const u32x4 v0 = ld16(src), v1 = ld16(src + 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[r][16 * q + 2 * i] = (uint16_t)(v0[i] & 0xFFFFu);
      tile[r][16 * q + 2 * i + 1] = (uint16_t)(v0[i] >> 16);
      tile[r][16 * q + 8 + 2 * i] = (uint16_t)(v1[i] & 0xFFFFu);
      tile[r][16 * q + 8 + 2 * i + 1] = (uint16_t)(v1[i] >> 16);
    }
  }
  __syncthreads();
  u32x4 o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = (uint32_t)tile[16 * q + 2 * i][r] | ((uint32_t)tile[16 * q + 2 * i + 1][r] << 16);
    o1[i] = (uint32_t)tile[16 * q + 8 + 2 * i][r] | ((uint32_t)tile[16 * q + 8 + 2 * i + 1][r] << 16);
  }
  uint16_t* dst = w_uvt + ((int64_t)h * kV + e0 + r) * kLat + c0 + 16 * q;
  st16(dst, o0);
  st16(dst + 8, o1);
}

// Head-batched product over 32-query tiles, for large batches:
//   C[t, h, col] = sum_k A[(t*64 + h)*K + k] * B[(h*NCOL + col)*K + k]
// (absorption: A = q_nope, B = W_UK, K = 192, NCOL = 512; up-projection:
// A = o_lat, B = W_UVt, K = 512, NCOL = 256).  grid (64 heads, groups of tpw
// tiles; head_gemm_tiles keeps >= 256 workgroups and amortises each
// workgroup's B load over up to 32 tiles); 8 waves, wave w owning columns [w*NCOL/8, +NCOL/8) with
// their B fragments resident.  The A rows of a tile (32 x K bf16) are read
// once per workgroup with coalesced 16-byte loads (consecutive threads,
// consecutive pieces of a row) into a double-buffered, padded LDS tile while
// the previous tile is computed; every wave takes its A fragments from LDS.
// Output blocks (32 queries x 32 columns) are staged in LDS and written as
// 16-byte pieces of output rows (bf16, round to nearest even, or fp32).
template <int K, int NCOL>
__global__ __launch_bounds__(512) void head_gemm_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        void* __restrict__ C, int out_f32, int T, int tpw) {
  constexpr int kCW = NCOL / 8, kNB = kCW / 32, kKS = K / 16, kRowLds = K + 8;
  constexpr int kChunks = 32 * K / 8;  // 16-byte pieces of an A tile
  constexpr int kCPT = (kChunks + 511) / 512;
  static_assert(kCW % 32 == 0 && K % 16 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t at[2][32 * kRowLds];
  __shared__ __attribute__((aligned(16))) float stage[8][32 * kUpStageRow];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int ntb = (T + 31) / 32;
  const int tb0 = blockIdx.y * tpw, tb1 = min(ntb, tb0 + tpw);
  if (tb0 >= tb1) return;
  bf16x8 bw[kNB][kKS];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const uint16_t* bp = B + ((int64_t)h * NCOL + wave * kCW + nb * 32 + n) * K + 8 * g;
#pragma unroll
    for (int j = 0; j < kKS; ++j) bw[nb][j] = as_bf16x8(ld16(bp + 16 * j));
  }
  u32x4 stg[kCPT];
  auto gload = [&](int tb) {
#pragma unroll
    for (int c = 0; c < kCPT; ++c) {
      const int lin = tid + 512 * c;
      if (kChunks % 512 == 0 || lin < kChunks) {
        const int r = lin / (K / 8), q = lin - r * (K / 8);
        const int t = min(tb * 32 + r, T - 1);
        stg[c] = ld16(A + ((int64_t)t * kHeads + h) * K + 8 * q);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < kCPT; ++c) {
      const int lin = tid + 512 * c;
      if (kChunks % 512 == 0 || lin < kChunks) {
        const int r = lin / (K / 8), q = lin - r * (K / 8);
        st16(&at[buf][r * kRowLds + 8 * q], stg[c]);
      }
    }
  };
  gload(tb0);
  lstore(0);
  __syncthreads();
  float* st = stage[wave];
  for (int tb = tb0; tb < tb1; ++tb) {
    const int buf = (tb - tb0) & 1;
    if (tb + 1 < tb1) gload(tb + 1);
    f32x16 acc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x16{};
    const uint16_t* ap = &at[buf][n * kRowLds + 8 * g];
#pragma unroll
    for (int j = 0; j < kKS; ++j) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(ap + 16 * j));
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[nb] = mfma32(a, bw[nb][j], acc[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      // element r of lane (g, n): query row 8(r/4) + 4g + r%4 of the tile, column n of block nb
#pragma unroll
      for (int r = 0; r < 16; ++r) st[(8 * (r >> 2) + 4 * g + (r & 3)) * kUpStageRow + n] = acc[nb][r];
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int row = lane >> 1, half = lane & 1;  // lane writes 16 columns of one row
      const int tr = tb * 32 + row;
      const float* sp = st + row * kUpStageRow + 16 * half;
      f32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const f32x4*>(sp + 4 * i);
      if (tr < T) {
        const int64_t o = ((int64_t)tr * kHeads + h) * NCOL + wave * kCW + nb * 32 + 16 * half;
        if (out_f32) {
          float* dst = reinterpret_cast<float*>(C) + o;
#pragma unroll
          for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(dst + 4 * i) = v[i];
        } else {
          uint16_t* dst = reinterpret_cast<uint16_t*>(C) + o;
          u32x4 p0, p1;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            p0[2 * i] = pack_bf16x2(v[i][0], v[i][1]);
            p0[2 * i + 1] = pack_bf16x2(v[i][2], v[i][3]);
            p1[2 * i] = pack_bf16x2(v[2 + i][0], v[2 + i][1]);
            p1[2 * i + 1] = pack_bf16x2(v[2 + i][2], v[2 + i][3]);
          }
          st16(dst, p0);
          st16(dst + 8, p1);
        }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next block's writes
    }
    if (tb + 1 < tb1) lstore(buf ^ 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- plan + launch
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Steps per stream of the decode core for a batch of T <= 16 queries at top-k
// k >= 1 (about 256 workgroups: ceil(128 / T) key splits per query), and its
// keys per split: 1-4 steps; splits of more than 4 steps take the ring form
// (NS = 8), keys per split a multiple of 128 (whole rounds of 4 steps).
static_assert(kMaxTopk / ((128 + kDecTMax - 1) / kDecTMax) <= kDecMaxKps, "ring splits fit s_idx");
static int dec_pair_steps(int T, int k, int* kps) {
  const int sp = (128 + T - 1) / T;
  const int pk = (k + sp - 1) / sp;
  const int ns = (pk + 2 * kDecKT - 1) / (2 * kDecKT);
  if (ns <= 4) {
    if (kps) *kps = 2 * kDecKT * ns;
    return ns;
  }
  const int rk = (pk + 8 * kDecKT - 1) / (8 * kDecKT) * (8 * kDecKT);
  if (kps) *kps = rk;
  return 8;
}

MlaPlan plan_mla(int T, int k) {
  MlaPlan p{};
  p.T = T;
  p.k = k;
  // Small batches split each query's keys so that about 256 workgroups run,
  // with at least 64 keys (2 tiles) per split.
  int s = 1;
  if (T > 0 && T < 256) s = (256 + T - 1) / T;
  const int cap = k / 64 > 32 ? k / 64 : 32;
  s = s < cap ? s : cap;
  const int max_s = (k + kKT - 1) / kKT;
  s = s < max_s ? s : max_s;
  if (s < 1) s = 1;
  int kps = (k + s - 1) / s;
  kps = (kps + kKT - 1) / kKT * kKT;
  p.keys_per_split = kps;
  p.splits = (k + kps - 1) / kps;
  // Decode core (batches of up to 16 queries)
  p.dec = T > 0 && T <= kDecTMax && k >= 1;
  if (p.dec) {
    dec_pair_steps(T, k, &p.dec_keys_per_split);
    p.dec_splits = (k + p.dec_keys_per_split - 1) / p.dec_keys_per_split;
  }
  const int max_splits = p.dec && p.dec_splits > p.splits ? p.dec_splits : p.splits;
  const size_t lat = (size_t)T * kHeads * kLat * sizeof(uint16_t);
  p.q_lat_off = 0;
  p.o_lat_off = align_up(lat, 256);
  size_t end = p.o_lat_off + align_up(lat, 256);
  if (max_splits > 1) {
    p.part_off = end;
    end += align_up((size_t)T * max_splits * kHeads * kLat * sizeof(uint16_t), 256);
    p.ml_off = end;
    end += align_up((size_t)T * max_splits * kHeads * 2 * sizeof(float), 256);
  }
  if (T >= kUpTMin) {
    p.wuvt_off = end;
    end += align_up((size_t)kHeads * kV * kLat * sizeof(uint16_t), 256);
  }
  p.total = end;
  return p;
}

hipError_t launch_sparse_mla(const LaunchBatch& b, const MlaPlan& p, const uint16_t* q_nope,
                             const uint16_t* q_rope, const void* kv, const uint16_t* w_uk,
                             const uint16_t* w_uv, const int32_t* idx, float scale, void* out,
                             int out_f32, void* ws, bool q_lat_ready, hipStream_t st) {
  char* base = static_cast<char*>(ws);
  const bool dec = p.dec && !b.kv_int4;
  const int S = dec ? p.dec_splits : p.splits;
  uint16_t* q_lat = reinterpret_cast<uint16_t*>(base + p.q_lat_off);
  uint16_t* o_lat = reinterpret_cast<uint16_t*>(base + p.o_lat_off);
  uint16_t* o_part = S > 1 ? reinterpret_cast<uint16_t*>(base + p.part_off) : nullptr;
  float* ml_part = S > 1 ? reinterpret_cast<float*>(base + p.ml_off) : nullptr;
  const int T = b.T;
  const int ntb = (T + 31) / 32;
  hipError_t e;
  if (!q_lat_ready) {
    const int nqg = (ntb + kAbsorbTilesPerWg - 1) / kAbsorbTilesPerWg;
    if (ntb <= 2)
      absorb_kernel<4><<<dim3(kHeads, nqg, 4), 256, 0, st>>>(q_nope, w_uk, q_lat, T);
    else
      head_gemm_kernel<kNope, kLat><<<dim3(kHeads, (ntb + head_gemm_tiles(ntb) - 1) / head_gemm_tiles(ntb)), 512,
                                        0, st>>>(q_nope, w_uk, q_lat, 0, T, head_gemm_tiles(ntb));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(T, p.splits);
  const int kps = p.keys_per_split;
  if (dec) {
    int dk;  // (the plan's dec_keys_per_split)
    const int ns = dec_pair_steps(T, p.k, &dk);
    const int dgrid = 16 * ((T * S + 7) / 8);
    const uint16_t* const kvb = static_cast<const uint16_t*>(kv);
#define DSA_DEC_LAUNCH(PG, NS)                                                                       \
  mla_decode_kernel<PG, NS><<<dgrid, kDecWaves * 64, 0, st>>>(b.q_seq, b.rows, q_lat, q_rope, kvb, idx, T, \
                                                               p.k, scale_log2, dk, S, o_lat, o_part, ml_part)
    if (b.paged()) {
      switch (ns) {
        case 1: DSA_DEC_LAUNCH(true, 1); break;
        case 2: DSA_DEC_LAUNCH(true, 2); break;
        case 3: DSA_DEC_LAUNCH(true, 3); break;
        case 4: DSA_DEC_LAUNCH(true, 4); break;
        default: DSA_DEC_LAUNCH(true, 8); break;
      }
    } else {
      switch (ns) {
        case 1: DSA_DEC_LAUNCH(false, 1); break;
        case 2: DSA_DEC_LAUNCH(false, 2); break;
        case 3: DSA_DEC_LAUNCH(false, 3); break;
        case 4: DSA_DEC_LAUNCH(false, 4); break;
        default: DSA_DEC_LAUNCH(false, 8); break;
      }
    }
#undef DSA_DEC_LAUNCH
  } else if (S == 1 && !b.kv_int4) {
    if (b.paged()) {
      int32_t* const entries = reinterpret_cast<int32_t*>(o_lat);
      ws_paged_entries_kernel<<<T, 256, 0, st>>>(b.q_seq, b.rows, idx, p.k, entries);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      mla_ws_kernel<true><<<T, kCoreThreads, 0, st>>>(b.q_seq, b.rows, q_lat, q_rope, static_cast<const uint16_t*>(kv),
                                                      entries, p.k, scale_log2, o_lat);
    } else {
      mla_ws_kernel<false><<<T, kCoreThreads, 0, st>>>(b.q_seq, b.rows, q_lat, q_rope,
                                                       static_cast<const uint16_t*>(kv), idx, p.k, scale_log2, o_lat);
    }
  } else if (b.paged() && b.kv_int4)
    mla_core_kernel<true, true><<<grid, kCoreThreads, 0, st>>>(b.q_seq, b.rows, q_lat, q_rope, kv, idx, p.k,
                                                               scale_log2, kps, S, o_lat, o_part, ml_part);
  else if (b.paged())
    mla_core_kernel<true, false><<<grid, kCoreThreads, 0, st>>>(b.q_seq, b.rows, q_lat, q_rope, kv, idx, p.k,
                                                                scale_log2, kps, S, o_lat, o_part, ml_part);
  else if (b.kv_int4)
    mla_core_kernel<false, true><<<grid, kCoreThreads, 0, st>>>(b.q_seq, b.rows, q_lat, q_rope, kv, idx, p.k,
                                                                scale_log2, kps, S, o_lat, o_part, ml_part);
  else
    mla_core_kernel<false, false><<<grid, kCoreThreads, 0, st>>>(b.q_seq, b.rows, q_lat, q_rope, kv, idx, p.k,
                                                                 scale_log2, kps, S, o_lat, o_part, ml_part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dec && S > 1) {  // the decode core's head-major partials: merge and up-projection in one launch
    const int tq = kMuQueries;
    merge_upproj_kernel<<<dim3(kHeads, kV / kUpEB, (T + tq - 1) / tq), kMuThreads, 0, st>>>(o_part, ml_part, S, w_uv,
                                                                                           out, out_f32, T, tq);
    return hipGetLastError();
  }
  if (S > 1) {
    if (S <= 8)
      mla_merge_kernel<8><<<dim3(T, 32), 256, 0, st>>>(o_part, ml_part, S, o_lat);
    else if (S <= 16)
      mla_merge_kernel<16><<<dim3(T, 32), 256, 0, st>>>(o_part, ml_part, S, o_lat);
    else
      mla_merge_kernel<32><<<dim3(T, 32), 256, 0, st>>>(o_part, ml_part, S, o_lat);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (T >= kUpTMin) {
    uint16_t* w_uvt = reinterpret_cast<uint16_t*>(base + p.wuvt_off);
    wuv_transpose_kernel<<<dim3(kHeads, kLat / 64, kV / 64), 256, 0, st>>>(w_uv, w_uvt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    head_gemm_kernel<kLat, kV><<<dim3(kHeads, (ntb + head_gemm_tiles(ntb) - 1) / head_gemm_tiles(ntb)), 512, 0,
                                 st>>>(o_lat, w_uvt, out, out_f32, T, head_gemm_tiles(ntb));
    return hipGetLastError();
  }
  upproj_kernel<<<dim3(kHeads, kV / kUpEB, (T + 32 * kUpMT - 1) / (32 * kUpMT)), 256, 0, st>>>(
      o_lat, w_uv, out, out_f32, T);
  return hipGetLastError();
}

}  // namespace dsa
