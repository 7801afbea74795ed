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
constexpr int kPartSlab = kHeads * kLat;  // fp16 values of one split partial
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

// s_waitcnt vmcnt(n) (n < 16), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
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
    tmax = fmaxf(tmax, xor_lane(tmax, 16));
    tmax = fmaxf(tmax, xor_lane(tmax, 32));
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
  float l_sum = l_part + xor_lane(l_part, 16);
  l_sum += xor_lane(l_sum, 32);
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
      // cache rows, so fp16 holds them to 2^-11) and keep the accumulator order
      // (see mla_merge_kernel): each store instruction writes 512 B of
      // consecutive memory.
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* dst = o_part + ((int64_t)t * S + sp) * kPartSlab + ((wave * 4 + j) * 4) * 256 + lane * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<u32x2*>(dst + e * 256) =
            u32x2{pack_f16x2(o[e][j][0] * inv, o[e][j][1] * inv), pack_f16x2(o[e][j][2] * inv, o[e][j][3] * inv)};
      if (wave == 0 && g == 0) {
        const int64_t base = ((int64_t)t * S + sp) * kHeads + h;
        ml_part[base * 2] = s_m[h];
        ml_part[base * 2 + 1] = L;
      }
    }
  }
}

// ---------------------------------------------------------------- merge
// Split partials of (query t, split s) form one slab of kHeads * kLat fp16
// values, each normalised by its split's sum l, in the core's accumulator
// order: element i of the 4-value group number ((w * 4 + j) * 4 + e) * 64 +
// lane is latent dim 64w + 16e + 4(lane / 16) + i of head 16j + lane % 16.
// ml_part[t][s][h] = (reference max m, sum l).  grid (T, 32): workgroup
// (t, 4w + j) combines latent dims 64w .. 64w+63 of heads 16j .. 16j+15, one
// group of every split per thread, weighting split s by 2^(m_s - max m) l_s.
__global__ __launch_bounds__(256) void mla_merge_kernel(const uint16_t* __restrict__ o_part,
                                                        const float* __restrict__ ml_part, int S,
                                                        uint16_t* __restrict__ o_lat) {
  const int t = blockIdx.x, w = blockIdx.y >> 2, j = blockIdx.y & 3, tid = threadIdx.x;
  const int lane = tid & 63, jj = tid >> 6;
  const int h = 16 * j + (lane & 15), g = lane >> 4;
  const float* ml = ml_part + ((int64_t)t * S * kHeads + h) * 2;
  const uint16_t* src = o_part + (int64_t)t * S * kPartSlab + (((w * 4 + j) * 4 + jj) * 64 + lane) * 4;
  // Splits in chunks of kMergeChunk whose (m, l) pairs and partials are all
  // requested before any is used (one memory latency per chunk).  Past S a
  // slot repeats split S - 1 with weight 0.  A later chunk with a larger
  // maximum rescales what is summed so far (with at most one chunk this is
  // the plain two-pass sum).
  constexpr int kMergeChunk = 32;
  float mstar = -1e30f, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kMergeChunk) {
    f32x2 m_l[kMergeChunk];
    u32x2 v[kMergeChunk];
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const int s = min(s0 + u, S - 1);
      m_l[u] = *reinterpret_cast<const f32x2*>(ml + (int64_t)s * kHeads * 2);
      v[u] = *reinterpret_cast<const u32x2*>(src + (int64_t)s * kPartSlab);
    }
    float cm = mstar;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) cm = s0 + u < S ? fmaxf(cm, m_l[u][0]) : cm;
    if (cm > mstar) {
      const float sc = exp2f(mstar - cm);
      L *= sc;
      acc *= sc;
      mstar = cm;
    }
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const float wgt = s0 + u < S ? exp2f(m_l[u][0] - mstar) * m_l[u][1] : 0.f;
      L += wgt;
      acc += wgt * f32x4{f16_lo(v[u].x), f16_hi(v[u].x), f16_lo(v[u].y), f16_hi(v[u].y)};
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
  const size_t lat = (size_t)T * kHeads * kLat * sizeof(uint16_t);
  p.q_lat_off = 0;
  p.o_lat_off = align_up(lat, 256);
  size_t end = p.o_lat_off + align_up(lat, 256);
  if (p.splits > 1) {
    p.part_off = end;
    end += align_up((size_t)T * p.splits * kHeads * kLat * sizeof(uint16_t), 256);
    p.ml_off = end;
    end += align_up((size_t)T * p.splits * kHeads * 2 * sizeof(float), 256);
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
  uint16_t* q_lat = reinterpret_cast<uint16_t*>(base + p.q_lat_off);
  uint16_t* o_lat = reinterpret_cast<uint16_t*>(base + p.o_lat_off);
  uint16_t* o_part = p.splits > 1 ? reinterpret_cast<uint16_t*>(base + p.part_off) : nullptr;
  float* ml_part = p.splits > 1 ? reinterpret_cast<float*>(base + p.ml_off) : nullptr;
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
  const int kps = p.keys_per_split, S = p.splits;
  if (b.paged() && b.kv_int4)
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
  if (p.splits > 1) {
    mla_merge_kernel<<<dim3(T, 32), 256, 0, st>>>(o_part, ml_part, p.splits, o_lat);
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
