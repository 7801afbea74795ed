// Lightning-indexer scoring on gfx950.
//
// score(t,s) = sum_{h<32} w[t,h] * ReLU(q_idx[t,h,:] . k_idx[s,:]),  s <= q_pos[t]
// (page "2026大模型架构概览（二）：GLM 5 DSV3.2 的 DSA 与 MoE 配置拆解", §2.2: one cheap score
// per query and history token, used only for ranking; page "（五）一万亿次点积砍到两千次：
// DSA 怎么破 N²", indexer section: 32 heads of 128-d dot products over every token).
//
// Both kernels put the 32 indexer heads of one query on the M side of a
// 32x32x16 bf16 MFMA and 32 keys on the N side; K = 128 is 8 MFMA steps.  The
// epilogue applies ReLU and the head weights in fp32 and folds the 32 head rows
// of each key column (16 per lane, then one cross-half lane exchange).
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "topk_plan.h"

namespace dsa {

// ---------------------------------------------------------------- decode scan
// One workgroup = one query x one slice of the row (slice_keys keys, a whole
// number of 128-key tiles; the slicing fills the chip in whole rounds).  A tile
// (32 KB) is read with fully coalesced 16-byte non-temporal loads (keys are
// touched once per decode step) into LDS, double buffered; each of the 4 waves
// then takes 32 keys of the tile as the MFMA B operand from LDS.  Reading the
// MFMA layout straight from HBM (2 lanes per 256-byte key row per load) was
// measured at about half the bandwidth of this coalesced form.
// With `lists` set, the workgroup also counts the top digit of its scores in
// LDS and writes the slice's sparse bin list for the split top-k.
// PAGED: the cache is paged (pages of >= 16 tokens, so every 16-key granule of
// a tile lies in one page).  Chunk c of every thread's tile load lies in
// granule c; each thread loads the 8 page ids of tile i + 2 into registers
// while tile i is computed (they complete with the key loads of tile i + 1),
// so key loads never wait on a lookup.
constexpr int kScanLds = kIdxDim + 8;  // bf16 per LDS key row (16 B pad)
constexpr int kGranule = 16;           // keys per page-table lookup (smallest page)

template <bool PAGED>
__global__ __launch_bounds__(256) void idx_scan_kernel(
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, CacheRows cr,
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ k_idx, float* __restrict__ scores, int64_t ld, int slice_keys,
    char* __restrict__ lists, SplitWs sw, const int32_t* __restrict__ row_mask) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kScanTile * kScanLds];
  __shared__ uint32_t hist[kTkBins / 2];
  __shared__ int wave_tot[4];
  const int t = blockIdx.x;
  if (row_mask != nullptr && row_mask[t] == 0) return;  // only the rows a mask names
  const int pos = q_pos[t];
  const int k0 = blockIdx.y * slice_keys;
  if (k0 > pos) return;
  const int kend = min(k0 + slice_keys, pos + 1);
  const int ntiles = (kend - k0 + kScanTile - 1) / kScanTile;
  const int seq = q_seq[t];
  const int64_t row0 = PAGED ? 0 : cr.seq_row0[seq];
  const int32_t* bt = PAGED ? cr.table + (int64_t)seq * cr.max_pages : nullptr;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // pages of the 8 granules of a tile (granules past pos: the page of pos)
  constexpr int kGr = kScanTile / kGranule;
  auto pid_fetch = [&](int tile, int p[kGr]) {
#pragma unroll
    for (int c = 0; c < kGr; ++c) p[c] = bt[min(k0 + tile * kScanTile + kGranule * c, pos) >> cr.page_shift];
  };
  const int g = lane >> 5, n = lane & 31;
  if (lists) {
#pragma unroll
    for (int i = 0; i < kTkBins / 2 / 256; ++i) hist[tid + 256 * i] = 0u;
  }

  // A operand: head n of query t, K-group g (dims 16j + 8g .. +8 at step j).
  bf16x8 qa[8];
  const uint16_t* qp = q_idx + ((int64_t)t * kIdxHeads + n) * kIdxDim + 8 * g;
#pragma unroll
  for (int j = 0; j < 8; ++j) qa[j] = as_bf16x8(ld16(qp + 16 * j));
  // Head weights of the accumulator rows this lane holds.
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = bf16_to_f32(w[t * kIdxHeads + 8 * (r >> 2) + 4 * g + (r & 3)]);

  u32x4 st[8];
  // Chunk c covers keys base + 16c + (tid >> 4): granule c.  A key clamped to
  // pos may be read from another row of granule c's page (never used).
  auto gload = [&](int tile, const int p[kGr]) {
    const int base = k0 + tile * kScanTile;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int lin = tid + 256 * c;  // 16-byte chunk of the 32 KB tile
      const int key = min(base + (lin >> 4), pos);  // rows past pos: never used
      int64_t row = row0 + key;
      if (PAGED) row = ((int64_t)p[c] << cr.page_shift) | (key & ((1 << cr.page_shift) - 1));
      st[c] = ld16_nt(k_idx + row * kIdxDim + (lin & 15) * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int lin = tid + 256 * c;
      st16(&ks[buf][(lin >> 4) * kScanLds + (lin & 15) * 8], st[c]);
    }
  };
  float* srow = scores + (int64_t)t * ld;
  int pa[kGr] = {}, pb[kGr] = {};  // pages of tiles tile + 1 and tile + 2 (PAGED)
  if (PAGED) {
    pid_fetch(0, pb);
    if (ntiles > 1) pid_fetch(1, pa);
  }
  gload(0, pb);
  // The query operands and head weights arrive here (their loads were issued
  // before tile 0's, which stay in flight).  Left to itself the compiler sinks
  // these loads to the loop entry and then, in every iteration, waits for the
  // loads issued since (the next tile's keys) before the first MFMA: the key
  // latency would sit on the compute path of every tile.
#pragma unroll
  for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(qa[j]));
#pragma unroll
  for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(wr[r]));
  lstore(0);
  __syncthreads();
  // Scores wait in registers and are written after the slice's last tile (or
  // every kWin tiles of a longer slice): written tile by tile, in among the
  // key reads, the 6.55 MB of scores of an 8 x 204,800 decode step cost ~7 us
  // of a ~68 us scan; held back they cost ~3 us.  win[i] holds the score of
  // tile tile - (kWin - 1 - i) (lanes 0-31; lanes 32-63 hold the same values).
  constexpr int kWin = 32;
  float win[kWin];
#pragma unroll
  for (int i = 0; i < kWin; ++i) win[i] = 0.f;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) gload(tile + 1, pa);
    if (PAGED && tile + 2 < ntiles) pid_fetch(tile + 2, pb);
    const uint16_t* bp = &ks[buf][(wave * 32 + n) * kScanLds + 8 * g];
    f32x16 acc = {};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc = mfma32(qa[j], as_bf16x8(*reinterpret_cast<const u32x4*>(bp + 16 * j)), acc);
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) part = fmaf(wr[r], relu(acc[r]), part);
    const float tot = part + xor_lane(part, 32);
    const int s = k0 + tile * kScanTile + wave * 32 + n;
    if (tile + 1 < ntiles) lstore(buf ^ 1);
    if (lists && g == 0 && s <= pos) hist16_add(hist, score_key(tot));
#pragma unroll
    for (int i = 0; i < kWin - 1; ++i) win[i] = win[i + 1];
    win[kWin - 1] = tot;
    if (tile == ntiles - 1 || (tile & (kWin - 1)) == kWin - 1) {
      // tiles first .. tile since the last write (the barrier below waits for
      // LDS only: no step waits for these stores)
      const int first = tile & ~(kWin - 1);
#pragma unroll
      for (int i = 0; i < kWin; ++i) {
        const int tt = tile - (kWin - 1 - i);
        const int si = k0 + tt * kScanTile + wave * 32 + n;
        if (g == 0 && tt >= first && si <= pos) srow[si] = win[i];
      }
    }
    if (PAGED) {
#pragma unroll
      for (int c = 0; c < kGr; ++c) pa[c] = pb[c];
    }
    lds_sync();
  }
  if (lists)
    write_bin_list<256>(hist,
                        reinterpret_cast<uint32_t*>(lists + (size_t)t * sw.per_query + sw.list_off +
                                                    (size_t)blockIdx.y * sw.list_stride),
                        wave_tot);
}

// ---------------------------------------------------------------- prefill GEMM
// One workgroup = kGemmQB consecutive queries x split_keys keys.  Each of the
// kGemmWaves waves keeps kGemmQPW queries (32 heads each) as resident A
// operands; key tiles of kGemmKT keys reach LDS by direct global->LDS loads
// (no register staging), double buffered, and are shared by the waves (one
// workgroup per CU; four waves per workgroup with two workgroups per CU
// measured slower).  Queries of one block normally share a sequence; a block
// that mixes sequences is processed once per distinct sequence.
//
// LDS holds a key row as 16 chunks of 16 B with chunk c of row r at slot
// c ^ (r & 15), so the B-fragment reads (32 rows, one chunk each, per
// instruction) spread over all banks without padding; a direct load writes
// lane L of a wave instruction to slot L of a 1 KB block, so each lane fetches
// the chunk that its slot holds.
// A tile is computed in groups of 64 keys.  The fragments of key block 0 of
// the next group are read as soon as the two MFMA chains that use block 0 of
// the current group are issued (likewise block 1); each chain's fold of its
// head rows follows the issue of the next chain, and the two chains of a
// query (keys 0-31 and 32-63 of a group) are summed and stored together
// through one lane-half swap (the last pair of a group after the next group's
// first chain, across the tile barrier too), so LDS latency and epilogue VALU
// overlap MFMA work.
constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kGemmQPW = 2;
constexpr int kGemmQB = kGemmWaves * kGemmQPW;
constexpr int kGemmKT = 256;  // keys per LDS tile (one barrier)
constexpr int kGemmGroups = kGemmKT / 64;
// Keys per workgroup: the whole context when the query blocks alone fill the
// chip (fewest workgroup prologues and no uneven last round: 5.59 ms against
// 5.96 ms with 8,192-key splits at 4,096 queries x 204,800 keys), else the
// context split so that about 256 workgroups run; at most 2^24 keys (store
// offsets of a split stay far below 2^32).
constexpr int kGemmMinWgs = 256;
constexpr int kGemmMaxSplit = 1 << 24;
inline int gemm_split_keys(int T, int max_ctx) {
  const int nqb = (T + kGemmQB - 1) / kGemmQB;
  int nsplit = nqb >= kGemmMinWgs ? 1 : (kGemmMinWgs + nqb - 1) / nqb;
  nsplit = max(nsplit, (int)(((int64_t)max_ctx + kGemmMaxSplit - 1) / kGemmMaxSplit));
  const int per = (int)(((int64_t)max_ctx + nsplit - 1) / nsplit);
  return (per + kGemmKT - 1) / kGemmKT * kGemmKT;
}
constexpr int kGemmLoads = kGemmKT * kIdxDim * 2 / (kGemmThreads * 16);  // direct loads per thread per tile
constexpr int kDlStride = 4 * kGemmWaves;  // key rows between a thread's successive direct loads

// What the GEMM produces (MODE):
//   kGemmScores      every score s <= q_pos into scores[t*ld + s];
//   kGemmSample      the scores of positions 0, R, 2R, ... <= q_pos (R = o.stride)
//                    into scores[t*ld + i] for position R*i;
//   kGemmCandidates  no score matrix: each query appends (monotone key, position)
//                    of every score >= theta[t] (s <= q_pos), in position order,
//                    to its list cand[t*cap ..] (entries past cap are counted, not
//                    written) and writes the count to cnt[t].  Needs one
//                    workgroup per query block over the whole context.
enum { kGemmScores = 0, kGemmSample = 1, kGemmCandidates = 2 };
struct GemmOut {
  float* scores;        // scores / sample scores
  int64_t ld;
  int stride;           // kGemmSample: positions per sample
  const float* theta;   // kGemmCandidates: per query threshold
  uint32_t* cand;       // kGemmCandidates: [T][cap][2] u32 (key, position)
  int cap;
  int* cnt;             // kGemmCandidates: [T]
};

template <bool PAGED, int MODE>
__global__ __launch_bounds__(kGemmThreads) void idx_gemm_kernel(
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, CacheRows cr,
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ k_idx, GemmOut o, int T, int split_keys) {
  float* const scores = o.scores;
  const int64_t ld = o.ld;
  // two buffers as two arrays: with distinct objects the compiler sees that
  // direct loads into one do not alias reads of the other, and does not make
  // those reads wait for the loads
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[kGemmKT * kIdxDim];
  __shared__ __attribute__((aligned(1024))) uint16_t ks1[kGemmKT * kIdxDim];
  __shared__ int s_seq[kGemmQB], s_pos[kGemmQB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level addresses stay scalar
  const int g = lane >> 5, n = lane & 31;
  const int t0 = blockIdx.x * kGemmQB;
  if (tid < kGemmQB) {
    const int t = t0 + tid;
    s_seq[tid] = t < T ? q_seq[t] : -1;
    // kGemmSample works in sample indices: sample i is position stride * i
    s_pos[tid] = t < T ? (MODE == kGemmSample ? q_pos[t] / o.stride : q_pos[t]) : -1;
  }
  __syncthreads();
  const int split0 = blockIdx.y * split_keys;
  int maxpos = -1;
#pragma unroll
  for (int i = 0; i < kGemmQB; ++i) maxpos = max(maxpos, s_pos[i]);
  if (split0 > maxpos) return;

  bf16x8 qa[kGemmQPW][8];
  float wr[kGemmQPW][16];
#pragma unroll
  for (int qi = 0; qi < kGemmQPW; ++qi) {
    const int tt = min(t0 + wave * kGemmQPW + qi, T - 1);
    const uint16_t* qp = q_idx + ((int64_t)tt * kIdxHeads + n) * kIdxDim + 8 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) qa[qi][j] = as_bf16x8(ld16(qp + 16 * j));
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[qi][r] = bf16_to_f32(w[tt * kIdxHeads + 8 * (r >> 2) + 4 * g + (r & 3)]);
  }

  // Direct load i of this thread: 1 KB block kGemmWaves i + wave of the tile
  // = rows kDlStride i + 4 wave .. +3; the lane's row and (swizzled) chunk.
  static_assert(kDlStride % 16 == 0, "the swizzle of a load's row does not depend on i");
  const int dl_row = 4 * wave + (lane >> 4);             // + kDlStride i
  const int dl_chunk = (lane & 15) ^ (dl_row & 15);
  // B-fragment read offsets (bf16 units) of key block nt of a group, step j:
  // row 32 nt + n (+ 64 per group), logical chunk 2j + g.
  int frag_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) frag_off[j] = n * kIdxDim + (((2 * j + g) ^ (n & 15)) << 3);
  // kGemmCandidates: per query of the wave, its threshold and list length so far
  // (wave-uniform; a query belongs to one sequence, so one pass below appends)
  float th[kGemmQPW];
  int ncand[kGemmQPW];
#pragma unroll
  for (int qi = 0; qi < kGemmQPW; ++qi) {
    th[qi] = 0.f;
    ncand[qi] = 0;
    if constexpr (MODE == kGemmCandidates) {
      const int tq = t0 + wave * kGemmQPW + qi;
      th[qi] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(o.theta[min(tq, T - 1)])));
    }
  }

  for (int i = 0; i < kGemmQB; ++i) {
    const int sq = s_seq[i];
    if (sq < 0) continue;
    bool seen = false;
    int hi = -1;
    for (int j = 0; j < kGemmQB; ++j) {
      if (j < i && s_seq[j] == sq) seen = true;
      if (s_seq[j] == sq) hi = max(hi, s_pos[j]);
    }
    if (seen) continue;
    const int kbeg = split0;
    const int kend = (int)min((int64_t)split0 + split_keys, (int64_t)hi + 1);
    if (kbeg >= kend) continue;
    const int64_t row0 = PAGED ? 0 : cr.seq_row0[sq];
    const int32_t* bt = PAGED ? cr.table + (int64_t)sq * cr.max_pages : nullptr;
    const int ntiles = (kend - kbeg + kGemmKT - 1) / kGemmKT;
    // PAGED: load i of a tile lies in granule (kGemmWaves i + wave) / 4 (16
    // keys, one page); the page ids of tile + 2 are loaded (into pv) while
    // tile is computed, and made scalar (pa, wave-uniform) once they have
    // arrived.  kGemmSample: consecutive keys of a tile are positions R apart,
    // so each lane loads the page of its own key's position (and keeps it).
    constexpr bool kLanePages = PAGED && MODE == kGemmSample;
    auto pid_fetch = [&](int tile, int p[kGemmLoads]) {
#pragma unroll
      for (int c = 0; c < kGemmLoads; ++c) {
        if constexpr (kLanePages)
          p[c] = bt[(min(kbeg + tile * kGemmKT + kDlStride * c + dl_row, hi) * o.stride) >> cr.page_shift];
        else
          p[c] = bt[min(kbeg + tile * kGemmKT + kGranule * ((kGemmWaves * c + wave) >> 2), hi) >> cr.page_shift];
      }
    };
    auto page_ready = [&](int v) __attribute__((always_inline)) -> int {
      if constexpr (kLanePages) return v;
      return __builtin_amdgcn_readfirstlane(v);
    };
    auto dma = [&](int tile, const int p[kGemmLoads], uint16_t* buf) {
      const int base = kbeg + tile * kGemmKT;
#pragma unroll
      for (int c = 0; c < kGemmLoads; ++c) {
        const int key = min(base + kDlStride * c + dl_row, hi);  // rows past hi: never stored
        const int64_t pos = MODE == kGemmSample ? (int64_t)key * o.stride : (int64_t)key;
        int64_t row = row0 + pos;
        if (PAGED) row = ((int64_t)p[c] << cr.page_shift) | (pos & ((1 << cr.page_shift) - 1));
        // (named pointers: the host pass rejects cast expressions as this builtin's operands)
        const uint16_t* const gsrc = k_idx + row * kIdxDim + dl_chunk * 8;
        uint16_t* const dst = buf + (kGemmWaves * c + wave) * 512;
        __builtin_amdgcn_global_load_lds(gsrc, dst, 16, 0, 0);
      }
    };
    // per query of the wave: a buffer resource over the keys of this split
    // that the query stores (s <= its position; none for another sequence).
    // Stores past its end are dropped by the hardware, so the epilogue stores
    // without a branch.
    __amdgpu_buffer_rsrc_t rs[kGemmQPW];
    int qlim[kGemmQPW];  // kGemmCandidates: last position the query keeps (-1: another sequence)
#pragma unroll
    for (int qi = 0; qi < kGemmQPW; ++qi) {
      const int local = wave * kGemmQPW + qi;
      const int lim = __builtin_amdgcn_readfirstlane(s_seq[local] == sq ? s_pos[local] : -1);
      qlim[qi] = lim;
      if constexpr (MODE != kGemmCandidates) {
        const int nrec = min(max(lim + 1 - kbeg, 0), split_keys) * 4;
        const uint64_t srow = reinterpret_cast<uint64_t>(scores + (int64_t)(t0 + local) * ld + kbeg);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)srow);
        const uint32_t hi32 = __builtin_amdgcn_readfirstlane((uint32_t)(srow >> 32));
        float* const base = reinterpret_cast<float*>(((uint64_t)hi32 << 32) | lo);
        rs[qi] = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, __builtin_amdgcn_readfirstlane(nrec), kBufferWord3);
      }
    }
    auto chain = [&](int qi, const bf16x8 b[8]) {
      f32x16 acc = {};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = mfma32(qa[qi][j], b[j], acc);
      return acc;
    };
    // Column n of a chain's accumulator is one key of query qi; lanes n and
    // n + 32 hold 16 of its 32 head rows each.  reduce() folds a lane's rows;
    // store_pair() takes the folds of the two chains of one query over keys
    // kb .. kb + 31 (a) and kb + 32 .. kb + 63 (b): one lane-half swap
    // (a's upper half for b's lower half) and one add leave the score of key
    // kb + l in lane l, and all 64 lanes store (offsets from kbeg).
    auto reduce = [&](int qi, const f32x16& acc) {
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part = fmaf(wr[qi][r], relu(acc[r]), part);
      return part;
    };
    auto store_pair = [&](int qi, float pa, float pb, int kb) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
      const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // a(l) + a(l + 32) | b(l - 32) + b(l)
      if constexpr (MODE == kGemmCandidates) {
        // keep key kbeg + kb + lane if it is causal for the query and at least
        // the threshold; the kept lanes append in lane (= position) order
        const int pos = kbeg + kb + lane;
        const bool keep = pos <= qlim[qi] && tot >= th[qi];
        const uint64_t m = __ballot(keep);
        if (m != 0) {
          const int before =
              (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          const int at = ncand[qi] + before;
          if (keep && at < o.cap) {
            uint32_t* const dst = o.cand + ((int64_t)(t0 + wave * kGemmQPW + qi) * o.cap + at) * 2;
            *reinterpret_cast<u32x2*>(dst) = u32x2{score_key(tot), (uint32_t)pos};
          }
          ncand[qi] += __builtin_popcountll(m);
        }
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), rs[qi], 4 * (kb + lane), 0, 0);
      }
    };
    auto frags = [&](const uint16_t* buf, int grp, int nt, bf16x8 b[8]) {
      const uint16_t* base = buf + (64 * grp + 32 * nt) * kIdxDim;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(base + frag_off[j]));
    };
    int pa[kGemmLoads] = {}, pv[kGemmLoads] = {};  // pages of tiles tile + 1 and tile + 2 (PAGED)
    if (PAGED) pid_fetch(0, pv);
    dma(0, pv, ks0);
    if (PAGED && ntiles > 1) {
      pid_fetch(1, pv);
#pragma unroll
      for (int c = 0; c < kGemmLoads; ++c) pa[c] = page_ready(pv[c]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct loads are in LDS
    __syncthreads();
    bf16x8 fa[8], fb[8];  // fragments of key blocks 0 and 1 of the current group
    f32x16 pend = {};          // accumulator of (query 1, block 1) of the previous group
    float pend_p = 0.f;        // fold of (query 1, block 0) of the previous group
    int pend_k = split_keys;   // their first key (split_keys: none, the stores are dropped)
    // tile in cur, tile + 1 loaded into nxt meanwhile
    auto tile_body = [&](const uint16_t* cur, uint16_t* nxt, int tile) {
      if (tile + 1 < ntiles) dma(tile + 1, pa, nxt);
      if (PAGED && tile + 2 < ntiles) pid_fetch(tile + 2, pv);
      frags(cur, 0, 0, fa);
      frags(cur, 0, 1, fb);
#pragma unroll
      for (int grp = 0; grp < kGemmGroups; ++grp) {
        const int kb = tile * kGemmKT + 64 * grp;
        // each fold follows the issue of the next chain, which runs meanwhile
        const f32x16 a0 = chain(0, fa);
        store_pair(1, pend_p, reduce(1, pend), pend_k);
        const f32x16 a1 = chain(1, fa);
        if (grp + 1 < kGemmGroups) frags(cur, grp + 1, 0, fa);
        const float p0 = reduce(0, a0);
        const f32x16 a2 = chain(0, fb);
        const float p1 = reduce(1, a1);
        const f32x16 a3 = chain(1, fb);
        if (grp + 1 < kGemmGroups) frags(cur, grp + 1, 1, fb);
        store_pair(0, p0, reduce(0, a2), kb);
        pend = a3;
        pend_p = p1;
        pend_k = kb;
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile + 1 are in LDS
      if (PAGED && tile + 2 < ntiles) {
#pragma unroll
        for (int c = 0; c < kGemmLoads; ++c) pa[c] = page_ready(pv[c]);
      }
      __syncthreads();                      // ... and every wave's; every wave is done with cur
    };
    for (int tile = 0; tile < ntiles; tile += 2) {
      tile_body(ks0, ks1, tile);
      if (tile + 1 < ntiles) tile_body(ks1, ks0, tile + 1);
    }
    store_pair(1, pend_p, reduce(1, pend), pend_k);
  }
  if constexpr (MODE == kGemmCandidates) {
#pragma unroll
    for (int qi = 0; qi < kGemmQPW; ++qi) {
      const int tq = t0 + wave * kGemmQPW + qi;
      if (lane == 0 && tq < T) o.cnt[tq] = ncand[qi];
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_index_scores(const LaunchBatch& b, const uint16_t* q_idx, const uint16_t* w,
                               const uint16_t* k_idx, float* scores, int64_t ld, bool gemm,
                               void* topk_ws, hipStream_t st, const int32_t* row_mask) {
  if (gemm) {
    const int split_keys = gemm_split_keys(b.T, b.max_ctx);
    dim3 grid((b.T + kGemmQB - 1) / kGemmQB, (int)(((int64_t)b.max_ctx + split_keys - 1) / split_keys));
    GemmOut o{};
    o.scores = scores;
    o.ld = ld;
    if (b.paged())
      idx_gemm_kernel<true, kGemmScores><<<grid, kGemmThreads, 0, st>>>(b.q_seq, b.q_pos, b.rows, q_idx, w, k_idx,
                                                                        o, b.T, split_keys);
    else
      idx_gemm_kernel<false, kGemmScores><<<grid, kGemmThreads, 0, st>>>(b.q_seq, b.q_pos, b.rows, q_idx, w, k_idx,
                                                                         o, b.T, split_keys);
  } else {
    const SplitWs sw = split_ws(b.T, b.max_ctx);
    char* lists = static_cast<char*>(topk_ws);
    if (b.paged())
      idx_scan_kernel<true><<<dim3(b.T, sw.S), 256, 0, st>>>(b.q_seq, b.q_pos, b.rows, q_idx, w, k_idx,
                                                             scores, ld, sw.slice_keys, lists, sw, row_mask);
    else
      idx_scan_kernel<false><<<dim3(b.T, sw.S), 256, 0, st>>>(b.q_seq, b.q_pos, b.rows, q_idx, w, k_idx,
                                                              scores, ld, sw.slice_keys, lists, sw, row_mask);
  }
  return hipGetLastError();
}

bool gemm_whole_context(int T, int max_ctx) {
  // (query blocks alone fill the chip: one workgroup per block over the whole context)
  return (T + kGemmQB - 1) / kGemmQB >= kGemmMinWgs && gemm_split_keys(T, max_ctx) >= max_ctx;
}

hipError_t launch_index_sample(const LaunchBatch& b, const uint16_t* q_idx, const uint16_t* w,
                               const uint16_t* k_idx, float* sample, int64_t ld_s, int stride, hipStream_t st) {
  const int n_s = (b.max_ctx - 1) / stride + 1;  // samples of the longest row
  const int split_keys = gemm_split_keys(b.T, n_s);
  dim3 grid((b.T + kGemmQB - 1) / kGemmQB, (n_s + split_keys - 1) / split_keys);
  GemmOut o{};
  o.scores = sample;
  o.ld = ld_s;
  o.stride = stride;
  if (b.paged())
    idx_gemm_kernel<true, kGemmSample><<<grid, kGemmThreads, 0, st>>>(b.q_seq, b.q_pos, b.rows, q_idx, w, k_idx, o,
                                                                      b.T, split_keys);
  else
    idx_gemm_kernel<false, kGemmSample><<<grid, kGemmThreads, 0, st>>>(b.q_seq, b.q_pos, b.rows, q_idx, w, k_idx, o,
                                                                       b.T, split_keys);
  return hipGetLastError();
}

hipError_t launch_index_candidates(const LaunchBatch& b, const uint16_t* q_idx, const uint16_t* w,
                                   const uint16_t* k_idx, const float* theta, uint32_t* cand, int cap, int* cnt,
                                   hipStream_t st) {
  const int split_keys = gemm_split_keys(b.T, b.max_ctx);
  if (split_keys < b.max_ctx) return hipErrorInvalidValue;  // needs whole-context workgroups
  dim3 grid((b.T + kGemmQB - 1) / kGemmQB, 1);
  GemmOut o{};
  o.theta = theta;
  o.cand = cand;
  o.cap = cap;
  o.cnt = cnt;
  if (b.paged())
    idx_gemm_kernel<true, kGemmCandidates><<<grid, kGemmThreads, 0, st>>>(b.q_seq, b.q_pos, b.rows, q_idx, w,
                                                                           k_idx, o, b.T, split_keys);
  else
    idx_gemm_kernel<false, kGemmCandidates><<<grid, kGemmThreads, 0, st>>>(b.q_seq, b.q_pos, b.rows, q_idx, w,
                                                                            k_idx, o, b.T, split_keys);
  return hipGetLastError();
}

}  // namespace dsa
