// Top-k selector on gfx950.
//
// Keeps the k best of the n = q_pos+1 scores of each query under (fp32 value
// descending, position ascending) and writes them as ascending positions,
// -1 padded (page "2026大模型架构概览（二）：GLM 5 DSV3.2 的 DSA 与 MoE 配置拆解", §2.2: the
// selector keeps the index_topk highest-scoring history keys; page "（五）一万亿次点积砍到
// 两千次：DSA 怎么破 N²": index_topk = 2048).
//
// Radix select over the monotone uint32 image of the scores with digits
// [31:20] | [19:8] | [7:0]:
//   1. histogram of the top digit -> bin b1 holding the k-th largest and the
//      count above it;
//   2. a position-ordered compaction of the row gives list A (top digit > b1:
//      all kept) and the candidates of bin b1 as (key, position);
//   3. the two lower digits are resolved on the candidates, the kept ones are
//      compacted in position order (list C) and A and C are merged;
//   4. if bin b1 holds more candidates than fit in LDS (heavy ties), the lower
//      digits are resolved with further passes over the row and a final
//      ordered compaction writes the output.
// Every compaction is a prefix sum in position order, so equal scores resolve
// to the lower positions and the output needs no sort.
//
// Two launch shapes compute the same result:
//   * one 512-thread workgroup per row (many rows, e.g. a prefill chunk);
//   * for few rows (decode), steps 1 and 2 are split over slices of the row:
//     each slice's sparse top-digit list (written by the key scan itself, or by
//     a histogram pass); then per slice the row histogram and the slice's output
//     offsets from the lists, and the compaction into global A / candidate
//     lists; then one workgroup per row runs steps 3/4.
#include "absorb.h"
#include "dsa_common.h"
#include "dsa_kernels.h"
#include "topk_plan.h"

namespace dsa {

constexpr int kTkThreads = 512;  // for k <= kTopkSmall two row workgroups fit a CU (LDS ~74 KB each)
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kPerThread = 16;                   // scores per thread per pass step
constexpr int kStep = kPerThread * kTkThreads;   // scores per pass step

constexpr int kSliceThreads = 256;

// KMAX: the largest k a launch handles.  List A holds fewer than k positions,
// list C at most min(k, candidates) of them.  With KMAX = kTopkSmall two row
// workgroups fit a CU; larger k (up to kMaxTopk) runs one per CU.
template <int KMAX>
struct TkShared {
  static constexpr int kListC = KMAX < kCandCap ? KMAX : kCandCap;
  uint32_t hist[kTkBins];
  int wave_tot[kTkWaves];
  int sel_bin, sel_above;
  alignas(16) uint32_t cand_key[kCandCap];  // 16-aligned: also staging for the absorb workgroups
  int cand_pos[kCandCap];
  int list_a[KMAX];
  int list_c[kListC];
};

// Finds the bin holding the krem-th largest element (1-based, counting from
// the highest bin) and the number of elements in higher bins (NT threads,
// NBINS bins; thread i owns a block of bins counted from the top).
template <int NT, int NBINS>
__device__ void find_bin(const uint32_t* hist, int krem, int* wave_tot, int* sel_bin, int* sel_above) {
  constexpr int kBpt = NBINS >= NT ? NBINS / NT : 1;
  const int tid = threadIdx.x;
  const int top = NBINS - 1 - tid * kBpt;
  // The block's total is read in a lane-rotated order (step b reads bin
  // (b + lane / 4) % kBpt of the block), which spreads the lanes of a read over
  // the LDS banks (blocks of consecutive lanes are kBpt words apart); only
  // the thread whose block holds the krem-th element reads it in order.
  int local = 0;
#pragma unroll
  for (int b = 0; b < kBpt; ++b) {
    const int e = (b + ((tid & 63) >> 2)) % kBpt;
    local += top - e >= 0 ? (int)hist[top - e] : 0;
  }
  int total;
  const int above = block_excl_scan<NT / 64>(local, wave_tot, total);
  if (local > 0 && above < krem && krem <= above + local) {
    uint32_t c[kBpt];
#pragma unroll
    for (int b = 0; b < kBpt; ++b) c[b] = top - b >= 0 ? hist[top - b] : 0u;
    int acc = above;
#pragma unroll
    for (int b = 0; b < kBpt; ++b) {
      if (acc + (int)c[b] >= krem) {
        *sel_bin = top - b;
        *sel_above = acc;
        break;
      }
      acc += (int)c[b];
    }
  }
  lds_sync();
}
template <int NBINS, int KMAX>
__device__ __forceinline__ void find_bin(TkShared<KMAX>& sh, int krem) {
  find_bin<kTkThreads, NBINS>(sh.hist, krem, sh.wave_tot, &sh.sel_bin, &sh.sel_above);
}

// kPerThread consecutive scores starting at i (i is a multiple of 4).
__device__ __forceinline__ void load_run(const float* row, int i, int n, uint32_t key[kPerThread],
                                         bool ok[kPerThread]) {
#pragma unroll
  for (int q = 0; q < kPerThread / 4; ++q) {
    const int b = i + 4 * q;
    if (b + 3 < n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + b);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[4 * q + e] = score_key(v[e]);
        ok[4 * q + e] = true;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ok[4 * q + e] = b + e < n;
        key[4 * q + e] = ok[4 * q + e] ? score_key(row[b + e]) : 0u;
      }
    }
  }
}

// Writes the union of two ascending, disjoint position lists (in LDS) to out
// in ascending order.  Thread i produces the contiguous output run
// [i * per, i * per + per): a binary search along the merge path finds how many
// entries of la precede the run's start, then the run is merged sequentially.
__device__ __forceinline__ void merge_lists(const int* la, int na, const int* lc, int nc, int32_t* out) {
  const int total = na + nc;
  const int per = (total + blockDim.x - 1) / blockDim.x;
  const int d = min((int)threadIdx.x * per, total), dend = min(d + per, total);
  int lo = max(0, d - nc), hi = min(d, na);
  while (lo < hi) {  // first i with la[i] > lc[d - 1 - i]: i entries of la precede output d
    const int mid = (lo + hi) >> 1;
    if (la[mid] < lc[d - 1 - mid]) lo = mid + 1; else hi = mid;
  }
  int i = lo, j = d - lo;
  int a = i < na ? la[i] : INT_MAX, c = j < nc ? lc[j] : INT_MAX;
  for (int o = d; o < dend; ++o) {
    if (a < c) {
      out[o] = a;
      ++i;
      a = i < na ? la[i] : INT_MAX;
    } else {
      out[o] = c;
      ++j;
      c = j < nc ? lc[j] : INT_MAX;
    }
  }
}

// Step 3: sh.cand_* holds c1 candidates in position order and sh.list_a the
// above1 positions above every candidate (ascending); krem = k - above1 of the
// candidates are kept.  With `window`, the candidates span several top-digit
// bins and the threshold bin among them is found first; otherwise all of them
// are in bin b1.
template <int KMAX>
__device__ void finish_from_candidates(TkShared<KMAX>& sh, uint32_t b1, int above1, int c1, int krem,
                                       int32_t* out, bool window = false) {
  const int tid = threadIdx.x;
  int krem1 = krem;
  if (window) {
    for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < c1; j += kTkThreads) atomicAdd(&sh.hist[sh.cand_key[j] >> 20], 1u);
    __syncthreads();
    find_bin<kTkBins>(sh, krem);
    b1 = (uint32_t)sh.sel_bin;
    krem1 = krem - sh.sel_above;
    __syncthreads();
  }
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int j = tid; j < c1; j += kTkThreads) {
    const uint32_t key = sh.cand_key[j];
    if ((key >> 20) == b1) atomicAdd(&sh.hist[(key >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  find_bin<kTkBins>(sh, krem1);
  const uint32_t b2 = (uint32_t)sh.sel_bin;
  const int krem2 = krem1 - sh.sel_above;
  __syncthreads();
  for (int i = tid; i < 256; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  const uint32_t pre12 = (b1 << 12) | b2;
  for (int j = tid; j < c1; j += kTkThreads) {
    const uint32_t key = sh.cand_key[j];
    if ((key >> 8) == pre12) atomicAdd(&sh.hist[key & 0xFFu], 1u);
  }
  __syncthreads();
  find_bin<256>(sh, krem2);
  const uint32_t b3 = (uint32_t)sh.sel_bin;
  const int r = krem2 - sh.sel_above;  // ties at the threshold key to keep (lowest positions)
  const uint32_t kstar = (b1 << 20) | (b2 << 8) | b3;
  // ordered compaction: thread tid takes candidates [kCE tid, kCE tid + kCE)
  // of a round of kCE * kTkThreads (one round holds all of kCandCap)
  constexpr int kCE = (kCandCap + kTkThreads - 1) / kTkThreads;
  int nG = 0, nE = 0;
  for (int base = 0; base < c1; base += kCE * kTkThreads) {
    const int j0 = base + kCE * tid;
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int e = 0; e < kCE; ++e) {
      if (j0 + e < c1) {
        const uint32_t key = sh.cand_key[j0 + e];
        gtm |= (key > kstar ? 1u : 0u) << e;
        eqm |= (key == kstar ? 1u : 0u) << e;
      }
    }
    int tot;
    const int ex = block_excl_scan<kTkWaves>((__builtin_popcount(gtm) << 16) | __builtin_popcount(eqm),
                                             sh.wave_tot, tot);
    int eg = nG + (ex >> 16), ee = nE + (ex & 0xFFFF);
#pragma unroll
    for (int e = 0; e < kCE; ++e) {
      if ((gtm >> e) & 1u) {
        sh.list_c[eg + min(ee, r)] = sh.cand_pos[j0 + e];
        ++eg;
      } else if ((eqm >> e) & 1u) {
        if (ee < r) sh.list_c[eg + ee] = sh.cand_pos[j0 + e];
        ++ee;
      }
    }
    nG += tot >> 16;
    nE += tot & 0xFFFF;
  }
  __syncthreads();
  merge_lists(sh.list_a, above1, sh.list_c, krem, out);
}

// Step 3 for a threshold bin whose c1 candidates (key, position pairs in
// position order) exceed the LDS capacity but sit in global memory (the split
// workspace): the same digit passes and ordered compaction, reading the
// candidates from global memory, 16 consecutive per thread per round.  List A
// is in sh.list_a; list C (krem <= KMAX entries) goes to the LDS of the unused
// candidate arrays.
template <int KMAX>
__device__ void finish_from_global_candidates(TkShared<KMAX>& sh, const uint32_t* __restrict__ cand,
                                              uint32_t b1, int above1, int c1, int krem, int32_t* out) {
  static_assert(KMAX <= 2 * kCandCap, "list C fits the candidate arrays");
  const int tid = threadIdx.x;
  int* list_c = reinterpret_cast<int*>(sh.cand_key);  // cand_key and cand_pos are contiguous
  constexpr int kPairs = kPerThread / 2;              // 16-byte loads (two candidates) per thread
  auto load = [&](int base, u32x4 v[kPairs]) {
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const int j = base + kPerThread * tid + 2 * u;
      v[u] = j < c1 ? *reinterpret_cast<const u32x4*>(cand + 2 * j) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // digit 2 (every candidate has top digit b1)
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int base = 0; base < c1; base += kStep) {
    u32x4 v[kPairs];
    load(base, v);
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const int j = base + kPerThread * tid + 2 * u;
      if (j < c1) atomicAdd(&sh.hist[(v[u].x >> 8) & 0xFFFu], 1u);
      if (j + 1 < c1) atomicAdd(&sh.hist[(v[u].z >> 8) & 0xFFFu], 1u);
    }
  }
  __syncthreads();
  find_bin<kTkBins>(sh, krem);
  const uint32_t b2 = (uint32_t)sh.sel_bin;
  const int krem2 = krem - sh.sel_above;
  __syncthreads();
  // digit 3
  for (int i = tid; i < 256; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  const uint32_t pre12 = (b1 << 12) | b2;
  for (int base = 0; base < c1; base += kStep) {
    u32x4 v[kPairs];
    load(base, v);
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const int j = base + kPerThread * tid + 2 * u;
      if (j < c1 && (v[u].x >> 8) == pre12) atomicAdd(&sh.hist[v[u].x & 0xFFu], 1u);
      if (j + 1 < c1 && (v[u].z >> 8) == pre12) atomicAdd(&sh.hist[v[u].z & 0xFFu], 1u);
    }
  }
  __syncthreads();
  find_bin<256>(sh, krem2);
  const int r = krem2 - sh.sel_above;  // ties at the threshold key to keep (lowest positions)
  const uint32_t kstar = (pre12 << 8) | (uint32_t)sh.sel_bin;
  // ordered compaction of the kept candidates into list C
  int nG = 0, nE = 0;
  for (int base = 0; base < c1; base += kStep) {
    u32x4 v[kPairs];
    load(base, v);
    const int j0 = base + kPerThread * tid;
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const uint32_t key = (e & 1) ? v[e >> 1].z : v[e >> 1].x;
      const bool ok = j0 + e < c1;
      gt += ok && key > kstar;
      eq += ok && key == kstar;
    }
    int tot;
    const int ex = block_excl_scan<kTkWaves>((gt << 16) | eq, sh.wave_tot, tot);  // <= kStep each
    int eg = nG + (ex >> 16), ee = nE + (ex & 0xFFFF);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (j0 + e >= c1) continue;
      const uint32_t key = (e & 1) ? v[e >> 1].z : v[e >> 1].x;
      const int pos = (int)((e & 1) ? v[e >> 1].w : v[e >> 1].y);
      if (key > kstar) {
        list_c[eg + min(ee, r)] = pos;
        ++eg;
      } else if (key == kstar) {
        if (ee < r) list_c[eg + ee] = pos;
        ++ee;
      }
    }
    nG += tot >> 16;
    nE += tot & 0xFFFF;
  }
  __syncthreads();
  merge_lists(sh.list_a, above1, list_c, krem, out);
}

// Step 4 (heavy ties): lower digits by passes over the row, then an ordered
// compaction straight to the output.
template <int KMAX>
__device__ void finish_from_row(TkShared<KMAX>& sh, const float* row, int n, uint32_t b1, int krem,
                                int32_t* out) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kStep) {
    uint32_t key[kPerThread];
    bool ok[kPerThread];
    load_run(row, base + kPerThread * tid, n, key, ok);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (ok[e] && (key[e] >> 20) == b1) atomicAdd(&sh.hist[(key[e] >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  find_bin<kTkBins>(sh, krem);
  const uint32_t b2 = (uint32_t)sh.sel_bin;
  const int krem2 = krem - sh.sel_above;
  __syncthreads();
  for (int i = tid; i < 256; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  const uint32_t pre = (b1 << 12) | b2;
  for (int base = 0; base < n; base += kStep) {
    uint32_t key[kPerThread];
    bool ok[kPerThread];
    load_run(row, base + kPerThread * tid, n, key, ok);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (ok[e] && (key[e] >> 8) == pre) atomicAdd(&sh.hist[key[e] & 0xFFu], 1u);
  }
  __syncthreads();
  find_bin<256>(sh, krem2);
  const int r = krem2 - sh.sel_above;
  const uint32_t kstar = (pre << 8) | (uint32_t)sh.sel_bin;
  int nG = 0, nE = 0;
  for (int base = 0; base < n; base += kStep) {
    const int i = base + kPerThread * tid;
    uint32_t key[kPerThread];
    bool ok[kPerThread];
    load_run(row, i, n, key, ok);
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      gt += ok[e] && key[e] > kstar;
      eq += ok[e] && key[e] == kstar;
    }
    int tot;
    const int ex = block_excl_scan<kTkWaves>((gt << 16) | eq, sh.wave_tot, tot);
    int eg = nG + (ex >> 16), ee = nE + (ex & 0xFFFF);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (!ok[e]) continue;
      if (key[e] > kstar) {
        out[eg + min(ee, r)] = i + e;
        ++eg;
      } else if (key[e] == kstar) {
        if (ee < r) out[eg + ee] = i + e;
        ++ee;
      }
    }
    nG += tot >> 16;
    nE += tot & 0xFFFF;
  }
}

// ---------------------------------------------------------------- sampled window
// Long rows: the top-digit histogram of a 1/16 sample of the row (every 16th
// block of 64 scores) locates the bin of the k-th largest score; one exact
// ordered pass then keeps everything above a window of one to three bins
// around it (list A) and collects the window's scores as candidates.  The pass checks
// that the k-th largest lies inside the window (A holds fewer than k, A plus
// the window at least k, the candidates fit); then the candidates are
// resolved as usual and the result is the same as the full histogram path's.
// Returns false (and the caller runs the full path) when the check fails.
constexpr int kSampleMinRow = 65536;
constexpr int kSampleBlock = 64;    // scores per sampled block
constexpr int kSampleStride = 16;   // one block in 16 is sampled

template <int KMAX>
__device__ bool window_select(TkShared<KMAX>& sh, const float* row, int64_t ld, int n, int k, int32_t* out) {
  const int tid = threadIdx.x;
  // Loads of 4 scores start at multiples of 4; those at or past the row's
  // stride ld (a multiple of 4, >= n) re-read its last 4, so every load is in
  // bounds and unconditional, and scores at or past n are masked where used.
  const int64_t last4 = ld - 4;
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  // ---- sample: 16 threads x 4 scores per sampled block, 64 blocks per step;
  // four steps' loads are issued before any is counted.  `act(key)` sees
  // every sampled score of the row, in the same order on every pass.
  auto sample_pass = [&](auto&& act) {
    constexpr int kBlocksPerStep = kTkThreads / (kSampleBlock / 4);
    constexpr int kU = 4;
    for (int m0 = 0; (int64_t)m0 * kSampleStride * kSampleBlock < n; m0 += kU * kBlocksPerStep) {
      f32x4 v[kU];
      int ii[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int m = m0 + u * kBlocksPerStep + tid / (kSampleBlock / 4);
        const int64_t i64 = (int64_t)m * kSampleStride * kSampleBlock + 4 * (tid % (kSampleBlock / 4));
        ii[u] = i64 < n ? (int)i64 : n;
        v[u] = *reinterpret_cast<const f32x4*>(row + min(i64, last4));
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ii[u] + e < n) act(score_key(v[u][e]));
    }
  };
  int ns = 0;
  sample_pass([&](uint32_t key) {
    atomicAdd(&sh.hist[key >> 20], 1u);
    ++ns;
  });
  int ns_tot;
  (void)block_excl_scan<kTkWaves>(ns, sh.wave_tot, ns_tot);
  // The k-th largest score of the row sits near rank ks of the ns_tot
  // sampled scores (counted from the top); that rank varies by about
  // sqrt(ks) between samples, so the window spans sample ranks ks -+ m with
  // m ~ 3 deviations: its top edge lies above the k-th score and its bottom
  // edge below it, except in rare rows (which take the full path).
  const int ks = max(1, (int)((int64_t)k * ns_tot / n));
  const int m = (int)(3.f * sqrtf((float)ks)) + 2;
  const int r_hi = max(ks - m, 1), r_lo = min(ks + m, ns_tot);
  find_bin<kTkBins>(sh, r_hi);
  const int bh = sh.sel_bin, ah = sh.sel_above;  // bin of rank r_hi, samples in higher bins
  find_bin<kTkBins>(sh, r_lo);
  const int bl = sh.sel_bin;                      // bin of rank r_lo
  // Window edges as 32-bit keys [key_lo, key_hi): whole top-digit bins, or,
  // when the window spans at most kSubBins / 256 bins, edges of sub-bins that
  // add the next 8 key bits (a second pass over the same sample counts the
  // sampled scores of those bins by sub-bin).
  constexpr int kSubBins = 1024;
  uint64_t key_hi = (uint64_t)(bh + 1) << 20;
  uint32_t key_lo = (uint32_t)bl << 20;
  if (bh - bl < kSubBins / 256) {
    const int btop = min(bl + kSubBins / 256 - 1, kTkBins - 1);  // top bin of the sub-bin range
    int a0 = ah;  // samples above the sub-bin range: above bh, less the bins bh+1..btop
    for (int bb = bh + 1; bb <= btop; ++bb) a0 -= (int)sh.hist[bb];
    __syncthreads();
    for (int i = tid; i < kSubBins; i += kTkThreads) sh.hist[i] = 0;
    __syncthreads();
    sample_pass([&](uint32_t key) {
      const int bin = (int)(key >> 20);
      if (bin >= bl && bin <= btop) atomicAdd(&sh.hist[((bin - bl) << 8) | ((key >> 12) & 0xFFu)], 1u);
    });
    __syncthreads();
    find_bin<kSubBins>(sh, r_hi - a0);
    const int sub_hi = sh.sel_bin;
    find_bin<kSubBins>(sh, r_lo - a0);
    const int sub_lo = sh.sel_bin;
    key_hi = ((uint64_t)((uint32_t)bl << 8) + (uint32_t)sub_hi + 1u) << 12;
    key_lo = (((uint32_t)bl << 8) + (uint32_t)sub_lo) << 12;
  }
  // ---- exact ordered pass: above the window -> A, inside -> candidates;
  // the scores of the next two steps are in flight while a step is compacted.
  // The window's edges become float thresholds, so a score is classified
  // by two compares into per-thread bit masks; keys are formed only for the
  // few scores that are kept.  Masks drop the scores past the row.
  const float thr_hi = key_hi >= (1ull << 32) ? __uint_as_float(0x7FC00000u) : key_floor((uint32_t)key_hi);
  const float thr_lo = key_floor(key_lo);
  int nA = 0, nC = 0;
  auto fetch = [&](int i, f32x4 nx[kPerThread / 4]) {
#pragma unroll
    for (int q = 0; q < kPerThread / 4; ++q) nx[q] = *reinterpret_cast<const f32x4*>(row + min((int64_t)i + 4 * q, last4));
  };
  static_assert(kPerThread <= 31, "valid-score mask");
  auto step = [&](int base, f32x4 nx[kPerThread / 4]) {
    const int i = base + kPerThread * tid;
    float f[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread / 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) f[4 * q + e] = nx[q][e];
    if (base + 2 * kStep < n) fetch(i + 2 * kStep, nx);
    uint32_t mA = 0, mW = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      mA |= (f[e] >= thr_hi ? 1u : 0u) << e;
      mW |= (f[e] >= thr_lo ? 1u : 0u) << e;
    }
    const int rem = n - i;  // scores of this thread inside the row
    const uint32_t valid = rem >= kPerThread ? (1u << kPerThread) - 1u : (rem > 0 ? (1u << rem) - 1u : 0u);
    mA &= valid;
    mW &= valid;
    const uint32_t mC = mW & ~mA;
    int tot;
    const int ex = block_excl_scan<kTkWaves>((__builtin_popcount(mA) << 16) | __builtin_popcount(mC),
                                             sh.wave_tot, tot);  // <= kStep each
    int oa = nA + (ex >> 16), oc = nC + (ex & 0xFFFF);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (!((mW >> e) & 1u)) continue;
      if ((mA >> e) & 1u) {
        if (oa < KMAX) sh.list_a[oa] = i + e;
        ++oa;
      } else {
        if (oc < kCandCap) {
          sh.cand_key[oc] = score_key(f[e]);
          sh.cand_pos[oc] = i + e;
        }
        ++oc;
      }
    }
    nA += tot >> 16;
    nC += tot & 0xFFFF;
  };
  f32x4 nxa[kPerThread / 4], nxb[kPerThread / 4];
  fetch(kPerThread * tid, nxa);
  if (kStep < n) fetch(kStep + kPerThread * tid, nxb);
  for (int base = 0; base < n; base += 2 * kStep) {
    step(base, nxa);
    if (base + kStep < n) step(base + kStep, nxb);
  }
  __syncthreads();
  if (!(nA < k && nA + nC >= k && nC <= kCandCap)) return false;  // uniform: every thread has the totals
  finish_from_candidates(sh, 0u, nA, nC, k - nA, out, true);
  return true;
}

// ---------------------------------------------------------------- one workgroup per row
template <int KMAX>
__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(const int32_t* __restrict__ q_pos,
                                                              const float* __restrict__ scores,
                                                              int64_t ld, int k,
                                                              int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ row_mask) {
  __shared__ TkShared<KMAX> sh;
  const int t = blockIdx.x, tid = threadIdx.x;
  if (row_mask != nullptr && row_mask[t] == 0) return;  // only the rows a mask names
  const int n = q_pos[t] + 1;
  int32_t* out = idx + (int64_t)t * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + (int64_t)t * ld;
  if (n >= kSampleMinRow && window_select(sh, row, ld, n, k, out)) return;
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kStep) {
    uint32_t key[kPerThread];
    bool ok[kPerThread];
    load_run(row, base + kPerThread * tid, n, key, ok);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (ok[e]) atomicAdd(&sh.hist[key[e] >> 20], 1u);
  }
  __syncthreads();
  find_bin<kTkBins>(sh, k);
  const uint32_t b1 = (uint32_t)sh.sel_bin;
  const int above1 = sh.sel_above;
  const int c1 = (int)sh.hist[b1];
  const int krem = k - above1;
  __syncthreads();
  if (c1 > kCandCap) {
    finish_from_row(sh, row, n, b1, krem, out);
    return;
  }
  int nA = 0, nC = 0;
  for (int base = 0; base < n; base += kStep) {
    const int i = base + kPerThread * tid;
    uint32_t key[kPerThread];
    bool ok[kPerThread];
    load_run(row, i, n, key, ok);
    int ca = 0, cc = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const uint32_t d = key[e] >> 20;
      ca += ok[e] && d > b1;
      cc += ok[e] && d == b1;
    }
    int tot;
    const int ex = block_excl_scan<kTkWaves>((ca << 16) | cc, sh.wave_tot, tot);
    int oa = nA + (ex >> 16), oc = nC + (ex & 0xFFFF);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (!ok[e]) continue;
      const uint32_t d = key[e] >> 20;
      if (d > b1) {
        sh.list_a[oa++] = i + e;
      } else if (d == b1) {
        sh.cand_key[oc] = key[e];
        sh.cand_pos[oc] = i + e;
        ++oc;
      }
    }
    nA += tot >> 16;
    nC += tot & 0xFFFF;
  }
  __syncthreads();
  finish_from_candidates(sh, b1, above1, c1, krem, out);
}

// ---------------------------------------------------------------- split path
// Workspace per query (SplitWs): the slice bin lists, a header {b1, above1,
// c1}, list A [kMaxTopk] and candidates (key, position) [kCandCapWs][2].

// Kernel 1 (grid T x S), only where the key scan did not write the lists:
// the sparse top-digit list of one slice of stored scores.
__global__ __launch_bounds__(kSliceThreads) void topk_slice_hist_kernel(
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int64_t ld, int k,
    char* __restrict__ ws, SplitWs w) {
  __shared__ uint32_t hist[kTkBins / 2];
  __shared__ int wave_tot[kSliceThreads / 64];
  const int t = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int n = q_pos[t] + 1;
  const int s0 = s * w.slice_keys;
  if (n <= k || s0 >= n) return;
  const float* row = scores + (int64_t)t * ld;
  for (int i = tid; i < kTkBins / 2; i += kSliceThreads) hist[i] = 0u;
  __syncthreads();
  const int end = min(n, s0 + w.slice_keys);
  for (int b = s0 + 4 * tid; b < end; b += 4 * kSliceThreads) {
    if (b + 3 < end) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + b);
#pragma unroll
      for (int e = 0; e < 4; ++e) hist16_add(hist, score_key(v[e]));
    } else {
      for (int e = 0; b + e < end; ++e) hist16_add(hist, score_key(row[b + e]));
    }
  }
  __syncthreads();
  write_bin_list<kSliceThreads>(
      hist, reinterpret_cast<uint32_t*>(ws + (size_t)t * w.per_query + w.list_off + (size_t)s * w.list_stride),
      wave_tot);
}

// Kernel 2 (grid T x S): every workgroup merges the row's slice lists into the
// row histogram (finds b1) and into the histogram of the earlier slices (its
// own output offsets), then compacts its slice into list A and the candidate
// list in position order.
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelKeys = 16;                       // consecutive scores per thread per step
constexpr int kSelStep = kSelKeys * kSelThreads;   // 4096 scores per step
constexpr int kSelBinsPT = kTkBins / kSelThreads;  // 16 bins per thread
constexpr int kListBatch = 16;                     // lists in flight per wave (64 per workgroup)

struct SelShared {
  uint32_t all[kTkBins];  // row histogram of the top digit
  uint32_t pre[kTkBins];  // the same over the slices before this one
  int wave_tot[kSelWaves];
  int wave_tot2[kSelWaves];
  int b1, above1, c1, offA, offC;
};

__global__ __launch_bounds__(kSelThreads) void topk_slice_select_kernel(
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int64_t ld, int k,
    char* __restrict__ ws, SplitWs w) {
  __shared__ SelShared sh;
  const int t = blockIdx.x, s = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  char* base = ws + (size_t)t * w.per_query;
  const char* lists = base + w.list_off;
  const float* row = scores + (int64_t)t * ld;
  const int s0 = s * w.slice_keys;
  // Loads that do not depend on the row length go out first.  Lists: wave v
  // reads lists v, v+4, ..., one 4-byte word per lane (word 0 = count); lists
  // past the row's end are stale and skipped below.  Scores: the first
  // kSelStep of the slice, 16 consecutive per thread (the slice starts inside
  // the row, and reads stop at ld).
  uint32_t word[kListBatch];
#pragma unroll
  for (int u = 0; u < kListBatch; ++u) {
    const int j = wave + kSelWaves * u;
    word[u] = j < w.S ? reinterpret_cast<const uint32_t*>(lists + (size_t)j * w.list_stride)[lane] : 0u;
  }
  // 16 scores from i0 on; groups of 4 past the row's stride (a multiple of 4)
  // re-read its last group: every load is in bounds and unconditional, and
  // scores at or past the slice's end are masked where they are used.
  const int64_t last4 = ld - 4;
  auto load16 = [&](int i0, float v[kSelKeys]) {
#pragma unroll
    for (int q = 0; q < kSelKeys / 4; ++q) {
      const int64_t b = min((int64_t)i0 + 4 * q, last4);
      const f32x4 x = *reinterpret_cast<const f32x4*>(row + b);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
    }
  };
  float v0[kSelKeys];
  load16(s0 + kSelKeys * tid, v0);
  const int n = q_pos[t] + 1;
  if (n <= k) return;
  const int S = (n + w.slice_keys - 1) / w.slice_keys;  // slices holding keys (<= kMaxSlices)
  if (s >= S) return;
  for (int i = tid; i < kTkBins / 4; i += kSelThreads) {
    reinterpret_cast<u32x4*>(sh.all)[i] = u32x4{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(sh.pre)[i] = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  // ---- merge the lists: row histogram, and histogram of the slices before s
  for (int j0 = 0; j0 < S; j0 += kSelWaves * kListBatch) {
    if (j0 > 0) {
#pragma unroll
      for (int u = 0; u < kListBatch; ++u) {
        const int j = j0 + wave + kSelWaves * u;
        word[u] = j < S ? reinterpret_cast<const uint32_t*>(lists + (size_t)j * w.list_stride)[lane] : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      const int j = j0 + wave + kSelWaves * u;
      if (j >= S) continue;  // wave-uniform
      const uint32_t* lst = reinterpret_cast<const uint32_t*>(lists + (size_t)j * w.list_stride);
      const int cnt = __builtin_amdgcn_readfirstlane(word[u]);  // lane 0 read word 0: the count
      for (int e0 = 0; e0 <= cnt; e0 += 64) {  // words e0 .. e0+63 (entries are words 1..cnt)
        const uint32_t ent = e0 == 0 ? word[u] : (e0 + lane <= cnt ? lst[e0 + lane] : 0u);
        const int widx = e0 + lane;
        if (widx >= 1 && widx <= cnt) {
          atomicAdd(&sh.all[ent >> 16], ent & 0xFFFFu);
          if (j < s) atomicAdd(&sh.pre[ent >> 16], ent & 0xFFFFu);
        }
      }
    }
  }
  __syncthreads();
  // ---- b1 and this slice's offsets from one scan over (row, earlier-slice)
  // counts in descending bin order; thread i owns bins 4095-16i-15 .. 4095-16i
  {
    const int lo_bin = kTkBins - kSelBinsPT * (tid + 1);
    // The thread's totals come from 16-byte reads in a lane-rotated order
    // (step q reads quarter (q + lane / 2) % 4 of the thread's bins), which
    // spreads a read over the LDS banks (consecutive lanes' bins are 64 bytes
    // apart); only the thread that holds the threshold bin reads them in order.
    uint32_t mine_all = 0, mine_pre = 0;
#pragma unroll
    for (int q = 0; q < kSelBinsPT / 4; ++q) {
      const int qq = (q + (lane >> 1)) & (kSelBinsPT / 4 - 1);
      const u32x4 a4 = reinterpret_cast<const u32x4*>(sh.all + lo_bin)[qq];
      const u32x4 p4 = reinterpret_cast<const u32x4*>(sh.pre + lo_bin)[qq];
      mine_all += a4[0] + a4[1] + a4[2] + a4[3];
      mine_pre += p4[0] + p4[1] + p4[2] + p4[3];
    }
    // both counts stay below 2^21, so the two scans are plain 32-bit scans
    const int inc_all = wave_inclusive_scan((int)mine_all), inc_pre = wave_inclusive_scan((int)mine_pre);
    if (lane == 63) {
      sh.wave_tot[wave] = inc_all;
      sh.wave_tot2[wave] = inc_pre;
    }
    __syncthreads();
    uint32_t above = (uint32_t)inc_all - mine_all, pre_above = (uint32_t)inc_pre - mine_pre;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
      above += i < wave ? (uint32_t)sh.wave_tot[i] : 0u;
      pre_above += i < wave ? (uint32_t)sh.wave_tot2[i] : 0u;
    }
    if (above < (uint32_t)k && (uint32_t)k <= above + mine_all) {
      uint32_t ca[kSelBinsPT], cp[kSelBinsPT];
#pragma unroll
      for (int e = 0; e < kSelBinsPT; ++e) {
        ca[e] = sh.all[lo_bin + e];
        cp[e] = sh.pre[lo_bin + e];
      }
#pragma unroll
      for (int e = kSelBinsPT - 1; e >= 0; --e) {
        if (above + ca[e] >= (uint32_t)k) {
          sh.b1 = lo_bin + e;
          sh.above1 = (int)above;
          sh.c1 = (int)ca[e];
          sh.offA = (int)pre_above;
          sh.offC = (int)cp[e];
          break;
        }
        above += ca[e];
        pre_above += cp[e];
      }
    }
    __syncthreads();
  }
  const uint32_t b1 = (uint32_t)sh.b1;
  const int above1 = sh.above1, c1 = sh.c1;
  if (s == 0 && tid == 0) {
    int* hdr = reinterpret_cast<int*>(base + w.hdr_off);
    hdr[0] = (int)b1;
    hdr[1] = above1;
    hdr[2] = c1;
  }
  if (c1 > kCandCapWs) return;  // heavy ties: the row's finish re-reads the row
  int offA = sh.offA, offC = sh.offC;
  // ---- ordered compaction of the slice, 16 consecutive scores per thread per step
  const float thr_hi = b1 + 1 >= (uint32_t)kTkBins ? __uint_as_float(0x7FC00000u) : key_floor((b1 + 1) << 20);
  const float thr_lo = key_floor(b1 << 20);
  int* list_a = reinterpret_cast<int*>(base + w.a_off);
  uint32_t* cand = reinterpret_cast<uint32_t*>(base + w.c_off);
  const int end = min(n, s0 + w.slice_keys);
  for (int c0 = s0; c0 < end; c0 += kSelStep) {
    const int i0 = c0 + kSelKeys * tid;
    float v[kSelKeys];
    if (c0 == s0) {
#pragma unroll
      for (int e = 0; e < kSelKeys; ++e) v[e] = v0[e];
    } else {
      load16(i0, v);
    }
    // classify against the float edges of bin b1 (bit masks), keys only for
    // the kept scores
    uint32_t mA = 0, mW = 0;
#pragma unroll
    for (int e = 0; e < kSelKeys; ++e) {
      const bool ok = i0 + e < end;
      mA |= (ok && v[e] >= thr_hi ? 1u : 0u) << e;
      mW |= (ok && v[e] >= thr_lo ? 1u : 0u) << e;
    }
    int tot;
    const int exs = block_excl_scan<kSelWaves>((__builtin_popcount(mA) << 16) | __builtin_popcount(mW & ~mA),
                                               sh.wave_tot, tot);  // < 4096 each
    int oa = offA + (exs >> 16), oc = offC + (exs & 0xFFFF);
#pragma unroll
    for (int e = 0; e < kSelKeys; ++e) {
      if (!((mW >> e) & 1u)) continue;
      if ((mA >> e) & 1u) {
        list_a[oa++] = i0 + e;
      } else {
        *reinterpret_cast<u32x2*>(cand + 2 * oc) = u32x2{score_key(v[e]), (uint32_t)(i0 + e)};
        ++oc;
      }
    }
    offA += tot >> 16;
    offC += tot & 0xFFFF;
  }
}

// Kernel 3 (grid T, plus 128 workgroups when an absorb job rides along): load
// list A and the candidates, resolve the lower digits, merge into the output.
// Workgroups T + 2h and T + 2h + 1, if launched, compute q_lat of head h for
// every query (each wave one block of 32 latent columns) on CUs the T row
// workgroups leave idle.
template <int KMAX>
__global__ __launch_bounds__(kTkThreads) void topk_finish_kernel(const int32_t* __restrict__ q_pos,
                                                                 const float* __restrict__ scores,
                                                                 int64_t ld, int k,
                                                                 int32_t* __restrict__ idx,
                                                                 const char* __restrict__ ws,
                                                                 SplitWs w, int T, AbsorbJob ab) {
  __shared__ TkShared<KMAX> sh;
  const int t = blockIdx.x, tid = threadIdx.x;
  if (t >= T) {  // the top-k LDS of this workgroup is free: per-wave staging for the absorption
    static_assert(kTkWaves * kAbsorbStage * sizeof(uint16_t) <= sizeof(sh.cand_key), "absorb staging");
    uint16_t* stage = reinterpret_cast<uint16_t*>(sh.cand_key) + (tid >> 6) * kAbsorbStage;
    // workgroup T + 2h + i: latent columns 256i .. 256i+255 of head h, one
    // block of 32 per wave
    const int j = t - T;
    absorb_wave(ab.q_nope, ab.w_uk, ab.q_lat, T, j >> 1, (j & 1) * (kLat / 2) + (tid >> 6) * 32, 0, (T + 31) / 32,
                stage);
    return;
  }
  const char* base = ws + (size_t)t * w.per_query;
  const int* list_a = reinterpret_cast<const int*>(base + w.a_off);
  const uint32_t* cand = reinterpret_cast<const uint32_t*>(base + w.c_off);
  // List A (fewer than k <= KMAX entries) and the first kCandCap candidates
  // (all an LDS finish can hold) are read together with the header; entries
  // past the counts are stale and unused (the workspace holds kMaxTopk entries
  // of A and kCandCapWs candidates).
  constexpr int kSpecA = KMAX / kTkThreads;
  constexpr int kSpecC = (kCandCap + kTkThreads - 1) / kTkThreads;
  static_assert(kSpecC * kTkThreads <= kCandCapWs, "speculative candidate reads stay in the workspace");
  int a_spec[kSpecA];
  u32x2 c_spec[kSpecC];
#pragma unroll
  for (int u = 0; u < kSpecA; ++u) a_spec[u] = list_a[tid + u * kTkThreads];
#pragma unroll
  for (int u = 0; u < kSpecC; ++u)
    c_spec[u] = *reinterpret_cast<const u32x2*>(cand + 2 * (tid + u * kTkThreads));
  const int n = q_pos[t] + 1;
  int32_t* out = idx + (int64_t)t * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int* hdr = reinterpret_cast<const int*>(base + w.hdr_off);
  const uint32_t b1 = (uint32_t)hdr[0];
  const int above1 = hdr[1];
  const int c1 = hdr[2];
  const int krem = k - above1;
  if (c1 > kCandCapWs) {
    finish_from_row(sh, scores + (int64_t)t * ld, n, b1, krem, out);
    return;
  }
#pragma unroll
  for (int u = 0; u < kSpecA; ++u) {
    const int i = tid + u * kTkThreads;
    if (i < above1) sh.list_a[i] = a_spec[u];
  }
  if (c1 > kCandCap) {  // candidates stay in the workspace
    __syncthreads();
    finish_from_global_candidates(sh, cand, b1, above1, c1, krem, out);
    return;
  }
#pragma unroll
  for (int u = 0; u < kSpecC; ++u) {
    const int i = tid + u * kTkThreads;
    if (i < c1) {
      sh.cand_key[i] = c_spec[u].x;
      sh.cand_pos[i] = (int)c_spec[u].y;
    }
  }
  __syncthreads();
  finish_from_candidates(sh, b1, above1, c1, krem, out);
}

// ---------------------------------------------------------------- launch
bool topk_split(int T, const void* ws) { return ws != nullptr && T > 0 && T < kSplitRows; }

size_t topk_workspace_bytes(int T, int max_ctx) {
  if (T <= 0 || T >= kSplitRows) return 0;
  return (size_t)T * split_ws(T, max_ctx).per_query;
}

hipError_t launch_topk(const LaunchBatch& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, bool lists_ready, const AbsorbJob* absorb, hipStream_t st,
                       const int32_t* row_mask) {
  const bool small = k <= kTopkSmall;
  if (!topk_split(b.T, ws) || row_mask != nullptr) {
    if (small)
      topk_row_kernel<kTopkSmall><<<b.T, kTkThreads, 0, st>>>(b.q_pos, scores, ld, k, idx, row_mask);
    else
      topk_row_kernel<kMaxTopk><<<b.T, kTkThreads, 0, st>>>(b.q_pos, scores, ld, k, idx, row_mask);
    return hipGetLastError();
  }
  const SplitWs w = split_ws(b.T, b.max_ctx);
  char* wsb = static_cast<char*>(ws);
  if (!lists_ready)
    topk_slice_hist_kernel<<<dim3(b.T, w.S), kSliceThreads, 0, st>>>(b.q_pos, scores, ld, k, wsb, w);
  topk_slice_select_kernel<<<dim3(b.T, w.S), kSelThreads, 0, st>>>(b.q_pos, scores, ld, k, wsb, w);
  const AbsorbJob ab = absorb ? *absorb : AbsorbJob{nullptr, nullptr, nullptr};
  static_assert(kTkWaves * 32 * 2 == kLat, "two absorb workgroups per head, a 32-column block per wave");
  const int grid = b.T + (absorb ? 2 * kHeads : 0);
  if (small)
    topk_finish_kernel<kTopkSmall><<<grid, kTkThreads, 0, st>>>(b.q_pos, scores, ld, k, idx, wsb, w, b.T, ab);
  else
    topk_finish_kernel<kMaxTopk><<<grid, kTkThreads, 0, st>>>(b.q_pos, scores, ld, k, idx, wsb, w, b.T, ab);
  return hipGetLastError();
}

// ---------------------------------------------------------------- candidate path
// For prefill chunks whose indexer GEMM keeps candidates instead of scores:
//   1. the GEMM scores a sample of each row, positions 0, R, 2R, ...;
//   2. topk_sample_threshold_kernel: per row of n > cap scores, theta = the
//      r-th largest sampled score with r = ceil(E * n_s / n), so that about E
//      of the row's scores lie at or above theta (E and cap are chosen on the
//      host, five sampling deviations from k and from cap); rows of n <= cap
//      keep every score (theta = -inf);
//   3. the GEMM keeps the scores >= theta as (key, position) in position order;
//   4. topk_cand_kernel selects the top k among them exactly (radix select as
//      above) when the row has between k and cap candidates and its threshold
//      bin fits in LDS.  Every score of the row's top k is then a candidate (at
//      least k scores are >= theta, so the k-th largest is too), so the result
//      equals the full path's.  Rows where this does not hold are flagged and
//      take the full path (scores by the key scan, then topk_row_kernel, both
//      limited to the flagged rows).
constexpr int kThrThreads = 256;

__global__ __launch_bounds__(kThrThreads) void topk_sample_threshold_kernel(
    const int32_t* __restrict__ q_pos, const float* __restrict__ sample, int64_t ld_s, int stride,
    int64_t target, int cap, float* __restrict__ theta) {
  __shared__ uint32_t hist[kTkBins];
  __shared__ int wave_tot[kThrThreads / 64];
  __shared__ int sel_bin, sel_above;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int pos = q_pos[t];
  const int n = pos + 1;
  if (n <= cap) {
    if (tid == 0) theta[t] = -INFINITY;
    return;
  }
  const int ns = pos / stride + 1;
  const int r = (int)min((int64_t)ns, max((int64_t)1, (target * ns + n - 1) / n));
  const float* row = sample + (int64_t)t * ld_s;
  // Radix select of the r-th largest sampled key: 12 + 12 + 8 bits; the
  // sampled scores are re-read from L2 on each pass.
  uint32_t prefix = 0;
  int krem = r;
  constexpr int shift[3] = {20, 8, 0};
  constexpr int nbins[3] = {kTkBins, kTkBins, 256};
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    for (int i = tid; i < kTkBins; i += kThrThreads) hist[i] = 0u;
    __syncthreads();
    const int sh = shift[p];
    const uint32_t hi_mask = p == 0 ? 0u : (0xFFFFFFFFu << (sh + (p == 1 ? 12 : 8)));
    for (int i = tid; i < ns; i += kThrThreads) {
      const uint32_t key = score_key(row[i]);
      if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> sh) & (nbins[p] - 1)], 1u);
    }
    __syncthreads();
    if (p < 2)
      find_bin<kThrThreads, kTkBins>(hist, krem, wave_tot, &sel_bin, &sel_above);
    else
      find_bin<kThrThreads, 256>(hist, krem, wave_tot, &sel_bin, &sel_above);
    prefix |= (uint32_t)sel_bin << sh;
    krem -= sel_above;
    __syncthreads();
  }
  if (tid == 0) theta[t] = key_floor(prefix);  // score >= theta  <=>  key >= prefix
}

template <int KMAX>
__global__ __launch_bounds__(kTkThreads) void topk_cand_kernel(
    const int32_t* __restrict__ q_pos, const uint32_t* __restrict__ cand, int cap, const int32_t* __restrict__ cnt,
    int k, int32_t* __restrict__ idx, int32_t* __restrict__ flags) {
  __shared__ TkShared<KMAX> sh;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int n = q_pos[t] + 1;
  int32_t* out = idx + (int64_t)t * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    if (tid == 0) flags[t] = 0;
    return;
  }
  const int c = cnt[t];
  if (c < k || c > cap) {  // the threshold missed: the row takes the full path
    if (tid == 0) flags[t] = 1;
    return;
  }
  const u32x2* cd = reinterpret_cast<const u32x2*>(cand) + (int64_t)t * cap;
  constexpr int kB = 8;  // candidates per thread per round of the histogram pass
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int b0 = 0; b0 < c; b0 += kB * kTkThreads) {
    uint32_t key[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int j = b0 + tid + u * kTkThreads;
      key[u] = j < c ? cd[j].x : 0u;
    }
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (b0 + tid + u * kTkThreads < c) atomicAdd(&sh.hist[key[u] >> 20], 1u);
  }
  __syncthreads();
  find_bin<kTkBins>(sh, k);
  const uint32_t b1 = (uint32_t)sh.sel_bin;
  int above = sh.sel_above;
  int cin = (int)sh.hist[b1];
  __syncthreads();
  // The candidates to resolve in LDS share a key prefix: the top digit b1, or,
  // when that bin holds more than fit, b1 and the next 12 bits (a second
  // histogram over the candidates of bin b1).  Keys with a larger prefix are
  // kept outright (list A).
  uint32_t prefix = b1;
  int pshift = 20;
  if (cin > kCandCap) {
    for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int b0 = 0; b0 < c; b0 += kB * kTkThreads) {
      uint32_t key[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int j = b0 + tid + u * kTkThreads;
        key[u] = j < c ? cd[j].x : 0u;
      }
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (b0 + tid + u * kTkThreads < c && (key[u] >> 20) == b1) atomicAdd(&sh.hist[(key[u] >> 8) & 0xFFFu], 1u);
    }
    __syncthreads();
    find_bin<kTkBins>(sh, k - above);
    prefix = (b1 << 12) | (uint32_t)sh.sel_bin;
    pshift = 8;
    above += sh.sel_above;
    cin = (int)sh.hist[sh.sel_bin];
    __syncthreads();
    if (cin > kCandCap) {  // more equal 20-bit prefixes than fit: the full path handles the row
      if (tid == 0) flags[t] = 1;
      return;
    }
  }
  // ordered compaction: thread tid takes candidates [base + kPerThread tid, +kPerThread)
  int nA = 0, nC = 0;
  for (int base = 0; base < c; base += kStep) {
    const int j0 = base + kPerThread * tid;
    u32x2 v[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) v[e] = j0 + e < c ? cd[j0 + e] : u32x2{0u, 0u};
    int ca = 0, cc = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const uint32_t d = v[e].x >> pshift;
      ca += j0 + e < c && d > prefix;
      cc += j0 + e < c && d == prefix;
    }
    int tot;
    const int ex = block_excl_scan<kTkWaves>((ca << 16) | cc, sh.wave_tot, tot);
    int oa = nA + (ex >> 16), oc = nC + (ex & 0xFFFF);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (j0 + e >= c) continue;
      const uint32_t d = v[e].x >> pshift;
      if (d > prefix) {
        sh.list_a[oa++] = (int)v[e].y;
      } else if (d == prefix) {
        sh.cand_key[oc] = v[e].x;
        sh.cand_pos[oc] = (int)v[e].y;
        ++oc;
      }
    }
    nA += tot >> 16;
    nC += tot & 0xFFFF;
  }
  __syncthreads();
  // (the LDS candidates all have top digit b1; their lower digits are resolved there)
  finish_from_candidates(sh, b1, above, cin, k - above, out);
  if (tid == 0) flags[t] = 0;
}

hipError_t launch_topk_candidates(const LaunchBatch& b, const float* sample, int64_t ld_s, int stride,
                                  int64_t target, int cap, float* theta, const uint32_t* cand, const int32_t* cnt,
                                  int k, int32_t* idx, int32_t* flags, hipStream_t st, bool threshold_only) {
  if (threshold_only) {
    topk_sample_threshold_kernel<<<b.T, kThrThreads, 0, st>>>(b.q_pos, sample, ld_s, stride, target, cap, theta);
    return hipGetLastError();
  }
  if (k <= kTopkSmall)
    topk_cand_kernel<kTopkSmall><<<b.T, kTkThreads, 0, st>>>(b.q_pos, cand, cap, cnt, k, idx, flags);
  else
    topk_cand_kernel<kMaxTopk><<<b.T, kTkThreads, 0, st>>>(b.q_pos, cand, cap, cnt, k, idx, flags);
  return hipGetLastError();
}

}  // namespace dsa
