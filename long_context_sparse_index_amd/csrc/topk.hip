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
//   * one 1024-thread workgroup per row (many rows, e.g. a prefill chunk);
//   * for few rows (decode), steps 1 and 2 are split over slices of the row:
//     slice suffix histograms; then per slice the row total (b1, the slice's
//     output offsets) and the compaction into global A / candidate lists; then
//     one workgroup per row runs steps 3/4.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkBins = 4096;
constexpr int kCandCap = 12288;
constexpr int kPerThread = 16;                   // scores per thread per pass step
constexpr int kStep = kPerThread * kTkThreads;   // scores per pass step

constexpr int kSlice = 8192;          // scores per slice in the split path
constexpr int kSliceThreads = 256;

struct TkShared {
  uint32_t hist[kTkBins];
  int wave_tot[kTkWaves];
  int sel_bin, sel_above;
  uint32_t cand_key[kCandCap];
  int cand_pos[kCandCap];
  int list_a[kMaxTopk];
  int list_c[kMaxTopk];
};

// Exclusive prefix sum over the workgroup in thread order; total in `total`.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = wave_tot[i];
    pre += (i < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return pre + incl - v;
}

// Finds the bin holding the krem-th largest element (1-based, counting from
// the highest bin) and the number of elements in higher bins.
__device__ void find_bin(TkShared& sh, int nbins, int krem) {
  const int tid = threadIdx.x;
  const int bpt = nbins >= kTkThreads ? nbins / kTkThreads : 1;
  const int top = nbins - 1 - tid * bpt;
  int local = 0;
  for (int b = 0; b < bpt; ++b) {
    const int bin = top - b;
    if (bin >= 0) local += (int)sh.hist[bin];
  }
  int total;
  const int above = block_excl_scan<kTkWaves>(local, sh.wave_tot, total);
  if (local > 0 && above < krem && krem <= above + local) {
    int acc = above;
    for (int b = 0; b < bpt; ++b) {
      const int bin = top - b;
      const int c = (int)sh.hist[bin];
      if (acc + c >= krem) {
        sh.sel_bin = bin;
        sh.sel_above = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
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

__device__ __forceinline__ int lower_bound(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Step 3: sh.cand_* holds the c1 candidates of bin b1 in position order and
// sh.list_a the above1 positions above it (ascending); krem = k - above1.
__device__ void finish_from_candidates(TkShared& sh, uint32_t b1, int above1, int c1, int krem,
                                       int32_t* out) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int j = tid; j < c1; j += kTkThreads) atomicAdd(&sh.hist[(sh.cand_key[j] >> 8) & 0xFFFu], 1u);
  __syncthreads();
  find_bin(sh, kTkBins, krem);
  const uint32_t b2 = (uint32_t)sh.sel_bin;
  const int krem2 = krem - sh.sel_above;
  __syncthreads();
  for (int i = tid; i < 256; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int j = tid; j < c1; j += kTkThreads) {
    const uint32_t key = sh.cand_key[j];
    if (((key >> 8) & 0xFFFu) == b2) atomicAdd(&sh.hist[key & 0xFFu], 1u);
  }
  __syncthreads();
  find_bin(sh, 256, krem2);
  const uint32_t b3 = (uint32_t)sh.sel_bin;
  const int r = krem2 - sh.sel_above;  // ties at the threshold key to keep (lowest positions)
  const uint32_t kstar = (b1 << 20) | (b2 << 8) | b3;
  int nG = 0, nE = 0;
  for (int base = 0; base < c1; base += kTkThreads) {
    const int j = base + tid;
    int gt = 0, eq = 0;
    if (j < c1) {
      const uint32_t key = sh.cand_key[j];
      gt = key > kstar;
      eq = key == kstar;
    }
    int tot;
    const int ex = block_excl_scan<kTkWaves>((gt << 16) | eq, sh.wave_tot, tot);
    const int eg = nG + (ex >> 16), ee = nE + (ex & 0xFFFF);
    if (gt) sh.list_c[eg + min(ee, r)] = sh.cand_pos[j];
    else if (eq && ee < r) sh.list_c[eg + ee] = sh.cand_pos[j];
    nG += tot >> 16;
    nE += tot & 0xFFFF;
  }
  __syncthreads();
  for (int i = tid; i < above1; i += kTkThreads) {
    const int a = sh.list_a[i];
    out[i + lower_bound(sh.list_c, krem, a)] = a;
  }
  for (int j = tid; j < krem; j += kTkThreads) {
    const int c = sh.list_c[j];
    out[j + lower_bound(sh.list_a, above1, c)] = c;
  }
}

// Step 4 (heavy ties): lower digits by passes over the row, then an ordered
// compaction straight to the output.
__device__ void finish_from_row(TkShared& sh, const float* row, int n, uint32_t b1, int krem,
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
  find_bin(sh, kTkBins, krem);
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
  find_bin(sh, 256, krem2);
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

// ---------------------------------------------------------------- one workgroup per row
__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(const int32_t* __restrict__ q_pos,
                                                              const float* __restrict__ scores,
                                                              int64_t ld, int k,
                                                              int32_t* __restrict__ idx) {
  __shared__ TkShared sh;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int n = q_pos[t] + 1;
  int32_t* out = idx + (int64_t)t * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + (int64_t)t * ld;
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
  find_bin(sh, kTkBins, k);
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
// Workspace, per query: slice suffix histograms [S][4096] u16 (entry b = number
// of the slice's scores whose top digit is >= b), a header {b1, above1, c1},
// list A [k_max] and candidates (key, position) [kCandCap][2].
struct SplitWs {
  int S;
  size_t hist_off, hdr_off, a_off, c_off, per_query;
};

__host__ __device__ inline SplitWs split_ws(int max_ctx) {
  SplitWs w;
  w.S = (max_ctx + kSlice - 1) / kSlice;
  size_t o = 0;
  w.hist_off = o;
  o += (size_t)w.S * kTkBins * sizeof(uint16_t);
  w.hdr_off = o;  // {b1, above1, c1, 0}
  o += 16;
  w.a_off = o;
  o += (size_t)kMaxTopk * sizeof(int);
  w.c_off = o;
  o += (size_t)kCandCap * 2 * sizeof(uint32_t);
  w.per_query = (o + 255) / 256 * 256;
  return w;
}

// Kernel 1 (grid T x S): suffix histogram of the top digit over one slice.
__global__ __launch_bounds__(kSliceThreads) void topk_slice_hist_kernel(
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int64_t ld, int k,
    char* __restrict__ ws, SplitWs w) {
  __shared__ uint32_t hist[kTkBins];
  __shared__ int wave_tot[kSliceThreads / 64];
  const int t = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int n = q_pos[t] + 1;
  const int s0 = s * kSlice;
  if (n <= k || s0 >= n) return;
  char* base = ws + (size_t)t * w.per_query;
  const float* row = scores + (int64_t)t * ld;
  for (int i = tid; i < kTkBins; i += kSliceThreads) hist[i] = 0;
  __syncthreads();
  const int end = min(n, s0 + kSlice);
#pragma unroll
  for (int q = 0; q < kSlice / (4 * kSliceThreads); ++q) {
    const int b = s0 + 4 * (tid + kSliceThreads * q);
    if (b + 3 < end) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + b);
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicAdd(&hist[score_key(v[e]) >> 20], 1u);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (b + e < end) atomicAdd(&hist[score_key(row[b + e]) >> 20], 1u);
    }
  }
  __syncthreads();
  // suffix sums: thread i owns bins 16i .. 16i+15; threads in descending bin order
  constexpr int kPerT = kTkBins / kSliceThreads;
  const int hi_t = kSliceThreads - 1 - tid;  // block of bins, scanned from the top
  uint32_t v[kPerT];
  int sum = 0;
#pragma unroll
  for (int e = kPerT - 1; e >= 0; --e) {
    v[e] = hist[hi_t * kPerT + e];
    sum += (int)v[e];
  }
  int tot;
  int run = block_excl_scan<kSliceThreads / 64>(sum, wave_tot, tot);  // scores in higher blocks
  uint16_t* dst = reinterpret_cast<uint16_t*>(base + w.hist_off) + (size_t)s * kTkBins;
  uint32_t out[kPerT];
#pragma unroll
  for (int e = kPerT - 1; e >= 0; --e) {
    run += (int)v[e];
    out[e] = (uint32_t)run;
  }
#pragma unroll
  for (int q = 0; q < kPerT / 8; ++q) {
    u32x4 pk;
#pragma unroll
    for (int d = 0; d < 4; ++d) pk[d] = out[8 * q + 2 * d] | (out[8 * q + 2 * d + 1] << 16);
    st16(dst + hi_t * kPerT + 8 * q, pk);
  }
}

// Kernel 2 (grid T x S): every workgroup sums the row's slice suffix
// histograms (finds b1 and its own output offsets) and compacts its slice into
// list A and the candidate list in position order.
struct SelShared {
  uint32_t hist[kTkBins];
  int wave_tot[kTkWaves];
  int sel_bin, sel_above;
};

__global__ __launch_bounds__(kTkThreads) void topk_slice_select_kernel(
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int64_t ld, int k,
    char* __restrict__ ws, SplitWs w) {
  __shared__ SelShared sh;
  const int t = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int n = q_pos[t] + 1;
  if (n <= k) return;
  const int S = (n + kSlice - 1) / kSlice;
  if (s >= S) return;
  char* base = ws + (size_t)t * w.per_query;
  const uint16_t* suf = reinterpret_cast<const uint16_t*>(base + w.hist_off);
  // ---- total suffix histogram; thread owns bins 4*tid .. 4*tid+3
  uint32_t acc[4] = {0u, 0u, 0u, 0u};
  for (int j = 0; j < S; ++j) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(suf + (size_t)j * kTkBins + 4 * tid);
    acc[0] += v.x & 0xFFFFu;
    acc[1] += v.x >> 16;
    acc[2] += v.y & 0xFFFFu;
    acc[3] += v.y >> 16;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) sh.hist[4 * tid + e] = acc[e];
  __syncthreads();
  // b1: the highest bin whose suffix count reaches k
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int b = 4 * tid + e;
    const uint32_t above = b + 1 < kTkBins ? sh.hist[b + 1] : 0u;
    if (sh.hist[b] >= (uint32_t)k && above < (uint32_t)k) {
      sh.sel_bin = b;
      sh.sel_above = (int)above;
    }
  }
  __syncthreads();
  const uint32_t b1 = (uint32_t)sh.sel_bin;
  const int above1 = sh.sel_above;
  const int c1 = (int)sh.hist[b1] - above1;
  if (s == 0 && tid == 0) {
    int* hdr = reinterpret_cast<int*>(base + w.hdr_off);
    hdr[0] = (int)b1;
    hdr[1] = above1;
    hdr[2] = c1;
  }
  const bool cand_fit = c1 <= kCandCap;
  const float* row = scores + (int64_t)t * ld;
  int* list_a = reinterpret_cast<int*>(base + w.a_off);
  uint32_t* cand = reinterpret_cast<uint32_t*>(base + w.c_off);
  if (cand_fit) {  // else the row's finish re-reads the row (heavy ties)
    // ---- this slice's offsets: sums over the earlier slices
    int ga = 0, gc = 0;
    for (int j = tid; j < s; j += kTkThreads) {
      const uint16_t* h = suf + (size_t)j * kTkBins;
      const int hb = h[b1];
      const int ha = b1 + 1 < kTkBins ? h[b1 + 1] : 0;
      ga += ha;
      gc += hb - ha;
    }
    int tot;
    (void)block_excl_scan<kTkWaves>((ga << 16) | gc, sh.wave_tot, tot);  // 16-bit halves: offsets < 65536
    int offA = tot >> 16, offC = tot & 0xFFFF;
    // ---- ordered compaction of the slice (8 consecutive scores per thread)
    constexpr int kPer = kSlice / kTkThreads;
    const int s0 = s * kSlice;
    const int end = min(n, s0 + kSlice);
    const int i0 = s0 + kPer * tid;
    uint32_t key[kPer];
    bool ok[kPer];
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const int b = i0 + 4 * q;
      if (b + 3 < end) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(row + b);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          key[4 * q + e] = score_key(v[e]);
          ok[4 * q + e] = true;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ok[4 * q + e] = b + e < end;
          key[4 * q + e] = ok[4 * q + e] ? score_key(row[b + e]) : 0u;
        }
      }
    }
    int ca = 0, cc = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const uint32_t d = key[e] >> 20;
      ca += ok[e] && d > b1;
      cc += ok[e] && d == b1;
    }
    const int ex = block_excl_scan<kTkWaves>((ca << 16) | cc, sh.wave_tot, tot);
    int oa = offA + (ex >> 16), oc = offC + (ex & 0xFFFF);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (!ok[e]) continue;
      const uint32_t d = key[e] >> 20;
      if (d > b1) {
        list_a[oa++] = i0 + e;
      } else if (d == b1) {
        *reinterpret_cast<u32x2*>(cand + 2 * oc) = u32x2{key[e], (uint32_t)(i0 + e)};
        ++oc;
      }
    }
  }
}

// Kernel 3 (grid T): load list A and the candidates, resolve the lower
// digits, merge into the output.
__global__ __launch_bounds__(kTkThreads) void topk_finish_kernel(const int32_t* __restrict__ q_pos,
                                                                 const float* __restrict__ scores,
                                                                 int64_t ld, int k,
                                                                 int32_t* __restrict__ idx,
                                                                 const char* __restrict__ ws,
                                                                 SplitWs w) {
  __shared__ TkShared sh;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int n = q_pos[t] + 1;
  int32_t* out = idx + (int64_t)t * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const char* base = ws + (size_t)t * w.per_query;
  const int* hdr = reinterpret_cast<const int*>(base + w.hdr_off);
  const uint32_t b1 = (uint32_t)hdr[0];
  const int above1 = hdr[1];
  const int c1 = hdr[2];
  const int krem = k - above1;
  if (c1 > kCandCap) {
    finish_from_row(sh, scores + (int64_t)t * ld, n, b1, krem, out);
    return;
  }
  const int* list_a = reinterpret_cast<const int*>(base + w.a_off);
  const uint32_t* cand = reinterpret_cast<const uint32_t*>(base + w.c_off);
  for (int i = tid; i < above1; i += kTkThreads) sh.list_a[i] = list_a[i];
  for (int j = tid; j < c1; j += kTkThreads) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(cand + 2 * j);
    sh.cand_key[j] = v.x;
    sh.cand_pos[j] = (int)v.y;
  }
  __syncthreads();
  finish_from_candidates(sh, b1, above1, c1, krem, out);
}

// ---------------------------------------------------------------- launch
// Rows below this count use the split path.
constexpr int kSplitRows = 128;

size_t topk_workspace_bytes(int T, int max_ctx) {
  if (T <= 0 || T >= kSplitRows) return 0;
  return (size_t)T * split_ws(max_ctx).per_query;
}

hipError_t launch_topk(const LaunchBatch& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, hipStream_t st) {
  if (b.T >= kSplitRows || ws == nullptr) {
    topk_row_kernel<<<b.T, kTkThreads, 0, st>>>(b.q_pos, scores, ld, k, idx);
    return hipGetLastError();
  }
  const SplitWs w = split_ws(b.max_ctx);
  char* wsb = static_cast<char*>(ws);
  topk_slice_hist_kernel<<<dim3(b.T, w.S), kSliceThreads, 0, st>>>(b.q_pos, scores, ld, k, wsb, w);
  topk_slice_select_kernel<<<dim3(b.T, w.S), kTkThreads, 0, st>>>(b.q_pos, scores, ld, k, wsb, w);
  topk_finish_kernel<<<b.T, kTkThreads, 0, st>>>(b.q_pos, scores, ld, k, idx, wsb, w);
  return hipGetLastError();
}

}  // namespace dsa
