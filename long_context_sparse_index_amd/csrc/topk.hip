// Top-k selector on gfx950: one workgroup (1024 threads) per query row.
//
// Keeps the k best of the n = q_pos+1 scores under (fp32 value descending,
// position ascending) and writes them as ascending positions, -1 padded
// (page "2026大模型架构概览（二）：GLM 5 DSV3.2 的 DSA 与 MoE 配置拆解", §2.2: the selector keeps the
// index_topk highest-scoring history keys; page "（五）一万亿次点积砍到两千次：DSA 怎么破 N²":
// index_topk = 2048).
//
// Radix select over the monotone uint32 image of the scores, digits
// [31:20] | [19:8] | [7:0]:
//   1. LDS histogram of the top digit over the row (global pass 1) -> bin b1
//      holding the k-th largest, and the count above it.
//   2. Fast path (bin b1 holds <= kCandCap scores): one more global pass does a
//      position-ordered compaction of "digit > b1" positions (all kept) into
//      list A and of the b1 candidates (key, position) into LDS.  The two lower
//      digits are resolved on the candidates in LDS, the kept candidates are
//      compacted in position order (list C) and A and C are merged.
//   3. Otherwise (heavy ties) the lower digits are resolved with further
//      global passes and a final ordered compaction writes the output.
// Every compaction is a block-wide prefix sum in position order, so equal
// scores resolve to the lower positions and the output needs no sort.
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkBins = 4096;
constexpr int kCandCap = 12288;

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
__device__ __forceinline__ int block_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTkWaves; ++i) {
    const int x = wave_tot[i];
    pre += (i < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return pre + incl - v;
}

// Finds the bin holding the krem-th largest element (1-based) of `hist`
// (counting from the highest bin) and the number of elements in higher bins.
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
  const int above = block_excl_scan(local, sh.wave_tot, total);
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

__device__ __forceinline__ void load4(const float* row, int i, int n, uint32_t key[4], bool ok[4]) {
  if (i + 3 < n) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[e] = score_key(v[e]);
      ok[e] = true;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ok[e] = i + e < n;
      key[e] = ok[e] ? score_key(row[i + e]) : 0u;
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

__global__ __launch_bounds__(kTkThreads) void topk_kernel(const int32_t* __restrict__ q_pos,
                                                          const float* __restrict__ scores,
                                                          int64_t ld, int k,
                                                          int32_t* __restrict__ idx) {
  __shared__ TkShared sh;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int n = q_pos[t] + 1;
  int32_t* out = idx + (int64_t)t * k;
  if (n <= k) {  // every position is kept
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + (int64_t)t * ld;
  constexpr int kStep = 4 * kTkThreads;

  // ---- pass 1: top digit histogram
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kStep) {
    uint32_t key[4];
    bool ok[4];
    load4(row, base + 4 * tid, n, key, ok);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ok[e]) atomicAdd(&sh.hist[key[e] >> 20], 1u);
  }
  __syncthreads();
  find_bin(sh, kTkBins, k);
  const uint32_t b1 = (uint32_t)sh.sel_bin;
  const int above1 = sh.sel_above;
  const int c1 = (int)sh.hist[b1];
  const int krem = k - above1;
  __syncthreads();

  if (c1 <= kCandCap) {
    // ---- pass 2: ordered compaction of the kept-for-sure and the candidates
    int nA = 0, nC = 0;
    for (int base = 0; base < n; base += kStep) {
      const int i = base + 4 * tid;
      uint32_t key[4];
      bool ok[4];
      load4(row, i, n, key, ok);
      int ca = 0, cc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!ok[e]) continue;
        const uint32_t d = key[e] >> 20;
        ca += d > b1;
        cc += d == b1;
      }
      int tot;
      const int ex = block_excl_scan((ca << 16) | cc, sh.wave_tot, tot);
      int oa = nA + (ex >> 16), oc = nC + (ex & 0xFFFF);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
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
    // ---- digit 2 on the candidates
    for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < c1; j += kTkThreads) atomicAdd(&sh.hist[(sh.cand_key[j] >> 8) & 0xFFFu], 1u);
    __syncthreads();
    find_bin(sh, kTkBins, krem);
    const uint32_t b2 = (uint32_t)sh.sel_bin;
    const int krem2 = krem - sh.sel_above;
    __syncthreads();
    // ---- digit 3
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
    // ---- ordered compaction of the kept candidates -> list C (krem entries)
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
      const int ex = block_excl_scan((gt << 16) | eq, sh.wave_tot, tot);
      const int eg = nG + (ex >> 16), ee = nE + (ex & 0xFFFF);
      if (gt) sh.list_c[eg + min(ee, r)] = sh.cand_pos[j];
      else if (eq && ee < r) sh.list_c[eg + ee] = sh.cand_pos[j];
      nG += tot >> 16;
      nE += tot & 0xFFFF;
    }
    __syncthreads();
    // ---- merge the two ascending lists
    for (int i = tid; i < above1; i += kTkThreads) {
      const int a = sh.list_a[i];
      out[i + lower_bound(sh.list_c, krem, a)] = a;
    }
    for (int j = tid; j < krem; j += kTkThreads) {
      const int c = sh.list_c[j];
      out[j + lower_bound(sh.list_a, above1, c)] = c;
    }
    return;
  }

  // ---- heavy-tie path: resolve the lower digits with global passes
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kStep) {
    uint32_t key[4];
    bool ok[4];
    load4(row, base + 4 * tid, n, key, ok);
#pragma unroll
    for (int e = 0; e < 4; ++e)
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
    uint32_t key[4];
    bool ok[4];
    load4(row, base + 4 * tid, n, key, ok);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ok[e] && (key[e] >> 8) == pre) atomicAdd(&sh.hist[key[e] & 0xFFu], 1u);
  }
  __syncthreads();
  find_bin(sh, 256, krem2);
  const int r = krem2 - sh.sel_above;
  const uint32_t kstar = (pre << 8) | (uint32_t)sh.sel_bin;
  int nG = 0, nE = 0;
  for (int base = 0; base < n; base += kStep) {
    const int i = base + 4 * tid;
    uint32_t key[4];
    bool ok[4];
    load4(row, i, n, key, ok);
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gt += ok[e] && key[e] > kstar;
      eq += ok[e] && key[e] == kstar;
    }
    int tot;
    const int ex = block_excl_scan((gt << 16) | eq, sh.wave_tot, tot);
    int eg = nG + (ex >> 16), ee = nE + (ex & 0xFFFF);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
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

hipError_t launch_topk(const LaunchBatch& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       hipStream_t st) {
  topk_kernel<<<b.T, kTkThreads, 0, st>>>(b.q_pos, scores, ld, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
