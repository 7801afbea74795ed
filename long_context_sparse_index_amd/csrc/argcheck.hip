// Device-side argument check: the preconditions the host cannot see (they sit
// in device arrays) checked by a kernel, for debugging callers.
//
// The selector keeps positions from the query's own history (page "2026大模型架构
// 概览（二）：GLM 5 DSV3.2 的 DSA 与 MoE 配置拆解", §2.2), so an index entry must be -1
// or a position 0 .. q_pos[t]; a query's visible positions must map to cache
// rows inside the caches.
#include "dsa.h"
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace dsa {

__global__ void argcheck_zero_kernel(uint32_t* flags) { *flags = 0u; }

// One workgroup per query (grid-stride over queries).  Bits of the result as in
// dsa.h (DSA_ARG_*).  A violation is recorded with one atomic OR per thread
// that saw one.
__global__ __launch_bounds__(256) void argcheck_kernel(int T, int num_seqs, int max_ctx, const int32_t* q_seq,
                                                       const int32_t* q_pos, CacheRows cr, int64_t cache_rows,
                                                       const int32_t* idx, int k, uint32_t* flags) {
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    const int seq = q_seq[t];
    const int pos = q_pos[t];
    uint32_t bad = 0;
    const bool seq_ok = seq >= 0 && seq < num_seqs;
    const bool pos_ok = pos >= 0 && pos < max_ctx;
    if (threadIdx.x == 0) {
      if (!seq_ok) bad |= DSA_ARG_Q_SEQ;
      if (!pos_ok) bad |= DSA_ARG_Q_POS;
      if (seq_ok && pos_ok && cr.page_shift == 0) {
        const int64_t r0 = cr.seq_row0[seq];
        if (r0 < 0 || (cache_rows > 0 && r0 + pos >= cache_rows)) bad |= DSA_ARG_CACHE_ROW;
      }
    }
    if (seq_ok && pos_ok && cr.page_shift != 0) {
      // every page holding positions 0 .. pos
      const int64_t pages = cache_rows > 0 ? cache_rows >> cr.page_shift : ((int64_t)1 << (31 - cr.page_shift));
      const int32_t* bt = cr.table + (int64_t)seq * cr.max_pages;
      for (int j = threadIdx.x; j <= (pos >> cr.page_shift); j += blockDim.x) {
        const int32_t pg = bt[j];
        if (pg < 0 || pg >= pages || pg >= ((int64_t)1 << (31 - cr.page_shift))) bad |= DSA_ARG_CACHE_ROW;
      }
    }
    if (idx != nullptr) {
      const int lim = pos_ok ? pos : max_ctx - 1;
      const int32_t* row = idx + (int64_t)t * k;
      for (int j = threadIdx.x; j < k; j += blockDim.x) {
        const int32_t v = row[j];
        if (v != -1 && (v < 0 || v > lim)) bad |= DSA_ARG_IDX;
      }
    }
    if (bad) atomicOr(flags, bad);
  }
}

hipError_t launch_argcheck(const LaunchBatch& b, int num_seqs, int64_t cache_rows, const int32_t* idx, int k,
                           uint32_t* flags, hipStream_t st) {
  argcheck_zero_kernel<<<1, 1, 0, st>>>(flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || b.T == 0) return e;
  const int grid = b.T < 65536 ? b.T : 65536;
  argcheck_kernel<<<grid, 256, 0, st>>>(b.T, num_seqs, b.max_ctx, b.q_seq, b.q_pos, b.rows, cache_rows, idx, k,
                                        flags);
  return hipGetLastError();
}

}  // namespace dsa
