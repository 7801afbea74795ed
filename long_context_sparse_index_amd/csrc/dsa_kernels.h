// Internal launch interface between the C ABI (dsa_abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Where token s of sequence b sits in the caches: row seq_row0[b] + s
// (contiguous, page_shift == 0), or row (table[b * max_pages + (s >> page_shift)]
// << page_shift) | (s & (2^page_shift - 1)) (paged, page_shift 4 .. 20).
struct CacheRows {
  const int64_t* seq_row0;
  const int32_t* table;
  int page_shift;
  int max_pages;
};

struct LaunchBatch {
  int T;                   // queries in this launch
  int max_ctx;             // host bound of q_pos + 1
  const int32_t* q_seq;    // [T] device
  const int32_t* q_pos;    // [T] device
  CacheRows rows;
  bool kv_int4;            // latent cache rows are INT4 (400 B) instead of bf16 (1152 B)
  bool paged() const { return rows.page_shift != 0; }
};

// INT4 latent cache: quantise `rows` bf16 cache rows into 400-byte rows.
hipError_t launch_quantize_kv_int4(const uint16_t* kv, int64_t rows, uint8_t* out, hipStream_t st);

// Device-side argument check (DSA_ARG_* bits into *flags, cleared first).
hipError_t launch_argcheck(const LaunchBatch& b, int num_seqs, int64_t cache_rows, const int32_t* idx, int k,
                           uint32_t* flags, hipStream_t st);

// Indexer scores.  gemm=true: tiled GEMM over blocks of consecutive queries;
// else the per-query key scan, which also writes the split top-k's slice bin
// lists into topk_ws when that is not null.
hipError_t launch_index_scores(const LaunchBatch& b, const uint16_t* q_idx, const uint16_t* w,
                               const uint16_t* k_idx, float* scores, int64_t ld, bool gemm,
                               void* topk_ws, hipStream_t st, const int32_t* row_mask = nullptr);
// True when the query blocks alone fill the chip and the indexer GEMM gives
// each one workgroup over the whole context (the condition of the candidate
// path below).
bool gemm_whole_context(int T, int max_ctx);
// Scores of the sampled positions 0, stride, 2 stride, ... <= q_pos[t] into
// sample[t * ld_s + i] (GEMM path, contiguous caches).
hipError_t launch_index_sample(const LaunchBatch& b, const uint16_t* q_idx, const uint16_t* w,
                               const uint16_t* k_idx, float* sample, int64_t ld_s, int stride, hipStream_t st);
// Indexer GEMM that keeps, per query t, the (monotone key, position) of every
// score >= theta[t] in position order in cand[t * cap ..] (u32 pairs; entries
// past cap counted but not written), the count in cnt[t].  Needs
// gemm_whole_context(T, max_ctx).
hipError_t launch_index_candidates(const LaunchBatch& b, const uint16_t* q_idx, const uint16_t* w,
                                   const uint16_t* k_idx, const float* theta, uint32_t* cand, int cap, int* cnt,
                                   hipStream_t st);

// Top-k selection.  Batches of few rows use a split path that needs
// topk_workspace_bytes(T, max_ctx) of workspace; with ws == nullptr every row
// runs on one workgroup (same result).  lists_ready: the key scan already
// wrote the slice bin lists into ws.
size_t topk_workspace_bytes(int T, int max_ctx);
bool topk_split(int T, const void* ws);
// Query absorption that the split top-k may run on its spare workgroups
// (q_lat = W_UK q_nope for the launch's T queries).
struct AbsorbJob {
  const uint16_t* q_nope;
  const uint16_t* w_uk;
  uint16_t* q_lat;
};
hipError_t launch_topk(const LaunchBatch& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, bool lists_ready, const AbsorbJob* absorb, hipStream_t st,
                       const int32_t* row_mask = nullptr);
// Candidate path (see topk.hip): threshold_only -> theta[t] from the sampled
// scores; else the exact top-k of each row's candidates, flags[t] = 1 for rows
// that must take the full path (row_mask of the key scan and launch_topk).
hipError_t launch_topk_candidates(const LaunchBatch& b, const float* sample, int64_t ld_s, int stride,
                                  int64_t target, int cap, float* theta, const uint32_t* cand, const int32_t* cnt,
                                  int k, int32_t* idx, int32_t* flags, hipStream_t st, bool threshold_only);

// Sparse MLA: workspace layout and launches.
struct MlaPlan {
  int T, k, splits, keys_per_split;
  // few queries with a bf16 cache: the decode core's key splits
  bool dec;
  int dec_splits, dec_keys_per_split;
  size_t q_lat_off, o_lat_off, part_off, ml_off, wuvt_off, total;
};
MlaPlan plan_mla(int T, int k);
hipError_t launch_sparse_mla(const LaunchBatch& b, const MlaPlan& p, const uint16_t* q_nope,
                             const uint16_t* q_rope, const void* kv, const uint16_t* w_uk,
                             const uint16_t* w_uv, const int32_t* idx, float scale, void* out,
                             int out_f32, void* ws, bool q_lat_ready, hipStream_t st);

}  // namespace dsa
