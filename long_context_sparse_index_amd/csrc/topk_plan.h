// Row slicing shared by the decode key scan and the split top-k, the layout of
// the split top-k workspace, and the workgroup primitives both use.
//
// A score row of n keys is cut into slices of `slice_keys` consecutive keys
// (a multiple of the 128-key scan tile).  Whoever produces a slice's scores (the
// key scan, or a histogram pass over stored scores) also writes the slice's
// top-digit histogram as a sparse list: u32 count, then `count` entries
// (bin << 16) | n_bin for the non-empty bins in ascending order, where bin is
// bits 31..20 of the monotone key of a score.  Sparse lists stay short because
// a row's scores populate few top-digit bins (a sign, an exponent and three
// mantissa bits), and a list never holds more entries than the slice has keys.
#pragma once

#include "dsa_common.h"

namespace dsa {

constexpr int kScanTile = 128;   // keys per scan tile and slice granularity
constexpr int kTkBins = 4096;    // top-digit bins
constexpr int kCandCap = 5120;   // candidates of the threshold bin(s) kept in LDS
constexpr int kCandCapWs = 32768;  // candidates of the threshold bin kept in the split workspace
constexpr int kSplitRows = 128;  // batches with fewer rows use the split top-k
constexpr int kMaxSlices = 1024; // slices per row
constexpr int kScanSlots = 512;  // resident key-scan workgroups (two per CU)

struct SplitWs {
  int S;               // slices per row (for max_ctx)
  int slice_keys;      // keys per slice
  size_t list_stride;  // bytes per slice list
  size_t list_off, hdr_off, a_off, c_off, per_query;
};

// Slicing for T rows of up to max_ctx keys: slices are 1..511 tiles long (so a
// slice's bin counts fit 16 bits) and a row has at most kMaxSlices of them.
// Among those, the longest slices are taken whose T x S workgroups fill the
// kScanSlots resident scan workgroups in whole rounds to >= 90%.
inline SplitWs split_ws(int T, int max_ctx) {
  const int tpr = (max_ctx + kScanTile - 1) / kScanTile;
  const int lo = tpr > 1024 ? (tpr + 1023) / 1024 : 1;
  const int hi = tpr < 511 ? tpr : 511;
  int best = hi;
  double best_eff = -1.0;
  for (int tpw = hi; tpw >= lo; --tpw) {
    const int S = (tpr + tpw - 1) / tpw;
    const double rounds = (double)T * S / (double)kScanSlots;
    const double full = rounds <= 1.0 ? 1.0 : (double)(long long)(rounds + 0.999999);
    const double eff = rounds / full;
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = tpw;
    }
    if (eff >= 0.9) {
      best = tpw;
      break;
    }
  }
  SplitWs w;
  w.slice_keys = best * kScanTile;
  w.S = (tpr + best - 1) / best;
  const int cap = w.slice_keys < kTkBins ? w.slice_keys : kTkBins;
  w.list_stride = ((size_t)(1 + cap) * sizeof(uint32_t) + 15) / 16 * 16;
  size_t o = 0;
  w.list_off = o;
  o += (size_t)w.S * w.list_stride;
  w.hdr_off = o;  // {b1, above1, c1, 0}
  o += 16;
  w.a_off = o;
  o += (size_t)kMaxTopk * sizeof(int);
  w.c_off = o;
  o += (size_t)kCandCapWs * 2 * sizeof(uint32_t);
  w.per_query = (o + 255) / 256 * 256;
  return w;
}

// Exclusive prefix sum over the workgroup (NW waves) in thread order; the
// workgroup total goes to `total`.  Contains two LDS barriers (global loads in
// flight stay in flight).
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) wave_tot[wave] = incl;
  lds_sync();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = wave_tot[i];
    pre += (i < wave) ? x : 0;
    tot += x;
  }
  lds_sync();
  total = tot;
  return pre + incl - v;
}

// LDS histogram of 16-bit counts: word i holds bin 2i (low half) and 2i+1.
__device__ __forceinline__ void hist16_add(uint32_t* hist, uint32_t key) {
  atomicAdd(&hist[key >> 21], 1u << ((key >> 16) & 16u));
}

// Writes the sparse list of a packed 16-bit LDS histogram (kTkBins bins) to
// `list` (global).  All NT threads of the workgroup call it after a barrier.
template <int NT>
__device__ __forceinline__ void write_bin_list(const uint32_t* hist, uint32_t* list, int* wave_tot) {
  constexpr int kWords = kTkBins / 2 / NT;
  const int tid = threadIdx.x;
  uint32_t v[kWords];
  int nz = 0;
#pragma unroll
  for (int i = 0; i < kWords; ++i) {
    v[i] = hist[tid * kWords + i];
    nz += ((v[i] & 0xFFFFu) != 0) + ((v[i] >> 16) != 0);
  }
  int total;
  int o = block_excl_scan<NT / 64>(nz, wave_tot, total);
#pragma unroll
  for (int i = 0; i < kWords; ++i) {
    const uint32_t b = 2u * (uint32_t)(tid * kWords + i);
    if (v[i] & 0xFFFFu) list[1 + o++] = (b << 16) | (v[i] & 0xFFFFu);
    if (v[i] >> 16) list[1 + o++] = ((b + 1u) << 16) | (v[i] >> 16);
  }
  if (tid == 0) list[0] = (uint32_t)total;
}

}  // namespace dsa
