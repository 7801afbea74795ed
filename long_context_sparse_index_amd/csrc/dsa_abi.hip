// C ABI of the DSA hot path: argument checks, workspace planning, query
// chunking and kernel launches on the caller's stream.  No allocation, no
// host synchronisation, nothing enqueued when a check fails.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "dsa.h"
#include "dsa_common.h"
#include "dsa_kernels.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// Upper bounds that keep every grid dimension and 32-bit index in range.
constexpr int32_t kMaxQueries = 1 << 21;
constexpr int32_t kMaxCtx = 1 << 21;  // 2,097,152 positions; row offsets fit 32 bits

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dsa_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    g_last_hip_error = (int32_t)(e != hipSuccess ? e : hipErrorNoDevice);
    return DSA_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int s = g_dev_state[dev].load(std::memory_order_relaxed);
    if (s == 1) return DSA_OK;
    if (s == 2) return DSA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return DSA_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? DSA_OK : DSA_ERR_DEVICE;
}

// log2 of a valid page size (16 .. 2^20, a power of two), else 0.
int page_shift(int32_t page_size) {
  for (int s = 4; s <= 20; ++s)
    if (page_size == (1 << s)) return s;
  return 0;
}

dsa_status check_batch(const dsa_batch* b) {
  if (!b) return DSA_ERR_NULL;
  if (b->num_queries < 0 || b->num_queries > kMaxQueries) return DSA_ERR_SHAPE;
  if (b->num_seqs < 1 || b->max_ctx < 1 || b->max_ctx > kMaxCtx) return DSA_ERR_SHAPE;
  if (b->kv_format != DSA_KV_BF16 && b->kv_format != DSA_KV_INT4) return DSA_ERR_UNSUPPORTED;
  if (b->page_size != 0) {
    if (page_shift(b->page_size) == 0) return DSA_ERR_SHAPE;
    if (b->max_pages < 1 || (int64_t)b->max_pages * b->page_size < b->max_ctx) return DSA_ERR_SHAPE;
    if ((int64_t)b->num_seqs * b->max_pages > ((int64_t)1 << 31)) return DSA_ERR_SHAPE;
  }
  if (b->num_queries > 0) {
    if (!b->q_seq || !b->q_pos) return DSA_ERR_NULL;
    if (b->page_size == 0 ? !b->seq_row0 : !b->block_table) return DSA_ERR_NULL;
  }
  return DSA_OK;
}

dsa_status check_scores(const dsa_batch* b, const void* scores, int64_t ld) {
  if (!scores) return DSA_ERR_NULL;
  if (ld < b->max_ctx) return DSA_ERR_SHAPE;
  if ((ld & 3) != 0 || !aligned16(scores)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

dsa_status launch_status(hipError_t e) {
  if (e == hipSuccess) return DSA_OK;
  g_last_hip_error = (int32_t)e;
  return DSA_ERR_LAUNCH;
}

dsa::LaunchBatch to_launch(const dsa_batch* b, int t0, int T) {
  dsa::LaunchBatch lb;
  lb.T = T;
  lb.max_ctx = b->max_ctx;
  lb.q_seq = b->q_seq + t0;
  lb.q_pos = b->q_pos + t0;
  lb.rows.seq_row0 = b->page_size == 0 ? b->seq_row0 : nullptr;
  lb.rows.table = b->page_size == 0 ? nullptr : b->block_table;
  lb.rows.page_shift = b->page_size == 0 ? 0 : page_shift(b->page_size);
  lb.rows.max_pages = b->page_size == 0 ? 0 : b->max_pages;
  lb.kv_int4 = b->kv_format == DSA_KV_INT4;
  return lb;
}

int64_t score_ld(int32_t max_ctx) { return ((int64_t)max_ctx + 3) / 4 * 4; }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool use_gemm(const dsa_batch* b) {
  return b->num_queries >= 8 && (int64_t)b->num_queries >= 8 * (int64_t)b->num_seqs;
}

// Candidate path of the prefill forward (page-4 §2.2: the selector keeps the
// index_topk best of the query's history; see topk.hip): every kCandStride-th
// position is scored first, and the indexer GEMM then keeps only the scores at
// or above a per-query threshold taken from that sample.  The threshold's
// sample rank puts about `target` of a row's scores above it, where target and
// the list capacity `cap` lie five sampling deviations (sqrt(target *
// kCandStride)) above k and below cap; rows outside [k, cap] take the full path.
constexpr int kCandStride = 128;
struct CandPlan {
  int64_t target;
  int cap;
  int64_t ld_s;  // sample-score row stride
};
CandPlan cand_plan(int32_t k, int32_t max_ctx) {
  const double R = kCandStride;
  const double x = (5.0 * std::sqrt(R) + std::sqrt(25.0 * R + 4.0 * k)) / 2.0;
  const double target = std::ceil(x * x);
  const double cap = target + 5.0 * std::sqrt(target * R);
  CandPlan c;
  c.target = (int64_t)target;
  c.cap = (int)((cap + 1023.0) / 1024.0) * 1024;
  c.ld_s = ((int64_t)(max_ctx - 1) / kCandStride + 1 + 3) / 4 * 4;
  return c;
}

// Workspace of dsa_forward for a chunk of T queries.  `cand`: the chunk takes
// the candidate path (its extra arrays follow the MLA workspace).
struct FwdPlan {
  size_t scores_off, idx_off, topk_off, mla_off, sample_off, theta_off, cnt_off, flags_off, cand_off, total;
  dsa::MlaPlan mla;
  CandPlan cp;
};
FwdPlan plan_forward(int32_t T, int32_t max_ctx, int32_t k, bool need_idx, bool cand) {
  FwdPlan f{};
  f.scores_off = 0;
  size_t end = align256((size_t)T * score_ld(max_ctx) * sizeof(float));
  f.idx_off = end;
  if (need_idx) end += align256((size_t)T * k * sizeof(int32_t));
  f.topk_off = end;
  end += align256(dsa::topk_workspace_bytes(T, max_ctx));
  f.mla_off = end;
  f.mla = dsa::plan_mla(T, k);
  end += f.mla.total;
  if (cand) {
    f.cp = cand_plan(k, max_ctx);
    f.sample_off = end;
    end += align256((size_t)T * f.cp.ld_s * sizeof(float));
    f.theta_off = end;
    end += align256((size_t)T * sizeof(float));
    f.cnt_off = end;
    end += align256((size_t)T * sizeof(int32_t));
    f.flags_off = end;
    end += align256((size_t)T * sizeof(int32_t));
    f.cand_off = end;
    end += align256((size_t)T * f.cp.cap * 2 * sizeof(uint32_t));
  }
  f.total = end;
  return f;
}

// The chunk of T queries takes the candidate path: indexer GEMM with one
// workgroup per query block over the whole context.
bool use_candidates(const dsa_batch* b, int32_t T, bool gemm) {
  return gemm && dsa::gemm_whole_context(T, b->max_ctx);
}

// The whole path over one workspace: query chunks sized to ws_bytes.
dsa_status forward_impl(const dsa_batch* batch, const dsa_bf16* q_idx, const dsa_bf16* w,
                        const dsa_bf16* k_idx, const dsa_bf16* q_nope, const dsa_bf16* q_rope,
                        const void* kv, const dsa_bf16* w_uk, const dsa_bf16* w_uv,
                        int32_t k, float softmax_scale, void* out, int32_t out_dtype,
                        int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

}  // namespace

// Scratch of dsa_forward_noalloc: the workspace of callers that cannot
// allocate, one copy per device for the life of the process.  Host code never
// uses this name as an address: the device address of each device's copy comes
// from hipGetSymbolAddress (scratch_address below).
constexpr size_t kNoAllocScratchBytes = (size_t)DSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of the current device's scratch (resolved once per device,
// with that device current).
dsa_status scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = (int32_t)(e != hipSuccess ? e : hipErrorInvalidDevice);
    return DSA_ERR_DEVICE;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        g_last_hip_error = (int32_t)(e != hipSuccess ? e : hipErrorInvalidSymbol);
        return DSA_ERR_DEVICE;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return DSA_OK;
}

}  // namespace

// Result word of the debug-mode device-argument check (DSA_CHECK_DEVICE_ARGS=1),
// one per device; its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint32_t argcheck_word[64];

namespace {

thread_local uint32_t g_last_arg_flags = 0;
std::mutex g_argcheck_mu;  // the word is shared by all calls on a device
std::atomic<void*> g_argword_ptr[kMaxDevices];

bool debug_device_args() {
  const char* e = std::getenv("DSA_CHECK_DEVICE_ARGS");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

// Debug mode: check the device-side preconditions of a call, wait for the
// result, and report DSA_ERR_DEVICE_ARGS before anything of the op is enqueued.
dsa_status debug_check(const dsa_batch* b, const int32_t* idx, int32_t k, hipStream_t st) {
  if (!debug_device_args()) return DSA_OK;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = (int32_t)(e != hipSuccess ? e : hipErrorInvalidDevice);
    return DSA_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_argcheck_mu);
  void* w = g_argword_ptr[dev].load(std::memory_order_relaxed);
  if (w == nullptr) {
    e = hipGetSymbolAddress(&w, HIP_SYMBOL(argcheck_word));
    if (e != hipSuccess || w == nullptr) {
      g_last_hip_error = (int32_t)(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return DSA_ERR_DEVICE;
    }
    g_argword_ptr[dev].store(w, std::memory_order_relaxed);
  }
  (void)hipGetLastError();
  e = dsa::launch_argcheck(to_launch(b, 0, b->num_queries), b->num_seqs, 0, idx, k, static_cast<uint32_t*>(w), st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  uint32_t flags = 0;
  if (e == hipSuccess) e = hipMemcpy(&flags, w, sizeof(flags), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return launch_status(e);
  if (flags == 0) return DSA_OK;
  g_last_arg_flags = flags;
  return DSA_ERR_DEVICE_ARGS;
}

}  // namespace

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

uint32_t dsa_last_device_arg_flags(void) { return g_last_arg_flags; }

dsa_status dsa_check_device_args(const dsa_batch* batch, const int32_t* idx, int32_t k, int64_t cache_rows,
                                 uint32_t* flags, void* stream) {
  dsa_status s = check_batch(batch);
  if (s != DSA_OK) return s;
  if (!flags) return DSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(flags) & 3u) != 0) return DSA_ERR_ALIGN;
  if (idx != nullptr && (k < 1 || k > DSA_MAX_TOPK)) return DSA_ERR_SHAPE;
  if (cache_rows < 0) return DSA_ERR_SHAPE;
  if ((s = check_device()) != DSA_OK) return s;
  (void)hipGetLastError();
  return launch_status(dsa::launch_argcheck(to_launch(batch, 0, batch->num_queries), batch->num_seqs, cache_rows,
                                            idx, idx ? k : 0, flags, (hipStream_t)stream));
}

int32_t dsa_last_hip_error(void) { return g_last_hip_error; }

const char* dsa_status_string(int32_t s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size argument is out of range";
    case DSA_ERR_ALIGN: return "a pointer or leading dimension is misaligned";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_UNSUPPORTED: return "unsupported option";
    case DSA_ERR_LAUNCH: return "kernel launch failed";
    case DSA_ERR_DEVICE: return "no gfx950 HIP device is current";
    case DSA_ERR_DEVICE_ARGS: return "a device-side argument violates its precondition (DSA_CHECK_DEVICE_ARGS)";
    default: return "unknown status";
  }
}

size_t dsa_workspace_bytes(int32_t op, int32_t num_queries, int32_t max_ctx, int32_t k) {
  if (num_queries < 0 || num_queries > kMaxQueries || max_ctx < 1 || max_ctx > kMaxCtx) return 0;
  switch (op) {
    case DSA_OP_INDEX_SCORES: return 0;
    case DSA_OP_TOPK: return dsa::topk_workspace_bytes(num_queries, max_ctx);
    case DSA_OP_SPARSE_MLA:
      if (k < 1 || k > DSA_MAX_TOPK) return 0;
      return dsa::plan_mla(num_queries, k).total;
    case DSA_OP_FORWARD:
      if (k < 1 || k > DSA_MAX_TOPK) return 0;
      // (the candidate path's arrays whenever such a chunk could take it)
      return plan_forward(num_queries, max_ctx, k, true, dsa::gemm_whole_context(num_queries, max_ctx)).total;
    default: return 0;
  }
}

dsa_status dsa_quantize_kv_int4(const dsa_bf16* kv, int64_t rows, uint8_t* kv_int4, void* stream) {
  if (rows < 0 || rows > ((int64_t)1 << 40)) return DSA_ERR_SHAPE;
  if (rows == 0) return DSA_OK;
  if (!kv || !kv_int4) return DSA_ERR_NULL;
  if (!aligned16(kv) || !aligned16(kv_int4)) return DSA_ERR_ALIGN;
  dsa_status s = check_device();
  if (s != DSA_OK) return s;
  (void)hipGetLastError();
  return launch_status(dsa::launch_quantize_kv_int4(kv, rows, kv_int4, (hipStream_t)stream));
}

dsa_status dsa_index_share_schedule(int32_t num_layers, int32_t num_dense, int32_t index_topk_freq,
                                    int32_t* source) {
  if (!source) return DSA_ERR_NULL;
  if (num_layers < 1 || num_dense < 1 || num_dense > num_layers || index_topk_freq < 1)
    return DSA_ERR_SHAPE;
  for (int32_t l = 0; l < num_layers; ++l) {
    if (l < num_dense) {
      source[l] = l;
      continue;
    }
    // Place of l in its run of index_topk_freq sparse layers; the run's last
    // layer is full, the others reuse the full layer just before the run.
    const int32_t r = (l - num_dense) % index_topk_freq;
    source[l] = r == index_topk_freq - 1 ? l : l - r - 1;
  }
  return DSA_OK;
}

dsa_status dsa_index_scores(const dsa_batch* batch, const dsa_bf16* q_idx, const dsa_bf16* w,
                            const dsa_bf16* k_idx, float* scores, int64_t ld_scores,
                            void* stream) {
  dsa_status s = check_batch(batch);
  if (s != DSA_OK) return s;
  if (batch->num_queries == 0) return DSA_OK;
  if (!q_idx || !w || !k_idx) return DSA_ERR_NULL;
  if ((s = check_scores(batch, scores, ld_scores)) != DSA_OK) return s;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx)) return DSA_ERR_ALIGN;
  if ((s = check_device()) != DSA_OK) return s;
  if ((s = debug_check(batch, nullptr, 0, (hipStream_t)stream)) != DSA_OK) return s;
  (void)hipGetLastError();
  return launch_status(dsa::launch_index_scores(to_launch(batch, 0, batch->num_queries), q_idx, w,
                                                k_idx, scores, ld_scores, use_gemm(batch), nullptr,
                                                (hipStream_t)stream));
}

dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  dsa_status s = check_batch(batch);
  if (s != DSA_OK) return s;
  if (batch->num_queries == 0) return DSA_OK;
  if ((s = check_scores(batch, scores, ld_scores)) != DSA_OK) return s;
  if (!idx) return DSA_ERR_NULL;
  if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_SHAPE;
  if (ws != nullptr) {
    if (!aligned16(ws)) return DSA_ERR_ALIGN;
    if (ws_bytes < dsa::topk_workspace_bytes(batch->num_queries, batch->max_ctx))
      return DSA_ERR_WORKSPACE;
  }
  if ((s = check_device()) != DSA_OK) return s;
  if ((s = debug_check(batch, nullptr, 0, (hipStream_t)stream)) != DSA_OK) return s;
  (void)hipGetLastError();
  return launch_status(dsa::launch_topk(to_launch(batch, 0, batch->num_queries), scores,
                                        ld_scores, k, idx, ws, false, nullptr,
                                        (hipStream_t)stream));
}

dsa_status dsa_sparse_mla_attn(const dsa_batch* batch, const dsa_bf16* q_nope,
                               const dsa_bf16* q_rope, const void* kv,
                               const dsa_bf16* w_uk, const dsa_bf16* w_uv, const int32_t* idx,
                               int32_t k, float softmax_scale, void* out, int32_t out_dtype,
                               void* ws, size_t ws_bytes, void* stream) {
  dsa_status s = check_batch(batch);
  if (s != DSA_OK) return s;
  if (batch->num_queries == 0) return DSA_OK;
  if (!q_nope || !q_rope || !kv || !w_uk || !w_uv || !idx || !out) return DSA_ERR_NULL;
  if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_SHAPE;
  if (out_dtype != DSA_OUT_BF16 && out_dtype != DSA_OUT_F32) return DSA_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return DSA_ERR_SHAPE;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(kv) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(out))
    return DSA_ERR_ALIGN;
  const dsa::MlaPlan plan = dsa::plan_mla(batch->num_queries, k);
  if (!ws) return DSA_ERR_NULL;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  if (ws_bytes < plan.total) return DSA_ERR_WORKSPACE;
  if ((s = check_device()) != DSA_OK) return s;
  if ((s = debug_check(batch, idx, k, (hipStream_t)stream)) != DSA_OK) return s;
  (void)hipGetLastError();
  return launch_status(dsa::launch_sparse_mla(to_launch(batch, 0, batch->num_queries), plan,
                                              q_nope, q_rope, kv, w_uk, w_uv, idx, softmax_scale,
                                              out, out_dtype == DSA_OUT_F32, ws, false,
                                              (hipStream_t)stream));
}

dsa_status dsa_forward(const dsa_batch* batch, const dsa_bf16* q_idx, const dsa_bf16* w,
                       const dsa_bf16* k_idx, const dsa_bf16* q_nope, const dsa_bf16* q_rope,
                       const void* kv, const dsa_bf16* w_uk, const dsa_bf16* w_uv,
                       int32_t k, float softmax_scale, void* out, int32_t out_dtype,
                       int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(batch, q_idx, w, k_idx, q_nope, q_rope, kv, w_uk, w_uv, k, softmax_scale, out,
                      out_dtype, idx_out, ws, ws_bytes, stream);
}

dsa_status dsa_forward_noalloc(const dsa_batch* batch, const dsa_bf16* q_idx, const dsa_bf16* w,
                               const dsa_bf16* k_idx, const dsa_bf16* q_nope, const dsa_bf16* q_rope,
                               const void* kv, const dsa_bf16* w_uk, const dsa_bf16* w_uv,
                               int32_t k, float softmax_scale, void* out, int32_t out_dtype,
                               int32_t* idx_out, void* stream) {
  dsa_status s = check_batch(batch);
  if (s != DSA_OK) return s;
  if (batch->num_queries == 0) return DSA_OK;
  if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_SHAPE;
  // One query must fit the scratch (the workspace of larger batches is chunked).
  if (plan_forward(1, batch->max_ctx, k, idx_out == nullptr, false).total > kNoAllocScratchBytes)
    return DSA_ERR_WORKSPACE;
  if ((s = check_device()) != DSA_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != DSA_OK) return s;
  return forward_impl(batch, q_idx, w, k_idx, q_nope, q_rope, kv, w_uk, w_uv, k, softmax_scale, out,
                      out_dtype, idx_out, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"

namespace {

dsa_status forward_impl(const dsa_batch* batch, const dsa_bf16* q_idx, const dsa_bf16* w,
                        const dsa_bf16* k_idx, const dsa_bf16* q_nope, const dsa_bf16* q_rope,
                        const void* kv, const dsa_bf16* w_uk, const dsa_bf16* w_uv,
                        int32_t k, float softmax_scale, void* out, int32_t out_dtype,
                        int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  dsa_status s = check_batch(batch);
  if (s != DSA_OK) return s;
  if (batch->num_queries == 0) return DSA_OK;
  if (!q_idx || !w || !k_idx || !q_nope || !q_rope || !kv || !w_uk || !w_uv || !out)
    return DSA_ERR_NULL;
  if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_SHAPE;
  if (out_dtype != DSA_OUT_BF16 && out_dtype != DSA_OUT_F32) return DSA_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return DSA_ERR_SHAPE;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx) || !aligned16(q_nope) ||
      !aligned16(q_rope) || !aligned16(kv) || !aligned16(w_uk) || !aligned16(w_uv) ||
      !aligned16(out))
    return DSA_ERR_ALIGN;
  const int32_t T = batch->num_queries;
  if (!ws) return DSA_ERR_NULL;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  const bool need_idx = idx_out == nullptr;
  const bool gemm = use_gemm(batch);
  auto plan = [&](int32_t c) {
    return plan_forward(c, batch->max_ctx, k, need_idx, use_candidates(batch, c, gemm));
  };
  // Largest chunk (by halving) for which both the full chunks and the last,
  // shorter one fit (a short chunk may use more key splits per query).
  auto fits = [&](int32_t c) {
    if (plan(c).total > ws_bytes) return false;
    const int32_t rem = T % c;
    return rem == 0 || plan(rem).total <= ws_bytes;
  };
  int32_t tc = T;
  while (tc > 1 && !fits(tc)) tc = (tc + 1) / 2;
  if (!fits(tc)) return DSA_ERR_WORKSPACE;
  if ((s = check_device()) != DSA_OK) return s;
  if ((s = debug_check(batch, nullptr, 0, (hipStream_t)stream)) != DSA_OK) return s;
  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  const int64_t ld = score_ld(batch->max_ctx);
  char* base = static_cast<char*>(ws);
  const size_t out_elem = out_dtype == DSA_OUT_F32 ? sizeof(float) : sizeof(uint16_t);
  for (int32_t t0 = 0; t0 < T; t0 += tc) {
    const int32_t n = T - t0 < tc ? T - t0 : tc;
    const bool cand = use_candidates(batch, n, gemm);
    const FwdPlan p = plan(n);
    const dsa::LaunchBatch lb = to_launch(batch, t0, n);
    float* scores = reinterpret_cast<float*>(base + p.scores_off);
    int32_t* idx = need_idx ? reinterpret_cast<int32_t*>(base + p.idx_off) : idx_out + (int64_t)t0 * k;
    const dsa_bf16* q_idx_c = q_idx + (int64_t)t0 * DSA_INDEX_HEADS * DSA_INDEX_DIM;
    const dsa_bf16* w_c = w + (int64_t)t0 * DSA_INDEX_HEADS;
    // The key scan writes the split top-k's slice lists as it goes.
    void* topk_ws = base + p.topk_off;
    const bool fused_lists = !gemm && dsa::topk_split(n, topk_ws);
    // With the split top-k, the query absorption runs on the finish kernel's
    // spare workgroups instead of its own launch.
    const dsa_bf16* q_nope_c = q_nope + (int64_t)t0 * DSA_HEADS * DSA_QK_NOPE_DIM;
    const bool ride = dsa::topk_split(n, topk_ws);
    const dsa::AbsorbJob job{q_nope_c, w_uk,
                             reinterpret_cast<uint16_t*>(base + p.mla_off + p.mla.q_lat_off)};
    hipError_t e;
    if (cand) {
      // sampled scores -> thresholds -> candidates -> exact top-k; flagged rows
      // take the full path (key scan and row top-k on those rows only)
      float* sample = reinterpret_cast<float*>(base + p.sample_off);
      float* theta = reinterpret_cast<float*>(base + p.theta_off);
      int32_t* cnt = reinterpret_cast<int32_t*>(base + p.cnt_off);
      int32_t* flags = reinterpret_cast<int32_t*>(base + p.flags_off);
      uint32_t* cl = reinterpret_cast<uint32_t*>(base + p.cand_off);
      e = dsa::launch_index_sample(lb, q_idx_c, w_c, k_idx, sample, p.cp.ld_s, kCandStride, st);
      if (e == hipSuccess)
        e = dsa::launch_topk_candidates(lb, sample, p.cp.ld_s, kCandStride, p.cp.target, p.cp.cap, theta,
                                        nullptr, nullptr, k, nullptr, nullptr, st, true);
      if (e == hipSuccess)
        e = dsa::launch_index_candidates(lb, q_idx_c, w_c, k_idx, theta, cl, p.cp.cap, cnt, st);
      if (e == hipSuccess)
        e = dsa::launch_topk_candidates(lb, sample, p.cp.ld_s, kCandStride, p.cp.target, p.cp.cap, theta, cl,
                                        cnt, k, idx, flags, st, false);
      if (e == hipSuccess)
        e = dsa::launch_index_scores(lb, q_idx_c, w_c, k_idx, scores, ld, false, nullptr, st, flags);
      if (e == hipSuccess) e = dsa::launch_topk(lb, scores, ld, k, idx, nullptr, false, nullptr, st, flags);
    } else {
      e = dsa::launch_index_scores(lb, q_idx_c, w_c, k_idx, scores, ld, gemm, fused_lists ? topk_ws : nullptr,
                                   st);
      if (e == hipSuccess)
        e = dsa::launch_topk(lb, scores, ld, k, idx, topk_ws, fused_lists, ride ? &job : nullptr, st);
    }
    if (e == hipSuccess)
      e = dsa::launch_sparse_mla(lb, p.mla, q_nope_c,
                                 q_rope + (int64_t)t0 * DSA_HEADS * DSA_QK_ROPE_DIM, kv, w_uk,
                                 w_uv, idx, softmax_scale,
                                 static_cast<char*>(out) + (size_t)t0 * DSA_HEADS * DSA_V_DIM * out_elem,
                                 out_dtype == DSA_OUT_F32, base + p.mla_off, ride, st);
    if (e != hipSuccess) return launch_status(e);
  }
  return DSA_OK;
}

}  // namespace
