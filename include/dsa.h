/*
 * dsa.h -- C ABI of the DSA sparse-attention hot path on AMD Instinct MI355X (gfx950).
 *
 * The method: a lightweight indexer scores every cached token of a query's
 * history, a top-k selector keeps index_topk (2048) positions, and multi-head
 * latent attention (MLA) runs over the kept positions only.
 *   - page "2026大模型架构概览（二）：GLM 5 DSV3.2 的 DSA 与 MoE 配置拆解", §2.1 (dimension
 *     table) and §2.2 (the indexer scores every query against all history and
 *     only ranks; the selector keeps the index_topk best; DSA is a filter in
 *     front of MLA, not a replacement);
 *   - page "（五）一万亿次点积砍到两千次：DSA 怎么破 N²", sections on the indexer
 *     (32 heads x 128-d dot products over every token), the full DSA flow
 *     (top-2048, then full attention over those only) and the cache (skipped
 *     tokens stay cached; DSA saves compute, not storage).
 *
 * Fixed dimensions (compile-time): indexer 32 heads x 128; attention 64 heads;
 * q/k 192 (nope) + 64 (rope); v 256; latent 512.  One cache row holds the
 * 512-d latent followed by the 64-d rope key (576 bf16 = 1152 B), one indexer
 * key per token (128 bf16 = 256 B).
 *
 * Conventions for every call below
 *   - All array pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors)
 *     unless stated; all arrays are dense row-major, innermost index last.
 *   - bf16 arrays are raw bit patterns (uint16_t).  bf16 arrays, the score
 *     matrix and the workspace must be 16-byte aligned (DSA_ERR_ALIGN).
 *   - Positions are sequence-local: query t belongs to sequence q_seq[t] and
 *     sits at position q_pos[t].  A query sees positions 0..q_pos[t] (itself
 *     included).  Token s of sequence b is cache row row(b, s) of both caches
 *     (the indexer keys k_idx and the latent cache kv):
 *       contiguous (page_size == 0): row(b, s) = seq_row0[b] + s;
 *       paged (page_size > 0):       row(b, s) = block_table[b*max_pages + s/page_size]
 *                                                * page_size + s % page_size
 *     (page 3, "GLM-5 7440亿参数，202K长上下文突破极限", section 六: paged KV caches for
 *     batched serving).  Paged rows must stay below 2^31.
 *   - Ownership: the caller owns every buffer.  The library allocates nothing,
 *     frees nothing and keeps no pointer after a call returns.  Work is
 *     enqueued on `stream` (a hipStream_t; NULL = default stream) and is not
 *     waited for: buffers must stay valid until the stream has passed it.
 *     Input caches and weights are never written.
 *   - Errors: every host-checkable precondition is checked before anything is
 *     enqueued, and a call that fails such a check enqueues nothing.
 *     DSA_ERR_LAUNCH reports a failed kernel launch (see dsa_last_hip_error);
 *     the kernels of the same call enqueued before the failing one (a call
 *     launches several, and dsa_forward one set per query chunk) stay
 *     enqueued, and the call's outputs are then unspecified.  Device-side
 *     preconditions (q_seq[t] < num_seqs, 0 <= q_pos[t] < rows of that
 *     sequence, every cache row and block_table page inside its allocation,
 *     idx entries in {-1} U [0, q_pos[t]]) are not checked: violating them is
 *     undefined.
 *   - num_queries == 0 is a valid empty call: DSA_OK, nothing enqueued.
 *   - Calls are re-entrant; the only library state is a per-device cache of
 *     the device check and a thread-local last HIP error.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 4

#define DSA_INDEX_HEADS 32
#define DSA_INDEX_DIM 128
#define DSA_HEADS 64
#define DSA_QK_NOPE_DIM 192
#define DSA_QK_ROPE_DIM 64
#define DSA_V_DIM 256
#define DSA_LATENT_DIM 512
#define DSA_KV_ROW 576           /* 512 latent | 64 rope */
#define DSA_INDEX_TOPK 2048      /* index_topk of the page-4 table */
#define DSA_MAX_TOPK 8192        /* largest k (page 4, §2.2 and §6.1, discuss index_topk 4096 and 8192) */

typedef uint16_t dsa_bf16;       /* raw bf16 bits */

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,         /* a required pointer is NULL */
  DSA_ERR_SHAPE = 2,        /* a size is out of range (counts, k, ld_scores, max_ctx) */
  DSA_ERR_ALIGN = 3,        /* a pointer or leading dimension is misaligned */
  DSA_ERR_WORKSPACE = 4,    /* workspace too small (see dsa_workspace_bytes) */
  DSA_ERR_UNSUPPORTED = 5,  /* an option value this build does not implement */
  DSA_ERR_LAUNCH = 6,       /* a kernel launch failed (dsa_last_hip_error) */
  DSA_ERR_DEVICE = 7,       /* the current HIP device is missing or is not gfx950 */
  DSA_ERR_DEVICE_ARGS = 8   /* DSA_CHECK_DEVICE_ARGS=1 found a device-side precondition violated
                               (see dsa_last_device_arg_flags); nothing of the op was enqueued */
} dsa_status;

/* Bits of a device-side argument check (dsa_check_device_args,
 * dsa_last_device_arg_flags). */
#define DSA_ARG_Q_SEQ 1u       /* some q_seq[t] outside [0, num_seqs) */
#define DSA_ARG_Q_POS 2u       /* some q_pos[t] outside [0, max_ctx) */
#define DSA_ARG_CACHE_ROW 4u   /* a visible position maps outside the caches: seq_row0[b] < 0 or
                                  seq_row0[b] + q_pos[t] >= cache_rows (contiguous), or a block_table
                                  entry of pages 0 .. q_pos[t]/page_size outside the pool (paged) */
#define DSA_ARG_IDX 8u         /* an idx entry that is neither -1 nor in [0, q_pos[t]] */

/* Output element type of the attention output. */
enum { DSA_OUT_BF16 = 0, DSA_OUT_F32 = 1 };

/* Latent-cache row formats (dsa_batch.kv_format).
 *   DSA_KV_BF16: 576 bf16 (512 latent | 64 rope), 1152 bytes.
 *   DSA_KV_INT4: 400 bytes (page 3, "GLM-5 7440亿参数，202K长上下文突破极限", section 六:
 *     INT4 KV-cache quantisation): bytes 0..255 the 512 latent values as 4-bit
 *     two's complement codes (element 2i in the low nibble of byte i); bytes
 *     256..271 eight bf16 scales, scale g for elements 64g .. 64g+63; bytes
 *     272..399 the 64 rope values in bf16.  Latent value = code * scale.
 *     dsa_quantize_kv_int4 writes this format. */
enum { DSA_KV_BF16 = 0, DSA_KV_INT4 = 1 };
#define DSA_KV_INT4_ROW_BYTES 400

/* Operation ids for dsa_workspace_bytes. */
enum { DSA_OP_INDEX_SCORES = 0, DSA_OP_TOPK = 1, DSA_OP_SPARSE_MLA = 2, DSA_OP_FORWARD = 3 };

/* Batch geometry and cache layout.  The struct itself is HOST memory, read
 * during the call. */
typedef struct dsa_batch {
  int32_t num_queries;       /* T >= 0 */
  int32_t num_seqs;          /* B >= 1 */
  int32_t max_ctx;           /* >= max_t(q_pos[t]) + 1, 1 .. 2^21: bounds grids and score rows */
  int32_t page_size;         /* 0: contiguous caches (seq_row0); else tokens per cache page,
                                a power of two, 16 .. 2^20 (block_table) */
  const int32_t* q_seq;      /* [T] device: sequence of each query */
  const int32_t* q_pos;      /* [T] device: position of each query (inclusive causal limit) */
  const int64_t* seq_row0;   /* contiguous: [B] device, first cache row of each sequence;
                                ignored when paged */
  const int32_t* block_table;/* paged: [B, max_pages] device, the page holding tokens
                                [j*page_size, (j+1)*page_size) of sequence b at [b*max_pages + j];
                                ignored when contiguous */
  int32_t max_pages;         /* paged: >= ceil(max_ctx / page_size); ignored when contiguous */
  int32_t kv_format;         /* DSA_KV_BF16 or DSA_KV_INT4: row format of kv (the indexer keys are bf16) */
} dsa_batch;

/*
 * Indexer scores (page-4 §2.2 "Lightning Indexer"; page-5 indexer section).
 * For each query t and s = 0..q_pos[t]:
 *   scores[t*ld_scores + s] = sum_{h<32} w[t,h] * max(0, sum_{d<128} q_idx[t,h,d] * k_idx[row(s),d])
 * in fp32 (bf16 products, fp32 accumulation).  Entries beyond q_pos[t] are
 * not written.
 *   q_idx [T,32,128] bf16, w [T,32] bf16, k_idx [rows,128] bf16,
 *   scores [T, ld_scores] fp32 with ld_scores >= max_ctx and ld_scores % 4 == 0.
 * Batches averaging >= 8 queries per sequence run as a tiled MFMA GEMM over
 * blocks of consecutive queries, others as a per-query key scan; both give
 * the same values.
 */
dsa_status dsa_index_scores(const dsa_batch* batch, const dsa_bf16* q_idx, const dsa_bf16* w,
                            const dsa_bf16* k_idx, float* scores, int64_t ld_scores,
                            void* stream);

/*
 * Top-k selector (page-4 §2.2 "Top-k Selector"; page-5: index_topk = 2048).
 * For each query t over scores[t, 0..q_pos[t]]: keeps the min(q_pos[t]+1, k)
 * largest under the total order (fp32 value descending, -0.0 == +0.0, then
 * position ascending) and writes them to idx[t*k .. t*k+k) in ascending
 * position order, padded with -1.  Bit-exact: equal inputs give equal outputs.
 * NaN scores are unsupported (unspecified result).
 *   scores [T, ld_scores] fp32 (as above), 1 <= k <= DSA_MAX_TOPK, idx [T,k] int32.
 *   Any k in range is a runtime choice (DSA_INDEX_TOPK is the tables' value);
 *   k above 2048 runs one row workgroup per CU instead of two.
 *   ws: NULL, or at least dsa_workspace_bytes(DSA_OP_TOPK, T, max_ctx, k) bytes
 *   (DSA_ERR_WORKSPACE otherwise).  Batches of few rows split each row over
 *   many workgroups when a workspace is given; with NULL every row runs on one
 *   workgroup.  Both give identical results.
 */
dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse MLA attention over the kept positions (page-5 DSA flow: full
 * Q.K.V over the kept tokens, softmax, weighted sum; page-4 §2.1 dims).
 * For query t and head h, over the entries j of idx[t, 0..k) that are >= 0:
 *   z_j  = softmax_scale * (q_nope[t,h] . (c_j W_UK[h]) + q_rope[t,h] . r_j)
 *   out[t,h] = sum_j softmax(z)_j * (c_j W_UV[h])
 * where c_j / r_j are the latent and rope parts of cache row seq_row0[b] + idx.
 * Computed in weight-absorbed form: q_lat = W_UK[h] q_nope (rounded to bf16),
 * logits against the latent, online softmax in fp32, the latent-weighted sum
 * (rounded to bf16) up-projected by W_UV[h]; fp32 accumulation throughout.
 * Batches of few queries split each query's kept positions over several
 * workgroups: each split's normalised weighted sum is then also held in bf16
 * (the latent's own type and range) before the splits are merged in fp32.
 *   q_nope [T,64,192], q_rope [T,64,64], w_uk [64,512,192], w_uv [64,512,256]:
 *   bf16.  kv: [rows,576] bf16, or [rows,400] bytes when batch->kv_format is
 *   DSA_KV_INT4 (the latent is then dequantised, code * scale, and rounded to
 *   bf16 as it is gathered).  idx [T,k] int32 (-1 = absent; any order).
 *   out [T,64,256]: bf16 (out_dtype DSA_OUT_BF16) or fp32 (DSA_OUT_F32).
 *   A query with no valid entry gets a zero output.
 *   ws: dsa_workspace_bytes(DSA_OP_SPARSE_MLA, T, max_ctx, k) bytes.
 */
dsa_status dsa_sparse_mla_attn(const dsa_batch* batch, const dsa_bf16* q_nope,
                               const dsa_bf16* q_rope, const void* kv,
                               const dsa_bf16* w_uk, const dsa_bf16* w_uv, const int32_t* idx,
                               int32_t k, float softmax_scale, void* out, int32_t out_dtype,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * The whole path (page-5 DSA flow): dsa_index_scores -> dsa_topk ->
 * dsa_sparse_mla_attn on one stream, in query chunks sized to the workspace.
 * Same inputs and outputs as the three calls.  idx_out [T,k] receives the
 * selection when not NULL (e.g. for reuse by later layers).
 *   ws: at least dsa_workspace_bytes(DSA_OP_FORWARD, 1, max_ctx, k) bytes;
 *   dsa_workspace_bytes(DSA_OP_FORWARD, T, max_ctx, k) runs T queries per chunk.
 */
dsa_status dsa_forward(const dsa_batch* batch, const dsa_bf16* q_idx, const dsa_bf16* w,
                       const dsa_bf16* k_idx, const dsa_bf16* q_nope, const dsa_bf16* q_rope,
                       const void* kv, const dsa_bf16* w_uk, const dsa_bf16* w_uv,
                       int32_t k, float softmax_scale, void* out, int32_t out_dtype,
                       int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same path and results, with no workspace argument.  Its workspace is a
 * static device array of DSA_NOALLOC_SCRATCH_BYTES (64 MiB) per device, held
 * from the first call on that device until the process ends; batches whose
 * workspace (dsa_workspace_bytes(DSA_OP_FORWARD, T, max_ctx, k)) exceeds it run
 * in query chunks that fit, as dsa_forward does with a small workspace.  The
 * call allocates and frees nothing.
 *   Every call on one device shares that device's array: calls that overlap on
 *   one device (several host threads, or several streams with work in flight at
 *   once) race and give undefined results; serialise them (one stream, or
 *   stream order).  Nothing in the array needs clearing between calls (every
 *   byte a call reads it has written first).
 *   Errors: as dsa_forward; DSA_ERR_WORKSPACE if one query's workspace exceeds
 *   the array (not reached for any valid max_ctx and k); DSA_ERR_DEVICE if the
 *   array's device address cannot be obtained.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)
dsa_status dsa_forward_noalloc(const dsa_batch* batch, const dsa_bf16* q_idx, const dsa_bf16* w,
                               const dsa_bf16* k_idx, const dsa_bf16* q_nope, const dsa_bf16* q_rope,
                               const void* kv, const dsa_bf16* w_uk, const dsa_bf16* w_uv,
                               int32_t k, float softmax_scale, void* out, int32_t out_dtype,
                               int32_t* idx_out, void* stream);

/*
 * INT4 latent cache (page 3, section 六; format at DSA_KV_INT4): quantises
 * `rows` bf16 cache rows kv [rows,576] into kv_int4 [rows,400] bytes.  Per
 * group of 64 latent values: scale = bf16(absmax / 7) and code =
 * clamp(rint(x / scale), -7, 7), both divisions correctly rounded in fp32,
 * ties to even (scale 0 gives code 0); rope copied.  Bit-exact.  Both arrays
 * device, 16-byte aligned, not overlapping; rows 0 .. 2^40 (0: nothing
 * enqueued; any count runs, the kernel strides over the rows).  Errors: DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_ALIGN, DSA_ERR_DEVICE,
 * DSA_ERR_LAUNCH.
 */
dsa_status dsa_quantize_kv_int4(const dsa_bf16* kv, int64_t rows, uint8_t* kv_int4, void* stream);

/*
 * IndexShare layer schedule (page 5, IndexShare section and the config fields
 * it lists: index_topk_freq 4, 78 layers of which the first 3 are dense, 21
 * layers with their own indexer and 57 that reuse one).  Host-only; writes
 * source[l] for l < num_layers (HOST array):
 *   source[l] == l  -> layer l runs its own indexer + top-k ("full": dsa_forward
 *                      with idx_out),
 *   source[l] <  l  -> layer l reuses the selection of full layer source[l]
 *                      ("shared": dsa_sparse_mla_attn on its own cache and
 *                      weights with that layer's idx).
 * Layers 0 .. num_dense-1 are full; the sparse layers after them form runs of
 * index_topk_freq consecutive layers whose last layer is full, and a shared
 * layer reuses the nearest full layer before it (a layer can only reuse a
 * selection that was computed earlier in the forward pass).  With
 * (78, 3, 4): full layers 0,1,2,6,10,...,74 (21), shared 3-5,7-9,...,75-77
 * (57).  index_topk_freq == 1 makes every layer full (DSA without sharing).
 * Errors: DSA_ERR_NULL (source NULL), DSA_ERR_SHAPE (num_layers < 1,
 * num_dense < 1 or > num_layers, index_topk_freq < 1).  Nothing is written on
 * error.
 */
dsa_status dsa_index_share_schedule(int32_t num_layers, int32_t num_dense, int32_t index_topk_freq,
                                    int32_t* source);

/*
 * Device-side argument check (the device-only preconditions listed at the top:
 * the selector keeps positions of the query's own history, page 4 §2.2).
 * Enqueues kernels on `stream` that set *flags (a device word, 4-byte aligned;
 * cleared first) to the DSA_ARG_* bits of every violated precondition, 0 when
 * all hold.  Reads only q_seq, q_pos, seq_row0 / block_table and idx, never the
 * caches.  idx [T,k] may be NULL (not checked; k is then ignored);
 * cache_rows > 0 bounds the rows of the caches (k_idx and kv; in pages of
 * page_size rows when paged), 0 leaves the upper row bound unchecked.
 * Errors: DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_ALIGN, DSA_ERR_DEVICE,
 * DSA_ERR_LAUNCH (host checks as for the ops).
 *
 * Debug mode: with the environment variable DSA_CHECK_DEVICE_ARGS=1 at the
 * time of a call, dsa_index_scores, dsa_topk, dsa_sparse_mla_attn, dsa_forward
 * and dsa_forward_noalloc first run this check (idx for dsa_sparse_mla_attn;
 * cache rows unchecked) into a word of the library, wait for `stream`, and return
 * DSA_ERR_DEVICE_ARGS, with nothing of the op enqueued, when any bit is set.
 * The wait makes such calls blocking (not usable under graph capture).
 */
dsa_status dsa_check_device_args(const dsa_batch* batch, const int32_t* idx, int32_t k, int64_t cache_rows,
                                 uint32_t* flags, void* stream);

/* DSA_ARG_* bits found by the debug-mode check of the last call on this thread
 * that returned DSA_ERR_DEVICE_ARGS (0 = none). */
uint32_t dsa_last_device_arg_flags(void);

/* Workspace bytes an op needs for num_queries queries (host only; 0 = none).
 * Returns 0 as well for invalid arguments (then the op itself reports them). */
size_t dsa_workspace_bytes(int32_t op, int32_t num_queries, int32_t max_ctx, int32_t k);

/* Static description of a status code (never NULL). */
const char* dsa_status_string(int32_t status);

/* DSA_ABI_VERSION of the built library. */
int32_t dsa_abi_version(void);

/* hipError_t of the last DSA_ERR_LAUNCH / DSA_ERR_DEVICE on this thread (0 = none). */
int32_t dsa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
