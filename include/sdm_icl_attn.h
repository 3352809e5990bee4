/*
 * sdm_icl_attn.h -- C ABI of the MI355X (gfx950) row-wise in-context-learning
 * (ICL) attention engine of tabular foundation models.
 *
 * What it computes
 * ----------------
 * Context rows are tokens that attend to one another without a causal mask;
 * query rows attend to the context keys/values only, either in the same call
 * or later from a cached K/V ("[FP8 3/4] Integrate FP8 attention and caching
 * into TabICLv2": model(context, labels, queries), model.fit(context, labels)
 * then model.predict(queries); walkthrough: Q/K/V come from one shared
 * projection and attention is scaled dot-product attention).  For a query
 * row i:
 *
 *     O_i = sum_{j < n} softmax_j( (q~_i . k_j) / sqrt(D) ) v_j
 *
 * where n is the number of valid (unmasked) context rows and q~ is the query
 * after the optional shared-length scaling ("Fuse shared-length query scaling
 * during inference", Problem identified / Solution):
 *
 *     NONE       q~ = q
 *     LOG        q~ = fp16(q * k_h)          k_h = fp16(fp32(L32 * c_h))
 *     GATED_LOG  q~ = fp16(fp16(q * k_h) * fp16(1 + fp16(tanh g)))
 *     L32 = fp32(ln(max(n, 1)))   (float32 length arithmetic, clamped log)
 *
 * With FP8 precision ("[FP8 3/4] ...", introduction) Q~, K and V are
 * quantised to OCP e4m3 with per-(batch, head) scales taken over the valid
 * context rows: s = amax/448, inv = 448/amax (amax = 0 gives 1), codes =
 * e4m3_rne(clamp(fp32(x * inv), -448, 448)), dequantised as code * s.  Q's
 * scale comes from the *scaled context* queries and query rows reuse it (and
 * saturate above it), so a row's result does not depend on how the queries
 * are split into batches.  Softmax and accumulation are fp32; outputs are
 * fp16.
 *
 * Conventions (all entry points)
 * ------------------------------
 * - Pointers named "device" are HIP device memory on the stream's device and
 *   stay owned by the caller; "host" pointers are read during the call only.
 * - Device fp16 row tensors (q, k, v, outputs) and the query workspace must be
 *   16-byte aligned (the kernels move them 16 bytes at a time), gates 2-byte
 *   and float arrays 4-byte aligned; a misaligned pointer is
 *   SDM_ICL_E_INVALID, found before anything touches the device.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   All device work is enqueued on it; no entry point synchronises the host
 *   unless stated (cache_export does).
 * - Every argument is validated on the host before anything is launched; a
 *   non-OK status leaves outputs untouched and sdm_icl_last_error() holds a
 *   message for the calling thread.  Errors of already-launched kernels show
 *   up as SDM_ICL_E_HIP from a later call or at the caller's next sync.
 * - head_dim must be 64 (the ICL width of the models on the pages is 8 x 64);
 *   other values return SDM_ICL_E_UNSUPPORTED.
 * - Only gfx950 devices are supported (SDM_ICL_E_DEVICE otherwise).
 */
#ifndef SDM_ICL_ATTN_H
#define SDM_ICL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sdm_icl_status;
#define SDM_ICL_OK            0
#define SDM_ICL_E_INVALID     1  /* bad argument: null pointer, size, mode/gate mismatch */
#define SDM_ICL_E_UNSUPPORTED 2  /* valid but not implemented (head_dim != 64, > 128 heads) */
#define SDM_ICL_E_DEVICE      3  /* pointer not on the stream's device, or not a gfx950 device */
#define SDM_ICL_E_OOM         4  /* device allocation failed */
#define SDM_ICL_E_HIP         5  /* a HIP runtime call failed */
#define SDM_ICL_E_STATE       6  /* released or unknown cache handle; workspace too small */

#define SDM_ICL_SCALE_NONE      0
#define SDM_ICL_SCALE_LOG       1
#define SDM_ICL_SCALE_GATED_LOG 2

#define SDM_ICL_PREC_FP16     0
#define SDM_ICL_PREC_FP8_E4M3 1
#define SDM_ICL_PREC_AUTO     2  /* FP8 iff n > 8192 valid context rows ("[FP8 3/4] ...", intro) */
#define SDM_ICL_PREC_SCOPED   3  /* an intermediate ICL layer under the opt-in FP8 scope: FP8 iff
                                    the calling thread's scope enables FP8 and n > 8192, else
                                    FP16 (see sdm_icl_scope_push); a final layer asks for FP16 */

/* Settings of an FP8 scope ("[FP8 3/4] ...", introduction and API example:
 * sdm.optimize(attention="fp8") is an opt-in scope that enables, disables or
 * inherits FP8 attention; using an FP8 cache outside the enabled scope is an
 * error and re-entering permits reuse; leaving a scope restores the previous
 * setting without touching caches). */
#define SDM_ICL_SCOPE_DISABLE 0
#define SDM_ICL_SCOPE_ENABLE  1
#define SDM_ICL_SCOPE_INHERIT 2

/* Opaque, library-owned, immutable after fit.  Holds n, the scaling factors,
 * the per-head FP8 scales and the K/V operands in a head-major layout. */
typedef struct sdm_icl_cache_s* sdm_icl_cache;

typedef struct {
  int32_t batch;           /* B >= 1 */
  int32_t rows_padded;     /* N_pad >= 1: allocated context rows per batch element */
  int32_t heads;           /* H, 1..128 */
  int32_t head_dim;        /* D, must be 64 */
  const int64_t* lengths;  /* host [B]: valid rows n_b, 1 <= n_b <= N_pad, one per batch
                              element (equal values = one shared length, the case the
                              pages' fused scaling covers; differing values make each
                              element behave as a batch of one with its own n_b, L32(n_b)
                              and k_h).  Rows n_b..N_pad-1 of element b are masked: not
                              keys, not in n_b, not in any amax, their outputs are 0 and
                              their contents are never read.  AUTO precision follows the
                              longest context, max n_b. */
  const void* q;           /* device fp16 [B, N_pad, H, D], row-major, row stride H*D */
  const void* k;           /* device fp16 [B, N_pad, H, D] */
  const void* v;           /* device fp16 [B, N_pad, H, D] */
  const void* gate;        /* device fp16 [B, N_pad, H]; non-NULL iff scale_mode == GATED_LOG */
  const float* head_coef;  /* host float32 [H] (c_h); non-NULL iff scale_mode != NONE */
  int32_t scale_mode;      /* SDM_ICL_SCALE_* */
  int32_t precision;       /* SDM_ICL_PREC_* */
  void* out_ctx;           /* device fp16 [B, N_pad, H, D] context self-attention output,
                              or NULL to only build the cache (model.fit) */
  void* stream;            /* hipStream_t */
} sdm_icl_fit_args;

typedef struct {
  int32_t batch, heads, head_dim;
  int32_t precision;       /* resolved: FP16 or FP8_E4M3, never AUTO */
  int32_t scale_mode;
  int32_t kv_splits;       /* KV-axis split count used by every query call (fixed at fit) */
  int64_t n_valid;         /* n (per-batch lengths: the longest, max n_b) */
  int64_t rows_alloc;      /* cache rows per (b, h): n_valid rounded up to the 64-row key tile */
  int64_t keys_per_split;  /* rows of each KV split (multiple of 64) */
  float length_scalar;     /* L32 (per-batch lengths: that of batch element 0) */
  uint64_t device_bytes;   /* bytes of device memory the cache holds */
  int32_t offloaded;       /* 1 while K/V live in pinned host memory (cache_offload) */
  int32_t stream_chunk_splits; /* splits per streamed chunk while offloaded, else 0 */
} sdm_icl_cache_info;

/* Build the K/V cache from the context (model.fit) and, if out_ctx != NULL,
 * also compute the context rows' self-attention (the context half of one
 * model call).  Allocates the cache with stream-ordered allocation on
 * args->stream; *out receives the handle only on SDM_ICL_OK.  Temporary
 * buffers of the call are freed stream-ordered before it returns. */
sdm_icl_status sdm_icl_attn_fit(const sdm_icl_fit_args* args, sdm_icl_cache* out);

/* Device workspace (bytes) that sdm_icl_attn_query needs for n_query rows:
 * the scaled (and quantised) query operand and, per KV split, (m, l) in fp32
 * and the split's normalised output row O / l in fp16.  The caller owns the
 * workspace, so the query itself allocates nothing (the caller-owned-buffer
 * rule of "... make trtllm::kda_decode inplace-only", walkthrough; the cached
 * predict of "[FP8 3/4] ...", introduction). */
sdm_icl_status sdm_icl_attn_query_workspace_size(sdm_icl_cache cache, int64_t n_query,
                                                 size_t* bytes);

/* Query rows attend to the cached context (model.predict); the rows of batch
 * element b attend to its n_b cached keys, scaled with its L32(n_b).  q: device fp16
 * [B, R, H, D]; gate: device fp16 [B, R, H], non-NULL iff the cache was fitted
 * with GATED_LOG (otherwise SDM_ICL_E_INVALID, the analogue of misusing an FP8
 * cache outside its scope); out: device fp16 [B, R, H, D].  workspace: caller
 * device memory of at least query_workspace_size(R) bytes.  Allocates nothing
 * and never synchronises.  The result of a row is bitwise independent of R
 * and of the other rows in the call (fixed KV split plan, fixed combine
 * order, context-derived Q scale).  R == 0 is a no-op.  Concurrent calls on
 * one cache with distinct workspaces are safe.  On a resident (not
 * offloaded) cache the call enqueues only kernel launches on `stream` (with
 * kernel timing off), so it can be captured into a graph and replayed; the
 * graph reads q, gate and the cache when it runs. */
sdm_icl_status sdm_icl_attn_query(sdm_icl_cache cache, const void* q, const void* gate,
                                  int64_t n_query, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* sdm_icl_attn_query for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, bit for bit, with the workspace
 * taken from a scratch array the library holds on each GPU (64 MiB per
 * device, SDM_ICL_NOALLOC_SCRATCH_BYTES, kept from the library's load until
 * the process ends).  The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine, no events (kernel timing is
 * skipped).  A query whose workspace (query_workspace_size) exceeds the
 * scratch array, e.g. 1,024 rows at 8 heads and 96 KV splits, returns
 * SDM_ICL_E_INVALID with the sizes in the message; an offloaded cache
 * returns SDM_ICL_E_UNSUPPORTED (its streamed chunks need staging space).
 * Every call on one GPU shares that GPU's array, so calls that overlap on
 * one GPU (on different streams, or from different threads without
 * ordering) race and may return wrong rows; calls ordered on one stream are
 * safe.  Nothing in the array needs clearing between calls: every byte a
 * call reads it wrote earlier in the same call.  Arguments and errors
 * otherwise as sdm_icl_attn_query. */
#define SDM_ICL_NOALLOC_SCRATCH_BYTES (64u << 20)
sdm_icl_status sdm_icl_attn_query_noalloc(sdm_icl_cache cache, const void* q, const void* gate,
                                          int64_t n_query, void* out, void* stream);

/* Shape, precision and split plan of a cache. */
sdm_icl_status sdm_icl_attn_cache_info(sdm_icl_cache cache, sdm_icl_cache_info* info);

/* Per-batch lengths n_b (host int64 [B]) and their length scalars L32(n_b)
 * (host float32 [B]) of a cache; either pointer may be NULL. */
sdm_icl_status sdm_icl_attn_cache_lengths(sdm_icl_cache cache, int64_t* host_lengths,
                                          float* host_length_scalars);

/* Copy the cached operands to host memory, so that a fitted cache can be
 * kept or moved to another device or process ("[FP8 3/4] ...", walkthrough:
 * the FP8 caches survive migration and chunking).
 * host_k / host_v: [B, H, n, D] elements with n = n_valid (rows n_b..n-1 of a
 * shorter batch element are 0), 1 byte (e4m3 code) in FP8 mode or
 * 2 bytes (fp16) in FP16 mode; host_scales: float32 [3, B, H] = s_q, s_k,
 * s_v, each fp32(amax/448) (all 1 in FP16 mode).  Any of the three may be
 * NULL.  Synchronises `stream`. */
sdm_icl_status sdm_icl_attn_cache_export(sdm_icl_cache cache, void* host_k, void* host_v,
                                         float* host_scales, void* stream);

typedef struct {
  int32_t batch;              /* B >= 1 */
  int32_t heads;              /* H, 1..128 */
  int32_t head_dim;           /* D, must be 64 */
  const int64_t* lengths;     /* host [B]: n_b >= 1 */
  int32_t scale_mode;         /* SDM_ICL_SCALE_* the cache was fitted with */
  int32_t precision;          /* FP16 or FP8_E4M3 (a resolved precision) */
  const float* head_coef;     /* host float32 [H] iff scale_mode != NONE */
  const void* host_k;         /* host [B, H, n, D], n = max n_b, as cache_export writes it:
                                 e4m3 codes (1 byte) or fp16; rows >= n_b are ignored */
  const void* host_v;         /* host [B, H, n, D], same element type */
  const float* host_scales;   /* host float32 [3, B, H]: s_q, s_k, s_v (all 1 for FP16) */
  void* stream;               /* hipStream_t */
} sdm_icl_import_args;

/* Rebuild a cache from what cache_export wrote (persistence, migration to
 * another device or process; the pages' FP8 caches are migrated and
 * preserved through chunking, "[FP8 3/4] ...", walkthrough).  FP8 codes and
 * scales are taken as they are; from each s = fp32(amax/448) the fp16 amax,
 * and with it the exact inverse scale, is recovered, so queries on the
 * imported cache reproduce those on the exported one bit for bit.  Scales
 * not of that form are SDM_ICL_E_INVALID, as are e4m3 NaN codes (0x7F,
 * 0xFF).  Allocates the cache on args->stream and synchronises that stream
 * before it returns. */
sdm_icl_status sdm_icl_attn_cache_import(const sdm_icl_import_args* args, sdm_icl_cache* out);

/* Host offload ("[FP8 3/4] ...", introduction: cache chunking and CPU
 * offloading are supported).  cache_offload moves the cache's K/V into pinned
 * host memory and keeps only scales, lengths and factors on the device;
 * cache_restore moves them back.  Both synchronise `stream` and are no-ops
 * when the cache is already in that state; no query may be in flight on the
 * cache meanwhile.  Queries on an offloaded cache stream K/V from host memory
 * in chunks of whole KV splits through two staging buffers in the caller's
 * workspace (query_workspace_size grows by 2 x 2 chunk buffers of K and V);
 * chunk_bytes bounds one chunk's K bytes (0: 64 MiB; at least one split),
 * copying on a stream the cache owns while the split kernel runs on
 * the caller's stream, then combine as usual: the results are bit-identical
 * to those of the resident cache.  Queries on one offloaded cache must not
 * overlap (the cache's copy stream and events are shared). */
sdm_icl_status sdm_icl_attn_cache_offload(sdm_icl_cache cache, size_t chunk_bytes, void* stream);
sdm_icl_status sdm_icl_attn_cache_restore(sdm_icl_cache cache, void* stream);

/* Free a cache (the end of a fitted cache's life: model.fit builds it,
 * model.predict reuses it, "[FP8 3/4] ...", introduction).  The memory is
 * returned stream-ordered on the stream the cache was fitted on; work on other streams that uses the cache must be complete
 * (or ordered before that stream) first.  A second release of the same handle
 * returns SDM_ICL_E_STATE. */
sdm_icl_status sdm_icl_attn_release(sdm_icl_cache cache);

/* The fused shared-length query scaling on its own ("Fuse shared-length query
 * scaling during inference", Solution: length preparation, per-head
 * conversion, query multiplication and optional gating in one kernel).
 * q: device fp16 [B, rows, H, D]; gate: device fp16 [B, rows, H] iff GATED_LOG;
 * key_length: the shared n (>= 0; the log is clamped at n <= 1);
 * head_coef: host float32 [H] unless NONE.  out: device, head-major
 * [B, H, rows, D]: fp16 when q_inv_scale is NULL, else e4m3 codes (1 byte)
 * of the scaled rows quantised with the device float32 inverse scales
 * q_inv_scale [B, H] (for a cache's queries, the Q inverse scales its fit
 * derived). */
sdm_icl_status sdm_icl_log_scale(const void* q, const void* gate, int32_t batch, int64_t rows,
                                 int32_t heads, int32_t head_dim, int64_t key_length,
                                 const float* head_coef, int32_t scale_mode,
                                 const float* q_inv_scale, void* out, void* stream);

/* The shared Q/K/V projection with the query scaling fused into its
 * epilogue ("[FP8 3/4] ...", walkthrough: Q/K/V come from one shared projection;
 * "Fuse shared-length query scaling during inference", Solution: the scaling
 * joins the producer of q instead of separate passes over it).
 *   x:    device fp16 [B, rows, in_features] hidden rows (in_features % 32 == 0)
 *   w:    device fp16 [3 * heads * head_dim, in_features]: a linear layer's
 *         [out, in] weight, rows producing Q, then K, then V
 *   bias: device fp16 [3 * heads * head_dim], or NULL
 *   q_out, k_out, v_out: device fp16 [B, rows, heads, head_dim] (row-major, the
 *         layout sdm_icl_attn_fit and sdm_icl_attn_query take)
 * Each output is x . w_n + b_n accumulated in float32 and rounded once to
 * fp16; q_out then takes scale_mode's scaling with key_length, head_coef and
 * gate ([B, rows, heads], GATED_LOG only) exactly as sdm_icl_log_scale would
 * apply it to the unscaled projection (bit for bit).  Rows projected this way
 * already carry the scaling: fit and query them with SDM_ICL_SCALE_NONE.
 * rows == 0 is a no-op.  Pointers as in the conventions above (x, w, outputs
 * 16-byte aligned, bias and gate 2-byte aligned). */
sdm_icl_status sdm_icl_qkv_project(const void* x, const void* w, const void* bias, int32_t batch,
                                   int64_t rows, int32_t in_features, int32_t heads, int32_t head_dim,
                                   int64_t key_length, const float* head_coef, int32_t scale_mode,
                                   const void* gate, void* q_out, void* k_out, void* v_out,
                                   void* stream);

/* ---- kernel timing (observability) -------------------------------------
 * When enabled, each kernel launch of the library is bracketed by two HIP
 * events recorded on the launch's own stream, grouped by kernel class:
 *   SDM_ICL_TIMING_CONTEXT  context self-attention (fit with out_ctx)
 *   SDM_ICL_TIMING_QUERY    cached-query split-KV attention
 *   SDM_ICL_TIMING_COMBINE  split combine
 *   SDM_ICL_TIMING_SCALE    fused q-scale (+quantise)
 *   SDM_ICL_TIMING_PREP     fit preparation (amax, scales, K/V pack)
 *   SDM_ICL_TIMING_PROJECT  Q/K/V projection (sdm_icl_qkv_project)
 * Off by default; enabling adds two event records per launch.
 * sdm_icl_timing_read waits for the recorded events of one class, returns
 * their summed duration in milliseconds and the launch count, and clears
 * that class. */
#define SDM_ICL_TIMING_CONTEXT 0
#define SDM_ICL_TIMING_QUERY   1
#define SDM_ICL_TIMING_COMBINE 2
#define SDM_ICL_TIMING_SCALE   3
#define SDM_ICL_TIMING_PREP    4
#define SDM_ICL_TIMING_PROJECT 5
sdm_icl_status sdm_icl_timing_enable(int32_t on);
sdm_icl_status sdm_icl_timing_read(int32_t kernel_class, double* total_ms, int64_t* launches);

/* ---- host-only helpers (no device work; usable without a GPU) ---------- */

/* L32 = fp32(ln(max(n, 1))). */
float sdm_icl_length_scalar(int64_t n);

/* k_h = fp16(fp32(L32(n) * c_h)) for h < heads, written as fp16 bit patterns. */
sdm_icl_status sdm_icl_head_factors(int64_t n, const float* head_coef, int32_t heads,
                                    uint16_t* out_fp16_bits);

/* Precision a fit with this n and request resolves to (AUTO: FP8 iff n > 8192). */
int32_t sdm_icl_select_precision(int64_t n, int32_t requested);

/* KV split plan for n valid keys and bh_count = batch * heads on a device with
 * num_cus compute units: about 3 * num_cus / bh_count splits of at least 4
 * key tiles each.  A pure function of (n, num_cus, bh_count), never of the
 * query count, so every query batch of a cache uses the same plan.  A cache
 * with per-batch lengths plans for the longest, max n_b; the splits past a
 * shorter element's n_b hold no keys of it and weigh 0 in its combine. */
sdm_icl_status sdm_icl_split_plan(int64_t n, int32_t num_cus, int32_t bh_count, int32_t* kv_splits,
                                  int64_t* keys_per_split);

/* Open a nested FP8 scope on the calling thread with one of the
 * SDM_ICL_SCOPE_* settings (INHERIT keeps the enclosing setting).  The
 * effective setting is that of the innermost scope that is not INHERIT,
 * disabled when there is none; a new thread starts with no scope.  It decides
 * SDM_ICL_PREC_SCOPED at fit, and a cache that resolved to FP8 that way can
 * only be queried or exported while the effective setting is ENABLE
 * (SDM_ICL_E_STATE otherwise); closing the scope changes no cache.  At most
 * 256 nested scopes (SDM_ICL_E_STATE beyond); an unknown setting is
 * SDM_ICL_E_INVALID. */
sdm_icl_status sdm_icl_scope_push(int32_t setting);

/* Close the innermost scope of the calling thread (SDM_ICL_E_STATE if none is
 * open). */
sdm_icl_status sdm_icl_scope_pop(void);

/* 1 if the calling thread's effective FP8 scope setting is ENABLE, else 0. */
int32_t sdm_icl_scope_fp8(void);

/* Message of the last non-OK status on this thread ("" if none): errors are
 * status codes, never exceptions across the boundary, like the RuntimeError
 * the pages raise for a misused FP8 cache ("[FP8 3/4] ...", walkthrough). */
const char* sdm_icl_last_error(void);

/* ABI version (major * 100 + minor): 102. */
int32_t sdm_icl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDM_ICL_ATTN_H */
