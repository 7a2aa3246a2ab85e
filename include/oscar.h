/*
 * oscar.h -- C ABI of the OSCAR 2-bit KV-cache hot path for MI355X (gfx950).
 *
 * OSCAR ("Offline Spectral Covariance-Aware Rotation", arXiv 2605.17757) stores
 * the history of the KV cache as per-token INT2 after a fixed, calibrated
 * rotation, and keeps sink and recent tokens in bf16.  Sources, cited by page
 * title and section:
 *   [IT] gist.science, Italian technical summary of arXiv 2605.17757, sections
 *        2.2.A (offline calibration) and 2.2.B (online serving).
 *   [ES] 7minutos.es article on OSCAR, sections "Lo que OSCAR hace diferente"
 *        (covariances, composite rotations, Lemma 1, bit reversal) and "El
 *        sistema de servicio: diseno de cache de precision mixta" (regions,
 *        write path, read path).
 *   [JA] gist.science, Japanese technical summary, sections 2.2.A and 2.2.B.
 *
 * Conventions
 *   - Every call returns oscar_status: OSCAR_OK (0) or a negative code.  No C++
 *     exception crosses this boundary.  oscar_last_error() returns a message for
 *     the last failing call on the calling thread.
 *   - "device" pointers are GPU memory owned by the caller; "host" pointers are
 *     CPU memory owned by the caller.  The library never allocates device memory.
 *   - Kernels are enqueued on the caller's HIP stream (hipStream_t passed as
 *     void*; NULL = the null stream) and run asynchronously.  A GPU fault shows
 *     up at the caller's next synchronisation.  Argument errors are detected on
 *     the host before anything is enqueued.
 *   - Row-vector convention: a head vector x (d channels) is rotated as
 *     x_rot = x R, with R stored row-major [d][d] in fp32.
 *   - A pool (oscar_pool) holds host bookkeeping only (free lists, reference
 *     counts, sequences); it is not thread-safe: callers serialise calls that
 *     take the same pool.  Launch functions keep no state and are reentrant.
 *   - Slots: a physical slot is page_id * page_size + slot_in_page (int32).
 *
 * Storage format of one (page, KV head) block, d channels, G channels per
 * group, NG = d / G, page_size = 16 tokens:
 *   INT2 block (2*(4*d + 64*NG) bytes: 1536 for d=128,G=32; 1280 for G=64):
 *     K codes  [16][d/4] bytes, token-major; byte b of token t is t*d/4 + b,
 *              and holds four 2-bit fields, field m at bits 2*m.  G = 64:
 *              field m of byte b is channel 4*b + m.  G = 32: byte
 *              b = 8*a + 4*w + i holds at field m the channel
 *              64*w + 32*(m/2) + 8*a + 4*(m%2) + i (every field position of
 *              the 4-byte word w of quarter a belongs to one group).
 *     K scale/zero  fp16 [16][NG][2] = (s, z) per token and group (token-major).
 *     V codes  [4][d] bytes by token quad: byte q*d + j holds channel j of
 *              tokens 4q..4q+3, token 4q+i at bits 2*i.
 *     V scale/zero  fp16 [NG][16][2] = (s, z) per group and token (group-major).
 *   BF16 block (4*16*d bytes): K as bf16 [16][d] (token-major), then V as
 *   bf16 [d][16] (channel-major).
 *   A layer's INT2 storage is [n_int2_pages][n_kv_heads][INT2 block]; its bf16
 *   storage is [n_bf16_pages][n_kv_heads][BF16 block].
 *
 * Regions of a request of length T ([ES] serving section; [IT] 2.2.B):
 *   positions [0, sink) are bf16 "sink" tokens, the last `recent` positions are
 *   bf16 "recent" tokens, everything between is INT2 history.  INT2 position p
 *   lives in INT2 logical page p/16, slot p%16.  Sink position p lives in bf16
 *   logical page p/16; recent position p lives in a ring of `recent` slots
 *   after the sink pages: bf16 logical slot 16*ceil(sink/16) + (p-sink)%recent.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t oscar_status;
#define OSCAR_OK 0
#define OSCAR_EINVAL (-1)        /* bad argument (null pointer, size, alignment, range) */
#define OSCAR_ENOMEM (-2)        /* a pool ran out of pages (host bookkeeping only) */
#define OSCAR_EHIP (-3)          /* the HIP runtime reported an error at launch */
#define OSCAR_EUNSUPPORTED (-4)  /* shape outside what the kernels are built for */

/* Shape of one attention layer and of the cache layout.
 * Supported: head_dim 128, page_size 16, group 32 or 64, n_q_heads a multiple
 * of n_kv_heads with n_q_heads / n_kv_heads * (head_dim / group) <= 64,
 * sink >= 0, recent >= 0 (recent a multiple of page_size or 0). */
typedef struct oscar_shape {
  int32_t head_dim;    /* d */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t group;       /* G: channels per quantisation group ([ES] write path; default there 64) */
  int32_t sink;        /* S0 ([ES] serving section; 64 there) */
  int32_t recent;      /* W  ([ES] serving section; 256 there) */
  int32_t page_size;   /* tokens per page */
  int32_t scale_bits;  /* storage of each group's scale and zero: 16 (or 0) two fp16; 8 two FP8 E4M3,
                          the lower-metadata format (G = 64 gives 2.25 history bits per element:
                          [ES] accuracy section, 2.28 / 2.38 bits per element) */
} oscar_shape;

/* Calibration state of one layer ([IT] 2.2.A: fixed rotations and clip
 * thresholds).  r_k / r_v: device fp32 [n_kv_heads][d][d], 16-byte aligned.
 * r_v may be NULL when R_V is folded into the model's weights ([ES] serving
 * section: the value rotation is absorbed offline into the projections): the
 * V vectors given to the write calls are then already rotated (W_V R_V), the
 * cache stores them as given (bf16 region) or quantises them unrotated (INT2
 * history), and the attention output stays in the rotated basis, for an
 * output projection R_V^T W_O.  This is the same as passing R_V = I, minus
 * the identity products.  r_k is required. */
typedef struct oscar_layer {
  const float* r_k;
  const float* r_v;
  float tau_k;         /* clip threshold for rotated keys (x_rot clamped to [-tau, tau]) */
  float tau_v;         /* Both finite and >= 0, and at most 65504 with fp16 scale and
                          zero (so that neither can overflow); calls taking a layer
                          return OSCAR_EINVAL otherwise. */
  const void* r_prep;  /* NULL, or device memory written by oscar_layer_prepare for
                          this r_k / r_v (256-byte aligned): the write calls then
                          load R's integer digits instead of deriving them in every
                          work group.  Prepare again after changing r_k or r_v. */
} oscar_layer;

/* Device storage of one layer (caller-owned; 256-byte aligned). */
typedef struct oscar_cache {
  void* int2_pages;
  int64_t n_int2_pages;
  void* bf16_pages;
  int64_t n_bf16_pages;
} oscar_cache;

typedef struct oscar_pool oscar_pool;
typedef struct oscar_seq oscar_seq;

const char* oscar_last_error(void);

/* Bytes of one (page, KV head) block. */
int64_t oscar_int2_block_bytes(const oscar_shape* shape);
int64_t oscar_bf16_block_bytes(const oscar_shape* shape);

/* ---- Offline calibration ([IT] 2.2.A; [ES] "Lo que OSCAR hace diferente") ----
 * Inputs (host, fp32): q [n][n_q_heads][d], k and v [n][n_kv_heads][d]: one
 * calibration sequence of n tokens.  For each KV head (its g = Hq/Hkv query
 * heads pooled): C_Q = sum q^T q / (n g); C_S = sum_h V^T S_h^T S_h V / (n g)
 * with S_h the causal softmax(Q_h K^T / sqrt(d)); eigenbases sorted by
 * decreasing eigenvalue, each eigenvector signed so its largest-magnitude entry
 * is positive; R_K = U_Q H P_br, R_V = U_S H P_br (H: orthonormal Sylvester
 * Walsh-Hadamard in natural order; P_br: bit-reversal permutation).  tau_k and
 * tau_v: the clip_pct_k / clip_pct_v quantile (linear interpolation) of
 * |x R| over all calibration tokens, KV heads and channels, using the fp32 R.
 * Computed in fp64 on the host; outputs (host): r_k_out, r_v_out fp32
 * [n_kv][d][d]; eig_k_out, eig_v_out fp64 [n_kv][d] (may be NULL); tau outputs.
 * Errors: OSCAR_EINVAL for null pointers, n < 1, bad shape or a quantile
 * outside (0, 1]. */
oscar_status oscar_calibrate_host(const oscar_shape* shape, int64_t n, const float* q, const float* k,
                                  const float* v, double clip_pct_k, double clip_pct_v, float* r_k_out,
                                  float* r_v_out, double* eig_k_out, double* eig_v_out, float* tau_k_out,
                                  float* tau_v_out);

/* The same calibration with the rotation chosen ([ES] the accuracy paragraph
 * and the paragraph before "Lo que OSCAR hace diferente"; [IT] 4: the pages'
 * baselines): OSCAR_ROTATION_OSCAR is oscar_calibrate_host;
 * OSCAR_ROTATION_IDENTITY is naive INT2, R = I; OSCAR_ROTATION_HADAMARD is the
 * data-oblivious Hadamard rotation R = H P_br (the composite with U = I).  The
 * two baselines do not read the covariances (eig outputs, when given, are set
 * to NaN); tau is the same quantile, taken under the chosen R.  The write and
 * read kernels take any of them unchanged.  Errors: as oscar_calibrate_host,
 * and OSCAR_EINVAL for an unknown rotation. */
#define OSCAR_ROTATION_OSCAR 0
#define OSCAR_ROTATION_IDENTITY 1
#define OSCAR_ROTATION_HADAMARD 2
oscar_status oscar_calibrate_host_rotation(const oscar_shape* shape, int32_t rotation, int64_t n, const float* q,
                                           const float* k, const float* v, double clip_pct_k, double clip_pct_v,
                                           float* r_k_out, float* r_v_out, double* eig_k_out, double* eig_v_out,
                                           float* tau_k_out, float* tau_v_out);

/* ---- Page pools and sequences (host bookkeeping; [IT] 2.2.B paged cache with
 * prefix caching; [ES] serving section) ---- */
oscar_status oscar_pool_create(const oscar_shape* shape, int64_t n_int2_pages, int64_t n_bf16_pages,
                               oscar_pool** out);
oscar_status oscar_pool_destroy(oscar_pool* pool);
/* Free pages left in each pool (either pointer may be NULL). */
oscar_status oscar_pool_free_pages(const oscar_pool* pool, int64_t* int2_free, int64_t* bf16_free);

oscar_status oscar_seq_create(oscar_pool* pool, oscar_seq** out);
/* Drops the sequence's page references; pages whose count reaches zero return
 * to the free lists. */
oscar_status oscar_seq_release(oscar_pool* pool, oscar_seq* seq);
int64_t oscar_seq_length(const oscar_seq* seq);

/* Plan the growth of `seq` by n_new tokens (positions T .. T+n_new-1), allocating
 * pages as needed.  Outputs (host arrays):
 *   int2_slots[n_new]  physical INT2 slot of each new token that goes straight to
 *                      the INT2 history, else -1;
 *   bf16_slots[n_new]  physical bf16 slot of each new sink/recent token, else -1;
 *   age_src[], age_dst[] (capacity n_new + recent): tokens that leave the recent
 *                      window: physical bf16 slot -> physical INT2 slot; *n_age
 *                      receives their count.
 * Execution order on the device: oscar_requant_from_bf16 (age-out) first, then
 * oscar_quant_write and oscar_bf16_write for the new tokens (a new recent token
 * may reuse the ring slot of a token that ages out).  On OSCAR_ENOMEM nothing is
 * changed. */
oscar_status oscar_seq_plan_append(oscar_pool* pool, oscar_seq* seq, int64_t n_new, int32_t* int2_slots,
                                   int32_t* bf16_slots, int32_t* age_src, int32_t* age_dst, int64_t* n_age);

/* New sequence equal to `parent` as it stands (prefix caching).  Sink pages and
 * full INT2 pages are shared by reference count; pages the child will write into
 * (the partly filled last INT2 page and the recent ring) are fresh copies.  The
 * caller must run the copies with oscar_copy_pages before writing to either
 * sequence: copy_src/copy_dst (host, capacity 64 + recent/16 each) receive
 * physical page ids and copy_kind 0 (INT2) or 1 (bf16); *n_copies their count. */
oscar_status oscar_seq_fork(oscar_pool* pool, const oscar_seq* parent, oscar_seq** child, int32_t* copy_src,
                            int32_t* copy_dst, int32_t* copy_kind, int64_t* n_copies);

/* Block tables for a batch (host outputs): int2_bt [n][max_int2_pages] and
 * bf16_bt [n][max_bf16_pages] physical page ids (-1 past the end), ctx_lens[n].
 * Errors: OSCAR_EINVAL if a sequence needs more pages than the row width. */
oscar_status oscar_block_tables(const oscar_pool* pool, const oscar_seq* const* seqs, int32_t n,
                                int32_t* int2_bt, int32_t max_int2_pages, int32_t* bf16_bt,
                                int32_t max_bf16_pages, int32_t* ctx_lens);

/* ---- Write path ([ES] serving section, write path; [IT] 2.2.B) ----
 * For each token i < n with int2_slots[i] >= 0 and each KV head h:
 *   x_rot = x R (fp64 accumulation of the exact bf16 x fp32 products);
 *   clamp to [-tau, tau]; per group of G channels: mn, mx,
 *   s = fp16((mx-mn)/3), z = fp16(mn) (fp64 arithmetic, one rounding to fp16,
 *   nearest-even); code = clamp(rint((x_rot - z)/s), 0, 3) (fp64, half-even),
 *   code = 0 where s == 0; a group holding NaN stores s = z = NaN, codes 0;
 * packed into the slot's INT2 block.  Inputs: k_bf16, v_bf16 device bf16
 * [n][n_kv_heads][d], contiguous, 16-byte aligned (EINVAL otherwise);
 * int2_slots device int32 [n].  Slots must be distinct within one call.
 * n == 0 is a no-op. */
oscar_status oscar_quant_write(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                               const void* k_bf16, const void* v_bf16, const int32_t* int2_slots, int64_t n,
                               void* stream);

/* Same quantisation for tokens already held in bf16 slots (tokens leaving the
 * recent window): src_bf16_slots / dst_int2_slots device int32 [n]. */
oscar_status oscar_requant_from_bf16(const oscar_shape* shape, const oscar_layer* layer,
                                     const oscar_cache* cache, const int32_t* src_bf16_slots,
                                     const int32_t* dst_int2_slots, int64_t n, void* stream);

/* R's integer digits for the write calls, prepared once per layer ([IT] 2.2.A:
 * R is fixed offline, so what the write path derives from it is too).  prep:
 * device, >= oscar_layer_prep_bytes(shape) bytes, 256-byte aligned, written on
 * `stream` (r_k / r_v of `layer`, NULL r_v meaning the identity); its contents
 * are the same as each write work group would derive.  Set layer->r_prep to it
 * for the write calls that follow on that stream.  OSCAR_EINVAL on a bad shape
 * or layer, a NULL, misaligned or short prep, before anything is enqueued. */
size_t oscar_layer_prep_bytes(const oscar_shape* shape);
oscar_status oscar_layer_prepare(const oscar_shape* shape, const oscar_layer* layer, void* prep, size_t prep_bytes,
                                 void* stream);

/* Copy bf16 K/V (unrotated) of tokens with bf16_slots[i] >= 0 into bf16 blocks
 * (sink and recent tokens).  k_bf16, v_bf16: device [n][n_kv_heads][d]. */
oscar_status oscar_bf16_write(const oscar_shape* shape, const oscar_cache* cache, const void* k_bf16,
                              const void* v_bf16, const int32_t* bf16_slots, int64_t n, void* stream);

/* Copy whole pages (all KV heads): kind 0 = INT2 storage, 1 = bf16 storage.
 * src, dst: device int32 [n] physical page ids. */
oscar_status oscar_copy_pages(const oscar_shape* shape, const oscar_cache* cache, int32_t kind,
                              const int32_t* src_pages, const int32_t* dst_pages, int64_t n, void* stream);

/* ---- Read path: mixed-precision paged decode attention ([ES] serving
 * section, read path; [IT] 2.2.B) ----
 * For each request b and query head h (KV head h / (Hq/Hkv)), over the T =
 * ctx_lens[b] positions of the request:
 *   o = sum_t softmax_t(q.k_t / sqrt(d)) v_t, with k_t, v_t the stored bf16
 *   values for sink/recent positions and (z + c s) R^T for INT2 positions.
 * The rotation is undone algebraically: logits of INT2 tokens use q R_K, and the
 * INT2 part of the value sum is multiplied by R_V^T once.  Split-K partials
 * (log-sum-exp) are merged by a second kernel.
 * Inputs (device): q bf16 [batch][n_q_heads][d]; int2_bt int32
 * [batch][max_int2_pages]; bf16_bt int32 [batch][max_bf16_pages]; ctx_lens
 * int32 [batch].  Output (device): out fp32 [batch][n_q_heads][d].
 * splits_int2 / splits_bf16: work items per (request, KV head) for the INT2 and
 * bf16 regions (0 = choose; up to four bf16 splits run inside the merging
 * kernel, one per wavefront).  workspace: device, >= oscar_decode_workspace_bytes
 * with the same arguments (for 0 it sizes the most the automatic count can take
 * in the current small-grid mode), 256-byte aligned.  T = 0 gives a zero row. */
size_t oscar_decode_workspace_bytes(const oscar_shape* shape, int32_t batch, int32_t splits_int2,
                                    int32_t splits_bf16);
oscar_status oscar_decode_attn(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                               const void* q, int32_t batch, const int32_t* int2_bt, int32_t max_int2_pages,
                               const int32_t* bf16_bt, int32_t max_bf16_pages, const int32_t* ctx_lens,
                               int32_t splits_int2, int32_t splits_bf16, float* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): oscar_decode_attn with the same arguments and results, minus the
 * workspace, which is a device array inside the library (one copy per GPU,
 * held until the process ends; its size is
 * oscar_decode_noalloc_max_workspace_bytes(), 64 MiB).  A call that needs more
 * (oscar_decode_workspace_bytes with the splits it resolves to) returns
 * OSCAR_EINVAL before enqueueing anything.  The call allocates nothing: the
 * first call on a device only looks up the array's address there.  Calls that
 * overlap on one GPU (other streams, other threads) share the array and race;
 * serialise them.  Nothing in the array needs clearing between calls. */
oscar_status oscar_decode_attn_noalloc(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                                       const void* q, int32_t batch, const int32_t* int2_bt, int32_t max_int2_pages,
                                       const int32_t* bf16_bt, int32_t max_bf16_pages, const int32_t* ctx_lens,
                                       int32_t splits_int2, int32_t splits_bf16, float* out, void* stream);
size_t oscar_decode_noalloc_max_workspace_bytes(void);

/* The same decode kernels over an all-bf16 cache (the comparison baseline):
 * position p of request b lives in bf16 logical page p/16 (bf16_bt row b),
 * slot p%16; sink/recent/INT2 regions are not used. */
oscar_status oscar_decode_attn_bf16_baseline(const oscar_shape* shape, const oscar_cache* cache, const void* q,
                                             int32_t batch, const int32_t* bf16_bt, int32_t max_bf16_pages,
                                             const int32_t* ctx_lens, int32_t splits, float* out,
                                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- Chunked prefill over the mixed cache ([IT] 2.2.B and [ES] serving
 * section: prefix-cached chunked prefill reads the same paged INT2 + bf16
 * cache) ----
 * Attention of a chunk of C new queries per request: query c of request b sits
 * at position T - C + c (T = ctx_lens[b], the length after the chunk's tokens
 * were written with the write calls) and attends every position up to its own,
 * each in the form the cache holds it (INT2 history through the rotations as in
 * decode, bf16 sink and recent values).  Inputs (device): q bf16
 * [batch][C][n_q_heads][d]; block tables and ctx_lens as for oscar_decode_attn.
 * Output (device): out fp32 [batch][C][n_q_heads][d].  C >= 1 and
 * ctx_lens[b] >= C.  A chunk longer than the recent window has its older
 * positions in INT2 like any history: its queries read them in that form,
 * each query only up to its own position.  The queries run in blocks (16 at
 * g = 4, G = 32), each block one pass over the history with one wavefront per
 * 16 (query head, group) rows.  splits as in decode (0 = choose; bf16 splits
 * default 1).  workspace: >= oscar_prefill_workspace_bytes with the same
 * batch, C and splits, 256-byte aligned. */
size_t oscar_prefill_workspace_bytes(const oscar_shape* shape, int32_t batch, int32_t chunk, int32_t splits_int2,
                                     int32_t splits_bf16);
oscar_status oscar_prefill_attn(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                                const void* q, int32_t batch, int32_t chunk, const int32_t* int2_bt,
                                int32_t max_int2_pages, const int32_t* bf16_bt, int32_t max_bf16_pages,
                                const int32_t* ctx_lens, int32_t splits_int2, int32_t splits_bf16, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Splits chosen when 0 is passed: the count whose work items fill two whole
 * rounds of the wavefronts the device runs at once, at most 128 and at least
 * 16 pages per split (deterministic for a given device and small-grid mode).
 * Where the small-grid form applies (oscar_decode_set_small_grid not 1, one
 * wavefront per work item) and the count whose INT2 items and four bf16 splits
 * fit two wavefronts per SIMD is at least 24, the count is that fit at most,
 * and the whole fit (past 128) when each of its splits keeps 24 pages. */
int32_t oscar_decode_auto_splits(const oscar_shape* shape, int32_t batch, int32_t max_int2_pages);

/* Form of the decode launches ([IT] 2.2.B split-K decode with a log-sum-exp
 * combine; the form changes only the work split, not what is computed).  On a
 * small grid (one request, say) the bf16 sink/recent splits run as extra
 * items of the INT2 kernel's launch, and the combine takes one work group per
 * (request, KV head, query head) instead of one per (request, KV head).
 * mode 0 (the default): that form when the INT2 items and the bf16 splits fit
 * two wavefronts per SIMD and one wavefront holds a work item's tiles; 1:
 * never; 2: whenever one wavefront holds a work item's tiles.  Process-wide
 * (every later decode and decode-step call, any thread); returns the previous
 * mode, or -1 (mode unchanged) for a mode outside 0..2.  Results of the two
 * forms differ only in fp32 summation order. */
int32_t oscar_decode_set_small_grid(int32_t mode);

/* INT2 splits oscar_prefill_attn chooses when 0 is passed, for a chunk of
 * `chunk` queries: the fewest whose work items fill their last round of the
 * device to at least 15/16, else the best-filled count; at most 64 and at
 * least 32 pages per split.  Returns 1 for an invalid shape or argument. */
int32_t oscar_prefill_auto_splits(const oscar_shape* shape, int32_t batch, int32_t max_int2_pages, int32_t chunk);

/* One decode step for a batch: grows each of the n sequences by one token
 * (host bookkeeping, as oscar_seq_plan_append with n_new = 1 per sequence).
 * Outputs (host, capacity n each): int2_slots / bf16_slots of the new tokens
 * (-1 where not that region); age_src / age_dst: the bf16 -> INT2 move of the
 * token of sequence i leaving the recent window (-1 if none), *n_age the number
 * of moves; ctx_lens: the new lengths; *tables_changed = 1 if any sequence
 * received a new page (its block table rows must be refreshed).  The four slot
 * arrays laid out as rows of one int32 [4][n] array are the step_slots of
 * oscar_decode_step.  On OSCAR_ENOMEM no sequence is changed. */
oscar_status oscar_plan_decode_step(oscar_pool* pool, oscar_seq* const* seqs, int32_t n, int32_t* int2_slots,
                                    int32_t* bf16_slots, int32_t* age_src, int32_t* age_dst, int32_t* n_age,
                                    int32_t* ctx_lens, int32_t* tables_changed);

/* One decode step, writes and attention in one call ([ES] serving section:
 * the fused write and read kernels; [IT] 2.2.B).  Before the attention of
 * oscar_decode_attn (same arguments, same result), and inside its first kernel,
 * each request b of the batch stores this step's token, per KV head:
 *   step_slots[3*batch + b] >= 0: the token in bf16 slot step_slots[2*batch + b]
 *     (leaving the recent window) is quantised into that INT2 slot, exactly as
 *     oscar_requant_from_bf16 does;
 *   step_slots[b] >= 0: the new token (k_new, v_new row b) is quantised into
 *     that INT2 slot, exactly as oscar_quant_write does;
 *   step_slots[batch + b] >= 0: the new token is copied into that bf16 slot
 *     (read after the leaving token, so the two may share a ring slot).
 * Inputs (device): k_new, v_new bf16 [batch][n_kv_heads][d]; step_slots int32
 * [4][batch] (-1 = nothing to do; out-of-range slots are skipped).  The
 * block tables and ctx_lens must already include the new token (as
 * oscar_plan_decode_step leaves them).  Errors as oscar_decode_attn. */
oscar_status oscar_decode_step(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                               const void* k_new, const void* v_new, const int32_t* step_slots, const void* q,
                               int32_t batch, const int32_t* int2_bt, int32_t max_int2_pages,
                               const int32_t* bf16_bt, int32_t max_bf16_pages, const int32_t* ctx_lens,
                               int32_t splits_int2, int32_t splits_bf16, float* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* oscar_decode_step with the step's small tables in host memory ([ES] serving
 * section, as above): step_slots int32 [4][batch] and ctx_lens int32 [batch]
 * are read on the host when the call is made and travel to the kernels inside
 * their launch arguments, so the step needs no copy of them to the device (a
 * serving loop passes the arrays oscar_plan_decode_step filled).  The caller
 * may reuse both arrays as soon as the call returns.  batch <= 64
 * (OSCAR_EINVAL otherwise: use oscar_decode_step).  Every other argument, the
 * writes and the result are those of oscar_decode_step. */
oscar_status oscar_decode_step_host_tables(const oscar_shape* shape, const oscar_layer* layer,
                                           const oscar_cache* cache, const void* k_new, const void* v_new,
                                           const int32_t* step_slots, const void* q, int32_t batch,
                                           const int32_t* int2_bt, int32_t max_int2_pages, const int32_t* bf16_bt,
                                           int32_t max_bf16_pages, const int32_t* ctx_lens, int32_t splits_int2,
                                           int32_t splits_bf16, float* out, void* workspace, size_t workspace_bytes,
                                           void* stream);

/* Instrumentation.  While enabled (on != 0), each decode launch made by the
 * calling thread records a pair of HIP events on its stream around the main
 * decode kernel (not the prologue or the combine).  oscar_profile_read waits
 * for the recorded events, returns the summed milliseconds and the launch
 * count, and clears the record (disabling first keeps it readable).  The
 * event pairs are created once per thread and reused after each read. */
oscar_status oscar_profile_enable(int32_t on);
oscar_status oscar_profile_read(double* main_ms, int64_t* launches);
/* The same, and the first cap launches' durations in milliseconds, in launch
 * order, into the host array ms_each (cap >= 0; ms_each may be NULL when cap
 * is 0).  The record is cleared even if timing one launch fails
 * (OSCAR_EHIP). */
oscar_status oscar_profile_read_each(float* ms_each, int64_t cap, double* main_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
