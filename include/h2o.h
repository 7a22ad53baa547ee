/*
 * h2o.h -- C ABI of the H2O chunked sparse-attention library for MI355X (gfx950).
 *
 * The method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
 * Attention" (montaan paper page).  A fixed-capacity KV cache per layer and KV
 * head holds N_C slots; slot j carries the token position t(b,h,j) and the H2O
 * score phi_h2o(b,h,j), the accumulated summed attention weights.  A chunk of S
 * query tokens attends to the filled slots and to its own causal keys; the same
 * computation returns the summed attention weights sum_i m_{b,h,i,j} ("Kernel
 * Support Needs"); those are added to the scores, and the chunk is written
 * into the slots of smallest score ("Improvements to Heavy-Hitter Oracle
 * (H2O)", item 2).
 *
 * Memory.  Every pointer is a device pointer allocated and owned by the caller.
 * The library never allocates or frees device memory, never synchronises the
 * device, and enqueues all work on `stream` (a hipStream_t; NULL = the null
 * stream).  Layouts are dense, row-major, no strides:
 *   q, out          [B][Hq][S][d]         dtype (bf16 or f32)
 *   k_new, v_new    [B][Hkv][S][d]        dtype
 *   cache->k, ->v   [B][Hkv][N_C][d]      dtype
 *   cache->pos      [B][Hkv][N_C]         int32, -1 marks an empty slot
 *   cache->score    [B][Hkv][N_C]         float32
 *   lse             [B][Hq][S]            float32, natural log
 *   colsum_cache    [B][Hkv][N_C]         float32
 *   colsum_new      [B][Hkv][S]           float32
 *   freed_slots     [B][Hkv][S]           int32
 * Query head h reads KV head h / (Hq/Hkv) (contiguous GQA groups).
 *
 * Errors.  Arguments are validated on the host before anything is enqueued; a
 * non-OK status means nothing was launched, and h2o_last_error() (thread-local)
 * describes it.  A failed launch returns H2O_ERR_HIP.  Faults inside kernels
 * surface at the caller's next synchronisation, as with any HIP work.  No C++
 * exception crosses this boundary.
 *
 * Threads.  The entry points keep no state between calls (apart from the
 * thread-local error text and the optional kernel timers) and may be called
 * from several threads; calls that write the same cache must be ordered by the
 * caller (same stream, or events).
 */
#ifndef H2O_H
#define H2O_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H2O_ABI_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define H2O_API __attribute__((visibility("default")))
#else
#define H2O_API
#endif

typedef enum {
    H2O_OK = 0,
    H2O_ERR_INVALID_ARG = -1,   /* null pointer, bad size, inconsistent shape   */
    H2O_ERR_UNSUPPORTED = -2,   /* valid but not implemented (head_dim, dtype)  */
    H2O_ERR_CAPACITY = -3,      /* the cache cannot take the chunk (see below)  */
    H2O_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required   */
    H2O_ERR_HIP = -5            /* a HIP runtime call or launch failed          */
} h2o_status_t;

typedef enum { H2O_F32 = 0, H2O_BF16 = 1 } h2o_dtype_t;

/* Ranking used to choose the slots to overwrite. */
typedef enum {
    H2O_SCORE_H2O = 0,        /* phi_h2o(b,h,j)                                    */
    H2O_SCORE_H2O_NORM = 1    /* phi_h2o(b,h,j) / (t - t(b,h,j)), t = P + S, formed
                                 in float32 ("Improvements to H2O", item 2)       */
} h2o_score_mode_t;

typedef struct {
    int32_t batch;            /* B >= 1                                  */
    int32_t n_q_heads;        /* Hq >= 1, a multiple of n_kv_heads       */
    int32_t n_kv_heads;       /* Hkv >= 1                                */
    int32_t head_dim;         /* d: 64 or 128                            */
    int32_t capacity;         /* N_C: 1 .. 32768 slots per (b, kv head)  */
    int32_t recent_window;    /* W >= 0: protected most recent positions */
    int32_t dtype;            /* h2o_dtype_t of q, k, v, out and the cache K/V */
} h2o_dims_t;

/* One layer's cache.  Slots [0, n_valid) are filled, for every (b, kv head).
 * n_valid lives on the host; h2o_evict_and_insert advances it. */
typedef struct {
    void    *k;
    void    *v;
    int32_t *pos;
    float   *score;
    int32_t  n_valid;
} h2o_cache_t;

/* Bytes of workspace h2o_chunk_attn and h2o_buffer_attn need for this chunk
 * length (enough for either): the split-over-slots partial results of the S = 1
 * path (bf16, d = 128, at most 32 query heads per KV head); or, for other
 * chunks, the partial summed weights of bf16 (4 * B * Hkv * (N_C + S) floats;
 * h2o_chunk_attn needs nothing else, and nothing at all without summed weights
 * or in f32) followed by the exclusion bits of h2o_buffer_attn
 * (B * Hkv * ceil(N_C / 64) 64-bit words).  The contents need no
 * initialisation and are not preserved. */
H2O_API size_t h2o_workspace_bytes(const h2o_dims_t *dims, int32_t chunk_len);

/*
 * Chunk attention with summed weights ("Kernel Support Needs").
 * Query row i (0 <= i < S) sits at position P + i, P = chunk_start.  Keys are
 * the filled slots j < n_valid and the chunk's own keys (position P + i').  Key
 * j is visible to row i iff 0 <= t(j) <= P + i (the implicit mask
 * -inf * 1[P+i < t(b,h,j)] of "Kernel Support Needs").  A cache filled by
 * h2o_evict_and_insert holds earlier tokens only, 0 <= t(j) < P, each visible
 * to every row, and chunk key i' is visible to rows i >= i'; a filled slot
 * marked -1 is never visible, and one holding a position at or after P is
 * visible from that row on (the kernels test positions per key tile, and take
 * the per-element mask only for tiles that hold such slots).  For every query
 * head h:
 *   out[b,h,i]  = sum_j softmax_j(sm_scale * q.k_j) v_j     (over visible keys)
 *   lse[b,h,i]  = log sum_j exp(sm_scale * q.k_j)
 * and for every KV head g, summing over its query heads and the S rows:
 *   colsum_cache[b,g,j] = sum_{h in g} sum_i m_{b,h,i,j}     j < n_valid (0 beyond)
 *   colsum_new[b,g,i']  = sum_{h in g} sum_i m_{b,h,i,i'}    chunk keys
 * bf16: MFMA inputs are bf16, accumulation and softmax fp32; the weights are
 * rounded to bf16 only for the product with V; summed weights are fp32.
 * colsum_cache and colsum_new may both be NULL: then only out and lse are
 * formed and the summed-weights work is skipped (a policy that does not rank
 * by attention, such as lastrec, needs no more).  Exactly one NULL is an error.
 * Requires 1 <= S, 0 <= n_valid <= N_C, chunk_start >= 0,
 * chunk_start + S <= INT32_MAX, sm_scale finite and > 0.  The cache is read only.
 */
H2O_API h2o_status_t h2o_chunk_attn(const h2o_dims_t *dims, const h2o_cache_t *cache,
                            int64_t chunk_start, int32_t chunk_len, float sm_scale,
                            const void *q, const void *k_new, const void *v_new,
                            void *out, float *lse, float *colsum_cache, float *colsum_new,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Score accumulation ("Improvements to H2O", item 2): the H2O score is the
 * running sum of summed attention weights.
 *   cache->score[b,g,j] += colsum_cache[b,g,j]   for j < cache->n_valid.
 */
H2O_API h2o_status_t h2o_update_scores(const h2o_dims_t *dims, const h2o_cache_t *cache,
                               const float *colsum_cache, void *stream);

/*
 * Eviction and insertion ("Improvements to H2O", item 2: new content overwrites
 * the slots with the smallest score).  With n = cache->n_valid, P = chunk_start:
 *   k = max(0, n + S - N_C) slots are evicted among the eligible ones
 *   E = { j < n : t(j) < P - W }, the k smallest by (score, slot index);
 *   targets = those victims and the empty slots [n, min(N_C, n+S)), ascending;
 *   chunk token i goes to targets[i]: K, V rows copied from k_new/v_new,
 *   t = P + i, score = colsum_new[b,g,i];  freed_slots[b,g,i] = targets[i];
 *   then cache->n_valid = min(N_C, n + S).
 * Returns H2O_ERR_CAPACITY (nothing launched) when k > 0 and S + W > N_C: with
 * distinct cached positions below P, |E| >= n - W, so S + W <= N_C guarantees
 * |E| >= k.  If the caller breaks that invariant and |E| < k on the device,
 * the shortfall is taken from the ineligible filled slots in slot order.
 * workspace may be NULL (none is needed).
 */
H2O_API h2o_status_t h2o_evict_and_insert(const h2o_dims_t *dims, h2o_cache_t *cache,
                                  int64_t chunk_start, int32_t chunk_len, int32_t score_mode,
                                  const void *k_new, const void *v_new,
                                  const float *colsum_new, int32_t *freed_slots,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * h2o_update_scores followed by h2o_evict_and_insert, in one call with the
 * same results bit for bit ("Improvements to H2O", item 2: accumulate, then
 * overwrite the smallest).  When slots are evicted (n + S > N_C) the score
 * update runs inside the selection, which reads every score anyway, so the
 * step takes one launch fewer; otherwise it runs on its own first.
 *   colsum_cache: [B][Hkv][N_C] fp32 device buffer, as for h2o_update_scores;
 *   the other arguments, the layouts, the errors (all returned before any
 *   launch) and the update of cache->n_valid are those of h2o_evict_and_insert.
 * score_mode is H2O_SCORE_H2O or H2O_SCORE_H2O_NORM.
 */
H2O_API h2o_status_t h2o_update_evict_and_insert(const h2o_dims_t *dims, h2o_cache_t *cache,
                                         const float *colsum_cache, int64_t chunk_start,
                                         int32_t chunk_len, int32_t score_mode,
                                         const void *k_new, const void *v_new,
                                         const float *colsum_new, int32_t *freed_slots,
                                         void *stream);

/*
 * One whole chunk step: h2o_chunk_attn followed by h2o_update_evict_and_insert,
 * with the same results bit for bit ("Kernel Support Needs": attention that
 * returns the summed weights; "Improvements to H2O", item 2: accumulate them
 * into the scores, then overwrite the slots of smallest score).  Arguments are
 * those of the two calls: colsum_cache and colsum_new (required) receive the
 * summed weights as from h2o_chunk_attn; the workspace is h2o_chunk_attn's
 * (h2o_workspace_bytes); score_mode, freed_slots, the cache update and the
 * advance of cache->n_valid are h2o_update_evict_and_insert's.  Every error of
 * either call (H2O_ERR_CAPACITY included) is returned before anything is
 * launched.  For S = 1 on the split decode path (bf16, d = 128) the score update
 * and each split's victim candidate are formed inside the kernel that forms the
 * summed weights, which already visits every slot, and one small launch merges
 * the output and inserts the token: one pass over the scores instead of two.
 * With at most four query heads per KV head, and when the device can hold the
 * whole split grid at once, that kernel is the attention launch itself: its
 * workgroups exchange their partial log-sum-exps within the launch (they wait
 * only for one another, so work on other streams delays but cannot block
 * them) and the logits never leave the chip.
 */
H2O_API h2o_status_t h2o_chunk_step(const h2o_dims_t *dims, h2o_cache_t *cache,
                            int64_t chunk_start, int32_t chunk_len, float sm_scale,
                            int32_t score_mode, const void *q, const void *k_new,
                            const void *v_new, void *out, float *lse, float *colsum_cache,
                            float *colsum_new, int32_t *freed_slots, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Insert-first buffer form ("Kernel Support Needs": attention over the fixed
 * N_C-slot buffer under the positional mask -inf * 1[P+i < t(b,h,j)]).  The
 * victims are chosen on the scores before the chunk and the chunk is written
 * into the targets before it attends, so it sees the slots that survive and
 * its own keys, causally -- never the slots it overwrites.  One chunk is:
 *   h2o_select_slots -> h2o_buffer_attn -> h2o_update_scores -> h2o_insert.
 *
 * h2o_select_slots: the targets of h2o_evict_and_insert (the k = max(0, n+S-N_C)
 * eligible slots of smallest (score, slot index) -- h2o or h2o-norm as
 * score_mode -- with the empty slots [n, min(N_C, n+S)), ascending) into
 * freed_slots, from the current scores.  The cache is not modified.  Errors
 * as h2o_evict_and_insert (H2O_ERR_CAPACITY when k > 0 and S + W > N_C).
 */
H2O_API h2o_status_t h2o_select_slots(const h2o_dims_t *dims, const h2o_cache_t *cache,
                              int64_t chunk_start, int32_t chunk_len, int32_t score_mode,
                              int32_t *freed_slots, void *stream);

/*
 * h2o_buffer_attn: the chunk attention of h2o_chunk_attn (same arguments,
 * layouts, precision and positional mask) over the buffer as it stands once the
 * chunk is written into freed_slots (the output of h2o_select_slots for this
 * cache, P and S): the targets below n_valid are not keys.  Equivalently, a
 * slot j of the buffer with position t(j) is visible to row i iff
 * t(j) <= P + i, the chunk's token i' sitting in slot freed_slots[b,g,i'].
 *   colsum_cache[b,g,j] = 0 for the slots being overwritten and j >= n_valid;
 *   colsum_new[b,g,i']  = the summed weight of chunk token i' (its slot's).
 * colsum_cache and colsum_new may both be NULL.  The workspace must hold
 * h2o_workspace_bytes(dims, chunk_len) bytes (the exclusion bits of the
 * overwritten slots live there).
 */
H2O_API h2o_status_t h2o_buffer_attn(const h2o_dims_t *dims, const h2o_cache_t *cache,
                             int64_t chunk_start, int32_t chunk_len, float sm_scale,
                             const void *q, const void *k_new, const void *v_new,
                             const int32_t *freed_slots, void *out, float *lse,
                             float *colsum_cache, float *colsum_new, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * h2o_insert: the insertion half of h2o_evict_and_insert for given targets:
 * chunk token i goes to freed_slots[b,g,i] (K, V copied, t = P + i, score =
 * colsum_new[b,g,i], or 0 when colsum_new is NULL); then
 * cache->n_valid = min(N_C, n + S).  freed_slots must come from
 * h2o_select_slots for the same cache, P and S.
 */
H2O_API h2o_status_t h2o_insert(const h2o_dims_t *dims, h2o_cache_t *cache, int64_t chunk_start,
                        int32_t chunk_len, const void *k_new, const void *v_new,
                        const float *colsum_new, const int32_t *freed_slots, void *stream);

/*
 * lastrec eviction and insertion ("Experimental Validation", the lr policy:
 * the first beta tokens and the last N_C - beta tokens stay in the cache).
 * With n = cache->n_valid, P = chunk_start, beta = sink_tokens:
 *   k = max(0, n + S - N_C) slots are evicted among E = { j < n : t(j) >= beta },
 *   the k of smallest position t(j) (positions are distinct: no ties);
 *   targets, insertion, freed_slots and n_valid as in h2o_evict_and_insert,
 *   except that an inserted slot gets score 0.  dims->recent_window is unused;
 *   the scores are neither read nor ranked.
 * Returns H2O_ERR_CAPACITY (nothing launched) when k > 0 and S + beta > N_C:
 * at most beta distinct cached positions lie below beta, so |E| >= n - beta,
 * and S + beta <= N_C guarantees |E| >= k.  If the caller breaks the
 * distinct-position invariant and |E| < k on the device, the shortfall is
 * taken from the other filled slots in slot order.  Requires sink_tokens >= 0.
 */
H2O_API h2o_status_t h2o_evict_and_insert_lastrec(const h2o_dims_t *dims, h2o_cache_t *cache,
                                          int64_t chunk_start, int32_t chunk_len,
                                          int32_t sink_tokens, const void *k_new,
                                          const void *v_new, int32_t *freed_slots,
                                          void *stream);

/*
 * Backward of the chunk attention (pass 1 of h2o_chunk_attn or h2o_buffer_attn)
 * with the cache decisions fixed: the policy's choices are replayed, not
 * differentiated ("Gradient Computation Strategy", item 1), so the keys and
 * the mask are those of the forward call and the gradient is that of masked
 * softmax attention.  Inputs: the cache as it stood for the forward call (K,
 * V, pos, n_valid), chunk_start, chunk_len, sm_scale, q, k_new, v_new, that
 * call's out and lse, dout = dL/dout ([B][Hq][S][d], dtype), and freed_slots
 * (NULL, or the h2o_buffer_attn targets: those slots are not keys).  With
 * m = softmax over the visible keys, D_i = sum_d dout[i,d] out[i,d] and
 * ds_ij = m_ij (dout_i . v_j - D_i), per query head h and KV head g = h / G:
 *   dq[b,h,i]        = sm_scale sum_j ds_ij k_j               [B][Hq][S][d]
 *   dk_cache[b,g,j]  = sm_scale sum_{h in g} sum_i ds_ij q_i  [B][Hkv][N_C][d]
 *   dv_cache[b,g,j]  = sum_{h in g} sum_i m_ij dout_i         [B][Hkv][N_C][d]
 *   dk_new, dv_new   the same for the chunk's own keys       [B][Hkv][S][d]
 * All gradients are float32; dk_cache and dv_cache are 0 for j >= n_valid and
 * at excluded slots.  bf16: MFMA inputs bf16 (the weights and ds rounded to
 * bf16 for their products), accumulation fp32.  The workspace must hold
 * h2o_backward_workspace_bytes(dims, chunk_len) bytes.  bf16 runs the dq
 * kernel on a second stream of the library (one per device, default
 * priority), forked from `stream` by an event and joined back to it before the
 * call returns: all the call's work is ordered with respect to `stream`, also
 * under HIP graph capture.  Concurrent calls on one device are serialised on
 * the host while they enqueue.
 */
H2O_API size_t h2o_backward_workspace_bytes(const h2o_dims_t *dims, int32_t chunk_len);
H2O_API h2o_status_t h2o_chunk_attn_backward(const h2o_dims_t *dims, const h2o_cache_t *cache,
                                     int64_t chunk_start, int32_t chunk_len, float sm_scale,
                                     const void *q, const void *k_new, const void *v_new,
                                     const void *out, const float *lse, const void *dout,
                                     const int32_t *freed_slots, float *dq, float *dk_new,
                                     float *dv_new, float *dk_cache, float *dv_cache,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * h2o_chunk_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus the workspace),
 * results, layouts, precision and errors as h2o_chunk_attn, from the same
 * kernels, so the outputs are bit-identical.  The workspace comes from a
 * static device array of the library, h2o_noalloc_scratch_bytes() bytes
 * (40 MiB) on each GPU, held until the process ends; its address on a device
 * is looked up once, at the first call on that device.  A call whose
 * workspace (h2o_workspace_bytes for a bf16 chunk with summed weights or a
 * decode step; none otherwise) exceeds it returns H2O_ERR_WORKSPACE before
 * anything is launched.  Calls no allocating routine.  Every call on one GPU
 * shares that GPU's array and leaves its contents behind (nothing in it must
 * start at zero): calls that overlap on one GPU (different streams, or host
 * threads without ordering) race on it and must be serialised by the caller.
 */
H2O_API size_t h2o_noalloc_scratch_bytes(void);
H2O_API h2o_status_t h2o_chunk_attn_noalloc(const h2o_dims_t *dims, const h2o_cache_t *cache,
                                    int64_t chunk_start, int32_t chunk_len, float sm_scale,
                                    const void *q, const void *k_new, const void *v_new,
                                    void *out, float *lse, float *colsum_cache,
                                    float *colsum_new, void *stream);

/* Thread-local description of the last non-OK status ("" if none). */
H2O_API const char *h2o_last_error(void);

/* H2O_ABI_VERSION of the loaded library. */
H2O_API int32_t h2o_abi_version(void);

/*
 * Optional per-kernel timing (a diagnostic, process-wide, not thread-safe).
 * While a timer is running, each launch of that kernel is bracketed by two HIP
 * events recorded on its launch stream (at most max_launches launches are
 * recorded).  h2o_kernel_timer_stop waits for those events and returns the sum
 * of their elapsed times and the number of launches recorded.
 */
typedef enum {
    H2O_KERNEL_ATTN = 0,      /* chunk attention: output + log-sum-exp          */
    H2O_KERNEL_COLSUM = 1,    /* summed attention weights (recompute pass)      */
    H2O_KERNEL_UPDATE = 2,    /* score accumulation                             */
    H2O_KERNEL_SELECT = 3,    /* eligibility + victim selection                 */
    H2O_KERNEL_INSERT = 4,    /* chunk insertion                                */
    H2O_KERNEL_DECODE = 5,    /* S = 1 attention (split over slots)             */
    H2O_KERNEL_DECODE_FINISH = 6, /* S = 1: merge of the splits (and summed weights
                                     when the attention launch did not form them) */
    H2O_KERNEL_BACKWARD = 7,  /* backward of the chunk attention (all its launches) */
    H2O_KERNEL_COUNT = 8
} h2o_kernel_id_t;

H2O_API h2o_status_t h2o_kernel_timer_start(int32_t kernel, int32_t max_launches);
H2O_API h2o_status_t h2o_kernel_timer_stop(int32_t kernel, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* H2O_H */
