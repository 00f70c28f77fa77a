/*
 * paged_attention.h -- C ABI of libpagedattn.so, an MI355X (gfx950) paged
 * attention operator.
 *
 * The operation ("Week 3 Day 5: Paged FlashAttention", sections "Keep the
 * Day 4 Interface", Task 1 and Task 2; "Week 2 Day 5: Fused Decode
 * Attention", Task 1): for every sequence b, query head h and query row l,
 *
 *   out[b,h,l,:] = sum_s softmax_s( scale * q[b,h,l,:] . K_b[s,:] ) * V_b[s,:]
 *
 * over the visible logical key positions s of sequence b, where
 *   - logical position s lives in physical page block_table[b, s / page_size]
 *     at slot s % page_size, i.e. K_b[s,:] = key_pages[page, kv_head, slot, :]
 *     (Task 1 of "Week 3 Day 5");
 *   - kv_head = h / (num_q_heads / num_kv_heads) (GQA head map, Task 1 of
 *     "Week 2 Day 5");
 *   - with causal != 0, key s is visible to row l iff
 *     s <= l + context_lens[b] - query_len (Task 2 of "Week 3 Day 5"), so the
 *     query_len rows are the last query_len positions of the context; with
 *     causal == 0 every s < context_lens[b] is visible.
 * Nothing is approximated: the kernels compute the same softmax as a dense
 * implementation would, tile by tile, so results differ from it by rounding
 * alone ("Week 3 Day 5", section "Why Optimize the Paged Path"). Arithmetic:
 * bf16 loads, fp32 dot products, softmax state and accumulation, bf16 (round
 * to nearest even) output.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays.
 *     bf16 is stored as 16-bit words. All index arrays are int32.
 *   - The caller owns every buffer. The library allocates nothing, keeps no
 *     pointer after returning, and has no global state besides the
 *     thread-local error message, a per-device cache of how many decode
 *     work items stay resident, a call counter that tags each call, and the
 *     per-device scratch array of paged_attention_static (a static device
 *     array, not an allocation). `out` must not alias any input.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; results are valid after the stream
 *     is synchronised.
 *   - Return value: PA_OK, or a negative PA_ERR_* code. Every argument check
 *     happens before any launch; on an error nothing is enqueued, nothing
 *     aborts, and paged_attention_last_error() describes the problem.
 */
#ifndef PAGED_ATTENTION_H_
#define PAGED_ATTENTION_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* null pointer, non-positive size, H_q % H_kv != 0,
                              max_pages * page_size < query_len, ... */
  PA_ERR_UNSUPPORTED = -2, /* head_dim not a multiple of 8 in [8, 256], or a size past a kernel limit */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  PA_ERR_LAUNCH = -4,      /* the HIP runtime rejected a launch */
  PA_ERR_METADATA = -5     /* paged_attention_check_metadata found bad data */
};

/* Which schedule runs. AUTO picks by query length (see paged_attention). */
enum {
  PA_SCHEDULE_AUTO = 0,
  PA_SCHEDULE_DECODE = 1,  /* short-query schedule, context split over work items */
  PA_SCHEDULE_PREFILL = 2, /* long-query MFMA tiled schedule: 128 packed query
                              rows x 64 keys per tile */
  PA_SCHEDULE_PREFILL_64X32 = 3 /* the same schedule at 64 packed query rows x
                              32 keys per tile, the tiling of the matrix kernel
                              in "Week 3 Day 5: Paged FlashAttention", Task 1,
                              for measurements against PREFILL (slower on
                              MI355X). Explicit only: head dims 64, 128 and
                              256, no explicit mask (PA_ERR_UNSUPPORTED
                              otherwise), never split, no workspace */
};

/*
 * paged_attention -- the operator (one call, "Week 3 Day 5", section "Keep
 * the Day 4 Interface"; the mask="causal" argument there is `causal`).
 *
 *   query        bf16 [batch, num_q_heads, query_len, head_dim]
 *   key_pages    bf16 [num_pages, num_kv_heads, page_size, head_dim]
 *   value_pages  bf16 [num_pages, num_kv_heads, page_size, head_dim]
 *   block_table  int32 [batch, max_pages]; entry j of row b is the physical
 *                page holding logical positions [j*page_size, (j+1)*page_size)
 *   context_lens int32 [batch]; number of logical K/V positions of sequence b
 *   out          bf16 [batch, num_q_heads, query_len, head_dim], written once
 *   scale        multiplier of q.k (typically 1/sqrt(head_dim)); any finite
 *                value: a negative scale is applied by negating q (exact in
 *                bf16), and 0 weights every visible key alike
 *   causal       0 or 1
 *   workspace    device scratch of at least
 *                paged_attention_workspace_bytes(...) bytes (may be NULL when
 *                that is 0). The decode schedule needs it; the prefill
 *                schedule needs it only to split the key ranges of a launch
 *                with fewer than 512 work items over several workgroups
 *                (without it, or when it is smaller, such a prefill runs
 *                unsplit -- a valid, slower result, not an error). Zero-fill
 *                a workspace once before its first use: its head holds
 *                arrival counters, which every successful call leaves at
 *                zero (a counter left by an interrupted call carries that
 *                call's tag and is ignored). The rest is scratch. Calls that
 *                share a workspace must be ordered on one stream.
 *
 * Device-data preconditions (not checked; see
 * paged_attention_check_metadata): for every b,
 * 1 <= context_lens[b] <= max_pages * page_size; with causal,
 * context_lens[b] >= query_len; 0 <= block_table[b,j] < num_pages for
 * j < ceil(context_lens[b] / page_size). Table entries past that and page
 * slots at or past context_lens[b] are never read and may hold anything.
 *
 * Dispatch (inside the library, "Week 3 Day 5", Task 4): a short query
 * (query_len * num_q_heads / num_kv_heads <= 4 rows per kv head) runs the
 * decode schedule, anything longer the prefill schedule -- the crossover
 * measured on MI355X over query lengths, contexts and GQA ratios. Supported:
 * head_dim any multiple of 8 from 8 to 256 ("Week 3 Day 5", Task 1, writes
 * its matrix kernel for head dim 128 and keeps generic controls for the
 * rest; here both schedules have instances for 64, 128 and 256, and any
 * other head dim runs the next larger instance with its extra dims masked),
 * page_size >= 1, any batch, GQA ratio and context length that fit int32.
 */
int paged_attention(const void* query, const void* key_pages, const void* value_pages,
                    const int32_t* block_table, const int32_t* context_lens, void* out,
                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t query_len,
                    int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t max_pages,
                    float scale, int32_t causal, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * paged_attention_ex -- paged_attention with the schedule and the number of
 * decode work items chosen by the caller (for tests of both schedules on
 * one input, "Week 3 Day 5", Task 3, and for tuning sweeps).
 *   schedule           PA_SCHEDULE_AUTO / _DECODE / _PREFILL /
 *                      _PREFILL_64X32. DECODE needs
 *                      query_len * num_q_heads / num_kv_heads <= 8.
 *   decode_work_items  the decode schedule cuts the total K/V work (sum of
 *                      context lengths times kv heads, in 64-key granules)
 *                      into contiguous ranges over this many work items,
 *                      sized by a cost model (a segment start costs extra;
 *                      with two resident per CU, the grid's second half
 *                      takes 12/16 of a first-half share); 0 = as many as
 *                      the GPU keeps resident at once (at most 2048);
 *                      otherwise 1 .. 65536. Ignored by the prefill
 *                      schedule.
 * Same arguments, preconditions and errors as paged_attention otherwise.
 */
int paged_attention_ex(const void* query, const void* key_pages, const void* value_pages,
                       const int32_t* block_table, const int32_t* context_lens, void* out,
                       int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t query_len,
                       int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t max_pages,
                       float scale, int32_t causal, void* workspace, size_t workspace_bytes,
                       int32_t schedule, int32_t decode_work_items, void* stream);

/*
 * paged_attention_masked -- paged_attention_ex with an explicit additive
 * mask beside the causal flag ("Week 2 Day 5: Fused Decode Attention",
 * Task 1: the primitive accepts explicit masks normalised to
 * [B * H_q, L, S]; Task 2, step 3: the scale, the optional mask and the
 * causal check are applied to each score):
 *
 *   score[b,h,l,s] = scale * q[b,h,l,:] . K_b[s,:] + mask[b,h,l,s]
 *
 * for the keys s that the context and (with causal) the causal rule leave
 * visible. The mask is in the units of the score (natural-log weights): -inf
 * removes a key, a finite value multiplies its weight by exp(value).
 *   mask          fp32, device. Entry (b, h, l, s) sits at element
 *                 b*mask_stride_b + h*mask_stride_h + l*mask_stride_l + s;
 *                 a stride of 0 broadcasts that axis (e.g. one mask row for
 *                 every query head). The buffer must hold
 *                 (B-1)*stride_b + (H_q-1)*stride_h + (L-1)*stride_l +
 *                 mask_len floats. Entries must not be NaN.
 *   mask_len      entries per mask row (the S axis), >= 1. A key at or past
 *                 mask_len has no entry and is absent, so a short mask never
 *                 leads to a read outside it.
 * A row whose every key is absent (or -inf) has no softmax; its output is
 * NaN, as 0 / 0 in the definition. Everything else -- arguments, layouts,
 * schedules, workspace, errors -- as paged_attention_ex; additionally
 * PA_ERR_INVALID for a NULL mask, a negative stride or mask_len < 1, or a
 * mask that overlaps `out`. The masked kernel instances hold the mask
 * entries in registers and run at lower occupancy than the unmasked ones.
 */
int paged_attention_masked(const void* query, const void* key_pages, const void* value_pages,
                           const int32_t* block_table, const int32_t* context_lens, const float* mask,
                           int64_t mask_stride_b, int64_t mask_stride_h, int64_t mask_stride_l,
                           int32_t mask_len, void* out, int32_t batch, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t query_len, int32_t head_dim, int32_t num_pages,
                           int32_t page_size, int32_t max_pages, float scale, int32_t causal,
                           void* workspace, size_t workspace_bytes, int32_t schedule,
                           int32_t decode_work_items, void* stream);

/*
 * Workspace bytes paged_attention (or paged_attention_ex with the same
 * schedule and decode_work_items) needs for these sizes; 0 when none is
 * needed.
 * Returns (size_t)-1 if the sizes are invalid (see
 * paged_attention_last_error). Pure host arithmetic, no device access.
 */
size_t paged_attention_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t query_len, int32_t head_dim, int32_t page_size,
                                       int32_t max_pages);
size_t paged_attention_workspace_bytes_ex(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t query_len, int32_t head_dim, int32_t page_size,
                                          int32_t max_pages, int32_t schedule, int32_t decode_work_items);

/*
 * The schedule PA_SCHEDULE_AUTO resolves to for these sizes (DECODE or
 * PREFILL), or a negative PA_ERR_* code. Pure host logic.
 */
int paged_attention_schedule(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t query_len, int32_t head_dim, int32_t page_size,
                             int32_t max_pages);

/*
 * paged_attention_check_metadata -- opt-in debug check of the device-data
 * preconditions above. Copies block_table and context_lens to the host on
 * `stream`, synchronises that stream, and returns PA_OK or PA_ERR_METADATA
 * (with the first offending entry in paged_attention_last_error()).
 */
int paged_attention_check_metadata(const int32_t* block_table, const int32_t* context_lens,
                                   int32_t batch, int32_t max_pages, int32_t num_pages,
                                   int32_t page_size, int32_t query_len, int32_t causal,
                                   void* stream);

/*
 * paged_kv_append -- writes the keys and values of new_len new tokens per
 * sequence into their page slots: the write half of the paged cache
 * ("Week 3 Day 5: Paged FlashAttention": logical position -> block_table ->
 * page and slot; the causal decode that follows a paged prefill needs the
 * new token's K/V in its page before paged_attention runs).
 *   key_new, value_new  bf16 [batch, num_kv_heads, new_len, head_dim], device
 *   key_pages, value_pages  bf16 [num_pages, num_kv_heads, page_size, head_dim],
 *                device, updated in place: only the new tokens' slots are
 *                written
 *   block_table  int32 [batch, max_pages], device
 *   context_lens int32 [batch], device: the context length AFTER the append,
 *                so token l of sequence b goes to logical position
 *                context_lens[b] - new_len + l (the convention paged_attention
 *                uses for query rows)
 * Device-data preconditions (not checked, but broken ones never cause a stray
 * write: a sequence with context_lens[b] < new_len is skipped, and so is a
 * token whose position falls past the block table or whose page id is not
 * a page of the pool):
 * new_len <= context_lens[b] <= max_pages * page_size; block_table[b, j] is
 * a page of the pool for every j the new positions touch; no two (sequence,
 * position) pairs of one call map to the same page slot.
 * The new K/V buffers must not overlap the pools, nor the two pools each
 * other. Asynchronous on `stream`; nothing is allocated. Returns PA_OK,
 * PA_ERR_INVALID, PA_ERR_UNSUPPORTED (head_dim not a multiple of 8 in [8, 256]) or
 * PA_ERR_LAUNCH;
 * nothing is launched unless every check passes.
 */
int paged_kv_append(const void* key_new, const void* value_new, void* key_pages, void* value_pages,
                    const int32_t* block_table, const int32_t* context_lens, int32_t batch,
                    int32_t num_kv_heads, int32_t new_len, int32_t head_dim, int32_t num_pages,
                    int32_t page_size, int32_t max_pages, void* stream);

/*
 * paged_attention_varlen -- the operator over a mixed batch in which every
 * sequence has its own number of query rows: prefill chunks and one-token
 * decodes in one call (the continuous-batching step that "Week 3 Day 5:
 * Paged FlashAttention", Task 4, measures on its serving trace; there the
 * dispatch picks the tiled prefill schedule for long queries and the vector
 * decode schedule for short ones -- here that choice is made per sequence).
 *
 *   query        bf16 [total_query, num_q_heads, head_dim], packed
 *                token-major: sequence b owns tokens
 *                [query_start[b], query_start[b + 1])
 *   query_start  int32 [batch + 1], device; L_b = query_start[b + 1] -
 *                query_start[b] is sequence b's query length (0 allowed:
 *                the sequence is skipped and its context is never read)
 *   out          bf16 [total_query, num_q_heads, head_dim], row t written
 *                once for every t of a sequence with L_b >= 1
 *   max_query_len  host bound on every L_b, 1 <= max_query_len <=
 *                total_query (sizes the prefill grid; no device read)
 *   key_pages, value_pages, block_table, context_lens, scale, causal: as for
 *                paged_attention; query row l of sequence b sits at logical
 *                position context_lens[b] - L_b + l.
 *   workspace    at least paged_attention_varlen_workspace_bytes(...) bytes,
 *                zero-filled once before first use (as for paged_attention:
 *                the decode part's counters and partials, then those of the
 *                prefill part's key-range split; a smaller workspace that
 *                still covers the decode part runs the prefill part unsplit).
 *
 * total_query == 0 is a valid empty call: nothing is enqueued, and query /
 * out may then be NULL.
 *
 * Device-data preconditions (not checked; see
 * paged_attention_varlen_check_metadata): query_start[0] == 0,
 * non-decreasing, query_start[batch] == total_query, every L_b <=
 * max_query_len; for each b with L_b >= 1 the preconditions of
 * paged_attention with query_len = L_b. A sequence whose offsets fall
 * outside [0, total_query] or whose length exceeds max_query_len is skipped
 * (its rows are not written), so broken offsets never cause a stray access.
 *
 * Dispatch, with group = num_q_heads / num_kv_heads: when group *
 * max_query_len <= 4 every sequence runs the decode schedule (the rule of
 * paged_attention); otherwise one-token queries run the decode schedule
 * (none when group > 4) and every longer query the prefill schedule -- the
 * decode schedule's cost grows with its widest sequence's rows. Two launches
 * on `stream`, the second only when some query is longer than the decode
 * bound.
 */
int paged_attention_varlen(const void* query, const void* key_pages, const void* value_pages,
                           const int32_t* block_table, const int32_t* context_lens, const int32_t* query_start,
                           void* out, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t total_query, int32_t max_query_len, int32_t head_dim, int32_t num_pages,
                           int32_t page_size, int32_t max_pages, float scale, int32_t causal, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * paged_attention_varlen_ex -- paged_attention_varlen with the split between
 * the two schedules and the decode work items chosen by the caller (tests run
 * one mixed batch through different splits; tuning sweeps).
 *   decode_max_len     -1: automatic (as paged_attention_varlen); 0: every
 *                      sequence takes the prefill schedule; k >= 1:
 *                      sequences with L_b <= k take the decode schedule,
 *                      which needs k * num_q_heads / num_kv_heads <= 8.
 *   decode_work_items  as for paged_attention_ex (0 = automatic).
 */
int paged_attention_varlen_ex(const void* query, const void* key_pages, const void* value_pages,
                              const int32_t* block_table, const int32_t* context_lens,
                              const int32_t* query_start, void* out, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t total_query, int32_t max_query_len,
                              int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t max_pages,
                              float scale, int32_t causal, void* workspace, size_t workspace_bytes,
                              int32_t decode_max_len, int32_t decode_work_items, void* stream);

/*
 * Workspace bytes paged_attention_varlen_ex needs for these sizes and
 * choices (decode_max_len = -1 and decode_work_items = 0 for
 * paged_attention_varlen); 0 when none is needed, (size_t)-1 if invalid.
 * Pure host arithmetic.
 */
size_t paged_attention_varlen_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t max_query_len, int32_t head_dim, int32_t page_size,
                                              int32_t max_pages, int32_t decode_max_len,
                                              int32_t decode_work_items);

/*
 * paged_attention_varlen_check_metadata -- opt-in debug check of the
 * mixed-batch preconditions above (copies the three index arrays to the
 * host on `stream` and synchronises it). Returns PA_OK, PA_ERR_INVALID,
 * PA_ERR_LAUNCH or PA_ERR_METADATA with the first offending entry in
 * paged_attention_last_error().
 */
int paged_attention_varlen_check_metadata(const int32_t* block_table, const int32_t* context_lens,
                                          const int32_t* query_start, int32_t batch, int32_t max_pages,
                                          int32_t num_pages, int32_t page_size, int32_t total_query,
                                          int32_t max_query_len, int32_t causal, void* stream);

/*
 * paged_attention_static -- paged_attention for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments and result as paged_attention, minus
 * the workspace: the decode schedule's counters and partial states (and the
 * split prefill's) live in a scratch array that the library holds on each
 * GPU until the process ends (paged_attention_static_scratch_bytes() bytes,
 * 64 MiB). The first call on a device looks the array up and zero-fills it
 * with one small kernel on `stream`; no call allocates (no hipMalloc, no
 * hipFree, no allocating library routine).
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents: calls that may overlap on one GPU (on different streams,
 * or from several threads without ordering) race on it and must be ordered
 * on one stream by the caller. Calls with a decode schedule that needs more
 * scratch than the array holds return PA_ERR_UNSUPPORTED before any launch;
 * a prefill whose key-range split needs more runs unsplit (a valid, slower
 * result).
 */
int paged_attention_static(const void* query, const void* key_pages, const void* value_pages,
                           const int32_t* block_table, const int32_t* context_lens, void* out, int32_t batch,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t query_len, int32_t head_dim,
                           int32_t num_pages, int32_t page_size, int32_t max_pages, float scale, int32_t causal,
                           void* stream);

/* Bytes of the per-GPU scratch array paged_attention_static uses. */
size_t paged_attention_static_scratch_bytes(void);

/* Message describing the last error returned on the calling thread ("" if none). */
const char* paged_attention_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_H_ */
