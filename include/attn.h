/*
 * attn.h - softmax attention with online (flash) softmax for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn.so.  Every pointer argument named q, k, v, o, *_pages, *_scales,
 * page_table, kv_lens and workspace is a DEVICE pointer; every call is asynchronous on
 * `stream` (a hipStream_t; NULL means the null stream) and returns as soon as the kernels
 * are queued.
 *
 * Problem statement.  The arguments follow the attention parameter block of
 * doppler (@simulatte/doppler 0.1.9->0.2.0, gpu/kernels/attention.js,
 * createAttentionUniformBuffer / executeAttention): numHeads, numKVHeads, headDim, kvLen,
 * seqLen, scale, causal, attnSoftcap, slidingWindow, pageSize, a page table and a
 * device-side kv length.  For one query row i at absolute position p_i, query head h,
 * KV head kvh = h / (num_heads / num_kv_heads) (contiguous groups):
 *
 *     visible(j)  =  j < kv_len  and  (!causal or j <= p_i)  and  (W == 0 or p_i - j < W)
 *     s_j         =  scale * <q_i, k_j>;   if attn_softcap > 0:  s_j = c * tanh(s_j / c)
 *     o_i         =  sum_{visible j} exp(s_j - m) v_j  /  sum_{visible j} exp(s_j - m)
 *
 * with m the row maximum.  A window of W keys includes the query's own position (doppler
 * run.js 0.1.0 clips kvLen to the window and sets kvStart = total - kvLen).  W = 0 and
 * c = 0 disable the window and the cap ("0 = disabled").  A row that sees no key cannot
 * occur for in-contract arguments; it would be written as zeros.
 *
 * Ownership.  All buffers are owned by the caller.  The library allocates nothing, frees
 * nothing, never synchronises and keeps no pointer after returning.  The caller keeps
 * every buffer alive until the queued work has completed on `stream`.  (The one piece of
 * device memory the library owns is the fixed scratch array of attn_decode_noalloc, part
 * of its loaded code object.)
 *
 * Errors.  Each entry point returns ATTN_OK (0) or a negative attn_status.  Argument
 * errors are detected on the host BEFORE any HIP call, so nothing is queued and no output
 * is touched.  ATTN_ERR_LAUNCH reports a failed kernel launch (hipGetLastError).  A
 * message for the last failure of the calling thread is returned by attn_last_error().
 * Faults during kernel execution surface at the caller's next synchronisation.
 *
 * Threading.  Re-entrant: the only mutable host state is thread-local (the error string
 * and the decode split override), apart from the per-device address of the scratch array,
 * looked up once under a lock.  Concurrent calls on different streams must use different
 * workspaces; concurrent attn_decode_noalloc calls on one GPU share its scratch and race.
 */
#ifndef TA03_ATTN_H
#define TA03_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, inconsistent sizes, bad value */
    ATTN_ERR_UNSUPPORTED = -2,   /* valid attention, but not a head_dim/dtype built here   */
    ATTN_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required             */
    ATTN_ERR_LAUNCH = -4         /* the HIP runtime refused the launch                     */
} attn_status;

typedef enum {
    ATTN_F32 = 0,                /* q, k, v, o in float32                                  */
    ATTN_F16 = 1                 /* q, k, v, o in IEEE float16                             */
} attn_dtype;

/*
 * Causal / sliding-window / bidirectional prefill with grouped KV heads and an optional
 * logit softcap (doppler attention.js, executeAttention with seqLen > 1; the tiled
 * prefill variants prefill, prefill_f16).
 *
 *   q, o : [seq_len, num_heads, head_dim]        token-major, dtype (doppler run.js:
 *   k, v : [kv_len, num_kv_heads, head_dim]      Q is [numTokens, numHeads*headDim], the
 *                                                cache is [kvLen, numKVHeads*headDim])
 *   Query row i sits at absolute position kv_len - seq_len + i (startPos = kvLen - seqLen).
 *   causal          : 0 or 1
 *   sliding_window  : W >= 0 keys including the query's own position; 0 = off
 *   attn_softcap    : c >= 0, finite; 0 = off
 *   scale           : finite, > 0 (doppler: 1/sqrt(headDim) or 1/sqrt(queryPreAttnScalar))
 *   head_dim        : 64, 128 or 256 (others: ATTN_ERR_UNSUPPORTED)
 *   Requires 1 <= seq_len <= kv_len, num_heads % num_kv_heads == 0, 16-byte aligned
 *   pointers.  f32 accumulation; the output is written in `dtype`.
 */
int attn_prefill(const void *q, const void *k, const void *v, void *o, int dtype,
                 int seq_len, int kv_len, int num_heads, int num_kv_heads, int head_dim,
                 int causal, int sliding_window, float attn_softcap, float scale,
                 void *stream);

/*
 * Chunked prefill against a cache whose length is read on the device (doppler
 * attention.js: kvLenSource = 1 takes kvLen from a buffer; run.js: a chunk of numTokens
 * new queries starts at startPos = currentSeqLen against kvLen = currentSeqLen +
 * numTokens cached keys).  The same computation as attn_prefill with kv_len = *kv_len,
 * for callers that capture the launch once (a HIP graph) and replay it as the cache grows.
 *
 *   q, o       : [seq_len, num_heads, head_dim]        token-major, dtype
 *   k, v       : [max_kv_len, num_kv_heads, head_dim]  capacity of the cache; rows at or
 *                past *kv_len are never read
 *   kv_len     : DEVICE pointer to one int32 L, read by the kernel when it runs; query row
 *                i sits at position L - seq_len + i.  Contract: seq_len <= L <= max_kv_len.
 *                Outside it every output row is NaN (loud, not silent).
 *   Other arguments and host-side checks as attn_prefill (with max_kv_len in place of
 *   kv_len); kv_len must be non-null and 4-byte aligned.
 */
int attn_prefill_device_kv_len(const void *q, const void *k, const void *v, void *o, int dtype,
                               int seq_len, int max_kv_len, const int32_t *kv_len,
                               int num_heads, int num_kv_heads, int head_dim, int causal,
                               int sliding_window, float attn_softcap, float scale,
                               void *stream);

/*
 * Bidirectional vision-tower self-attention (rullama 0.5.0, src/backend/dispatch/
 * attention.rs, vision_attention_chained and the head-major flash variant
 * vision_attention_flash_sub_hpd_chained): no mask, every patch sees every patch.
 *
 *   q, k, v, o : float16 [num_heads, num_patches, head_dim]   (head-major, "HPD")
 *   head_dim   : 64, 128 or 256;  num_patches >= 1;  scale finite > 0.
 *   f32 accumulation, float16 output.
 */
int attn_vision(const void *q, const void *k, const void *v, void *o,
                int num_patches, int num_heads, int head_dim, float scale, void *stream);

/*
 * Single-token decode over a contiguous float16 KV cache with float32 query (doppler
 * attention.js: decode is seqLen == 1; the _f16kv variants take f32 Q with f16 K/V).
 *
 *   q, o : float32 [num_heads, head_dim]
 *   k, v : float16 [num_kv_heads, kv_len, head_dim]   (head-major cache)
 *   The query sits at position kv_len - 1 and sees keys [max(0, kv_len - W), kv_len - 1].
 *   Device-data range: the products run on f16 matrix operands holding q * scale * log2(e)
 *   (q * scale under a cap) split into a high and a low f16 part, so every element of that
 *   must stay below 65504 in magnitude (|q| below about 5e5 at scale 1/sqrt(128)); this
 *   holds for the decode and tiered entry points alike.
 *   workspace : device memory of at least attn_decode_workspace_bytes(1, num_heads,
 *               num_kv_heads, head_dim, kv_len) bytes, 256-byte aligned, ZERO-FILLED by the
 *               caller once when allocated; the kernels leave it zeroed again on completion
 *               (self-resetting arrival counters), so it can be reused call after call on
 *               one stream.  One workspace per stream that runs decode concurrently.
 */
int attn_decode(const float *q, const void *k, const void *v, float *o,
                int num_heads, int num_kv_heads, int head_dim, int kv_len,
                int sliding_window, float attn_softcap, float scale,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation, kernels and
 * result as attn_decode, with the split partials and arrival counters in a library-owned
 * device array of ATTN_DECODE_SCRATCH_BYTES (4 MiB) per GPU instead of a caller workspace.
 * The array is part of the loaded code object, so each GPU the library runs on holds one
 * until the process ends; this entry point allocates and frees nothing.
 *
 *   Arguments, layouts and host-side checks as attn_decode, minus the workspace.  A shape
 *   whose split partials need more than ATTN_DECODE_SCRATCH_BYTES (attn_decode_workspace_bytes
 *   (1, num_heads, num_kv_heads, head_dim, kv_len) > 4 MiB, e.g. more than about 240 splits
 *   of 32 heads at head_dim 128) is refused with ATTN_ERR_UNSUPPORTED before any HIP call.
 *   The arrival counters are cleared on `stream` by a small kernel before every launch.
 *   All calls on one GPU share its array: calls whose execution overlaps on one GPU (two
 *   streams, or two threads) race and give wrong results; serialise them.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)4 << 20)
int attn_decode_noalloc(const float *q, const void *k, const void *v, float *o,
                        int num_heads, int num_kv_heads, int head_dim, int kv_len,
                        int sliding_window, float attn_softcap, float scale, void *stream);

/*
 * Single-token decode over a ring-buffer f16 cache that keeps the newest tokens of a
 * sliding-window layer (doppler attention.js / run.js: kvLayout = 1 "ring" for a
 * SlidingWindowKVCache, kvStart = totalSeqLen - kvLen with kvLen clipped to the window).
 * The pages name the layout but not its index map; the reading adopted here is the plain
 * one: the token at absolute position t lives at row t mod ring_len.
 *
 *   q, o      : float32 [num_heads, head_dim]
 *   k, v      : float16 [num_kv_heads, ring_len, head_dim]  (head-major ring)
 *   total_len : tokens seen so far (>= 1); the query sits at position total_len - 1
 *   sliding_window : W, 0 <= W <= ring_len; the query sees the newest E tokens,
 *               E = W if W > 0 else ring_len, i.e. positions [max(0, total_len - E),
 *               total_len - 1].  Rows holding other positions are never read.
 *   workspace : as attn_decode, sized by attn_decode_workspace_bytes(1, num_heads,
 *               num_kv_heads, head_dim, ring_len).
 *   Other arguments, checks and errors as attn_decode; W > ring_len is ATTN_ERR_INVALID_ARG.
 */
int attn_decode_ring(const float *q, const void *k, const void *v, float *o,
                     int num_heads, int num_kv_heads, int head_dim, int ring_len,
                     int total_len, int sliding_window, float attn_softcap, float scale,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Batched single-token decode over a paged, symmetric-int8 KV cache with float32 query
 * (doppler attention.js: kvLayout paged with pageSize and kvPageTable, kvLenSource = 1
 * reading kvLen from a buffer; executeAttentionTieredQuant: packed int8 K/V with separate
 * K and V scale buffers, f32 Q required).
 *
 *   q, o        : float32 [batch, num_heads, head_dim]
 *   k_pages,
 *   v_pages     : int8    [num_pages, num_kv_heads, page_size, head_dim]
 *   k_scales,
 *   v_scales    : float32 [num_pages, num_kv_heads, page_size]; value = q8 * scale.
 *                 Pages and scales are head-major within a page, so the page_size rows
 *                 and scales one KV head needs from a page are contiguous.
 *   page_table  : int32   [batch, max_pages_per_seq]; logical page -> physical page
 *   kv_lens     : int32   [batch], in DEVICE memory
 *   page_size   : 16
 *   Device-data contract: 1 <= kv_lens[b] <= max_pages_per_seq * page_size and
 *   page_table[b][0 .. ceil(kv_lens[b]/16) - 1] in [0, num_pages).  Entries past that are
 *   never read.  A kv_lens[b] outside its range makes row b of o NaN (nothing is read for
 *   it); page-table entries out of range are clamped into [0, num_pages) so a bad table
 *   gives wrong numbers, never an out-of-bounds access.
 *   workspace: as for attn_decode, sized by attn_decode_workspace_bytes(batch, num_heads,
 *   num_kv_heads, head_dim, max_pages_per_seq * page_size).
 */
int attn_decode_paged_q8(const float *q, const int8_t *k_pages, const int8_t *v_pages,
                         const float *k_scales, const float *v_scales,
                         const int32_t *page_table, const int32_t *kv_lens, float *o,
                         int batch, int num_heads, int num_kv_heads, int head_dim,
                         int page_size, int num_pages, int max_pages_per_seq,
                         int sliding_window, float attn_softcap, float scale,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Single-token decode over a tiered cache of one sequence (doppler attention.js:
 * executeAttentionTieredQuant, with coldLen, hotLen, hotWindow, hotStart; run.js passes
 * the tiers of a 'tiered' KV cache): the oldest cold_len positions sit in a paged
 * symmetric-int8 cold tier with separate K and V scales, the newest hot_len positions in an
 * f16 ring (the hot tier).  One online softmax runs over both tiers.
 *
 *   q, o           : float32 [num_heads, head_dim]
 *   hot_k, hot_v   : float16 [num_kv_heads, hot_window, head_dim]; position p in
 *                    [cold_len, cold_len + hot_len) lives at row (hot_start + p - cold_len)
 *                    mod hot_window (the pages give hotStart and hotWindow but print no index
 *                    formula; this is the plain reading).  Unused if hot_len == 0.
 *   cold_k_pages,
 *   cold_v_pages   : int8 [num_pages, num_kv_heads, page_size, head_dim]
 *   cold_k_scales,
 *   cold_v_scales  : float32 [num_pages, num_kv_heads, page_size] (head-major within a
 *                    page, as attn_decode_paged_q8); value = q8 * scale
 *   cold_page_table: int32 [max_pages]; logical page i (positions 16 i .. 16 i + 15) ->
 *                    physical page.  Unused if cold_len == 0.
 *   page_size      : 16
 *   The query sits at position cold_len + hot_len - 1 and sees the newest W positions
 *   (W = sliding_window, 0 = all), across both tiers.  Rows holding other positions, and
 *   page-table entries past ceil(cold_len / 16), are never read; out-of-range page-table
 *   entries are clamped into [0, num_pages).
 *   Requires hot_len <= hot_window,
 *   0 <= hot_start < hot_window when hot_len > 0, cold_len <= max_pages * page_size, and
 *   cold_len + hot_len >= 1; otherwise ATTN_ERR_INVALID_ARG before any HIP call.
 *   workspace: as for attn_decode, sized by attn_decode_workspace_bytes(1, num_heads,
 *   num_kv_heads, head_dim, cold_len + hot_len).
 */
int attn_decode_tiered_q8(const float *q, const void *hot_k, const void *hot_v,
                          const int8_t *cold_k_pages, const int8_t *cold_v_pages,
                          const float *cold_k_scales, const float *cold_v_scales,
                          const int32_t *cold_page_table, float *o,
                          int num_heads, int num_kv_heads, int head_dim,
                          int cold_len, int hot_len, int hot_window, int hot_start,
                          int page_size, int num_pages, int max_pages,
                          int sliding_window, float attn_softcap, float scale,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Conformer block-local self-attention with a relative-position term (rullama 0.5.0,
 * src/backend/dispatch/attention.rs, block_local_attention_chained: the audio conformer's
 * attention over chunks of chunk_size queries, each attending over a context of
 * context_size keys, max_past before and max_future after, with a sinusoidal position
 * table through a linear projection, an optional logit cap, head_dim 128).  float32.
 *
 *   q_pad    : [padded_len, num_heads * 128]  queries, already projected and scaled per
 *              dimension (the kernel applies no further scale); row i is position i
 *   k_padded,
 *   v_padded : [kv_rows, num_heads * 128]  row r holds position r - pad_left; the rows of
 *              positions outside [0, seq) are padding and never read
 *   pos_proj : [max_span, num_heads * 128]  row j belongs to the key j - max_past positions
 *              from the query (row max_past: the query's own position).  The pages name this
 *              projection but not its indexing; this is the reading adopted.
 *   attn_out : [padded_len, num_heads * 128]; rows >= seq are computed like the others (the
 *              caller trims them); a row with no visible key is written as zeros
 *   Query i sees key t iff i - max_past <= t <= i + max_future and 0 <= t < seq;
 *   s = q_i . k_t + q_i . pos_proj[t - i + max_past]; if logit_cap > 0, s = c tanh(s / c);
 *   o_i = softmax-weighted sum of the visible v_t.
 *   Requires head_dim == 128 (else ATTN_ERR_UNSUPPORTED), 1 <= seq <= padded_len,
 *   padded_len a multiple of chunk_size, max_span == max_past + max_future + 1,
 *   context_size == chunk_size + max_past + max_future, pad_left == max_past,
 *   kv_rows >= pad_left + seq, logit_cap finite >= 0 (else ATTN_ERR_INVALID_ARG), and
 *   max_past + max_future <= 28 (else ATTN_ERR_UNSUPPORTED: the key window of 16 queries
 *   and the position rows are staged in 64 KB of LDS).
 */
int attn_block_local(const float *q_pad, const float *k_padded, const float *v_padded,
                     const float *pos_proj, float *attn_out,
                     int seq, int padded_len, int kv_rows, int num_heads, int head_dim,
                     int chunk_size, int context_size, int max_span, int max_past,
                     int max_future, int pad_left, float logit_cap, void *stream);

/*
 * Tiered decode with an int8 cold tier stored contiguously ("packed", no page table), as
 * doppler attention.js executeAttentionTieredQuant binds it (packed int8 cold K and V, K and V
 * scale buffers, packedStride, f32 Q required, no page table).  The same computation and
 * readings as attn_decode_tiered_q8; only the cold tier's addressing differs.
 *
 *   cold_k, cold_v          : int8 [num_kv_heads, cold_capacity, head_dim]; position p <
 *                             cold_len of KV head h at row h * cold_capacity + p (the pages'
 *                             packedStride, the row pitch of the packed tier, is fixed by this
 *                             head-major layout: head_dim bytes per row, cold_capacity rows per
 *                             head)
 *   cold_k_scales,
 *   cold_v_scales           : float32 [num_kv_heads, cold_capacity]; value = q8 * scale
 *   Requires cold_capacity >= cold_len; other arguments and errors as attn_decode_tiered_q8
 *   (the workspace is sized the same way).
 */
int attn_decode_tiered_q8_packed(const float *q, const void *hot_k, const void *hot_v,
                                 const int8_t *cold_k, const int8_t *cold_v,
                                 const float *cold_k_scales, const float *cold_v_scales, float *o,
                                 int num_heads, int num_kv_heads, int head_dim,
                                 int cold_len, int hot_len, int hot_window, int hot_start,
                                 int cold_capacity, int sliding_window, float attn_softcap,
                                 float scale, void *workspace, size_t workspace_bytes, void *stream);

/* Cold-tier layouts of attn_decode_tiered_f16, with the codes of the pages' coldLayout. */
typedef enum {
    ATTN_COLD_CONTIGUOUS = 0,    /* [num_kv_heads, cold_capacity, head_dim], no page table    */
    ATTN_COLD_PAGED = 2          /* 16-token pages [num_pages, num_kv_heads, 16, head_dim]     */
} attn_cold_layout;

/*
 * Tiered decode with an f16 cold tier (doppler attention.js executeAttentionTiered /
 * createTieredAttentionUniformBuffer: f16 hot and cold K/V, coldLen, hotLen, hotWindow,
 * hotStart, coldPageTable, coldPageSize, coldLayout 2 = paged / 0 = contiguous, hotLayout
 * 1 = ring; doppler run.js passes coldLayout = coldPageTable ? 2 : 0).  The same positions,
 * window, cap and readings as attn_decode_tiered_q8; the cold tier holds f16 rows.
 *
 *   q, o           : float32 [num_heads, head_dim]
 *   hot_k, hot_v   : float16 ring [num_kv_heads, hot_window, head_dim], as attn_decode_tiered_q8
 *   cold_layout    : ATTN_COLD_PAGED: cold_k, cold_v float16 [num_pages, num_kv_heads, 16,
 *                    head_dim] (head-major within a page), cold_page_table int32
 *                    [cold_capacity / 16] mapping logical page i (positions 16 i .. 16 i + 15)
 *                    to a physical page (out-of-range entries are clamped into [0, num_pages));
 *                    cold_capacity must be a multiple of 16 and page_size 16.
 *                    ATTN_COLD_CONTIGUOUS: cold_k, cold_v float16 [num_kv_heads, cold_capacity,
 *                    head_dim]; cold_page_table must be NULL; page_size and num_pages unused.
 *   Requires cold_len <= cold_capacity; other arguments and errors as attn_decode_tiered_q8.
 */
int attn_decode_tiered_f16(const float *q, const void *hot_k, const void *hot_v,
                           const void *cold_k, const void *cold_v, const int32_t *cold_page_table,
                           float *o, int num_heads, int num_kv_heads, int head_dim,
                           int cold_len, int hot_len, int hot_window, int hot_start,
                           int cold_layout, int cold_capacity, int page_size, int num_pages,
                           int sliding_window, float attn_softcap, float scale,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace bytes needed by attn_decode (batch = 1) and attn_decode_paged_q8 for the
 * given shape (split partials and arrival counters).  Returns 0 for invalid sizes,
 * including shapes whose query (batch * num_heads * head_dim) or cache (max_kv_len *
 * num_kv_heads * head_dim) would exceed 2^40 elements, which the decode entry points refuse
 * with ATTN_ERR_INVALID_ARG.  Honours the calling thread's split override
 * (attn_set_decode_split).
 */
size_t attn_decode_workspace_bytes(int batch, int num_heads, int num_kv_heads, int head_dim,
                                   int max_kv_len);

/*
 * Test and tuning hook: force the number of KV tokens each decode workgroup handles
 * (a positive multiple of 16), for the calling thread; 0 restores the built-in plan.
 * Split-KV results agree within rounding for every split size.
 * Returns ATTN_OK or ATTN_ERR_INVALID_ARG.
 */
int attn_set_decode_split(int tokens_per_split);

/* Message for the calling thread's last failed call ("" if none).  Valid until the next
 * call on this thread. */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TA03_ATTN_H */
