/*
 * gqa.h -- C ABI of libgqa: single-token grouped-query-attention (GQA) decode over a KV cache on
 * AMD MI355X (gfx950).
 *
 * The operation.  For every batch entry b and query head h, with G = Hq / Hkv and j = floor(h / G):
 *
 *     s_t        = scale * k_descale * dot(q[b,h,:], k_cache[b,j,t,:])     for t in [0, seq_lens[b])
 *     out[b,h,:] = v_descale * sum_t softmax(s)_t * v_cache[b,j,t,:]
 *
 * i.e. ordinary scaled dot-product attention per query head, where each contiguous group of G query
 * heads shares one K head and one V head ("Grouped-Query Attention: How Sharing KV Heads Shrinks
 * Inference Memory", section "How grouped-query attention works"; "Grouped Query Attention (GQA):
 * Efficient Multi-Head Attention", Worked example 2).  One decode step attends over the cached K/V
 * of the tokens already in the cache ("Grouped Query Attention (GQA): Efficient Multi-Head
 * Attention", section "The bottleneck: autoregressive decoding ..."); here those are exactly the first
 * seq_lens[b] positions of the cache, and the new token's rows are stored by gqa_append_kv before
 * the call (or by the fused gqa_decode_append entry points further down).  A sequence
 * with seq_lens[b] == 0 gets an all-zero output row.  The cache is read once per KV head for all G
 * query heads of its group; nothing is expanded to Hq heads ("Grouped Query Attention: Why 8 KV
 * Heads Decide Your Batch Size", sections "Why does GQA speed up decode, not just save memory?" and
 * "Why doesn't GQA speed up my fine-tuned model?").
 *
 * Memory layout (all row-major, contiguous, device memory, 16-byte aligned base pointers):
 *     q        [B, Hq, d]        dtype q_dtype
 *     k_cache  [B, Hkv, L, d]    dtype kv_dtype   (L = allocated cache length per sequence)
 *     v_cache  [B, Hkv, L, d]    dtype kv_dtype
 *     seq_lens [B]               int32, each in [0, L] (values outside are clamped on the device)
 *     out      [B, Hq, d]        dtype out_dtype
 *
 * Supported dtype combinations (q / kv / out): f32 / f32 / {f32, bf16}; bf16 / bf16 / {bf16, f32};
 * bf16 / fp8-e4m3 / {bf16, f32}.  The fp8 cache is the OCP e4m3fn format with per-tensor descales
 * (real value = stored * descale), as in "Grouped-Query Attention: How Sharing KV Heads Shrinks
 * Inference Memory", section "FP8 KV cache: the other factor of two".  Head dims: 64 and 128.
 * Group sizes: G = Hq / Hkv in [1, 64] for bf16 and fp8 caches, [1, 32] for f32 caches.  Accumulation
 * is fp32; a bf16 out is rounded to nearest even.
 *
 * Ownership and threading.  The caller owns every buffer, the workspace included.  The library never
 * allocates or frees device memory and keeps no mutable global state besides cached device
 * attributes.  gqa_decode only enqueues work on the given stream and returns; it never synchronises.
 * Two calls that run at the same time must not share a workspace.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GQA_F32 = 0, GQA_BF16 = 1, GQA_FP8_E4M3 = 2 } gqa_dtype_t;

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1, /* null or misaligned pointer, bad dimension, Hq % Hkv != 0, overflow */
  GQA_ERR_UNSUPPORTED = 2, /* head dim, group size or dtype combination outside the list above */
  GQA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than gqa_decode_workspace_bytes() */
  GQA_ERR_HIP = 4          /* the HIP runtime reported an error while enqueueing */
} gqa_status_t;

typedef struct {
  int32_t B, Hq, Hkv, L, d;
  int32_t q_dtype, kv_dtype, out_dtype; /* gqa_dtype_t values */
  float k_descale, v_descale;           /* 1.0 for f32 and bf16 caches */
  int32_t num_workgroups; /* workgroups that split the cache: 0 = library's choice, else
                             1..65536.  The choice is 256, except for groups of more than 16 query
                             heads that are not split into sub-groups (below): min(256, max(64,
                             8 * B * Hkv)).  Results do not depend on it beyond rounding.
                             Bf16 and fp8 caches: a group of more than 16 query heads with few
                             (batch, KV head) pairs (at most 32 sub-group segments, 64 above 32
                             heads) runs as 2, 3 or 4 sub-groups of at most 16 heads, each of
                             which reads its KV head's cache; the choice depends on the
                             shape only. */
} gqa_shape_t;

/* Validates a shape (dimensions, divisibility, dtypes, workgroup count, 32-bit offsets).
 * Host only; no HIP call.  Returns GQA_OK, GQA_ERR_INVALID_ARG or GQA_ERR_UNSUPPORTED. */
gqa_status_t gqa_shape_check(const gqa_shape_t* shape);

/* Bytes of device workspace gqa_decode needs for this shape: a 256-byte header, a fixed 1 MiB area
 * of counters (one per (batch, KV head); B * Hkv may not exceed 2^18), then two partial-result slots
 * per workgroup.  0 if the shape is invalid.  Host only.
 *
 * Header: bytes 0-7 hold a tag that only gqa_workspace_init writes; bytes 8-11 are a uint32 error
 * count.  Bytes 12-15 (uint32, zero after initialisation) are merge-route flags for tests: bit 0
 * makes every workgroup publish its piece of a shared segment, never merging the last piece from
 * registers; bit 1 makes the decodes count, in bytes 16-19, the segments merged from registers.
 * The output is bitwise the same for any value of the flags.  The merge of a (batch, KV head) segment that several workgroups share is done by the one
 * that finishes last, found with the segment's counter, so the counters must start at zero. */
size_t gqa_decode_workspace_bytes(const gqa_shape_t* shape);

/* Initialises a workspace: clears the error count and the whole counter area (every counter, not
 * only this shape's) and writes the tag.  Required once before the first decode on a workspace;
 * every decode that completes leaves the counters at zero again, so the workspace then serves later
 * calls of any shape that fits in it, on one stream at a time.  Zero-filling is not initialisation.
 * A decode, paged decode or fused append-decode given a workspace without the tag (for instance
 * fresh memory from hipMalloc) does no work: every output row becomes NaN, no counter and no cache
 * row is written, and each of its workgroups adds one to the header's error count.  The check does
 * not see a counter area overwritten after initialisation (the result is then undefined);
 * initialise again after writing into the workspace.  Enqueues one small kernel on `stream` (a
 * hipStream_t, NULL = the default stream); returns GQA_ERR_WORKSPACE if workspace_bytes is below
 * this shape's requirement. */
gqa_status_t gqa_workspace_init(void* workspace, size_t workspace_bytes, const gqa_shape_t* shape,
                                void* stream);

/* Enqueues the decode described at the top of this header on `stream` (a hipStream_t; NULL = the
 * default stream).  scale is typically 1/sqrt(d) ("Grouped Query Attention (GQA): Efficient
 * Multi-Head Attention", Worked example 2) and must be finite.  All checks that do not need device
 * data run first and return an error before any HIP call; seq_lens is read on the device only. */
gqa_status_t gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, float scale, void* out, const gqa_shape_t* shape,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Decode without a caller workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same operation, arguments,
 * checks and kernels as gqa_decode, but the workspace is a fixed array of GQA_STATIC_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends; no call allocates or frees memory.
 * The first call on a device looks the array up and initialises it with a small kernel on `stream`;
 * later calls find its counters back at zero.  (A first call made while `stream` is being captured
 * into a graph puts the initialisation into the graph, and the next call outside a capture
 * initialises the array again.)  Shapes whose workspace (gqa_decode_workspace_bytes)
 * exceeds GQA_STATIC_SCRATCH_BYTES return GQA_ERR_WORKSPACE before any HIP call; a HIP error while
 * setting the array up returns GQA_ERR_HIP.  All calls on one GPU share its array, so calls that
 * overlap in time on one GPU (on different streams or from several threads without ordering) race
 * and give undefined results: order them on one stream.
 */
#define GQA_STATIC_SCRATCH_BYTES (24u << 20)

gqa_status_t gqa_decode_static(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, float scale, void* out, const gqa_shape_t* shape,
                               void* stream);

/* ------------------------------------------------------------------------------------------------
 * Paged cache.  Serving engines keep the cache in fixed-size pages handed out on demand ("Grouped
 * Query Attention: Why 8 KV Heads Decide Your Batch Size", section "What should you do about it?",
 * lists paged allocation among the levers; "Grouped-Query Attention: How Sharing KV Heads Shrinks
 * Inference Memory" cites the PagedAttention paper among its references).  The operation is the
 * decode above over the un-paged cache: position t of sequence b is row t % block_size of physical
 * page block_table[b][t / block_size].
 *
 * Memory layout (device memory; q, pages and out 16-byte aligned, tables 4-byte aligned):
 *     q            [B, Hq, d]                              dtype q_dtype
 *     k_pages      [num_blocks, Hkv, block_size, d]        dtype kv_dtype (bf16 or fp8-e4m3)
 *     v_pages      [num_blocks, Hkv, block_size, d]        dtype kv_dtype
 *     block_table  [B, max_blocks]                         int32 physical page numbers
 *     seq_lens     [B]                                     int32 in [0, max_blocks * block_size]
 *     out          [B, Hq, d]                              dtype out_dtype
 * Each (page, KV head) is one contiguous block_size x d run, so whole 16-position tiles of one KV
 * head come from one page.  Only the entries of pages that hold positions below seq_lens[b] are read;
 * the rest of a row may hold anything.  A page number outside [0, num_blocks) in a read entry is a
 * caller error: the kernel reads zeros for that page instead of faulting, so the output row is then
 * meaningless but no memory outside the pools is touched.
 */
typedef struct {
  int32_t B, Hq, Hkv, d;
  int32_t block_size; /* positions per page: a power of two, 16 .. 4096 */
  int32_t max_blocks; /* entries per block_table row; sequences hold at most max_blocks * block_size */
  int32_t num_blocks; /* pages in each of k_pages and v_pages */
  int32_t q_dtype, kv_dtype, out_dtype;
  float k_descale, v_descale;
  int32_t num_workgroups; /* as in gqa_shape_t */
} gqa_paged_shape_t;

/* Validates a paged shape: the checks of gqa_shape_check with L = max_blocks * block_size, plus the
 * page geometry above.  f32 caches are not supported paged (GQA_ERR_UNSUPPORTED).  Host only. */
gqa_status_t gqa_paged_shape_check(const gqa_paged_shape_t* shape);

/* Workspace bytes for gqa_decode_paged (same layout as gqa_decode_workspace_bytes); 0 if invalid. */
size_t gqa_decode_paged_workspace_bytes(const gqa_paged_shape_t* shape);

/* gqa_workspace_init for a paged shape. */
gqa_status_t gqa_paged_workspace_init(void* workspace, size_t workspace_bytes,
                                      const gqa_paged_shape_t* shape, void* stream);

/* Enqueues the paged decode on `stream`; same contract as gqa_decode otherwise (asynchronous, all
 * host-checkable errors returned before any HIP call, seq_lens and block_table read on the device). */
gqa_status_t gqa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* seq_lens, float scale, void* out,
                              const gqa_paged_shape_t* shape, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------------------------------------------------
 * Cache append: stores the new token's K and V rows before the decode that attends to them.  Row
 * (b, j) of k_new / v_new ([B, Hkv, d], new_dtype GQA_F32 or GQA_BF16, 16-byte aligned) goes to
 * position positions[b] (int32 [B], device) of sequence b, KV head j, converted to the cache's
 * format: f32 as is; bf16 rounded to nearest even (overflow to infinity, NaN to 0x7FC0 with its
 * sign); fp8-e4m3 as the code of x / descale (k_descale for K, v_descale for V, binary32 division)
 * rounded to nearest even and saturated at +-448, NaN to 0x7F with its sign ("Grouped-Query
 * Attention: How Sharing KV Heads Shrinks Inference Memory", section "FP8 KV cache: the other
 * factor of two": real value = stored * descale).  A negative position skips the sequence.  A
 * position >= L (dense) or >= max_blocks * block_size, or whose page-table entry lies outside
 * [0, num_blocks) (paged), writes nothing for that sequence and adds one to *skipped_count (device
 * int32, may be NULL).  Nothing else in the cache is touched.  Descales must be positive and finite.
 * Enqueued on `stream`; asynchronous.  The shapes describe the cache as for the decode entry points
 * (their q_dtype and out_dtype must still form a supported combination).
 */
gqa_status_t gqa_append_kv(const void* k_new, const void* v_new, int32_t new_dtype, void* k_cache,
                           void* v_cache, const gqa_shape_t* shape, const int32_t* positions,
                           int32_t* skipped_count, void* stream);
gqa_status_t gqa_append_kv_paged(const void* k_new, const void* v_new, int32_t new_dtype, void* k_pages,
                                 void* v_pages, const int32_t* block_table, const gqa_paged_shape_t* shape,
                                 const int32_t* positions, int32_t* skipped_count, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Append fused into the decode.  One decoding step stores the new token's K and V rows and then
 * attends over the cache that now holds them ("Grouped Query Attention (GQA): Efficient Multi-Head
 * Attention", section "The bottleneck: autoregressive decoding is not attention's finest hour").
 * These entry points do both in one launch: the result equals gqa_append_kv (new_dtype GQA_BF16,
 * positions[b] = seq_lens[b] - 1) followed by gqa_decode (or gqa_decode_paged) with the same
 * seq_lens, bit for bit, in both the cache and out.
 *   - seq_lens[b] counts the new token: its rows k_new[b] and v_new[b] ([B, Hkv, d] bf16, 16-byte
 *     aligned, device) go to position seq_lens[b] - 1 of sequence b, converted to the cache's format
 *     as gqa_append_kv converts bf16 rows (fp8-e4m3 caches divide by the shape's k_descale and
 *     v_descale), and the decode attends over positions [0, min(seq_lens[b], L)).
 *   - seq_lens[b] <= 0 writes nothing (and the output row is zero, as in the decode).  seq_lens[b] > L
 *     (L = max_blocks * block_size when paged) writes nothing, attends over all L positions and adds
 *     one to *skipped_count; so does a new position whose page-table entry lies outside
 *     [0, num_blocks) (that page then reads as zeros, as in gqa_decode_paged).  skipped_count is a
 *     device int32 (4-byte aligned) or NULL.
 *   - The cache is written at the new position only; the kernel that attends reads the new rows from
 *     registers, so no ordering between the write and the read is needed.
 *   - q_dtype must be GQA_BF16 and kv_dtype GQA_BF16 or GQA_FP8_E4M3 (else GQA_ERR_UNSUPPORTED);
 *     out_dtype, the workspace and every other argument are as for gqa_decode / gqa_decode_paged,
 *     with the same errors, returned before any HIP call.  Enqueued on `stream`; asynchronous.
 */
gqa_status_t gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                               void* v_cache, const int32_t* seq_lens, float scale, void* out,
                               const gqa_shape_t* shape, int32_t* skipped_count, void* workspace,
                               size_t workspace_bytes, void* stream);
gqa_status_t gqa_decode_append_paged(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                     void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                                     float scale, void* out, const gqa_paged_shape_t* shape,
                                     int32_t* skipped_count, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* KV-cache bytes per token: 2 (one K and one V tensor) * layers * kv_heads * head_dim * dtype_bytes
 * ("Grouped Query Attention: Why 8 KV Heads Decide Your Batch Size", section "Why does GQA decide
 * your batch size?").  Computed in 64-bit; host only. */
uint64_t gqa_kv_bytes_per_token(uint32_t layers, uint32_t kv_heads, uint32_t head_dim,
                                uint32_t dtype_bytes);

/* ------------------------------------------------------------------------------------------------
 * Prefill.  Attention of a whole prompt of S tokens over itself, the scaled_dot_product_attention
 * call with enable_gqa (and is_causal) of "Grouped Query Attention: Why 8 KV Heads Decide Your Batch
 * Size", section "Why doesn't GQA speed up my fine-tuned model?":
 *
 *     out[b,h,i,:] = sum_{t < n_i} softmax_t(scale * dot(q[b,h,i,:], k[b,j,t,:])) * v[b,j,t,:],
 *     j = floor(h / G), n_i = i + 1 when causal, S otherwise.
 *
 * Layout (device memory, 16-byte aligned): q [B, Hq, S, d], k and v [B, Hkv, S, d] (bf16), out
 * [B, Hq, S, d] (bf16 rounded to nearest even, or f32).  Each K/V tile is read once per workgroup and
 * serves the G query heads of its group; nothing is expanded to Hq heads.  Supported: d in {64, 128},
 * any G = Hq / Hkv up to 64 (a workgroup takes floor(256 / G) positions of all G heads).  No workspace.
 * Enqueued on `stream`; asynchronous.
 */
typedef struct {
  int32_t B, Hq, Hkv, S, d;
  int32_t dtype;     /* of q, k, v: GQA_BF16 */
  int32_t out_dtype; /* GQA_BF16 or GQA_F32 */
  int32_t causal;    /* 1: position i sees positions <= i; 0: every position */
} gqa_prefill_shape_t;

gqa_status_t gqa_prefill_shape_check(const gqa_prefill_shape_t* shape);
gqa_status_t gqa_prefill(const void* q, const void* k, const void* v, float scale, void* out,
                         const gqa_prefill_shape_t* shape, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Serving planners (host only, no HIP call).
 *
 * Tensor-parallel head sharding ("Grouped Query Attention: Why 8 KV Heads Decide Your Batch Size",
 * section "What breaks when num_kv_heads is smaller than your tensor-parallel degree?";
 * "Grouped-Query Attention: How Sharing KV Heads Shrinks Inference Memory", section "Why not always go
 * to one KV head?"): rank r of tp_size takes query heads [r * Hq / tp, (r + 1) * Hq / tp) and holds
 * every KV head they read (h -> h / G, G = Hq / Hkv).  When tp_size exceeds Hkv, or neither divides
 * the other, a KV head is held by several ranks: *kv_heads_held (summed over ranks) then exceeds Hkv,
 * and the ratio is the replication factor.  Requires Hq % Hkv == 0 and Hq % tp_size == 0, else
 * GQA_ERR_INVALID_ARG.  ranks (tp_size entries) and kv_heads_held may each be NULL.
 * A rank's KV bytes per token: gqa_kv_bytes_per_token(layers, kv_head_end - kv_head_begin, ...).
 */
typedef struct {
  int32_t q_head_begin, q_head_end;   /* query heads [begin, end) */
  int32_t kv_head_begin, kv_head_end; /* KV heads [begin, end) held by the rank */
} gqa_tp_rank_t;

gqa_status_t gqa_tp_plan(int32_t num_q_heads, int32_t num_kv_heads, int32_t tp_size, gqa_tp_rank_t* ranks,
                         int32_t* kv_heads_held);

/* Sequences of context_tokens that fit in free_bytes of cache: free / (bytes_per_token * context),
 * rounded down, 0 when either factor is 0 ("Grouped Query Attention: Why 8 KV Heads Decide Your Batch
 * Size", section "Why does GQA decide your batch size?").  Exact for all 64-bit inputs. */
uint64_t gqa_max_concurrency(uint64_t free_bytes, uint64_t bytes_per_token, uint64_t context_tokens);

/* Cached tokens that fit in free_bytes: free / bytes_per_token rounded down (0 if bytes_per_token is 0). */
uint64_t gqa_max_cached_tokens(uint64_t free_bytes, uint64_t bytes_per_token);

/* Test helper: writes the number of seq_lens entries outside [0, L] to *bad_count (device memory).
 * Enqueued on `stream`; does not synchronise.  Returns GQA_ERR_INVALID_ARG for null or misaligned
 * pointers or B <= 0. */
gqa_status_t gqa_validate_seq_lens(const int32_t* seq_lens, int32_t B, int32_t L, int32_t* bad_count,
                                   void* stream);

/* Measurement helper: streams `bytes` (a multiple of 16, 16-byte aligned) from `src` with
 * non-temporal 16-byte loads and writes one 32-bit word per workgroup into `sink` (at least
 * gqa_stream_read_sink_words() words).  Used to calibrate achievable read bandwidth. */
gqa_status_t gqa_stream_read(const void* src, size_t bytes, void* sink, void* stream);
size_t gqa_stream_read_sink_words(void);

/* Static description of a status code. */
const char* gqa_status_string(gqa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
