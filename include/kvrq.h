/*
 * kvrq.h -- C ABI of the MI355X (gfx950) rotated INT4 paged KV cache.
 *
 * The library implements the hot path of SAW-INT4 ("System-Aware 4-Bit
 * KV-Cache Quantization for Real-World LLM Serving"):
 *
 *   kv_rotquant_write     one fused launch that rotates each K (and/or V) head
 *                         row by a block-diagonal Walsh-Hadamard matrix,
 *                         quantises it token-wise to INT4 and stores the codes
 *                         and fp16 parameters straight into a paged cache
 *                         (wispaper.ai blog, section 3: the rotation is fused
 *                         into the KV-cache write operator, no separate
 *                         launch; fugumt.com abstract: a fused
 *                         rotation-quantisation kernel that writes into paged
 *                         KV-cache layouts);
 *   kv_int4_paged_decode  decode attention over that cache: the query is
 *                         rotated by the same matrix (wispaper.ai blog,
 *                         section 3, third consequence: the rotated dot
 *                         product equals the original one), INT4 pages are
 *                         de-quantised on the fly, the V rotation is undone on
 *                         the output;
 *   kv_int4_paged_decode_step  the write of one new token per sequence
 *                         fused into the decode that reads it;
 *   kv_int4_paged_extend  causal attention of a chunk of new query tokens
 *                         over the same cache (chunked prefill);
 *   kvrq_pool_*           a host page allocator and page table for the fixed-
 *                         size pages the pages insist on (wispaper.ai blog,
 *                         section 1: PagedAttention needs uniform pages).
 *
 * Conventions for every call:
 *   - Return value: kvrq_status, 0 = KVRQ_OK.  On failure a description is
 *     available from kvrq_last_error() (thread-local, valid until the next
 *     failing call on the same thread).  No C++ exception crosses the ABI.
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call touches no device memory and makes no HIP call.
 *   - Device pointers are plain addresses of device memory owned by the
 *     caller.  The library never allocates or frees device memory and never
 *     synchronises the device; hot-path calls are asynchronous on the HIP
 *     stream passed as `stream` (a hipStream_t; NULL = the null stream).
 *   - The hot-path calls put only kernel launches on that stream (no memset,
 *     copy, event or host wait), so a caller may record them into a HIP
 *     graph during stream capture and replay it; the buffers recorded (and,
 *     for the workspace calls, the zero state of the workspace's counters,
 *     which every call restores) must stay valid for the replays.
 *   - A launch failure is reported as KVRQ_EHIP with the HIP error string.
 *   - head_dim must be 128.  Rotation blocks are 0 (no rotation, plain INT4)
 *     or 16, 32, 64, 128.  Page sizes are powers of two; the decode needs a
 *     multiple of 16.
 *
 * Cache layout (per layer, separate K and V pools):
 *   codes   uint8   [num_pages][num_kv_heads][page_size][head_dim/2]
 *           byte i of a row holds channel 2i in its low nibble and channel
 *           2i+1 in its high nibble (a 2-bit pool: [..][head_dim/4], byte i
 *           holds channels 4i..4i+3 at bits 0, 2, 4, 6);
 *   params  uint16  [num_pages][num_kv_heads][page_size][2]
 *           binary16 bit patterns (scale, zero); a row de-quantises as
 *           code * scale + zero in the rotated basis.
 * A token position `pos` of a sequence lives at slot = page * page_size +
 * pos % page_size, with page = the sequence's page for pos / page_size.
 */
#ifndef KVRQ_H
#define KVRQ_H

#include <stddef.h>
#include <stdint.h>

#if defined(KVRQ_BUILDING_LIBRARY)
#define KVRQ_API __attribute__((visibility("default")))
#else
#define KVRQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvrq_status;

/* split_tokens value of the decode calls that selects the balanced grid (see
 * kv_int4_paged_decode). */
#define KVRQ_SPLIT_BALANCED (-1)

enum {
    KVRQ_OK = 0,
    KVRQ_EINVAL = 1,        /* null pointer, negative size, bad alignment, bad shape */
    KVRQ_EUNSUPPORTED = 2,  /* valid request outside what the library implements */
    KVRQ_ENOPAGES = 3,      /* the page pool cannot satisfy a request */
    KVRQ_EHIP = 4,          /* a HIP launch or runtime error */
    KVRQ_EWORKSPACE = 5     /* workspace too small */
};

/* Static name of a status code ("KVRQ_OK", ...). Never NULL. */
KVRQ_API const char *kvrq_status_str(kvrq_status s);

/* Text of the last failure on this thread ("" if none). Never NULL. */
KVRQ_API const char *kvrq_last_error(void);

/* Geometry of one layer's cache.  k_block / v_block: rotation block of the
 * K and V rows (0 = no rotation), the block sizes 16..128 of the pages
 * (wispaper.ai blog, section 2, block-diagonal bullet).  k_bits / v_bits:
 * code width of each pool, 4 (0 means 4) or 2.  The 2-bit variant is the
 * open question of the pages (wispaper.ai blog, section 5, limitations:
 * whether the rotation keeps 2-bit accurate, perhaps with mixed precision);
 * it quantises with 3 levels instead of 15 and stores four codes per byte,
 * channel d at bit 2 (d % 4) of byte d / 4, in 32-byte rows.  K and V may
 * differ (mixed precision). */
typedef struct {
    int32_t head_dim;      /* D, must be 128 */
    int32_t num_kv_heads;  /* Hkv >= 1 */
    int32_t page_size;     /* P tokens per page, power of two, 1..1024 */
    int32_t num_pages;     /* pages in each pool, >= 1; num_pages * num_kv_heads *
                              page_size must not exceed 2^32 */
    int32_t k_block;       /* 0, 16, 32, 64 or 128 */
    int32_t v_block;       /* 0, 16, 32, 64 or 128 */
    int32_t k_bits;        /* 0 or 4: INT4; 2: 2-bit */
    int32_t v_bits;        /* 0 or 4: INT4; 2: 2-bit */
} kvrq_cache_desc;

/* Device buffers of one layer's cache (caller-allocated, layout above).
 * All four must be 16-byte aligned. */
typedef struct {
    uint8_t *k_codes;
    uint8_t *v_codes;
    uint16_t *k_params;
    uint16_t *v_params;
} kvrq_cache_buffers;

/* Bytes of the K codes pool, the V codes pool and ONE params pool for `d`
 * (K and V each need a params pool).  Validates `d`.  Any output may be
 * NULL. */
KVRQ_API kvrq_status kvrq_cache_sizes(const kvrq_cache_desc *d, size_t *k_codes_bytes,
                                      size_t *v_codes_bytes, size_t *params_bytes);

/* ------------------------------------------------------------------------
 * Host page pool and page table (host memory only; one pool per cache;
 * not thread-safe).  Pages are handed out from a free list whose initial
 * order is the identity (shuffle_seed == 0) or a permutation drawn from a
 * 64-bit seed (scattered pages, as a long-running server would see).
 * ------------------------------------------------------------------------ */
typedef struct kvrq_pool kvrq_pool;

/* Create a pool of num_pages pages of page_size tokens for up to max_seqs
 * sequences of at most max_pages_per_seq pages each.  *out receives the
 * pool; release it with kvrq_pool_destroy. */
KVRQ_API kvrq_status kvrq_pool_create(int32_t num_pages, int32_t page_size, int32_t max_seqs,
                             int32_t max_pages_per_seq, uint64_t shuffle_seed, kvrq_pool **out);

/* Free a pool (NULL is ignored). */
KVRQ_API void kvrq_pool_destroy(kvrq_pool *p);

/* Grow sequence `seq` to hold new_len tokens, taking pages from the free
 * list.  All or nothing: on KVRQ_ENOPAGES (pool exhausted or the sequence
 * would exceed max_pages_per_seq) nothing changes.  new_len below the
 * current length is KVRQ_EINVAL. */
KVRQ_API kvrq_status kvrq_seq_extend(kvrq_pool *p, int32_t seq, int32_t new_len);

/* Return all pages of `seq` to the free list and set its length to 0. */
KVRQ_API kvrq_status kvrq_seq_release(kvrq_pool *p, int32_t seq);

/* Current length of `seq` in tokens, or -1 for a bad pool or index. */
KVRQ_API int32_t kvrq_seq_len(const kvrq_pool *p, int32_t seq);

/* Slots of positions first_pos .. first_pos+count-1 of `seq` into the host
 * array slots_out[count].  The positions must lie below the sequence's
 * length (extend first). */
KVRQ_API kvrq_status kvrq_slots(const kvrq_pool *p, int32_t seq, int32_t first_pos, int32_t count,
                       int32_t *slots_out);

/* Export the page table: table_out[max_seqs][max_pages_per_seq] (host,
 * -1 beyond each sequence's pages) and seq_lens_out[max_seqs] (host; may
 * be NULL). */
KVRQ_API kvrq_status kvrq_page_table(const kvrq_pool *p, int32_t *table_out, int32_t *seq_lens_out);

/* Number of free pages, or -1 for a NULL pool. */
KVRQ_API int32_t kvrq_pool_free_pages(const kvrq_pool *p);

/* ------------------------------------------------------------------------
 * Hot path
 * ------------------------------------------------------------------------ */

/* Fused rotation + token-wise INT4 write (K~ = quant(K H_blk), V~ =
 * quant(V H_blk); wispaper.ai blog, section 3 core formula).
 *   k, v            device bf16 [num_tokens][num_kv_heads][head_dim]; token
 *                   t of head h starts at element t*token_stride + h*head_dim;
 *                   16-byte aligned, strides multiples of 8 elements
 *   num_tokens      T >= 0 (T == 0 launches nothing)
 *   slot_mapping    device int32 [T]; slot < 0 or slot >= num_pages*page_size
 *                   skips the token; slots must be unique within a call
 *                   (duplicates race; not checked)
 * For every written row (token t, head h, tensor X) with block b:
 *   y = H_b x in fp32 (butterflies of width 1, 2, ..., b/2, then * fp32(1/sqrt b)),
 *   scale = fp16((max y - min y) / 15), zero = fp16(min y),
 *   code_d = clamp(round_half_even((y_d - zero) * fp32(1 / scale)), 0, 15)  (0 if
 *   scale == 0), with scale and zero the stored fp16 values widened to fp32 and the
 *   reciprocal rounded to fp32 (not a true division: the two can differ by one code at a
 *   rounding boundary).
 * One launch on `stream`; rows are independent (no atomics). */
KVRQ_API kvrq_status kv_rotquant_write(const kvrq_cache_desc *d, const kvrq_cache_buffers *b,
                              const void *k, const void *v, int64_t num_tokens,
                              int64_t k_token_stride, int64_t v_token_stride,
                              const int32_t *slot_mapping, void *stream);

/* Workspace bytes kv_int4_paged_decode needs for num_seqs sequences of at
 * most max_seq_len tokens with num_q_heads query heads and the given
 * split_tokens (0 = automatic, KVRQ_SPLIT_BALANCED, or a split size, as in the
 * decode call).  0 when a single split covers max_seq_len: the split kernel
 * then writes the output itself and the workspace may be NULL. */
KVRQ_API kvrq_status kv_int4_paged_decode_workspace(const kvrq_cache_desc *d, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t max_seq_len,
                                           int32_t split_tokens, size_t *bytes);

/* Paged INT4 decode attention (one query token per sequence).
 *   q               device bf16 [num_seqs][num_q_heads][head_dim], unrotated
 *   num_q_heads     multiple of num_kv_heads, at most 16 per KV head; query
 *                   head g reads KV head g / (num_q_heads / num_kv_heads)
 *   page_table      device int32 [num_seqs][max_pages_per_seq]; an entry
 *                   outside [0, num_pages) is read as page 0 (garbage
 *                   output, never an out-of-bounds access)
 *   seq_lens        device int32 [num_seqs]; tokens 0..L-1 are attended;
 *                   L above max_seq_len is clamped to it; L <= 0 gives a
 *                   zero row
 *   max_seq_len     host bound on every L, used to plan the splits
 *   sm_scale        softmax scale; <= 0 selects 1/sqrt(head_dim)
 *   split_tokens    how the (sequence, KV head, token) work is cut:
 *                   0 = automatic; a multiple of 128 = split workgroups of that
 *                   many tokens (four waves each); KVRQ_SPLIT_BALANCED = the
 *                   balanced grid: one resident round of workgroups, each
 *                   taking an equal share of every sequence's 32-token tiles
 *                   in (sequence, KV head, tile) order (at most 1024
 *                   sequences and 16384 sequence x KV head pairs, else
 *                   KVRQ_EUNSUPPORTED).  The automatic choice is the balanced
 *                   grid when num_seqs * num_kv_heads * max_seq_len reaches
 *                   2^22 tokens (work for several rounds of split
 *                   workgroups) and the shape fits it; otherwise splits of
 *                   4 x clamp(S * Hkv * max_seq_len / 8192, 256, 1024) tokens,
 *                   raised to keep at most 64 splits
 *   out             device fp32 [num_seqs][num_q_heads][head_dim]
 *   workspace       device scratch of workspace_bytes >= the size reported by
 *                   kv_int4_paged_decode_workspace (16-byte aligned; unused,
 *                   and may be NULL, when that size is 0).  Its first 64 KiB
 *                   are split counters that must be zero before the first
 *                   call that uses the workspace (allocate it zero-filled, or
 *                   clear it once); every decode, decode-step and extend call
 *                   leaves them zero, so a workspace reused call after call
 *                   on one stream needs no further clearing.  Calls that may
 *                   overlap in time need workspaces of their own.
 * Computes, per sequence s and query head g (KV head h):
 *   q' = H_bK q,  score_t = sm_scale * q'.(code_t * scale_t + zero_t),
 *   o' = sum_t softmax(score)_t (V code_t * scale_t + zero_t),  out = H_bV o'.
 * One launch on `stream` for the balanced grid, when a single split covers
 * max_seq_len, or when every split workgroup fits on the device at once,
 * there are at most 16 splits and num_seqs * num_kv_heads <= 16384: the last
 * workgroup of each (sequence, KV head) to finish merges the partials (the
 * counters elect it).  Otherwise two launches: the split-K partials, then the
 * combine. */
KVRQ_API kvrq_status kv_int4_paged_decode(const kvrq_cache_desc *d, const kvrq_cache_buffers *b,
                                 const void *q, int32_t num_seqs, int32_t num_q_heads,
                                 const int32_t *page_table, int32_t max_pages_per_seq,
                                 const int32_t *seq_lens, int32_t max_seq_len, float sm_scale,
                                 int32_t split_tokens, float *out, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* kv_int4_paged_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The split counters and partials live in the library's own static device
 * array of 32 MiB per GPU (kept until the process ends); the call allocates and frees
 * nothing.  A decode whose workspace (kv_int4_paged_decode_workspace with the same
 * arguments) exceeds 32 MiB is rejected with KVRQ_EWORKSPACE before any HIP call; the
 * Qwen3-32B-like shape (256 sequences, 64 query and 8 KV heads) needs ~17 MiB.  The first
 * call on a device looks the array up and clears its counters with a small kernel on
 * `stream`; every call leaves them zero.  All calls on one GPU share the array: calls that
 * may overlap in time on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Arguments, results and launches are those of
 * kv_int4_paged_decode. */
KVRQ_API kvrq_status kv_int4_paged_decode_noalloc(const kvrq_cache_desc *d,
                                                  const kvrq_cache_buffers *b, const void *q,
                                                  int32_t num_seqs, int32_t num_q_heads,
                                                  const int32_t *page_table,
                                                  int32_t max_pages_per_seq, const int32_t *seq_lens,
                                                  int32_t max_seq_len, float sm_scale,
                                                  int32_t split_tokens, float *out, void *stream);

/* Fused decode step: write each sequence's new token and decode over it, in
 * one pass of the decode's split kernel (plus its combine).  For the
 * small-batch, latency-bound regime the pages serve next to the
 * high-concurrency one (fugumt.com abstract: serving must support both, and
 * the fused kernel matches plain INT4 across concurrency levels), where a
 * separate write launch of a few hundred rows costs as much as its launch.
 *   k_new, v_new    device bf16 [num_seqs][num_kv_heads][head_dim], one new
 *                   token per sequence, token strides as in kv_rotquant_write
 *   new_slots       device int32 [num_seqs]: the slot of position
 *                   seq_lens[s] - 1 of sequence s (the same slot its page
 *                   table gives); a negative slot writes nothing
 *   the rest        as in kv_int4_paged_decode; seq_lens counts the new token
 * The workgroup whose split holds position seq_lens[s] - 1 of sequence s and
 * KV head h encodes that head's K and V rows exactly as kv_rotquant_write
 * does (bit-identical cache bytes), stores them, and only then reads its
 * tiles; no other workgroup reads that position.  A sequence with
 * seq_lens[s] <= 0 writes nothing.  Preconditions (device data, not checked):
 * seq_lens[s] <= max_seq_len (a longer one is clamped, and its new row is
 * written but not attended), and new_slots[s] equal to the slot the page
 * table gives for position seq_lens[s] - 1 (otherwise the decode reads
 * whatever that position holds).
 * Output, workspace (zero-filled before its first use) and launches are
 * those of kv_int4_paged_decode with the same arguments
 * (kv_int4_paged_decode_workspace gives the size). */
KVRQ_API kvrq_status kv_int4_paged_decode_step(const kvrq_cache_desc *d, const kvrq_cache_buffers *b,
                                               const void *k_new, const void *v_new,
                                               int64_t k_token_stride, int64_t v_token_stride,
                                               const int32_t *new_slots, const void *q,
                                               int32_t num_seqs, int32_t num_q_heads,
                                               const int32_t *page_table, int32_t max_pages_per_seq,
                                               const int32_t *seq_lens, int32_t max_seq_len,
                                               float sm_scale, int32_t split_tokens, float *out,
                                               void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes kv_int4_paged_extend needs (arguments as in that call;
 * split_tokens 0 = automatic); 0, and the workspace may be NULL, when the
 * key range is not split (the usual case for chunks of many rows). */
KVRQ_API kvrq_status kv_int4_paged_extend_workspace(const kvrq_cache_desc *d, int32_t num_seqs,
                                                    int32_t num_q_heads, int32_t total_q,
                                                    int32_t max_q_len, int32_t max_seq_len,
                                                    int32_t split_tokens, size_t *bytes);

/* Paged INT4 extend (chunked prefill) attention: several new query tokens per
 * sequence, causal, over the same rotated INT4 cache -- the attention of the
 * prefill side of a serving engine (fugumt.com abstract: fused attention
 * execution over paged layouts).  The new tokens' K and V must already be in
 * the cache (kv_rotquant_write first).
 *   q               device bf16 [total_q][num_q_heads][head_dim], unrotated;
 *                   rows qo_start[s] .. qo_start[s+1]-1 are the last
 *                   n_s = qo_start[s+1] - qo_start[s] tokens of sequence s
 *   qo_start        device int32 [num_seqs + 1]; qo_start[0] = 0,
 *                   non-decreasing, qo_start[num_seqs] = total_q, every
 *                   n_s <= max_q_len and n_s <= seq_lens[s] (preconditions on
 *                   device data: violating rows get unspecified values, never
 *                   an out-of-bounds access)
 *   seq_lens        device int32 [num_seqs]: tokens in the cache, new ones
 *                   included (clamped to max_seq_len)
 *   max_q_len       host bound on every n_s (plans the grid); <= max_seq_len
 *   other arguments as in kv_int4_paged_decode
 *   out             device fp32 [total_q][num_q_heads][head_dim]
 * Row i of sequence s sits at position p = seq_lens[s] - n_s + i and its
 * output is the decode of the sequence's first p + 1 tokens with that row's
 * query (tokens after p are masked).  Two launches on `stream` (one when the
 * key range is not split).  The workspace is laid out as the decode's: its
 * first 64 KiB are left as they are, so one workspace can serve both. */
KVRQ_API kvrq_status kv_int4_paged_extend(const kvrq_cache_desc *d, const kvrq_cache_buffers *b,
                                          const void *q, int32_t total_q, int32_t num_seqs,
                                          int32_t num_q_heads, const int32_t *qo_start,
                                          const int32_t *page_table, int32_t max_pages_per_seq,
                                          const int32_t *seq_lens, int32_t max_seq_len,
                                          int32_t max_q_len, float sm_scale, int32_t split_tokens,
                                          float *out, void *workspace, size_t workspace_bytes,
                                          void *stream);

/* ------------------------------------------------------------------------
 * Measurement helpers (same conventions)
 * ------------------------------------------------------------------------ */

/* Unquantised reference write: bf16 rows copied into a paged bf16 cache
 * k_cache/v_cache [num_pages][num_kv_heads][page_size][head_dim] at the same
 * slots (the BF16 KV-cache baseline the pages compare against; wispaper.ai
 * blog, section 4).  Only head_dim, num_kv_heads, page_size and num_pages
 * of `d` are used. */
KVRQ_API kvrq_status kvrq_bf16_paged_write(const kvrq_cache_desc *d, void *k_cache, void *v_cache,
                                  const void *k, const void *v, int64_t num_tokens,
                                  int64_t k_token_stride, int64_t v_token_stride,
                                  const int32_t *slot_mapping, void *stream);

/* Plain device copy of `bytes` bytes (multiple of 16, both pointers 16-byte
 * aligned; one 16-byte element per lane): the streaming kernel used to measure
 * achievable HBM bandwidth and to calibrate byte counters. */
KVRQ_API kvrq_status kvrq_device_copy(void *dst, const void *src, size_t bytes, void *stream);

/* Streaming read of `bytes` bytes (multiple of 16, src 16-byte aligned): non-temporal
 * loads, eight waves per CU, nothing written but possibly one word at `sink` (a device
 * uint32; in practice never).  The ceiling a read-only kernel such as the decode can reach,
 * measured the same way on the same device. */
KVRQ_API kvrq_status kvrq_device_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Page-gather read: every byte of the cache pages listed in `pages` (device int32
 * [num_list]; ids outside [0, num_pages) read page 0) -- K codes, V codes and both
 * parameter pools of all KV heads -- in list order, with non-temporal loads, nothing
 * computed and nothing written but possibly one word at `sink` (a device uint32; in
 * practice never).  A decode's page table walked in sequence order gives the decode's
 * own bytes in the decode's order: the ceiling of a read-only kernel over a
 * page-scattered cache (the pages are fixed-size and scattered by the allocator;
 * wispaper.ai blog, section 1), next to kvrq_device_read's ceiling over contiguous
 * memory.  Reads num_list * num_kv_heads * page_size * 136 bytes.
 *   pattern 0: whole pages per wave, 16-byte loads (num_kv_heads * page_size a
 *              multiple of 128);
 *   pattern 1: per (page, KV head) block of 16 tokens, one workgroup per KV head and
 *              share of the list, two 32-token tiles in flight per wave, with the
 *              decode's own load shapes (16-byte K loads, 4-byte V and parameter loads);
 *   pattern 2: as 1 with 16-byte V loads;
 *   pattern 3: as 1 with four 32-token tiles in flight per wave (page_size a
 *              multiple of 16 for 1 to 3).
 * Patterns 1 to 3 may read a wave's last blocks again past the end of its share (in
 * flight only).  4-bit pools only (KVRQ_EUNSUPPORTED otherwise); wgs_per_cu (1..4)
 * workgroups of four waves per CU; a bad pattern, grid size, NULL `pages` or `sink`, or a
 * sink not 4-byte aligned is KVRQ_EINVAL, checked before any launch.  Asynchronous on
 * `stream`. */
KVRQ_API kvrq_status kvrq_paged_read(const kvrq_cache_desc *d, const kvrq_cache_buffers *b,
                                     const int32_t *pages, int64_t num_list, int32_t pattern,
                                     int32_t wgs_per_cu, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVRQ_H */
