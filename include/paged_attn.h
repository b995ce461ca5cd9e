/*
 * paged_attn.h — C ABI of libpagedattn.so: attention over a paged KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * The cache has the shape (2, num_blocks, block_size, num_kv_heads,
 * head_size); key_cache and value_cache below are its two halves, each a
 * contiguous [num_blocks, block_size, num_kv_heads, head_size] array
 * [vLLM flash_attn.py (e2f56c3), FlashAttentionBackend.get_kv_cache_shape;
 * FlashAttentionImpl.forward, kv_cache.unbind(0)].  A sequence's logical
 * token j lives at (block_table[b][j / block_size], j % block_size)
 * [Aphrodite flash_attn.py, FlashAttentionMetadata, block_tables].
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers, except where a parameter says
 *    otherwise.  Integer sizes and scalars are passed by value from the host.
 *  - The caller owns every buffer, outputs included; the library allocates
 *    nothing and keeps no state between calls (the one exception is the
 *    fixed scratch array of paged_attn_decode_noalloc, below).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without synchronising.
 *  - Return value: PA_OK, or a negative code.  Arguments are validated on the
 *    host before anything is enqueued; on a validation error nothing is
 *    written.  pa_last_error() gives a message for the last failure of the
 *    calling thread.
 *  - Contents of device arrays (slot ids, block ids, lengths) are trusted:
 *    an out-of-range block id or slot is undefined behaviour
 *    (pa_check_indices counts such entries, for tests and debugging).
 *  - dtype of q / key / value / out: PA_F16 or PA_BF16.  All arithmetic is
 *    fp32; outputs are rounded to nearest-even.
 *  - kv_cache_dtype: the caches' element type, either dtype itself or
 *    PA_FP8_E4M3 [vLLM flash_attn.py (e2f56c3), get_fp8_dtype_for_flashattn:
 *    "fp8" / "fp8_e4m3" is float8_e4m3fn; FlashAttentionImpl.forward, the
 *    kv_cache_dtype, k_scale and v_scale of reshape_and_cache_flash and the
 *    k/v descales of the attention call].  An fp8 cache holds one-byte OCP
 *    e4m3 codes (same shape, 1 byte per element) and takes two device fp32
 *    scalars k_scale / v_scale: the code of an element x is x / scale
 *    (fp32, correctly rounded) rounded to the nearest e4m3 value, ties to
 *    even, saturating at +-448 (NaN stays NaN); the attention reads
 *    value(code) * scale.  With a 16-bit cache k_scale / v_scale are
 *    ignored (may be NULL).
 *  - q_scale (attention calls): NULL, or with an fp8 cache a device fp32
 *    scalar that makes q an fp8 query: q then holds one-byte e4m3 codes
 *    (same shape, e.g. from scaled_fp8_quant with this scale) and the
 *    attention reads value(code) * q_scale [vLLM flash_attn.py (v0.9.0.1
 *    docs), FlashAttentionImpl.forward, the fp8 branch:
 *    ops.scaled_fp8_quant(query, layer._q_scale) and q_descale; vLLM
 *    flash_attn.py (e2f56c3), "queries are quantized in the attention
 *    layer"].  Every score is multiplied by q_scale * k_scale; dtype is then
 *    the dtype of out.  q_scale with a 16-bit cache is PA_ERR_UNSUPPORTED.
 *    With q_scale NULL an fp8 cache is attended by a 16-bit query (another
 *    backend's option, which keeps the query unquantised).
 *  - head_size must be 64, 128 or 256; block_size a positive multiple of 16
 *    and at most 256; num_heads a multiple of num_kv_heads.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F16 = 0, PA_BF16 = 1, PA_F32 = 2, PA_FP8_E4M3 = 3 } pa_dtype_t;

enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,      /* bad argument (NULL pointer, inconsistent sizes) */
  PA_ERR_UNSUPPORTED = -2,  /* valid request this library does not implement */
  PA_ERR_HIP = -3           /* the HIP runtime reported an error on launch */
};

/*
 * reshape_and_cache — write the K and V rows of new tokens into their cache
 * slots [vLLM flash_attn.py (e2f56c3), FlashAttentionImpl.forward, the
 * reshape_and_cache_flash call; Aphrodite flash_attn.py, the
 * reshape_and_cache_flash custom op].
 *
 *   key, value      [>= num_tokens rows, num_kv_heads, head_size]; row i
 *                   starts at key + i * key_token_stride (elements); heads
 *                   and head elements are contiguous within a row.
 *   key_cache,
 *   value_cache     [num_blocks, block_size, num_kv_heads, head_size].
 *   slot_mapping    int64 [num_tokens]; token i goes to block
 *                   slot / block_size, offset slot % block_size.  A negative
 *                   slot is padding and is skipped.  num_tokens is the length
 *                   of slot_mapping; key/value may hold more (padded) rows.
 *   dtype           of key / value (PA_F16 or PA_BF16).
 *   kv_cache_dtype  dtype: rows are copied bit-exactly (kv_cache_dtype
 *                   "auto", no conversion); PA_FP8_E4M3: each element is
 *                   quantised with k_scale (keys) or v_scale (values) as
 *                   described above, and the caches hold the codes.
 *   Two tokens mapped to the same slot race (the caller must not do that).
 *   num_tokens == 0 is a no-op.
 */
int reshape_and_cache(const void* key, const void* value,
                      int64_t key_token_stride, int64_t value_token_stride,
                      void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int64_t num_tokens,
                      int64_t num_blocks, int block_size, int num_kv_heads,
                      int head_size, pa_dtype_t dtype,
                      pa_dtype_t kv_cache_dtype, const float* k_scale,
                      const float* v_scale, void* stream);

/*
 * paged_attn_prefill — variable-length attention of new query tokens over
 * the paged cache (prefill chunks, or any mix of query lengths)
 * [vLLM flash_attn.py (e2f56c3), FlashAttentionImpl.forward, the
 * flash_attn_varlen_func call with block_table and seqused_k].
 *
 *   out             [total_q, num_heads, head_size] (dtype).
 *   lse             nullable; fp32 [num_heads, total_q], natural log.
 *   q               [total_q, num_heads, head_size] (dtype), contiguous.
 *   cu_seqlens_q    int32 [num_seqs + 1]: queries of sequence b are rows
 *                   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1.
 *   seq_lens        int32 [num_seqs]: keys of sequence b (context + its new
 *                   tokens, which must already be in the cache); the query
 *                   rows are the LAST positions: row t of b sits at position
 *                   p = seq_lens[b] - q_len_b + t.
 *   block_table     int32, row b at block_table + b * block_table_stride.
 *   max_seqlen_q    host upper bound of the query lengths (sizes the grid).
 *   max_seqlen_k    host upper bound of seq_lens.
 *   scale           softmax scale applied to q.k.
 *   causal          nonzero: key j visible to position p iff j <= p.
 *   window_left     -1: none; else also require j >= p - window_left (a
 *                   sliding window w is passed as w - 1).
 *   softcap         0: off; else s = softcap * tanh(s / softcap) on the
 *                   scaled score.
 *   alibi_slopes    nullable; fp32 [num_heads]; adds -slope_h * |p - j|
 *                   after the softcap.
 *   sinks           nullable; fp32 [num_heads] attention-sink logits [vLLM
 *                   flash_attn.py (e2f56c3), FlashAttentionImpl sinks,
 *                   passed to the kernel as s_aux]: each adds e^{sink_h} to
 *                   its head's softmax denominator and no value, so
 *                   out = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sink_h})
 *                   and lse = ln(sum_j e^{s_j} + e^{sink_h}).
 *   Query head h reads KV head h / (num_heads / num_kv_heads).
 *   A query that sees no key gets out = 0 and lse = -inf (lse = sink_h
 *   with sinks).
 *   kv_cache_dtype, k_scale, v_scale: a 16-bit cache (= dtype) or an fp8
 *                   cache with its scales (see the conventions above); the
 *                   K scale multiplies every score and the V scale the
 *                   result, and the products run on the 16-bit values of
 *                   the codes (exact), as for a 16-bit cache.
 *   PA_ERR_UNSUPPORTED also for num_seqs > 65535, more than 128 query heads
 *   per KV head, max_seqlen_k >= 2^24, num_kv_heads * max_seqlen_q >= 2^31
 *   or num_kv_heads * (total_q + num_seqs) >= 2^31 (grid limits).  The
 *   grid is sized from total_q, so cu_seqlens_q[num_seqs] must not exceed
 *   total_q (q's row count).
 */
int paged_attn_prefill(void* out, float* lse, const void* q,
                       const void* key_cache, const void* value_cache,
                       const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                       const int32_t* block_table, int64_t block_table_stride,
                       int num_seqs, int64_t total_q, int max_seqlen_q,
                       int max_seqlen_k, int num_heads, int num_kv_heads,
                       int head_size, int block_size, int64_t num_blocks,
                       float scale, int causal, int window_left, float softcap,
                       const float* alibi_slopes, const float* sinks,
                       pa_dtype_t dtype, pa_dtype_t kv_cache_dtype,
                       const float* k_scale, const float* v_scale,
                       const float* q_scale, void* stream);

/*
 * paged_attn_decode — one query token per sequence over the paged cache,
 * optionally split along the keys [Aphrodite flash_attn.py,
 * FlashAttentionImpl.forward, the flash_attn_with_kvcache decode call;
 * vLLM flash_attn.py (e2f56c3), FlashAttentionMetadataBuilder, num_splits
 * and its [num_splits, num_heads, num_tokens, head_size] intermediates;
 * vLLM flashinfer.py, FlashInferMetadataBuilder, fixed_split_size].
 *
 *   q               [num_seqs, num_heads, head_size] (dtype); the query of
 *                   sequence b sits at position seq_lens[b] - 1.
 *   seq_lens        int32 [num_seqs]; block_table as for prefill.
 *   num_splits == 1 writes out [num_seqs, num_heads, head_size] (dtype) and,
 *                   if lse != NULL, lse fp32 [num_heads, num_seqs].
 *   num_splits  > 1 writes only part_out fp32 [num_splits, num_seqs,
 *                   num_heads, head_size] and part_lse fp32 [num_splits,
 *                   num_heads, num_seqs]; out and lse are not touched (may be
 *                   NULL).  Every sequence is cut into the same fixed,
 *                   block-aligned chunks sized from the batch bound:
 *                   c = block_size * ceil(ceil(max_seq_len / num_splits) /
 *                   block_size); split p of sequence b covers keys
 *                   [p*c, min((p+1)*c, L)), and the last split also takes
 *                   any keys past num_splits*c (so a loose max_seq_len
 *                   still covers the sequence).  An empty split writes
 *                   part_out = 0, part_lse = -inf.  Combine with
 *                   merge_attn_states(out, lse, part_out, part_lse,
 *                   num_splits, num_seqs, num_heads, head_size, PA_F32, ...).
 *   max_seq_len     host upper bound of seq_lens (sizes the splits).
 *   window_left, softcap, alibi_slopes, sinks as for prefill.  With
 *   num_splits > 1 the sinks join split 0 only, so the merged result
 *   counts each once.  num_splits <= 256.
 *   kv_cache_dtype, k_scale, v_scale: a 16-bit cache (= dtype) or an fp8
 *   cache with its scales (see the conventions above); the K scale
 *   multiplies every score and the V scale the result.
 *   num_heads / num_kv_heads must be at most 128 [vLLM flash_attn.py
 *   (e2f56c3), FlashAttentionImpl.__init__: any num_queries_per_kv =
 *   num_heads / num_kv_heads].
 */
int paged_attn_decode(void* out, float* lse, float* part_out, float* part_lse,
                      const void* q, const void* key_cache,
                      const void* value_cache, const int32_t* seq_lens,
                      const int32_t* block_table, int64_t block_table_stride,
                      int num_seqs, int max_seq_len, int num_heads,
                      int num_kv_heads, int head_size, int block_size,
                      int64_t num_blocks, float scale, int window_left,
                      float softcap, const float* alibi_slopes,
                      const float* sinks, int num_splits, pa_dtype_t dtype,
                      pa_dtype_t kv_cache_dtype, const float* k_scale,
                      const float* v_scale, const float* q_scale, void* stream);

/*
 * paged_attn_decode_merged — paged_attn_decode with the splits merged
 * inside the same launch: out [num_seqs, num_heads, head_size] (dtype) and,
 * if lse != NULL, lse fp32 [num_heads, num_seqs] receive what
 * paged_attn_decode followed by merge_attn_states(out, lse, part_out,
 * part_lse, num_splits, ...) gives, the same arithmetic in the same order
 * [vLLM flash_attn.py (e2f56c3), FlashAttentionMetadataBuilder, the
 * split-KV intermediates; merge_attn_states].  Every split writes its
 * partial result to part_out / part_lse (as paged_attn_decode, except
 * that splits without visible keys write nothing); the split of a
 * (sequence, group of query heads) that finishes last merges the partials
 * of its group, counting arrivals in split_counters.
 *
 *   split_counters  int32 [num_seqs * num_heads], device, caller-owned
 *                   workspace that must be all zero on entry (e.g. once,
 *                   after allocation); every call leaves it all zero.
 *                   Calls that overlap on one counters array race.
 *   part_out, part_lse as for paged_attn_decode (overwritten workspace).
 *   num_splits == 1: the plain single-pass decode (the workspaces are not
 *   used and may be NULL).  Other arguments and errors as paged_attn_decode.
 *   One launch instead of two; every split item then waits for its
 *   device-coherent partial stores and its count before it ends, which on
 *   MI355X costs more than the separate merge launch for a 64-sequence,
 *   8-split batch (145 us against 130 + 6 us).
 */
int paged_attn_decode_merged(void* out, float* lse, float* part_out, float* part_lse,
                             int32_t* split_counters, const void* q,
                             const void* key_cache, const void* value_cache,
                             const int32_t* seq_lens, const int32_t* block_table,
                             int64_t block_table_stride, int num_seqs, int max_seq_len,
                             int num_heads, int num_kv_heads, int head_size, int block_size,
                             int64_t num_blocks, float scale, int window_left, float softcap,
                             const float* alibi_slopes, const float* sinks, int num_splits,
                             pa_dtype_t dtype, pa_dtype_t kv_cache_dtype,
                             const float* k_scale, const float* v_scale,
                             const float* q_scale, void* stream);

/*
 * paged_attn_decode_noalloc — for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): paged_attn_decode with num_splits parts followed by
 * merge_attn_states into out / lse, with the fp32 partial results kept in a
 * fixed device array of the library instead of caller workspace.  Nothing
 * is allocated by the call.
 *
 *   Arguments as for paged_attn_decode without part_out / part_lse; out is
 *   required and receives the merged result [num_seqs, num_heads, head_size]
 *   (dtype), lse (nullable) fp32 [num_heads, num_seqs].  num_splits == 1
 *   writes out directly and uses no scratch.
 *   Limit: num_splits * num_seqs * num_heads * (head_size + 1) * 4 bytes (plus
 *   up to 255 bytes of alignment) must fit the 32 MiB scratch, else
 *   PA_ERR_UNSUPPORTED and nothing is enqueued.
 *   The scratch is one array per GPU, held until the process ends and
 *   shared by every call on that GPU: calls that overlap on one GPU (two
 *   streams, or two threads) race on it.  Its contents are fully rewritten
 *   by each call before they are read; nothing needs clearing.
 */
int paged_attn_decode_noalloc(void* out, float* lse, const void* q,
                              const void* key_cache, const void* value_cache,
                              const int32_t* seq_lens, const int32_t* block_table,
                              int64_t block_table_stride, int num_seqs,
                              int max_seq_len, int num_heads, int num_kv_heads,
                              int head_size, int block_size, int64_t num_blocks,
                              float scale, int window_left, float softcap,
                              const float* alibi_slopes, const float* sinks,
                              int num_splits, pa_dtype_t dtype,
                              pa_dtype_t kv_cache_dtype, const float* k_scale,
                              const float* v_scale, const float* q_scale,
                              void* stream);

/*
 * merge_attn_states — combine partial attention results by their
 * log-sum-exp [vLLM flash_attn.py (e2f56c3), cascade_attention and
 * _forward_with_dcp, merge_attn_states(out, a_out, a_lse, b_out, b_lse)].
 *
 *   parts_out       [num_parts, num_tokens, num_heads, head_size] in
 *                   parts_dtype (PA_F32, PA_F16 or PA_BF16).
 *   parts_lse       fp32 [num_parts, num_heads, num_tokens], natural log.
 *   out             [num_tokens, num_heads, head_size] in out_dtype
 *                   (PA_F32, PA_F16 or PA_BF16).
 *   out_lse         nullable; fp32 [num_heads, num_tokens].
 *   Per (t, h): M = max_p lse_p, w_p = exp(lse_p - M),
 *   out = sum_p w_p out_p / sum_p w_p, out_lse = M + ln(sum_p w_p); if every
 *   part is -inf, out = 0 and out_lse = -inf.  1 <= num_parts <= 256.
 */
int merge_attn_states(void* out, float* out_lse, const void* parts_out,
                      const float* parts_lse, int num_parts,
                      int64_t num_tokens, int num_heads, int head_size,
                      pa_dtype_t parts_dtype, pa_dtype_t out_dtype,
                      void* stream);

/*
 * paged_attn_cascade — causal prefill of a batch whose sequences share their
 * first common_prefix_len keys, computed the cascade way [vLLM flash_attn.py
 * (e2f56c3), cascade_attention]: every query against the shared prefix once
 * (non-causal, through block_table row 0), each sequence's queries against
 * its own keys after the prefix (causal, through the rest of its row), and
 * the log-sum-exp merge of the two.  The result equals paged_attn_prefill
 * with causal = 1 on the same batch; the shared prefix is read once for the
 * batch rather than once per sequence.
 *
 *   Arguments as for paged_attn_prefill (16-bit or fp8 cache; causal, no
 *   window, no ALiBi: the page's cascade supports neither), plus
 *   sinks              nullable, as for prefill; folded into the prefix
 *                      part only (the page adds s_aux to the prefix LSE);
 *   common_prefix_len  > 0, a multiple of block_size, below max_seqlen_k.
 *                      The caller guarantees (device data, not checked):
 *                      the first common_prefix_len / block_size entries of
 *                      every block-table row are the same blocks, and every
 *                      sequence's queries come after the prefix
 *                      (seq_len - query_len >= common_prefix_len).
 *   max_prefix_splits  1..255: the workspaces hold max_prefix_splits + 1
 *                      partial results.  The prefix pass may split the
 *                      prefix keys into up to max_prefix_splits parts (it
 *                      does when there are few queries, as in a decode
 *                      batch, so that the pass fills the GPU); the suffix
 *                      pass may split each sequence's own keys into up to 4
 *                      (when there are few sequences), the prefix then
 *                      taking correspondingly fewer;
 *   parts_out          workspace [max_prefix_splits + 1, total_q, num_heads,
 *                      head_size] of dtype (prefix parts, then the suffix
 *                      parts);
 *   parts_lse          fp32 workspace [max_prefix_splits + 1, num_heads,
 *                      total_q];
 *   work_ints          reserved, nullable, not accessed.
 *   Workspaces are caller-owned and overwritten; num_kv_heads * (total_q +
 *   num_seqs) must be below 2^31.
 */
int paged_attn_cascade(void* out, float* lse, const void* q,
                       const void* key_cache, const void* value_cache,
                       const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                       const int32_t* block_table, int64_t block_table_stride,
                       int num_seqs, int64_t total_q, int max_seqlen_q,
                       int max_seqlen_k, int num_heads, int num_kv_heads,
                       int head_size, int block_size, int64_t num_blocks,
                       float scale, float softcap, const float* sinks,
                       int common_prefix_len, int max_prefix_splits,
                       void* parts_out, float* parts_lse,
                       int32_t* work_ints, pa_dtype_t dtype,
                       pa_dtype_t kv_cache_dtype, const float* k_scale,
                       const float* v_scale, const float* q_scale, void* stream);

/*
 * scaled_fp8_quant — quantise a 16-bit tensor to fp8 (e4m3) codes with a
 * static per-tensor scale, as the attention layer does to the query when
 * the cache is fp8 [vLLM flash_attn.py (v0.9.0.1 docs),
 * FlashAttentionImpl.forward, ops.scaled_fp8_quant(query, layer._q_scale)].
 *
 *   input     num_elems elements of dtype (PA_F16 / PA_BF16), contiguous.
 *   out       num_elems one-byte codes: out[i] = code of input[i] / *scale,
 *             rounded as the cache codes are (see the conventions above).
 *   scale     device fp32 scalar (the attention's q_scale / q_descale).
 *   num_elems == 0 is a no-op.
 */
int scaled_fp8_quant(void* out, const void* input, const float* scale,
                     int64_t num_elems, pa_dtype_t dtype, void* stream);

/*
 * pa_use_cascade — HOST-side decision whether a batch should take
 * paged_attn_cascade rather than the plain path [vLLM flash_attn.py
 * (e2f56c3), use_cascade_attention].  The page's support checks, in its
 * order: no cascade when common_prefix_len < 256, with ALiBi, a sliding
 * window or chunked local attention, with fewer than 8 requests, or with
 * decode context parallelism (dcp_world_size > 1).  Then, as on the page, a
 * batch that would not take split-KV decode (a request with more than one
 * query, or one query head per KV head) takes the cascade.  For a decode
 * batch the page compares CTA waves of its kernels on `num_sms`
 * multiprocessors; here the comparison is between time models of this
 * library's two paths on MI355X (paged_attn_decode with splits +
 * merge_attn_states against paged_attn_cascade), calibrated on measured
 * times of decode batches of 8..128 requests with 256..8192 shared keys:
 * fixed costs, unique and re-read K/V bytes, the prefix pass's MFMA work
 * and a cost per request.  (On every measured batch the cascade was the
 * faster path, so there the decision is the support checks'.)
 *
 *   query_lens, seq_lens  HOST int32 [num_reqs]: new queries and keys
 *                         (including the prefix) of each request.
 *   kv_elem_bytes         2 for a 16-bit cache, 1 for fp8.
 *   Returns 1 (use the cascade), 0 (do not), or a negative code.  No
 *   device work.
 */
int pa_use_cascade(int common_prefix_len, const int32_t* query_lens,
                   const int32_t* seq_lens, int num_reqs, int num_heads,
                   int num_kv_heads, int head_size, int kv_elem_bytes,
                   int use_alibi, int use_sliding_window,
                   int use_local_attention, int dcp_world_size);

/*
 * pa_local_virtual_batches — HOST-side rewriting of a batch for chunked
 * local attention [vLLM flash_attn.py (v0.9.0.1 docs),
 * make_local_attention_virtual_batches]: positions are cut into chunks of
 * attn_chunk_size tokens and a query sees only the keys of its own chunk up
 * to itself.  Each (sequence, chunk holding some of its queries) becomes one
 * virtual sequence whose queries are those rows (same order: q and out stay
 * as they are), whose keys run from the chunk start to its last query, and
 * whose block-table row is the sequence's row from the chunk's first block
 * (attn_chunk_size / block_size entries, clipped to the last column).
 * paged_attn_prefill (causal) over the virtual batch is the chunked
 * attention of the original one.
 *
 *   All arrays are HOST arrays.  query_start_loc int32 [num_seqs + 1],
 *   seq_lens int32 [num_seqs] (keys, >= the sequence's queries),
 *   block_table int32 rows of block_table_stride entries of which the first
 *   block_table_cols are valid.  attn_chunk_size a positive multiple of
 *   block_size.
 *   Outputs (all NULL: only count; else all given, caller-owned, room for
 *   max_virtual sequences): seqlens_q_local [V], cu_seqlens_q_local [V + 1],
 *   seqlens_k_local [V], block_table_local [V, attn_chunk_size / block_size].
 *   Returns V >= 0, the number of virtual sequences, or a negative code
 *   (nothing written on error).  No device work.
 */
int pa_local_virtual_batches(int attn_chunk_size, int block_size,
                             const int32_t* query_start_loc,
                             const int32_t* seq_lens, int num_seqs,
                             const int32_t* block_table,
                             int64_t block_table_stride, int block_table_cols,
                             int max_virtual, int32_t* seqlens_q_local,
                             int32_t* cu_seqlens_q_local,
                             int32_t* seqlens_k_local,
                             int32_t* block_table_local);

/*
 * pa_check_indices — debug validation of the device index arrays that the
 * calls above trust (their contents are undefined behaviour when out of
 * range).  Optional, for tests and debugging; not on the hot path.
 * [vLLM flash_attn.py (e2f56c3), FlashAttentionImpl.forward: slot_mapping
 * addresses cache slots, block_table maps each sequence's logical blocks;
 * Aphrodite flash_attn.py, FlashAttentionMetadata, block_tables.]
 *
 *   slot_mapping    int64 [num_tokens] or NULL when num_tokens == 0.
 *   block_table     int32 rows of block_table_stride entries, one per
 *                   sequence; seq_lens int32 [num_seqs].  Both may be NULL
 *                   when num_seqs == 0.
 *   counts          int32 [3], device, caller-owned; overwritten with
 *     counts[0]  slots >= num_blocks * block_size (negative slots are
 *                padding and allowed);
 *     counts[1]  block ids outside [0, num_blocks) among the entries a call
 *                reads: the first ceil(seq_lens[b] / block_size) of row b
 *                (padding past them is not looked at);
 *     counts[2]  sequences with a negative length, or with more blocks than
 *                a row holds (their rows are not read).  A row holds
 *                block_table_stride entries: the calls take no separate
 *                count of valid columns, so the stride is the row length
 *                they may read up to (a caller whose table has fewer valid
 *                columns than its stride must keep seq_lens within them).
 *   Enqueued on `stream` like the other calls; read counts after it.
 *   block_size a positive multiple of 16; num_blocks > 0.
 */
int pa_check_indices(const int64_t* slot_mapping, int64_t num_tokens,
                     const int32_t* block_table, int64_t block_table_stride,
                     const int32_t* seq_lens, int num_seqs, int64_t num_blocks,
                     int block_size, int32_t* counts, void* stream);

/*
 * pa_trace_set — timeline tracing, for profiling (not part of the
 * attention path).  Only the trace build of the library
 * (libpagedattn_trace.so, built with PA_TRACE=1) records anything; the
 * regular library returns PA_ERR_UNSUPPORTED.  buffer: NULL (off), or a
 * device array of 16 uint64 per workgroup of the largest prefill / decode
 * launch that follows; each workgroup writes shader-clock times of its
 * phases (entry, work item known, key loop start, key loop end, results
 * stored), its CU's HW_ID and XCC_ID, the key tiles or steps it ran, its
 * item (sequence << 32 | query tile or split) and each wave's end time.
 * The times of different shader engines are not on one clock.  Process-
 * wide setting; launches that overlap share the buffer.
 */
int pa_trace_set(void* buffer);

/* Message describing the last non-OK return on the calling thread ("" if
 * none).  The string is owned by the library and valid until the next call
 * on this thread. */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
