/*
 * pa.h — paged-KV decode attention for AMD Instinct MI355X (gfx950).
 *
 * A plain C ABI: every buffer is a pointer to caller-allocated DEVICE memory,
 * every size is a plain integer, and the stream is a hipStream_t passed as
 * void* (NULL = the default stream).  No HIP or framework types appear here.
 *
 * The problem, as the source pages frame it:
 *   - a batch of sequences, each with its own context length (Dragon
 *     "Inference Service" developer guide, "vLLM Integration": max_num_seqs
 *     and max_model_len bound the batch and the context);
 *   - one shared pool of fixed-size KV pages addressed through per-sequence
 *     block tables (llm-d router blog post, engine metric spec: page_size and
 *     num_pages; vLLM "EngineCoreClient" page, "Archivos clave":
 *     num_gpu_blocks and block_size reported as the real cache capacity);
 *   - pages shared across sequences by prefix reuse (llm-d blog post,
 *     prefix-cache producer section); the device code only ever reads them;
 *   - decode attention, named there as paged attention under continuous
 *     batching and described as memory-bandwidth bound (llm-d blog post,
 *     opening section and the disaggregated P/D paragraph).
 *
 * Pool layout (page_size = 16 tokens, "head-major": a page id selects one
 * contiguous block holding every kv head, and each (page, kv head) tile is
 * itself contiguous):
 *     k_cache[num_pages][num_kv_heads][16][head_dim]     key rows per slot
 *     v_cache[num_pages][num_kv_heads][head_dim][16]     value columns per slot
 * Token position t of sequence b is stored at page block_tables[b][t / 16],
 * in-page slot t % 16.  Element types: float32 or bf16 (PA_DTYPE_*); query,
 * output, key/value inputs and both pools share one element type.
 *
 * Attention (the reading taken of the pages, which never write the formula):
 *     out[b][h] = sum_{t < L_b} softmax_t(scale * q[b][h] . k[b][t][g]) v[b][t][g]
 *     with g = h / (num_q_heads / num_kv_heads)   (contiguous GQA groups).
 * Accumulation is in float32; bf16 outputs are rounded to nearest even.
 *
 * Ownership and ordering: the library never allocates, frees or
 * synchronizes.  Each call validates its arguments on the host, enqueues its
 * kernels on `stream` and returns; buffers must stay alive and unmodified
 * until the stream has passed the call (the same lifetime rule the vLLM
 * EngineCoreClient page describes for tensors in flight, "Archivos clave",
 * SyncMPClient send path).  Results are deterministic: they depend only on
 * the logical token order, never on physical page placement or sharing.
 *
 * Errors (TensorRT Edge-LLM "HTTP Inference Server Architecture", "Extension
 * Rules": unsupported options are rejected, never silently ignored):
 *   PA_ERR_INVALID_ARGUMENT  a NULL pointer, a negative count, or
 *                            inconsistent sizes; nothing was launched;
 *   PA_ERR_UNSUPPORTED       head_dim not 64/128, page_size not 16, an
 *                            unknown dtype, or a GQA group above 16;
 *                            nothing was launched;
 *   PA_ERR_LAUNCH            the HIP launch itself failed.
 * Device data (block-table entries, lengths, slots) is not validated on the
 * host, since that would need a synchronization.  Kernels skip out-of-range
 * page ids and slots instead of faulting; the affected outputs are then
 * unspecified.  Device faults surface asynchronously at the caller's next
 * synchronization and leave the HIP context unusable (compare the vLLM
 * EngineCoreClient page, "Límites y fallos": engine death is detected late
 * and is final).
 */
#ifndef PA_H
#define PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,
  PA_ERR_UNSUPPORTED = 2,
  PA_ERR_LAUNCH = 3,
  PA_ERR_SCRATCH_LIMIT = 4
} pa_status;

typedef enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 } pa_dtype;

#define PA_PAGE_SIZE 16
#define PA_MAX_GQA_GROUP 16
/* Size of the per-GPU scratch array of pa_chunk_attention_split_noalloc. */
#define PA_SCRATCH_BYTES (64 * 1024 * 1024)

/*
 * pa_reshape_and_cache — the slot-mapped cache write.
 *
 * For every token t in [0, num_tokens) with slot = slot_mapping[t] >= 0:
 *     k_cache[slot / 16][h][slot % 16][:]  = key[t][h][:]
 *     v_cache[slot / 16][h][:][slot % 16]  = value[t][h][:]    for every kv head h.
 * A negative slot writes nothing (padding tokens).  Slots at or beyond
 * num_pages * 16 are skipped.  The copy is bit-exact.
 *
 *   key, value     [num_tokens][num_kv_heads][head_dim], contiguous.
 *   k_cache,
 *   v_cache        the pools, layout above.
 *   slot_mapping   int64 [num_tokens], device.
 *
 * Single writer: non-negative slots must be distinct and must not lie in a
 * page that another sequence's block table also references (a shared prefix
 * page is read-only; TensorRT Edge-LLM "HTTP Inference Server
 * Architecture", "Request Lifecycle": one writer owns retained pages).
 * Violations give unspecified pool contents.  num_tokens == 0 is a no-op.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                         int head_dim, int page_size, int64_t num_pages, int dtype,
                         void* stream);

/*
 * pa_decode — one query token per sequence attends over its paged context.
 *
 *   out            [num_seqs][num_q_heads][head_dim] (dtype); written only
 *                  when partition_size == 0.
 *   query          [num_seqs][num_q_heads][head_dim] (dtype).
 *   k_cache,
 *   v_cache        the pools, [num_pages] pages, layout above.
 *   block_tables   int32 [num_seqs][max_pages_per_seq]; entries at and past
 *                  ceil(L_b / 16) never affect the result (padding may hold
 *                  -1).  Column 0 of every row is read even when L_b = 0:
 *                  in batches of up to 1024 sequences, a sequence whose
 *                  first page also starts another sequence (prefix reuse)
 *                  has its pages loaded through the caches and every other
 *                  sequence streams its pages with the nontemporal hint;
 *                  larger batches load every page through the caches.
 *   context_lens   int32 [num_seqs]; L_b counts every cached token of
 *                  sequence b, including one appended this step.  0 yields a
 *                  zero output.  Lengths above 16 * max_pages_per_seq are
 *                  clamped to it; with split-KV, each partition past the
 *                  clamped context but below min(ceil(L_b / partition_size),
 *                  max_num_partitions) gets an empty partial (out 0, max
 *                  -inf, sum 0), so pa_decode_reduce merges the clamped
 *                  context.
 *   scale          multiplies q . k before the softmax (normally 1/sqrt(D)).
 *   partition_size 0: single pass, `out` is written directly and the partial
 *                  buffers may be NULL.  Otherwise a positive multiple of 16:
 *                  split-KV — the context of every sequence is cut at
 *                  multiples of partition_size tokens from position 0 and each
 *                  partition p < ceil(L_b / partition_size) writes
 *                      partial_max[b][h][p] = m   (a reference score, in
 *                                                  the units of scale*q.k)
 *                      partial_sum[b][h][p] = sum_t exp(s_t - m)
 *                      partial_out[b][h][p][:] = sum_t exp(s_t - m) v_t / partial_sum
 *                  over its tokens; pa_decode_reduce then produces `out`.
 *                  m need not be the exact maximum; any reference that keeps
 *                  the exponentials finite gives the same merged result.
 *   max_num_partitions  partition dimension of the partial buffers (>= 1 when
 *                  splitting).  Partitions at or beyond it are not computed
 *                  and their rows are never written; the merge then covers
 *                  the first max_num_partitions * partition_size tokens.
 *   partial_out    float32 [num_seqs][num_q_heads][max_num_partitions][head_dim]
 *   partial_max,
 *   partial_sum    float32 [num_seqs][num_q_heads][max_num_partitions]
 *
 * Requirements: num_q_heads % num_kv_heads == 0, the group
 * num_q_heads / num_kv_heads <= 16, head_dim in {64, 128}, page_size == 16.
 * num_seqs == 0 is a no-op.
 */
int pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
              int num_q_heads, int num_kv_heads, int head_dim, int page_size,
              int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
              int max_num_partitions, float* partial_out, float* partial_max,
              float* partial_sum, int dtype, void* stream);

/*
 * pa_chunk_attention — several new query tokens per sequence, causal.
 *
 * The step beside decode that chunked prefill and the verification of
 * drafted tokens run (llm-d blog post, the two phases of inference and the
 * disaggregated P/D paragraph; TensorRT Edge-LLM "HTTP Inference Server
 * Architecture", "Model Loading": an optional draft checkpoint).  Sequence b
 * has q_len_b = query_start[b + 1] - query_start[b] new tokens: the last
 * q_len_b positions of its context, whose K/V are already in the pools (write
 * them with pa_reshape_and_cache first).  Query row query_start[b] + i is
 * the token at position p = L_b - q_len_b + i and attends to positions 0..p:
 *     out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . k[b][t][g]) v[b][t][g]
 * With q_len_b = 1 for every b this is pa_decode's single-pass result.
 *
 *   out            [num_query_tokens][num_q_heads][head_dim], bf16; rows of
 *                  every sequence are written.
 *   query          [num_query_tokens][num_q_heads][head_dim], bf16.
 *   query_start    int32 [num_seqs + 1], device: nondecreasing, query_start[0]
 *                  = 0, query_start[num_seqs] = num_query_tokens.
 *   max_query_len  host bound on q_len_b (sizes the grid); 0 <= q_len_b <=
 *                  min(max_query_len, L_b) is required of the device data (a
 *                  sequence with no new token has no rows).
 *   the rest       as in pa_decode (pools, block tables, context lengths,
 *                  scale, page size).
 * Results are deterministic and do not depend on page placement.  With
 * max_query_len * (num_q_heads / num_kv_heads) above 64 a kernel that stages
 * K/V in LDS for 128 or 256 columns at a time runs instead of the 16-column
 * one: the same results to rounding, so bits can change with max_query_len
 * across that bound.  A sequence
 * whose q_len_b exceeds L_b gets unspecified rows, and one whose rows fall
 * outside [0, num_query_tokens) gets none written (no fault either way).  bf16 only:
 * PA_DTYPE_F32 returns PA_ERR_UNSUPPORTED.  max_query_len above
 * num_query_tokens, or a NULL pointer, returns PA_ERR_INVALID_ARGUMENT;
 * num_seqs, num_query_tokens or max_query_len of 0 is a no-op.
 */
int pa_chunk_attention(void* out, const void* query, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, int num_seqs, int num_query_tokens,
                       int max_query_len, int num_q_heads, int num_kv_heads, int head_dim,
                       int page_size, int max_pages_per_seq, int64_t num_pages, float scale,
                       int dtype, void* stream);

/*
 * pa_chunk_attention_split — pa_chunk_attention as split-KV work units and
 * their log-sum-exp merge, in one call, for callers that want the split
 * decode's partial layout per new token (or, through the _noalloc form
 * below, no caller workspace).  The same contraction as pa_chunk_attention;
 * the partitions and their merge are those of pa_decode (split) and
 * pa_decode_reduce, per new token.
 *
 *   partition_size      tokens per partition, a positive multiple of 16.
 *   max_num_partitions  partition slots per row: ceil(L_b / partition_size)
 *                       <= max_num_partitions is required of the device data.
 *   partial_out         [num_query_tokens][num_q_heads][max_num_partitions][head_dim]
 *                       fp32 (16-byte aligned); partial_max, partial_sum
 *                       [num_query_tokens][num_q_heads][max_num_partitions]
 *                       fp32: caller-owned workspace, overwritten.  A token
 *                       whose position precedes a whole partition gets an
 *                       empty partial there (o = 0, max = -inf, sum = 0).
 *   the rest            as in pa_chunk_attention.
 * Results match pa_chunk_attention to rounding (the partial sums group the
 * keys by partition) and are deterministic.  Errors as for
 * pa_chunk_attention, plus PA_ERR_INVALID_ARGUMENT for partition_size <= 0
 * or not a multiple of 16, max_num_partitions < 1, or a NULL or misaligned
 * workspace.
 */
int pa_chunk_attention_split(void* out, const void* query, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables,
                             const int32_t* context_lens, const int32_t* query_start,
                             int num_seqs, int num_query_tokens, int max_query_len,
                             int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                             int max_pages_per_seq, int64_t num_pages, float scale,
                             int partition_size, int max_num_partitions, float* partial_out,
                             float* partial_max, float* partial_sum, int dtype, void* stream);

/*
 * pa_chunk_attention_split_noalloc — pa_chunk_attention_split without the
 * caller's workspace, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The split partials live in a fixed array of PA_SCRATCH_BYTES
 * (64 MiB) per GPU, part of the library's device image, held until the
 * process ends; its address is looked up once per device, on the first call
 * with that device current.  The call allocates and frees nothing.
 *
 * Arguments, results and errors as for pa_chunk_attention_split, without
 * partial_out / partial_max / partial_sum.  The partials take
 * num_query_tokens * num_q_heads * max_num_partitions * (head_dim + 2) * 4
 * bytes; a call that needs more than PA_SCRATCH_BYTES returns
 * PA_ERR_SCRATCH_LIMIT and launches nothing (e.g. 64 sequences x 8 drafted
 * tokens x 32 heads x 6 partitions at head_dim 128 take 51 MB).  Nothing in
 * the array needs to start at any value: every partial the merge reads is
 * written earlier in the same call.  Every call on one GPU shares that GPU's
 * array: calls that may overlap on one GPU (different streams without
 * ordering between them, or several host threads) race and give unspecified
 * results; calls ordered on one stream are safe.
 */
int pa_chunk_attention_split_noalloc(void* out, const void* query, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* query_start,
                                     int num_seqs, int num_query_tokens, int max_query_len,
                                     int num_q_heads, int num_kv_heads, int head_dim,
                                     int page_size, int max_pages_per_seq, int64_t num_pages,
                                     float scale, int partition_size, int max_num_partitions,
                                     int dtype, void* stream);

/*
 * pa_decode_append — one decode step in one call: write each sequence's new
 * token into the pool, then attend over every cached token.
 *
 * The result (pool and outputs, bit for bit) equals pa_reshape_and_cache(key,
 * value, k_cache, v_cache, slot_mapping, num_tokens = num_seqs, ...) followed
 * by pa_decode(...) with the other arguments as given, provided every
 * slot_mapping[b] is either negative (nothing written) or the slot of the
 * sequence's last position, block_tables[b][(L_b - 1) / 16] * 16 +
 * (L_b - 1) % 16 (the step that appends token L_b - 1 and attends over it;
 * any other slot gives unspecified results).
 *   key, value    [num_seqs][num_kv_heads][head_dim], dtype; key 16-byte aligned.
 *   slot_mapping  [num_seqs] int64, device.
 * For bf16 the write happens inside the decode launch: the work unit that
 * reads a sequence's last page stores the new K row and V column first and
 * then streams that page (one kernel instead of two).  fp32 runs the two
 * kernels back to back.  Errors as for pa_decode, plus
 * PA_ERR_INVALID_ARGUMENT for a NULL key, value or slot_mapping.
 */
int pa_decode_append(void* out, const void* query, const void* key, const void* value,
                     const int64_t* slot_mapping, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                     int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                     int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
                     int max_num_partitions, float* partial_out, float* partial_max,
                     float* partial_sum, int dtype, void* stream);

/*
 * pa_decode_cascade — split-KV decode that reads pages shared by a group of
 * sequences once per group (prefix reuse: llm-d blog post, prefix-cache
 * sections; requests with a common prompt prefix point at the same pages).
 *
 * Group g's members are group_seqs[group_start[g] .. group_start[g + 1]) (batch
 * indices).  They hold the same physical page ids in block-table columns
 * 0 .. group_partitions[g] * (partition_size / 16) - 1, and every token of
 * those pages lies inside every member's context.  For each such partition and
 * kv head one work unit reads the pages once and computes every member's
 * partial for it: the members' query heads are the columns of the matrix
 * tiles, up to 32 per wave.  In the same launch, units of four waves per
 * (sequence, partition, kv head) compute each sequence's partitions from
 * seq_first_partition[b] on (0 for sequences in no group).  With
 * key/value/slot_mapping non-NULL those units also write the step's new
 * token, as pa_decode_append does.  The partial arrays end up as pa_decode
 * (split) writes them: merge them with pa_decode_reduce.
 *
 *   num_groups, max_group_size, max_group_partitions  host bounds that size
 *               the grid: groups of more members or partitions are not fully
 *               computed (unspecified results).  max_group_partitions must
 *               not exceed max_num_partitions.
 *   max_suffix_partitions  host bound on min(ceil(L_b / partition_size),
 *               max_num_partitions) - seq_first_partition[b] over the batch:
 *               the grid holds that many partitions per sequence, counted
 *               from its first.  A smaller value than the
 *               true maximum leaves partitions uncomputed (unspecified
 *               results); 0 means max_num_partitions (always enough, at the
 *               cost of workgroups that find nothing to do).  Units whose
 *               partition would reach max_num_partitions are skipped.
 *               pa_pager_prefix_groups returns it.
 *   group_start [num_groups + 1], group_seqs, group_partitions [num_groups],
 *   seq_first_partition [num_seqs]: int32, device.  seq_first_partition[b]
 *               must equal group_partitions of b's group (0 outside groups).
 *   Other arguments as for pa_decode with partition_size > 0.
 * Results match pa_decode (split) to rounding.  The shared partitions'
 * partials sum their pages in another order, so bits differ, but they are
 * deterministic.  Members outside [0, num_seqs) are skipped.  bf16 only:
 * other dtypes return PA_ERR_UNSUPPORTED.  num_groups == 0 is pa_decode (or
 * pa_decode_append).  Host-checkable errors as for pa_decode, plus
 * PA_ERR_INVALID_ARGUMENT for partition_size 0, a negative bound, NULL group
 * arrays with num_groups > 0, or key/value/slot_mapping given only in part.
 */
int pa_decode_cascade(const void* query, const void* key, const void* value,
                      const int64_t* slot_mapping, void* k_cache, void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                      int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
                      int max_num_partitions, float* partial_out, float* partial_max,
                      float* partial_sum, int num_groups, int max_group_size,
                      int max_group_partitions, int max_suffix_partitions,
                      const int32_t* group_start, const int32_t* group_seqs,
                      const int32_t* group_partitions, const int32_t* seq_first_partition,
                      int dtype, void* stream);

/*
 * pa_decode_valu — pa_decode with the vector-ALU kernel forced.
 *
 * Same arguments, layouts, results contract and errors as pa_decode.  For
 * bf16, pa_decode runs the QK^T and P.V products on the matrix cores; this
 * variant runs them on the vector ALU (bf16 pairs with fp32 accumulation,
 * P rounded to bf16 as on the matrix cores).  It exists to measure and
 * cross-check the two designs; fp32 pa_decode already uses it, with every
 * product in fp32.
 */
int pa_decode_valu(void* out, const void* query, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                   int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                   int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
                   int max_num_partitions, float* partial_out, float* partial_max,
                   float* partial_sum, int dtype, void* stream);

/*
 * pa_decode_reduce — merge split-KV partials by log-sum-exp.
 *
 * For every (b, h) with n = min(ceil(L_b / partition_size), max_num_partitions):
 *     M = max_p partial_max[b][h][p],  w_p = partial_sum[b][h][p] * exp(partial_max[b][h][p] - M)
 *     out[b][h][:] = sum_p w_p partial_out[b][h][p][:] / sum_p w_p
 * with the numerator accumulated in increasing p and the denominator summed
 * in a fixed tree order (deterministic); n == 0 writes zeros.  Buffers as in pa_decode;
 * out is dtype (bf16 rounded to nearest even).
 */
int pa_decode_reduce(void* out, const float* partial_out, const float* partial_max,
                     const float* partial_sum, const int32_t* context_lens, int num_seqs,
                     int num_q_heads, int head_dim, int partition_size,
                     int max_num_partitions, int dtype, void* stream);

/*
 * pa_export_pages / pa_import_pages — move whole KV pages between a pool and
 * one contiguous buffer: the on-GPU half of handing a sequence's KV cache
 * from the engine that computed it to the one that decodes it (llm-d blog
 * post, disaggregated prefill/decode section: the KV computed by the prefill
 * pods is transferred to the decode pods; the network half is not here).
 *
 *   buffer      [2][num_ids][num_kv_heads * 16 * head_dim] elements of dtype:
 *               section 0 holds the K blocks, section 1 the V blocks, of
 *               page_ids[0], page_ids[1], ... in that order.  Each block is
 *               the pool page's own bytes (K [Hkv][16][D], V [Hkv][D][16]),
 *               so a receiving pool of the same shape takes it unchanged.
 *               Export writes it; import reads it.  16-byte aligned.
 *   buffer_bytes  size of `buffer`; must be at least
 *               2 * num_ids * num_kv_heads * 16 * head_dim * element size.
 *   page_ids    [num_ids] int32, device (a block-table row serves directly:
 *               a sequence of length L exports its first ceil(L / 16) ids).
 *   k_cache, v_cache, num_kv_heads, head_dim, page_size, num_pages, dtype:
 *               the pool, as for pa_reshape_and_cache.
 *
 * Bit copies: slots past a sequence's length travel as they are (they are
 * never read by attention).  An id outside [0, num_pages) is skipped: export
 * leaves that id's buffer blocks unwritten, import writes nothing for it.
 * Import writes exactly the listed pages; ids must be distinct, and no other
 * call may read or write those pages until the stream passes this one (the
 * single-writer rule of pa_reshape_and_cache).  num_ids == 0 is a no-op that
 * examines no pointer (an empty tensor's address may be NULL).
 * Errors: a NULL pointer, a negative count, a short buffer or misalignment
 * returns PA_ERR_INVALID_ARGUMENT; head_dim, page_size or dtype outside the
 * supported set returns PA_ERR_UNSUPPORTED.
 */
int pa_export_pages(void* buffer, int64_t buffer_bytes, const void* k_cache, const void* v_cache,
                    const int32_t* page_ids, int64_t num_ids, int num_kv_heads, int head_dim,
                    int page_size, int64_t num_pages, int dtype, void* stream);
int pa_import_pages(const void* buffer, int64_t buffer_bytes, void* k_cache, void* v_cache,
                    const int32_t* page_ids, int64_t num_ids, int num_kv_heads, int head_dim,
                    int page_size, int64_t num_pages, int dtype, void* stream);

/* Human-readable name of a pa_status value (static storage). */
const char* pa_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
