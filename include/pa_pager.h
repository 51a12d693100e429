/*
 * pa_pager.h — host-side owner of the KV page pool: which physical page holds
 * which tokens of which sequence.  Plain C ABI over a C++ implementation
 * (libpa_pager.so); no GPU calls.  It produces exactly what the device calls
 * in pa.h consume: block tables, context lengths and slot mappings, plus the
 * page copies a copy-on-write needs.
 *
 * What the pages ask of this part:
 *   - the cache is a fixed number of fixed-size pages (llm-d router blog
 *     post, engine metric spec: page_size and num_pages; vLLM
 *     "EngineCoreClient" page, "Archivos clave": num_gpu_blocks and
 *     block_size reported as the real capacity);
 *   - a request whose prompt prefix is already cached skips recomputing it,
 *     and the engine announces which prefixes it holds through allocation
 *     and eviction events (llm-d blog post, prefix-cache scorer and the
 *     precise KV-cache producer section);
 *   - page ownership and reuse rules live in one native owner with a
 *     single-writer contract (TensorRT Edge-LLM "HTTP Inference Server
 *     Architecture", "Request Lifecycle" on context reuse and "Extension
 *     Rules" on page ownership).
 *
 * Policy (deterministic; a plain model of it lives with the tests):
 *   - A FULL page is identified by the chained hash of every token from the
 *     sequence start through its last token (64-bit; an entry also stores
 *     its 16 tokens and its parent's hash and is only reused when both
 *     match).  Full pages are registered when they are allocated full (a
 *     prompt) or become full (appends), unless the same hash is already
 *     registered.  A partial page is never shared by prefix reuse.
 *   - Adding a sequence reuses the longest run of registered full pages that
 *     matches its prompt from the start, then allocates the rest.
 *   - A page is free (reference count 0) or in use.  Free pages that hold a
 *     registered full page stay reusable ("cached") until evicted.
 *   - Allocation takes the lowest-numbered free page that holds nothing
 *     registered; if there is none, it evicts the cached page released
 *     longest ago (LRU) and unregisters it.  If every page is in use, the
 *     call fails with PA_PAGER_OUT_OF_PAGES and changes nothing.
 *   - Releasing a sequence drops its pages from its last to its first, so
 *     that its deepest pages are evicted first.
 *   - Single writer: a page is written (a token slot) only while exactly one
 *     sequence holds it.  Appending to a partial tail page that a fork
 *     shares first moves the appending sequence onto a fresh page; the call
 *     reports (src, dst) and the caller copies page src to dst on the device
 *     (pa_export_pages then pa_import_pages, say) before writing the slot.
 *
 * Thread safety: none; one owner thread per pager (the single-writer rule).
 */
#ifndef PA_PAGER_H
#define PA_PAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_PAGER_OK = 0,
  PA_PAGER_INVALID_ARGUMENT = 1,  /* NULL pointer, negative count, bad size */
  PA_PAGER_OUT_OF_PAGES = 2,      /* every page is in use; nothing changed */
  PA_PAGER_UNKNOWN_SEQUENCE = 3,  /* no live sequence has that id */
  PA_PAGER_SEQUENCE_EXISTS = 4,   /* the id is already live */
  PA_PAGER_SEQUENCE_FULL = 5      /* the sequence would exceed max_pages_per_seq */
} pa_pager_status;

typedef enum { PA_PAGER_EVENT_STORED = 0, PA_PAGER_EVENT_REMOVED = 1 } pa_pager_event_kind;

typedef struct pa_pager pa_pager;

typedef struct {
  int64_t num_pages;
  int64_t in_use;            /* pages held by at least one sequence */
  int64_t cached_free;       /* free pages still holding a registered full page */
  int64_t empty_free;        /* free pages holding nothing registered */
  int64_t registered;        /* registered full pages (in use or cached) */
  int64_t live_sequences;
  int64_t prefix_hit_tokens; /* tokens served from registered pages since creation */
  int64_t evictions;         /* cached pages evicted since creation */
  int64_t cow_copies;        /* copy-on-write page moves since creation */
} pa_pager_stats;

/* A pool of num_pages pages of page_size (16) tokens; a sequence may hold
 * at most max_pages_per_seq pages.  Returns NULL on a bad argument. */
pa_pager* pa_pager_create(int64_t num_pages, int page_size, int max_pages_per_seq);
void pa_pager_destroy(pa_pager* pager);

/* Start sequence `seq_id` with prompt tokens[0..n).  slot_mapping[t]
 * (int64, n entries, host memory) receives the pool slot of token t
 * (page * page_size + offset); *num_cached receives how many leading tokens
 * already sit in reused pages (a multiple of page_size): the caller writes
 * K/V only for tokens num_cached..n-1, on the stream before any attention
 * call that reads them. */
int pa_pager_add_sequence(pa_pager* pager, int64_t seq_id, const int32_t* tokens, int64_t n,
                          int64_t* slot_mapping, int64_t* num_cached);

/* Reserve the slot of one new token of `seq_id`.  *copy_src / *copy_dst
 * receive -1, or the pages to copy on the device before the slot is
 * written (copy-on-write of a shared tail page). */
int pa_pager_append(pa_pager* pager, int64_t seq_id, int32_t token, int64_t* slot,
                    int64_t* copy_src, int64_t* copy_dst);

/* One decode step's appends: token tokens[i] to sequence seq_ids[i], in
 * order, with slot and copy results as for pa_pager_append (arrays of n,
 * host memory).  Stops at the first failing append and returns its status;
 * *num_done receives how many appends were made (all of them on success). */
int pa_pager_append_batch(pa_pager* pager, const int64_t* seq_ids, const int32_t* tokens,
                          int64_t n, int64_t* slots, int64_t* copy_src, int64_t* copy_dst,
                          int64_t* num_done);

/* `child` starts as a copy of `parent` sharing all of its pages. */
int pa_pager_fork(pa_pager* pager, int64_t parent, int64_t child);

/* End `seq_id` and release its pages (last to first). */
int pa_pager_free_sequence(pa_pager* pager, int64_t seq_id);

/* Block-table rows and context lengths of n live sequences, in the layout
 * pa_decode reads: tables[n][max_pages_per_seq] (int32, padded with -1),
 * context_lens[n] (int32).  Host memory. */
int pa_pager_block_tables(const pa_pager* pager, const int64_t* seq_ids, int64_t n,
                          int32_t* tables, int32_t* context_lens);

int pa_pager_get_stats(const pa_pager* pager, pa_pager_stats* out);

/* Move up to `capacity` pending events, oldest first, into kinds/pages/hashes
 * (host arrays); *count receives how many were written.  STORED: a full page
 * was registered (hash = its chained hash); REMOVED: a cached page was
 * evicted and unregistered. */
int pa_pager_drain_events(pa_pager* pager, int32_t* kinds, int64_t* pages, uint64_t* hashes,
                          int64_t capacity, int64_t* count);

/* Groups of sequences that share their first pages, in the form
 * pa_decode_cascade (pa.h) takes.  block_tables [num_seqs][max_pages_per_seq]
 * and context_lens [num_seqs] are host int32 arrays (the rows a batch's
 * decode reads).  Sequences are grouped when they hold the same page id in
 * column 0.  A group's shared prefix is the longest run of columns from 0 in
 * which every member holds the first member's page id, counting only pages
 * that lie wholly before each member's last token (so the page that receives
 * the step's token is never in it), in whole partitions of
 * pages_per_partition pages.  Groups of one member or of no whole partition
 * are dropped.  Groups are ordered by their first member and members by batch
 * index.  Outputs (host; sized for the worst case): group_start [num_seqs +
 * 1], group_seqs [num_seqs], group_partitions [num_seqs], seq_first_partition
 * [num_seqs] (0 outside groups); *num_groups, *max_group_size,
 * *max_group_partitions, and *max_suffix_partitions: the most partitions any
 * sequence has from its seq_first_partition on (ceil(min(ceil(L / 16),
 * max_pages_per_seq) / pages_per_partition) - first), the bound
 * pa_decode_cascade sizes its grid by. */
int pa_pager_prefix_groups(const int32_t* block_tables, const int32_t* context_lens,
                           int64_t num_seqs, int max_pages_per_seq, int pages_per_partition,
                           int32_t* group_start, int32_t* group_seqs, int32_t* group_partitions,
                           int32_t* seq_first_partition, int64_t* num_groups,
                           int64_t* max_group_size, int64_t* max_group_partitions,
                           int64_t* max_suffix_partitions);

/* Chained hash of one full page: the value registered for a page whose
 * parent has hash `parent` (0 for the first page) and whose tokens are
 * tokens[0..page_size).  Exposed so a router can compute prefix keys. */
uint64_t pa_pager_page_hash(uint64_t parent, const int32_t* tokens, int page_size);

#ifdef __cplusplus
}
#endif

#endif /* PA_PAGER_H */
