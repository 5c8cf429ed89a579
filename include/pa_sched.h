/*
 * Host-side KV-cache block manager and step planner of libpa.so: the part of
 * an engine step that decides which tokens run and where their keys and
 * values live, producing exactly the inputs pa_cache_write / pa_forward_ex
 * take (page "Inside vLLM: Anatomy of a High-Throughput LLM Inference
 * System", sections "Scheduler", "Chunked prefill", "Prefix Caching" and
 * "Run forward pass").
 *
 *  - Block pool: a doubly linked queue of free blocks popped from the left;
 *    freed blocks are appended on the right (a request's blocks last to
 *    first, so its earliest blocks stay cached longest). Every block has a
 *    reference count.
 *  - Prefix caching: every full block of a request's tokens gets a hash of
 *    (previous block's hash, its 16 token ids); computed full blocks are
 *    recorded in a hash -> block map. A new request reuses the longest run
 *    of leading blocks found in the map (at least its last token is always
 *    computed). A cached block stays valid in the free queue and is dropped
 *    from the map only when the queue hands it out again (lazy
 *    invalidation). Lookups compare the stored token ids and parent hash, so
 *    a hash collision never returns a wrong block.
 *  - Scheduling: running requests first (decode first), then waiting ones in
 *    arrival order, under a token budget per step; new tokens per request per
 *    step are capped by long_prefill_token_threshold (> 0: chunked prefill;
 *    a prompt longer than the remaining budget is chunked regardless).
 *    allocate_slots needs ceil((computed + new) / 16) blocks per request;
 *    when the pool runs short for a running request, the most recently
 *    admitted running request is preempted (its blocks freed, its tokens
 *    recomputed later), and a waiting request that does not fit stops the
 *    step's admissions.
 *
 * Not thread safe: one handle per engine thread. All pointers are host
 * pointers. Functions return PA_OK (0) or a negative PA_ERR_* code with the
 * reason in pa_last_error().
 */
#ifndef PA_SCHED_H_
#define PA_SCHED_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched;

/* Creates a planner over a pool of num_blocks blocks of block_size (16)
 * tokens. max_num_batched_tokens: the token budget per step (> 0);
 * max_num_seqs: most running requests (> 0); long_prefill_token_threshold:
 * most new tokens of one request per step (<= 0: no cap but the budget);
 * enable_prefix_caching: 0 or 1. Returns NULL on an invalid argument. */
pa_sched* pa_sched_create(int64_t num_blocks, int32_t block_size,
                          int32_t max_num_batched_tokens, int32_t max_num_seqs,
                          int32_t long_prefill_token_threshold, int32_t enable_prefix_caching);
void pa_sched_destroy(pa_sched* s);

/* Queues a request (its prompt token ids are copied). Ids must be unique
 * among live requests; max_new_tokens >= 1. */
int pa_sched_add_request(pa_sched* s, int64_t request_id, const int32_t* prompt,
                         int32_t prompt_len, int32_t max_new_tokens);

/* Plans the next step: which requests run and how many new tokens each.
 * Writes the step's sizes: rows (num_seqs), new tokens (num_tokens) and the
 * most blocks any row's table holds (max_blocks). A step with no rows is
 * valid (nothing to run). Each call plans a new step; pa_sched_update must
 * follow a step with rows before the next one is planned. */
int pa_sched_schedule(pa_sched* s, int32_t* num_seqs, int32_t* num_tokens, int32_t* max_blocks);

/* The planned step's kernel inputs, rows in schedule order (running
 * requests first). Arrays are caller-owned:
 *   request_ids      [num_seqs]
 *   query_start_loc  [num_seqs + 1] (exclusive prefix sum of new tokens)
 *   seq_lens         [num_seqs] tokens in the cache after the step's write
 *   block_table      [num_seqs][table_cols] (table_cols >= max_blocks);
 *                    entries past a row's blocks are -1
 *   slot_mapping     [num_tokens] cache slot of each new token
 *   token_ids        [num_tokens], positions [num_tokens] (position in its
 *                    request) — any of the last three may be NULL, and
 *                    every array but query_start_loc when num_seqs is 0 */
int pa_sched_step_inputs(const pa_sched* s, int64_t* request_ids, int32_t* query_start_loc,
                         int32_t* seq_lens, int32_t* block_table, int32_t table_cols,
                         int64_t* slot_mapping, int32_t* token_ids, int32_t* positions);

/* Ends the planned step: the new tokens' keys and values are now in the
 * cache. sampled[i] is the token produced by row i; it is used only for
 * rows whose request computed all its known tokens (a finished prefill or a
 * decode row). A request that has produced max_new_tokens tokens finishes
 * and frees its blocks. */
int pa_sched_update(pa_sched* s, const int32_t* sampled);

/* Ends a live request early (frees its blocks). */
int pa_sched_finish_request(pa_sched* s, int64_t request_id);

typedef struct {
  int64_t num_free_blocks;     /* blocks in the free queue (cached or not) */
  int64_t num_cached_blocks;   /* entries of the hash -> block map */
  int32_t num_waiting;
  int32_t num_running;
  int32_t num_finished;
  int32_t pad_;
  int64_t num_steps;
  int64_t prefix_hit_tokens;   /* tokens taken from the cache at admission */
  int64_t num_preemptions;
} pa_sched_stats;
int pa_sched_get_stats(const pa_sched* s, pa_sched_stats* out);

/* A live request's blocks (returns their count, copying at most cap), or a
 * negative code if the id is unknown; its tokens computed so far. */
int32_t pa_sched_request_blocks(const pa_sched* s, int64_t request_id, int32_t* blocks,
                                int32_t cap);
int32_t pa_sched_request_computed(const pa_sched* s, int64_t request_id);
/* Reference count of a block (-1 if out of range). */
int32_t pa_sched_block_ref_count(const pa_sched* s, int32_t block);

/*
 * Leading blocks that every row of a planned step shares (host arrays as
 * pa_sched_step_inputs fills them; section "Prefix Caching": requests with
 * the same prompt prefix reference the same full blocks): the largest P
 * such that every row's first P table entries equal row 0's and every row
 * keeps at least one key past 16 * P, so that its new token lies in a block
 * of its own. 0 when a row does not hold exactly one query token (the
 * shared-prefix calls take decode rows only) or on bad arguments. The
 * shared-prefix calls (pa_write_and_forward_shared_prefix) apply to the
 * step when it is above 0.
 */
int32_t pa_sched_shared_prefix_blocks(const int32_t* query_start_loc, const int32_t* seq_lens,
                                      const int32_t* block_table, int32_t num_seqs,
                                      int32_t table_cols);

#ifdef __cplusplus
}  // extern "C"
#endif

#endif  // PA_SCHED_H_
