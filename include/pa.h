/*
 * pa.h - C ABI of the paged-attention hot path for MI355X (gfx950).
 *
 * The operations come from the pages "Inside vLLM: Anatomy of a
 * High-Throughput LLM Inference System" (bilingual copy at s.sunxiunan.com,
 * Chinese translation at uml.org.cn, part-2 copy on the chengshu blog):
 *
 *   - the KV cache is carved into blocks of 16 tokens (section "Scheduler");
 *     one block of one standard layer holds 2 * block_size * num_kv_heads *
 *     head_size * dtype_bytes bytes (uml.org.cn, section "LLM Engine 构造函数");
 *   - each step builds block tables and a slot_mapping, flattens all
 *     sequences into one super sequence, and runs paged attention in which
 *     positions and masks keep every sequence to its own tokens (section
 *     "Run forward pass");
 *   - the forward pass writes the new tokens' keys and values into the paged
 *     KV memory (section "Prefix Caching"), and one step may hold decode rows
 *     and chunks of long prompts side by side (sections "Scheduler" and
 *     "Chunked prefill").
 *
 * Conventions for every entry point:
 *   - Tensors are row-major and contiguous; "device" pointers point to HIP
 *     device memory of the current device; element type bf16 unless stated.
 *   - The caller owns every buffer, including the workspace. The library
 *     keeps no pointer to them after a call returns and allocates no device
 *     memory on the hot path (pa_cache_write, pa_forward); its only state is
 *     a second stream and two events per device, made by the first large
 *     mixed call (see pa_forward_ex).
 *   - pa_cache_write and pa_forward only enqueue work ordered on `stream` (a
 *     hipStream_t; NULL = the null stream) and return: no device-to-host
 *     copy, no synchronisation. A large mixed batch runs part of its work
 *     on the second stream, forked from and joined back into `stream`
 *     within the call. Call pa_cache_write for a step's tokens before
 *     pa_forward on the same stream.
 *   - Host-known arguments are checked before anything is launched; a
 *     negative pa_status is returned and pa_last_error() describes it.
 *     Device-resident metadata (slots, lengths, tables) is trusted on the hot
 *     path; pa_validate_inputs checks it synchronously.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,         /* a required pointer is NULL                          */
  PA_ERR_SHAPE = -2,        /* a size is out of range or sizes disagree            */
  PA_ERR_UNSUPPORTED = -3,  /* valid but not built: head_size, group size, block   */
  PA_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned                    */
  PA_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required          */
  PA_ERR_HIP = -6,          /* a HIP runtime call or kernel launch failed          */
  PA_ERR_INVALID_DATA = -7  /* pa_validate_inputs found inconsistent metadata      */
} pa_status;

/* Tokens per KV-cache block; the only block size the kernels accept. */
#define PA_BLOCK_SIZE 16

/*
 * Bytes of one KV-cache block of one layer (key and value together):
 * 2 * block_size * num_kv_heads * head_size * dtype_bytes
 * (uml.org.cn translation, section "LLM Engine 构造函数"). Pure host
 * arithmetic; returns -1 if an argument is not positive.
 */
int64_t pa_kv_block_bytes(int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                          int32_t dtype_bytes);

/*
 * KV-cache write (section "Run forward pass": slot_mapping; section "Prefix
 * Caching": the forward pass populates the allocated blocks).
 *
 *   k, v          device, bf16 [num_tokens, num_kv_heads, head_size]
 *   slot_mapping  device, int64 [num_tokens]; token t goes to row
 *                 slot % block_size of block slot / block_size; slot < 0
 *                 skips the token (padding)
 *   k_cache,      device, bf16 [num_blocks, block_size, num_kv_heads,
 *   v_cache       head_size], written in place
 *
 * The copy is bit-exact. Caller contract (not checked on this path): every
 * slot is < num_blocks * block_size and no two tokens share a slot.
 * num_tokens == 0 is a no-op. Requires block_size == 16, head_size a multiple
 * of 8, 16-byte aligned k, v, k_cache, v_cache.
 */
int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                   int64_t num_blocks, int32_t block_size, void* stream);

/*
 * Workspace bytes pa_forward needs for these sizes: a fixed region of
 * PA_WORKSPACE_COUNTER_BYTES at the start holding per-row arrival counters
 * of the decode rows (zero before the first call, left zero by every call,
 * never written with anything else), then partial results of decode rows
 * split between workgroups and the work list of prefill tiles. Depends only
 * on its arguments (and on the tuning overrides read once per process);
 * returns 0 if an argument is out of range or the sizes are not supported.
 * The hints are those the forward call will pass: max_query_len_hint with
 * 1 < hint <= 16 / (num_q_heads / num_kv_heads) plans for rows of several
 * query tokens on the decode path; max_seq_len_hint <= 0 means "unknown"
 * (max_blocks_per_seq * 16 is used).
 */
#define PA_WORKSPACE_COUNTER_BYTES (256u * 1024u)
size_t pa_forward_workspace_bytes(int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_size,
                                  int32_t max_blocks_per_seq, int32_t max_query_len_hint,
                                  int32_t max_seq_len_hint);

/*
 * Paged attention over a flattened varlen batch (section "Run forward pass",
 * step 3; chunked rows per section "Chunked prefill").
 *
 *   q                device, bf16 [num_tokens, num_q_heads, head_size]
 *   k_cache, v_cache device, bf16 [num_blocks, 16, num_kv_heads, head_size]
 *   block_table      device, int32 [num_seqs, max_blocks_per_seq]; only the
 *                    first ceil(seq_lens[s] / 16) entries of row s are read
 *   seq_lens         device, int32 [num_seqs]: tokens in the cache for
 *                    sequence s after this step's write (context + new)
 *   query_start_loc  device, int32 [num_seqs + 1]: exclusive prefix sum of
 *                    the per-sequence query counts; [0] = 0, [S] = num_tokens
 *   scale            softmax scale applied to q.k (e.g. 1/sqrt(head_size))
 *   out              device, bf16 [num_tokens, num_q_heads, head_size]
 *   max_query_len_hint, max_seq_len_hint
 *                    host upper bounds of q_len and seq_len over the batch;
 *                    <= 0 = unknown (num_tokens and max_blocks_per_seq * 16
 *                    are used). A hint below the true maximum is a contract
 *                    violation (rows past it are not computed).
 *   workspace        device, >= pa_forward_workspace_bytes(...) bytes,
 *                    16-byte aligned. Its first PA_WORKSPACE_COUNTER_BYTES
 *                    must be zero before its first use (every call leaves
 *                    them zero); the rest is scratch that each call writes
 *                    before it reads. Calls that share a workspace must be
 *                    ordered on one stream.
 *
 * Query row i of sequence s (i < q_len = qsl[s+1] - qsl[s]) sits at position
 * c + i with c = seq_lens[s] - q_len and attends to keys 0..c+i of its own
 * sequence; query head h reads KV head h / (num_q_heads / num_kv_heads).
 * Rows with q_len == 0 produce nothing; rows with q_len == 1 take the decode
 * path (for large batches the rows' blocks are shared out evenly between
 * workgroups; small batches, or more than 4096 rows, split rows into fixed
 * partitions), rows with q_len > 1 the prefill path. When 1 <
 * max_query_len_hint <= 16 / (num_q_heads / num_kv_heads) (for instance
 * rows verifying a few speculated tokens) every row takes the decode path
 * (either schedule, chosen as for single-token rows), its q_len * G query
 * columns sharing each K/V block, and no prefill launch is made. A batch
 * of at most 256 (row, KV head) pairs that makes a prefill launch and has
 * no row longer than 128 keys (by max_seq_len_hint, else
 * max_blocks_per_seq * 16) runs its single-token rows on the prefill path
 * too, so no decode launch is made, unless a flag of pa_forward_ex names
 * the decode schedule.
 * Output is fp32-accumulated and rounded to bf16 (round to nearest even).
 * Tuning overrides, read once per process (for sweeps; out-of-range values
 * are ignored): PA_DECODE_STREAM (0 / 1 = always the partitioned / the
 * even-share decode schedule where it fits), PA_DECODE_STREAM_WGS
 * (even-share workgroups, 1..512), PA_DECODE_PART_TOKENS (tokens per decode
 * partition, a multiple of 16, at least 128), PA_DECODE_WAVES (waves per
 * partitioned decode workgroup, 1..16 within the head size's limit),
 * PA_DECODE_PREFETCH (blocks in flight per wave at head_size 64, 2..3),
 * PA_SHORT_BATCH_TILES (0 = single-token rows of a batch of short rows keep
 * the decode launch).
 * Requires block_size == 16, head_size in {64, 128}, num_q_heads /
 * num_kv_heads in {1, 2, 4, 8, 16}. Caller contract: 0 <= q_len <= seq_len
 * <= max_blocks_per_seq * 16 and the first ceil(seq_len / 16) table entries
 * of each row are valid block ids.
 */
int pa_forward(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* seq_lens,
               const int32_t* query_start_loc, float scale, void* out, int32_t num_tokens,
               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
               int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
               int32_t max_query_len_hint, int32_t max_seq_len_hint, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * pa_forward with option flags (pa_forward is pa_forward_ex with flags 0).
 *
 *   PA_FORWARD_SHARED_BLOCKS  some physical blocks appear in more than one
 *       row's table (prefix caching: blocks with a reference count above one,
 *       section "Prefix Caching"). KV is then read through the caches so the
 *       shared blocks are served from them; without the flag V is read with
 *       streaming (nontemporal) loads, the faster choice for blocks read once.
 *       Either way the results are identical.
 *
 *   PA_FORWARD_DECODE_EVEN_SHARES, PA_FORWARD_DECODE_PARTITIONED
 *       force the decode rows' schedule: every workgroup takes an equal share
 *       of all rows' blocks (rows cut by a share are merged by the share that
 *       finishes them last), or rows are split into fixed partitions merged
 *       by a combine pass. Without either the library picks by batch size.
 *       EVEN_SHARES falls back to partitions when num_seqs > 4096. The
 *       results agree to rounding order; each schedule is deterministic.
 *
 *   PA_FORWARD_SERIAL
 *       keep every launch of a mixed batch on `stream`, one part after the
 *       other (see below). The results are the same either way up to the
 *       decode rows' rounding order (their shares differ).
 *
 * Unknown flag bits, or both schedule flags, return PA_ERR_UNSUPPORTED.
 *
 * Mixed batches (section "Scheduler": one step holds decode rows, bound by
 * memory bandwidth, and prefill rows, bound by compute): when the decode
 * rows take even shares and num_tokens - num_seqs >= 1024, the prefill
 * tiles that see many keys run on a second stream that the library makes
 * for the device on the first such call (default priority; kept until the
 * process ends), forked from `stream` after the call's cache write and tile
 * planner and joined back into `stream` by events before the call returns,
 * while the decode's shares (160 of them, PA_MIXED_DECODE_WGS overrides),
 * then the tiles that see few keys, run on `stream` and leave CUs to the
 * long prefill tiles. Work enqueued on `stream` after the call still
 * sees all of its results. Calls made while `stream` is being captured
 * into a graph, calls whose `stream` belongs to a device other than the
 * current one, calls with PA_FORWARD_SERIAL, pa_write_and_forward_noalloc
 * and every process with PA_MIXED_OVERLAP=0 keep all launches on `stream`.
 */
#define PA_FORWARD_SHARED_BLOCKS 1u
#define PA_FORWARD_DECODE_EVEN_SHARES 2u
#define PA_FORWARD_DECODE_PARTITIONED 4u
#define PA_FORWARD_SERIAL 8u

int pa_forward_ex(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* seq_lens,
                  const int32_t* query_start_loc, float scale, void* out, int32_t num_tokens,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                  int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                  int32_t max_query_len_hint, int32_t max_seq_len_hint, void* workspace,
                  size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * The step's KV write and its attention in one call: the same results as
 * pa_cache_write(k, v, slot_mapping, k_cache, v_cache, num_tokens,
 * num_kv_heads, head_size, num_blocks, block_size, stream) followed by
 * pa_forward_ex(q, k_cache, v_cache, ..., flags, stream) (the write feeds the
 * forward pass, section "Prefix Caching"; both per section "Run forward
 * pass"). When max_query_len_hint == 1 (every row is a decode row) and the
 * decode rows take the partitioned schedule (with at most 8 waves per
 * workgroup where the head size needs the registers; the default takes 4),
 * a single launch does both: each row's workgroups write its new token into
 * the caches and read that token from k and v rather than from the slot
 * being written. A batch with prefill rows writes in the launch of the
 * tile planner (which the prefill tiles, and any decode launch, follow);
 * otherwise the write is a launch of its own ahead of the forward launches.
 *
 *   k, v, slot_mapping   as for pa_cache_write (k, v: bf16 [num_tokens,
 *                        num_kv_heads, head_size]; slot_mapping int64
 *                        [num_tokens], < 0 skips a token)
 *   everything else      as for pa_forward_ex; k_cache, v_cache are written
 *
 * Caller contract of the single launch (the pages' slot mapping): token
 * qsl[s] of decode row s is its position seq_lens[s] - 1, slot_mapping of it
 * (when >= 0) is that position's slot in row s's blocks, and no other row of
 * the call reads a slot being written (a block being appended to is not
 * shared). A token whose slot is < 0 is not written and is read from the
 * cache, as in the two-call sequence. Errors as for pa_cache_write and
 * pa_forward_ex; on an error nothing is launched.
 */
int pa_write_and_forward(const void* k, const void* v, const int64_t* slot_mapping,
                         void* k_cache, void* v_cache, const void* q, const int32_t* block_table,
                         const int32_t* seq_lens, const int32_t* query_start_loc, float scale,
                         void* out, int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks,
                         int32_t max_query_len_hint, int32_t max_seq_len_hint, void* workspace,
                         size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * pa_write_and_forward without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The workspace is the library's own fixed device array of
 * PA_NOALLOC_SCRATCH_BYTES bytes, one per device (held until the process
 * ends). Arguments, results and errors are those of pa_write_and_forward
 * with workspace and workspace_bytes left out; the call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).
 *
 *   - Sizes whose pa_forward_workspace_bytes(...) exceeds
 *     PA_NOALLOC_SCRATCH_BYTES are rejected with PA_ERR_WORKSPACE before
 *     anything is launched (the named workloads of this library need at
 *     most about 33 MiB).
 *   - The first call on a device, with that device current, looks up the
 *     array's address and enqueues a fill kernel on `stream` that clears its
 *     counter region; make that first call outside graph capture. Every
 *     call leaves the counter region zero again.
 *   - Every call on one device shares that device's array: calls that
 *     overlap on one device (different streams, or host threads, without
 *     ordering between them) race. Order them on one stream.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int pa_write_and_forward_noalloc(const void* k, const void* v, const int64_t* slot_mapping,
                                 void* k_cache, void* v_cache, const void* q,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* query_start_loc, float scale, void* out,
                                 int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                 int32_t max_blocks_per_seq, int64_t num_blocks,
                                 int32_t max_query_len_hint, int32_t max_seq_len_hint,
                                 uint32_t flags, void* stream);

/*
 * Decode rows whose tables all begin with the same prefix_blocks blocks
 * (a shared prompt prefix; section "Prefix Caching": a cached block is
 * referenced by every request that shares it). The prefix's keys are
 * attended once for all rows together: their query tokens are stacked as
 * the rows of matrix-core tiles (G heads each), chunk by chunk of the
 * prefix, leaving partial results per row; each row's own blocks after the
 * prefix run on the partitioned decode schedule, whose last workgroup per
 * (row, KV head) merges both (the log-sum-exp identity). Results agree with
 * pa_forward_ex to rounding order.
 *
 *   q ... out, sizes, num_blocks   as for pa_forward_ex, with num_tokens =
 *                    num_seqs: every row is a decode row (query_start_loc
 *                    = 0, 1, ..., num_seqs)
 *   prefix_blocks    leading table entries shared by every row (>= 1);
 *                    row 0's entries are the ones read
 *   max_seq_len_hint as for pa_forward_ex; must exceed 16 * prefix_blocks
 *   workspace        >= pa_shared_prefix_workspace_bytes(...) bytes, 16-byte
 *                    aligned; its first PA_WORKSPACE_COUNTER_BYTES must be
 *                    zero before its first use (every call leaves them
 *                    zero), the rest is scratch written before it is read;
 *                    calls sharing a workspace must be ordered on one stream
 *   flags            0 or PA_FORWARD_SHARED_BLOCKS
 *
 * Caller contract (not checked): every row's first prefix_blocks table
 * entries equal row 0's, and seq_lens[s] > 16 * prefix_blocks (the row's
 * new token lies past the prefix, in a block of its own). Errors as for
 * pa_forward_ex; on an error nothing is launched.
 */
size_t pa_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_size,
                                        int32_t max_blocks_per_seq, int32_t prefix_blocks,
                                        int32_t max_seq_len_hint);
int pa_forward_shared_prefix(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* query_start_loc, float scale, void* out,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_blocks, int32_t prefix_blocks, int32_t max_seq_len_hint,
                             void* workspace, size_t workspace_bytes, uint32_t flags,
                             void* stream);

/*
 * The step's KV write and the shared-prefix decode in one call: the same
 * results as pa_cache_write(k, v, slot_mapping, k_cache, v_cache, num_seqs,
 * num_kv_heads, head_size, num_blocks, block_size, stream) followed by
 * pa_forward_shared_prefix(...) (section "Run forward pass": the new tokens
 * are written through the slot mapping before attention reads them;
 * section "Prefix Caching" for the shared blocks). The write rides in the
 * prefix pass's launch, which reads only the prefix's blocks; the rows'
 * own blocks are read by the launch after it.
 *
 *   k, v, slot_mapping   as for pa_cache_write, one token per row (k, v:
 *                        bf16 [num_seqs, num_kv_heads, head_size];
 *                        slot_mapping int64 [num_seqs], < 0 skips a token)
 *   everything else      as for pa_forward_shared_prefix; k_cache, v_cache
 *                        are written
 *
 * Caller contract (not checked), beyond pa_forward_shared_prefix's: no slot
 * being written lies in the prefix's blocks (each row's new token sits past
 * the prefix, in a block of its own). Errors as for pa_cache_write and
 * pa_forward_shared_prefix; on an error nothing is launched.
 */
int pa_write_and_forward_shared_prefix(const void* k, const void* v, const int64_t* slot_mapping,
                                       void* k_cache, void* v_cache, const void* q,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* query_start_loc, float scale, void* out,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_size,
                                       int32_t block_size, int32_t max_blocks_per_seq,
                                       int64_t num_blocks, int32_t prefix_blocks,
                                       int32_t max_seq_len_hint, void* workspace,
                                       size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * Synchronous check of the device-resident metadata that the hot path
 * trusts (for tests and debugging; copies to the host and waits on
 * `stream`). Checks: query_start_loc starts at 0, never decreases and ends at
 * num_tokens; 0 <= q_len <= seq_len <= max_blocks_per_seq * 16; the table
 * entries a row reads are in [0, num_blocks); hints, when given, bound the
 * true maxima; and, if slot_mapping is not NULL, every slot of its
 * num_write_tokens entries is < num_blocks * 16 and no slot repeats.
 * Returns PA_OK or PA_ERR_INVALID_DATA (or an argument error).
 */
int pa_validate_inputs(const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* query_start_loc, const int64_t* slot_mapping,
                       int32_t num_tokens, int32_t num_seqs, int32_t max_blocks_per_seq,
                       int64_t num_blocks, int32_t block_size, int32_t num_write_tokens,
                       int32_t max_query_len_hint, int32_t max_seq_len_hint, void* stream);

/*
 * Synchronous check of the shared-prefix calls' caller contract (section
 * "Prefix Caching": a cached block is shared by reference, only full blocks
 * are shared, and a request's new tokens go into blocks of its own), for
 * tests and debugging; copies to the host and waits on `stream`. Checks:
 * every row's first prefix_blocks table entries equal row 0's; every row's
 * seq_len is above 16 * prefix_blocks and at most max_blocks_per_seq * 16;
 * and, if slot_mapping (int64 [num_seqs], one new token per row) is not
 * NULL, no slot >= 0 lies in one of the prefix's blocks. Returns PA_OK or
 * PA_ERR_INVALID_DATA (or an argument error); pa_last_error() names the
 * first row that breaks the contract.
 */
int pa_validate_shared_prefix(const int32_t* block_table, const int32_t* seq_lens,
                              const int64_t* slot_mapping, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t prefix_blocks, void* stream);

/*
 * Read probe for measurement harnesses (not part of the attention path):
 * reads every K and V block that rows 0..num_seqs-1 cover (the first
 * ceil(seq_lens[s] / 16) entries of each table row, the blocks a forward
 * call reads for them; section "Run forward pass"), whole and once, with
 * no arithmetic, so a decode kernel's bandwidth can be set beside what the
 * memory system delivers for the same scattered blocks. Bytes read:
 * sum over rows of ceil(seq_len / 16) * 2 * 16 * num_kv_heads * head_size
 * * 2.
 *
 *   k_cache, v_cache   device, bf16 [num_blocks, 16, num_kv_heads, head_size],
 *                      16-byte aligned; only read
 *   block_table        device, int32 [num_seqs, max_blocks_per_seq]; ids
 *                      outside [0, num_blocks) are clamped into it
 *   seq_lens           device, int32 [num_seqs], each <= max_blocks_per_seq * 16
 *   waves              waves per workgroup, 1..16
 *   blocks_per_workgroup  table columns per workgroup, >= 1; the grid is
 *                      num_seqs x ceil(max_blocks_per_seq / blocks_per_workgroup)
 *   sink               device, 4 bytes; written only if the XOR of all data
 *                      read by one thread equals 0x9e3779b9 (keeps the
 *                      loads from being optimised away)
 *
 * Enqueues one launch on `stream` and returns; PA_ERR_* on a bad argument.
 */
int pa_probe_block_read(const void* k_cache, const void* v_cache, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                        int32_t head_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                        int32_t waves, int32_t blocks_per_workgroup, uint32_t* sink,
                        void* stream);

/*
 * Kernel timing for measurement harnesses (not for the hot path). After
 * pa_profile_begin, every kernel the library launches is bracketed by HIP
 * events on its stream; pa_profile_end stops recording, waits for those
 * events and returns, per kernel class, the number of launches and their
 * summed elapsed time (event to event, on the launch stream). Begin resets
 * the totals. Recording is process-wide and off by default; while it is off
 * a launch pays one atomic flag read. Events are created on first use and
 * reused.
 */
#define PA_KERNEL_CACHE_WRITE 0   /* pa_cache_write                            */
#define PA_KERNEL_DECODE 1        /* decode rows: partitions                   */
#define PA_KERNEL_COMBINE 2       /* decode rows: split-K merge                */
#define PA_KERNEL_PREFILL 3       /* prefill tiles seeing many keys            */
#define PA_KERNEL_PREFILL_SHORT 4 /* prefill tiles seeing few keys             */
#define PA_KERNEL_PLAN 5          /* prefill tile planner                      */
#define PA_KERNEL_PREFIX 6        /* shared-prefix pass (pa_forward_shared_prefix) */
#define PA_KERNEL_WRITE_PLAN 7    /* KV write + tile planner in one launch     */
#define PA_KERNEL_CLASSES 8

typedef struct pa_profile {
  int64_t launches[PA_KERNEL_CLASSES];
  double total_ms[PA_KERNEL_CLASSES];
} pa_profile;

int pa_profile_begin(void);
int pa_profile_end(pa_profile* out);  /* out may be NULL */

/* Message of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version string. */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
