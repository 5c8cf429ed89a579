// Host-side launchers of the gfx950 kernels; called by the C ABI layer after
// it has validated every host-known argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Brackets one kernel launch of class `cls` (PA_KERNEL_*) with timing events
// when pa_profile_begin has enabled recording; otherwise no-ops.
void profile_begin(int cls, hipStream_t stream);
void profile_end(int cls, hipStream_t stream);

// Read probe: the rows' K and V blocks read whole, no arithmetic.
hipError_t launch_block_read_probe(const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_kv_heads, int32_t head_size,
                                   int32_t max_blocks_per_seq, int64_t num_blocks, int32_t waves,
                                   int32_t blocks_per_wg, uint32_t* sink, hipStream_t stream);
hipError_t launch_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                              void* k_cache, void* v_cache, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_size, hipStream_t stream);

struct ForwardArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;
  void* out;
  float scale;
  int32_t num_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq;
  int32_t max_query_len, max_seq_len;  // resolved upper bounds (hints or defaults)
};

// Decode rows (q_len == 1). Stream schedule: stream_wgs workgroups each take
// an equal share of all decode rows' blocks, stream_heads KV heads per
// workgroup (grid y covers the rest), waves / stream_heads waves per head;
// rows split between shares are merged by the last share through counters.
// Partitioned schedule: one workgroup per (row, KV head, partition); rows of
// several partitions are merged by a combine kernel.
struct DecodePlan {
  bool stream;            // stream schedule (else partitioned)
  int32_t stream_wgs;     // stream: workgroups (grid x)
  int32_t stream_heads;   // stream: KV heads per workgroup (divides waves)
  int32_t part_tokens;    // partitioned: tokens per partition (multiple of 16)
  int32_t num_parts_max;  // partitioned: partitions per row (grid z; workspace stride)
  int32_t waves;          // waves per workgroup (1..decode_max_waves)
  int32_t heads_per_wg;   // partitioned: KV heads per workgroup (divides Hkv and waves)
  int32_t prefetch;       // register ring depth in 16-token blocks (2, or 3 at D = 64)
  bool stream_v;          // V through nontemporal loads (blocks not shared)
  float* ws_o;            // partial outputs: stream [wgs][2][Hq][D], partitioned [S][parts][Hq][D]
  float* ws_ml;           // partial (max in log2 units, sum): same rows, 2 floats each
  int32_t* counters;      // stream: [S][groups] arrival counters, zero between calls
  // Partitioned schedule after a shared-prefix pass: keys start at
  // tok_base, partition p is stored as partial part_base + p, and every row
  // leaves partials for the combine (even with one partition).
  int32_t tok_base;
  int32_t part_base;
  // Partitioned schedule: rows of 1..qmax query tokens (qmax * G <= 16)
  // take the decode path; partials are laid out per query token.
  int32_t qmax;
  // Partitioned schedule: the last workgroup of a split row merges its
  // partials through `counters` ([S][Hkv], zero between calls) instead of a
  // combine launch.
  bool fused_combine;
  // Fused write (partitioned schedule, decode rows only): the decode launch
  // also writes each row's new token and reads it from knew / vnew.
  bool fused_write;
  const void* knew;
  const void* vnew;
  const int64_t* slot_mapping;
  void* k_cache_w;
  void* v_cache_w;
};
hipError_t launch_decode(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream);
// Most waves a decode workgroup may hold for this head size and ring depth,
// of the fused-write variant or the others (0: head size not built).
int32_t decode_max_waves(int32_t head_size, int32_t prefetch, bool fused_write = false);
// LDS bytes of one stream-schedule workgroup.
size_t decode_stream_lds_bytes(int32_t head_size, int32_t waves, int32_t num_seqs);

// Prefill rows (q_len > 1): a planner writes the tile list, then the tiles run.
struct PrefillPlan {
  int32_t tile_queries;        // query tokens per list-A tile
  int32_t split_tile_queries;  // query tokens per list-B tile
  int32_t bound_a;       // entries of list A (tiles seeing many keys)
  int32_t bound_b;       // entries of list B (tiles seeing few keys)
  int32_t* tiles_a;      // [bound_a][2] (sequence, first query row) or -1
  int32_t* tiles_b;      // [bound_b][2]
  int32_t* counts;       // [2] tiles the planner put in lists A and B
  bool all_rows;         // list single-token rows too (no decode launch follows)
};
// The planner (one workgroup), then the tiles it listed; the tiles may go to
// another stream ordered after the planner.
hipError_t launch_prefill_plan(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream);
// The KV write of a.num_tokens tokens and the planner in one launch.
hipError_t launch_write_and_plan(const ForwardArgs& a, const PrefillPlan& p, const void* k,
                                 const void* v, const int64_t* slot_mapping, void* k_cache,
                                 void* v_cache, hipStream_t stream);
hipError_t launch_prefill_tiles(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream);
// Query tokens per prefill tile for a given group size (MFMA rows / G), for
// tiles whose rows see many keys (list A) and few (list B).
int32_t prefill_tile_queries(int32_t group);
int32_t prefill_split_tile_queries(int32_t group);
// Decode rows per workgroup of the shared-prefix pass.
int32_t prefix_tile_rows(int32_t group);
// Upper bound on list-B tiles per row.
int32_t prefill_split_tiles_per_row(int32_t group);
// Tiles whose rows see more keys than this go to list A (none can when no
// row is longer).
int32_t prefill_split_keys();

// Shared-prefix pass: the first prefix_keys keys of every decode row come
// from the same blocks (row 0's table); chunks of chunk_keys keys are
// attended for all rows at once and leave partials 0 .. chunks-1 of each row.
struct PrefixPlan {
  int32_t chunks;
  int32_t chunk_keys;     // multiple of 64
  int32_t prefix_keys;    // 16 * prefix blocks
  int32_t num_parts_max;  // partials per row in the workspace (prefix + suffix)
  float* ws_o;
  float* ws_ml;
  // The step's KV write in the same launch (write_tokens 0: none): token t
  // of knew / vnew ([write_tokens][Hkv][D]) goes to slot slot_mapping[t] of
  // k_cache_w / v_cache_w, never a slot of the prefix's blocks.
  int32_t write_tokens;
  const void* knew;
  const void* vnew;
  const int64_t* slot_mapping;
  void* k_cache_w;
  void* v_cache_w;
};
hipError_t launch_prefix(const ForwardArgs& a, const PrefixPlan& p, hipStream_t stream);

// Workspace layout shared by pa_forward and pa_forward_workspace_bytes.
struct WorkspaceLayout {
  bool stream_ok, stream_default;  // even shares fit / are the default schedule
  int32_t qmax;                    // query tokens per decode row (see DecodePlan)
  bool fused_combine;              // partitioned rows merge in the kernel
  int32_t stream_wgs, stream_heads, stream_waves, waves, prefetch;
  int32_t part_tokens, num_parts_max, tile_queries, bound_a, bound_b;
  size_t off_ctr, off_o, off_ml, off_counts, off_tiles_a, off_tiles_b, total;
};
bool plan_workspace(int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_size, int32_t max_blocks_per_seq,
                    int32_t max_query_len_hint, int32_t max_seq_len_hint, WorkspaceLayout* out);

}  // namespace pa
