// Host-side launchers of the gfx950 kernels; called by the C ABI layer after
// it has validated every host-known argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

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

// Decode rows (q_len == 1): split-K partials or direct output, then combine.
struct DecodePlan {
  int32_t part_tokens;    // tokens per split-K partition (multiple of 16)
  int32_t num_parts_max;  // partitions reserved per row in the workspace
  float* ws_o;            // [S][num_parts_max][Hq][D] unnormalised partial outputs
  float* ws_ml;           // [S][num_parts_max][Hq][2] running max (log2 units) and sum
};
hipError_t launch_decode(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream);

// Prefill rows (q_len > 1): a planner writes the tile list, then the tiles run.
struct PrefillPlan {
  int32_t tile_queries;  // query tokens per tile
  int32_t tile_bound;    // entries in the tile list (upper bound on tiles)
  int32_t* tiles;        // [tile_bound] (sequence << 16 | tile index) or -1
};
hipError_t launch_prefill(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream);
// Query tokens per prefill tile for a given group size (128 MFMA rows / G).
int32_t prefill_tile_queries(int32_t group);

// Workspace layout shared by pa_forward and pa_forward_workspace_bytes.
struct WorkspaceLayout {
  int32_t part_tokens, num_parts_max, tile_queries, tile_bound;
  size_t off_o, off_ml, off_tiles, total;
};
bool plan_workspace(int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_size, int32_t max_blocks_per_seq,
                    int32_t max_seq_len_hint, WorkspaceLayout* out);

}  // namespace pa
