// KV write of one 16-byte chunk, shared by the cache-write kernel and the
// launch that writes and plans in one (pa_write_and_forward).
#pragma once

#include "common.h"

namespace pa {

// KV write of one 16-byte chunk: chunk i of the new tokens' K and V rows
// (chunks_per_token = Hkv * D / 8 per token; a token's Hkv * D values are
// one contiguous run both in k / v and in its cache row) moves to the slot
// that slot_mapping names. A negative slot (a padding token) moves nothing.
__device__ __forceinline__ void write_kv_chunk(const u32x4* __restrict__ k,
                                               const u32x4* __restrict__ v,
                                               const int64_t* __restrict__ slot_mapping,
                                               u32x4* __restrict__ k_cache,
                                               u32x4* __restrict__ v_cache, int64_t i,
                                               int32_t chunks_per_token) {
  const int64_t t = i / chunks_per_token;
  const int32_t c = (int32_t)(i - t * chunks_per_token);
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;
  const int64_t dst = slot * chunks_per_token + c;
  const u32x4 kv = __builtin_nontemporal_load(k + i);
  const u32x4 vv = __builtin_nontemporal_load(v + i);
  k_cache[dst] = kv;
  v_cache[dst] = vv;
}

}  // namespace pa
