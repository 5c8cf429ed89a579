// KV-cache write: every new token's key and value rows are copied into the
// slot its slot_mapping entry names (pages "Inside vLLM: Anatomy of a
// High-Throughput LLM Inference System", section "Run forward pass" for the
// slot mapping and section "Prefix Caching" for the forward pass filling the
// paged KV memory). A token's Hkv*D values are one contiguous run both in k/v
// and in the cache row, so the copy is a run of 16-byte moves per token.
#include "common.h"
#include "kernels.h"
#include "kv_write.h"

namespace pa {

// One thread moves one 16-byte chunk of K and the matching chunk of V.
// chunks_per_token = Hkv * D / 8.
__global__ __launch_bounds__(256) void cache_write_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, int64_t total_chunks, int32_t chunks_per_token) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total_chunks) write_kv_chunk(k, v, slot_mapping, k_cache, v_cache, i, chunks_per_token);
}

hipError_t launch_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                              void* k_cache, void* v_cache, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_size, hipStream_t stream) {
  const int32_t chunks_per_token = num_kv_heads * head_size / 8;
  const int64_t total = (int64_t)num_tokens * chunks_per_token;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  profile_begin(PA_KERNEL_CACHE_WRITE, stream);
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const u32x4*)k, (const u32x4*)v, slot_mapping, (u32x4*)k_cache,
                     (u32x4*)v_cache, total, chunks_per_token);
  profile_end(PA_KERNEL_CACHE_WRITE, stream);
  return hipGetLastError();
}

}  // namespace pa
