// Read probe: every K and V block of the rows' contexts read once, whole,
// with no arithmetic. A decode step reads the same blocks (section "Run
// forward pass" of the pages "Inside vLLM: Anatomy of a High-Throughput LLM
// Inference System": the block table names them), so the probe's rate is
// what the memory system delivers for that scattered-block pattern, the
// ceiling a decode kernel's bandwidth is compared with.
#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

// One workgroup per (row, chunk of blocks_per_wg table columns); its waves
// take the chunk's blocks in turn, each reading a whole block of K and of V
// (16 * Hkv * D bf16 each) in 1 KiB wave-wide steps, eight steps per cache
// in flight. Block ids are clamped into the pool, so a bad table entry
// cannot send a load outside it. The loads feed an XOR whose value is
// stored only if it equals a fixed constant, which keeps them live while
// writing (almost) nothing.
__global__ __launch_bounds__(1024) void block_read_probe_kernel(
    const u32x4* __restrict__ k_cache, const u32x4* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    int32_t MB, int64_t num_blocks, int32_t block_vecs, int32_t blocks_per_wg,
    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int W = blockDim.x / kWave;
  const int s = blockIdx.x;
  const int nb = (seq_lens[s] + kBlock - 1) / kBlock;
  const int b0 = blockIdx.y * blocks_per_wg;
  const int b1 = min(nb, b0 + blocks_per_wg);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int b = b0 + w; b < b1; b += W) {
    int64_t id = block_table[(int64_t)s * MB + b];
    id = id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
    const u32x4* kp = k_cache + id * block_vecs;
    const u32x4* vp = v_cache + id * block_vecs;
    for (int i0 = 0; i0 < block_vecs; i0 += 8 * kWave) {
      u32x4 r[16];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = min(i0 + u * kWave + lane, block_vecs - 1);
        r[u] = __builtin_nontemporal_load(kp + i);
        r[8 + u] = __builtin_nontemporal_load(vp + i);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) acc ^= r[u];
    }
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

hipError_t launch_block_read_probe(const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_kv_heads, int32_t head_size,
                                   int32_t max_blocks_per_seq, int64_t num_blocks, int32_t waves,
                                   int32_t blocks_per_wg, uint32_t* sink, hipStream_t stream) {
  const int32_t block_vecs = kBlock * num_kv_heads * head_size / 8;
  dim3 grid(num_seqs, (max_blocks_per_seq + blocks_per_wg - 1) / blocks_per_wg);
  hipLaunchKernelGGL(block_read_probe_kernel, grid, dim3(waves * kWave), 0, stream,
                     (const u32x4*)k_cache, (const u32x4*)v_cache, block_table, seq_lens,
                     max_blocks_per_seq, num_blocks, block_vecs, blocks_per_wg, sink);
  return hipGetLastError();
}

}  // namespace pa
