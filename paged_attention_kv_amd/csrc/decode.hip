// Decode rows of the flattened batch (one query token per sequence): paged
// attention over the sequence's whole context, split over the context into
// partitions whose partial softmax states are merged by a combine kernel.
//
// What is computed follows the pages "Inside vLLM: Anatomy of a
// High-Throughput LLM Inference System": section "Scheduler" (decode requests
// attend over all earlier, already cached KV and are bound by memory
// bandwidth; blocks hold 16 tokens) and section "Run forward pass" (block
// tables index the paged KV memory; each sequence sees only its own tokens).
//
// Work decomposition (gfx950): a workgroup is one (sequence, partition) and
// holds one wave per KV head, so a workgroup streams whole 16-token blocks
// (all heads of a block are contiguous in [NB, 16, Hkv, D]). Each wave keeps
// the G query heads of its KV head in MFMA operands:
//   S^T[16 tokens x 16 heads] = K[16 x D] . Q^T[D x 16]   (16x16x32 bf16 MFMA,
//                                                          K straight from HBM)
//   O^T[D x 16 heads]       += V^T[D x 16] . P^T[16 x 16] (16x16x16 bf16 MFMA,
//                                                          V transposed via LDS)
// The S^T accumulator layout (lane: head l%16, tokens 4*(l/16)+r) is exactly
// the B operand layout of the second product, so P never leaves registers,
// and the per-head softmax statistics are lane-local except for one max
// across the four 16-lane groups per block.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kMaxWavesPerGroup = 8;
constexpr int kMaxPartTokens = 64 * kBlock;  // one table entry per lane

template <int D>
struct DecodeShape {
  static constexpr int kKChunks = D / 32;  // 16-byte K chunks per lane per block = QK MFMAs
  static constexpr int kVChunks = D / 32;  // 16-byte V chunks per lane per block
  static constexpr int kDTiles = D / 16;   // PV MFMAs per block
  // Padded LDS row of V (elements): rows 16B aligned, and consecutive rows 8
  // banks apart so the four rows of one transpose read do not collide.
  static constexpr int kLdsRow = D + 16;
  static constexpr int kLdsWave = kBlock * kLdsRow;
};

template <int D>
__global__ __launch_bounds__(kMaxWavesPerGroup * kWave) void decode_partition_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    uint16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    float scale_log2, int32_t Hq, int32_t Hkv, int32_t G, int32_t MB, int32_t part_tokens,
    int32_t num_parts_max, int32_t waves_per_group) {
  using Sh = DecodeShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kMaxWavesPerGroup * Sh::kLdsWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int s = blockIdx.y;
  const int part = blockIdx.x;
  const int g = blockIdx.z * waves_per_group + w;
  if (g >= Hkv) return;
  const int t0 = qsl[s];
  if (qsl[s + 1] - t0 != 1) return;  // not a decode row
  const int L = seq_lens[s];
  const int tok_begin = part * part_tokens;
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + part_tokens);
  const int nparts = (L + part_tokens - 1) / part_tokens;
  const int b_begin = tok_begin / kBlock;
  const int nblk = (tok_end + kBlock - 1) / kBlock - b_begin;

  const int hl = lane & 15;   // head within the group (MFMA column)
  const int grp = lane >> 4;  // 16-lane group
  const int qh = g * G + hl;
  const int64_t kv_row = (int64_t)Hkv * D;  // elements between consecutive tokens of a block

  // Q^T as the B operand: lane holds head hl, d = 32*i + 8*grp + e.
  bf16x8 qv[Sh::kKChunks];
  {
    const u32x4* qp = (const u32x4*)(q + ((int64_t)t0 * Hq + qh) * D) + grp;
#pragma unroll
    for (int i = 0; i < Sh::kKChunks; ++i) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qv[i] = as_bf16x8(hl < G ? qp[4 * i] : z);
    }
  }

  // This partition's block ids: lane j holds entry b_begin + j.
  const int my_blk = lane < nblk ? block_table[(int64_t)s * MB + b_begin + lane] : 0;

  uint16_t* vl = lds + w * Sh::kLdsWave;
  const uint16_t* kbase = k_cache + (int64_t)g * D + 8 * grp + (int64_t)hl * kv_row;
  f32x4 o[Sh::kDTiles];
#pragma unroll
  for (int mi = 0; mi < Sh::kDTiles; ++mi) o[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;

  auto load_block = [&](int j, u32x4 (&kk)[Sh::kKChunks], u32x4 (&vv)[Sh::kVChunks]) {
    const int64_t blk = __builtin_amdgcn_readlane(my_blk, j);
    const int64_t boff = blk * kBlock * kv_row;
    const u32x4* kp = (const u32x4*)(kbase + boff);
#pragma unroll
    for (int i = 0; i < Sh::kKChunks; ++i) kk[i] = kp[4 * i];
#pragma unroll
    for (int jj = 0; jj < Sh::kVChunks; ++jj) {
      const int c = jj * kWave + lane;
      const int row = c / (D / 8);
      const int col8 = c % (D / 8);
      vv[jj] = *(const u32x4*)(v_cache + boff + row * kv_row + (int64_t)g * D + col8 * 8);
    }
  };

  auto process_block = [&](int j, const u32x4 (&kk)[Sh::kKChunks],
                           const u32x4 (&vv)[Sh::kVChunks]) {
    const int tokb = (b_begin + j) * kBlock;
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < Sh::kKChunks; ++i) sacc = mfma_16x16x32(as_bf16x8(kk[i]), qv[i], sacc);
    float sv[4];
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tokb + 4 * grp + r;
      sv[r] = tok < tok_end ? sacc[r] * scale_log2 : -INFINITY;
      bm = fmaxf(bm, sv[r]);
    }
    bm = max_across_groups(bm);
    const float mn = fmaxf(m, bm);
    const float alpha = fast_exp2(m - mn);
    float p[4];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(sv[r] - mn);
      ps += p[r];
    }
    lsum = lsum * alpha + ps;
    m = mn;
#pragma unroll
    for (int mi = 0; mi < Sh::kDTiles; ++mi) o[mi] *= alpha;

    // V block into this wave's LDS slice, rows past the sequence zeroed.
#pragma unroll
    for (int jj = 0; jj < Sh::kVChunks; ++jj) {
      const int c = jj * kWave + lane;
      const int row = c / (D / 8);
      const int col8 = c % (D / 8);
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4*)(vl + row * Sh::kLdsRow + col8 * 8) = (tokb + row < L) ? vv[jj] : z;
    }
    wave_lds_fence();
    i16x4 phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint16_t h, l;
      split_bf16(p[r], h, l);
      phi[r] = (short)h;
      plo[r] = (short)l;
    }
    // A operand V^T[d = 16*mi + hl][token 4*grp + r] by transpose reads.
    const uint16_t* vrow = vl + (4 * grp + hl / 4) * Sh::kLdsRow + 4 * (hl % 4);
#pragma unroll
    for (int mi = 0; mi < Sh::kDTiles; ++mi) {
      const i16x4 a = lds_read_tr16(vrow + 16 * mi);
      o[mi] = mfma_16x16x16(a, phi, o[mi]);
      o[mi] = mfma_16x16x16(a, plo, o[mi]);
    }
    wave_lds_fence();
  };

  u32x4 k0[Sh::kKChunks], v0[Sh::kVChunks], k1[Sh::kKChunks], v1[Sh::kVChunks];
  load_block(0, k0, v0);
  for (int j = 0; j < nblk; j += 2) {
    if (j + 1 < nblk) load_block(j + 1, k1, v1);
    process_block(j, k0, v0);
    if (j + 1 >= nblk) break;
    if (j + 2 < nblk) load_block(j + 2, k0, v0);
    process_block(j + 1, k1, v1);
  }

  const float ltot = sum_across_groups(lsum);
  if (hl >= G) return;
  if (nparts == 1) {
    const float inv = 1.0f / ltot;
    uint16_t* op = out + ((int64_t)t0 * Hq + qh) * D + 4 * grp;
#pragma unroll
    for (int mi = 0; mi < Sh::kDTiles; ++mi) {
      u32x2 pr = {pack_bf16x2(o[mi][0] * inv, o[mi][1] * inv),
                  pack_bf16x2(o[mi][2] * inv, o[mi][3] * inv)};
      *(u32x2*)(op + 16 * mi) = pr;
    }
  } else {
    const int64_t base = ((int64_t)s * num_parts_max + part) * Hq + qh;
    float* wo = ws_o + base * D + 4 * grp;
#pragma unroll
    for (int mi = 0; mi < Sh::kDTiles; ++mi) *(f32x4*)(wo + 16 * mi) = o[mi];
    if (grp == 0) {
      ws_ml[base * 2 + 0] = m;
      ws_ml[base * 2 + 1] = ltot;
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Merge the partitions of one decode row and one query head:
// M = max_p m_p, out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// summed in partition order (deterministic). One wave per (row, head).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, uint16_t* __restrict__ out,
    int32_t Hq, int32_t part_tokens, int32_t num_parts_max) {
  constexpr int kPer = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int s = blockIdx.y;
  const int qh = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (qh >= Hq) return;
  const int t0 = qsl[s];
  if (qsl[s + 1] - t0 != 1) return;
  const int L = seq_lens[s];
  const int np = (L + part_tokens - 1) / part_tokens;
  if (np <= 1) return;
  const int64_t row0 = (int64_t)s * num_parts_max * Hq + qh;  // partition p at row0 + p*Hq

  float M = -INFINITY;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    const int p = p0 + lane;
    if (p < np) M = fmaxf(M, ws_ml[(row0 + (int64_t)p * Hq) * 2]);
  }
  M = wave_max(M);

  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float wl = 0.f;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    const int p = p0 + lane;
    float wgt = 0.f;
    if (p < np) {
      const int64_t r = row0 + (int64_t)p * Hq;
      wgt = fast_exp2(ws_ml[r * 2] - M);
      wl += wgt * ws_ml[r * 2 + 1];
    }
    const int cnt = min(kWave, np - p0);
    for (int k = 0; k < cnt; ++k) {
      const float wk = __shfl(wgt, k);
      const float* op = ws_o + (row0 + (int64_t)(p0 + k) * Hq) * D;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] += wk * op[lane + kWave * e];
    }
  }
  const float W = wave_sum(wl);
  const float inv = 1.0f / W;
  uint16_t* op = out + ((int64_t)t0 * Hq + qh) * D;
#pragma unroll
  for (int e = 0; e < kPer; ++e) op[lane + kWave * e] = float_to_bf16_bits(acc[e] * inv);
}

template <int D>
hipError_t launch_decode_d(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream) {
  const int waves = a.num_kv_heads < kMaxWavesPerGroup ? a.num_kv_heads : kMaxWavesPerGroup;
  const int groups = (a.num_kv_heads + waves - 1) / waves;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  dim3 grid(p.num_parts_max, a.num_seqs, groups);
  hipLaunchKernelGGL(decode_partition_kernel<D>, grid, dim3(waves * kWave), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                     (const uint16_t*)a.v_cache, a.block_table, a.seq_lens, a.query_start_loc,
                     (uint16_t*)a.out, p.ws_o, p.ws_ml, scale_log2, a.num_q_heads,
                     a.num_kv_heads, a.num_q_heads / a.num_kv_heads, a.max_blocks_per_seq,
                     p.part_tokens, p.num_parts_max, waves);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.num_parts_max <= 1) return hipSuccess;
  dim3 cgrid((a.num_q_heads + 3) / 4, a.num_seqs);
  hipLaunchKernelGGL(decode_combine_kernel<D>, cgrid, dim3(256), 0, stream, a.seq_lens,
                     a.query_start_loc, p.ws_o, p.ws_ml, (uint16_t*)a.out, a.num_q_heads,
                     p.part_tokens, p.num_parts_max);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (p.part_tokens <= 0 || p.part_tokens % kBlock || p.part_tokens > kMaxPartTokens)
    return hipErrorInvalidValue;
  switch (a.head_size) {
    case 64: return launch_decode_d<64>(a, p, stream);
    case 128: return launch_decode_d<128>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
