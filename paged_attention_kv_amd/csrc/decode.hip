// Decode rows of the flattened batch (one query token per sequence): paged
// attention over the sequence's whole context, split over the context into
// partitions whose partial softmax states are then merged.
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
// the B operand layout of the second product, so P never leaves registers.
// Blocks stream through a ring of NBUF register buffers whose loads are
// issued unconditionally (indices clamped), so the compiler's wait counts
// only ever wait for the block being consumed.
//
// Softmax: scores are kept in log2 units against a per-head reference max m.
// m is only recomputed (one max across the four 16-lane groups) and the
// accumulators rescaled when some score exceeds m by more than 2^kLazy; in
// between, weights are exp2(s - m) <= 2^kLazy, which bf16 hi+lo parts and the
// fp32 accumulators carry without loss.
//
// Split-K merge: a partition that is not its row's only one writes
// (m, l, o) to the workspace. With `fused`, the last workgroup of a row to
// finish (an atomic counter per row, reset by that workgroup) merges the
// partitions itself; otherwise a separate combine kernel does it.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kMaxWavesPerGroup = 8;
constexpr int kMaxPartTokens = 64 * kBlock;  // one table entry per lane
constexpr float kLazy = 8.0f;                // log2 of the largest unnormalised weight

template <int D>
struct DecodeShape {
  static constexpr int kKChunks = D / 32;  // 16-byte K chunks per lane per block = QK MFMAs
  static constexpr int kVChunks = D / 32;  // 16-byte V chunks per lane per block
  static constexpr int kDTiles = D / 16;   // PV MFMAs per block (per P part)
  // Padded LDS row of V (elements): rows 16B aligned, and consecutive rows 8
  // banks apart so the four rows of one transpose read do not collide.
  static constexpr int kLdsRow = D + 16;
  static constexpr int kLdsWave = kBlock * kLdsRow;
};

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

// Merge the np <= kMaxFusedParts partitions of one query head of a decode
// row: M = max_p m_p, out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// summed in partition order. All loads are issued before the first use, so
// the merge costs one memory round trip. Produces the four d of quad d4.
constexpr int kMaxFusedParts = 16;
template <int D>
__device__ __forceinline__ void merge_head_quad(const float* __restrict__ ws_o,
                                                const float* __restrict__ ws_ml,
                                                uint16_t* __restrict__ out, int64_t row0,
                                                int32_t Hq, int np, int64_t out_off, int d4) {
  float mv[kMaxFusedParts], lv[kMaxFusedParts];
  f32x4 ov[kMaxFusedParts];
#pragma unroll
  for (int p = 0; p < kMaxFusedParts; ++p) {
    if (p < np) {
      const int64_t r = row0 + (int64_t)p * Hq;
      mv[p] = load_coherent(ws_ml + r * 2);
      lv[p] = load_coherent(ws_ml + r * 2 + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[p][e] = load_coherent(ws_o + r * D + 4 * d4 + e);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kMaxFusedParts; ++p)
    if (p < np) M = fmaxf(M, mv[p]);
  float W = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < kMaxFusedParts; ++p) {
    if (p < np) {
      const float w = fast_exp2(mv[p] - M);
      W += w * lv[p];
      acc += w * ov[p];
    }
  }
  const float inv = 1.0f / W;
  u32x2 pr = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *(u32x2*)(out + out_off + 4 * d4) = pr;
}

template <int D, int NBUF, bool kStreamV>
__global__ __launch_bounds__(kMaxWavesPerGroup * kWave) void decode_partition_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    uint16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int32_t* __restrict__ counters, float scale_log2, int32_t Hq, int32_t Hkv, int32_t G,
    int32_t MB, int32_t part_tokens, int32_t num_parts_max, int32_t waves_per_group,
    int32_t fused) {
  using Sh = DecodeShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kMaxWavesPerGroup * Sh::kLdsWave];
  __shared__ int32_t last_flag;

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int s = blockIdx.y;
  const int part = blockIdx.x;
  const int g = blockIdx.z * waves_per_group + w;
  const bool active = g < Hkv;  // wave-uniform; idle waves still meet the barriers
  // This partition's block ids (lane j: entry part*part_tokens/16 + j), read
  // before the row's length is known so the two loads overlap; the index is
  // kept inside the row, and lanes past the partition are never used.
  const int b_begin = part * (part_tokens / kBlock);
  const int my_blk = (lane < part_tokens / kBlock && b_begin + lane < MB)
                         ? block_table[(int64_t)s * MB + b_begin + lane] : 0;
  // Workgroup-uniform exits, all before any barrier.
  const int t0 = qsl[s];
  if (qsl[s + 1] - t0 != 1) return;  // not a decode row
  const int L = seq_lens[s];
  const int tok_begin = part * part_tokens;
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + part_tokens);
  const int nparts = (L + part_tokens - 1) / part_tokens;
  const int nblk = (tok_end + kBlock - 1) / kBlock - b_begin;

  const int hl = lane & 15;   // head within the group (MFMA column)
  const int grp = lane >> 4;  // 16-lane group
  const int qh = g * G + hl;
  const int64_t kv_row = (int64_t)Hkv * D;  // elements between consecutive tokens of a block

  f32x4 o[Sh::kDTiles];
#pragma unroll
  for (int mi = 0; mi < Sh::kDTiles; ++mi) o[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;

  if (active) {
    // Q^T as the B operand: lane holds head hl, d = 32*i + 8*grp + e.
    bf16x8 qv[Sh::kKChunks];
    {
      const u32x4* qp = (const u32x4*)(q + ((int64_t)t0 * Hq + qh) * D) + grp;
#pragma unroll
      for (int i = 0; i < Sh::kKChunks; ++i) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        qv[i] = as_bf16x8(hl < G ? qp[4 * i] : z);
      }
    }
    uint16_t* vl = lds + w * Sh::kLdsWave;
    const uint16_t* kbase = k_cache + (int64_t)g * D + 8 * grp + (int64_t)hl * kv_row;
    const uint16_t* vbase = v_cache + (int64_t)g * D;

    // Loads block min(j, nblk-1): always issued, so the wait counts stay exact.
    // Unless blocks are shared between rows, V goes through nontemporal
    // (streaming) loads: each V load covers whole rows and is read once, and
    // measured faster that way. K keeps plain loads: two of its loads cover
    // the two halves of one 128-byte line, which streaming loads re-fetch.
    auto load_block = [&](int j, u32x4 (&kk)[Sh::kKChunks], u32x4 (&vv)[Sh::kVChunks]) {
      const int jj = min(j, nblk - 1);
      const int64_t blk = __builtin_amdgcn_readlane(my_blk, jj);
      const int64_t boff = blk * kBlock * kv_row;
      const u32x4* kp = (const u32x4*)(kbase + boff);
#pragma unroll
      for (int i = 0; i < Sh::kKChunks; ++i) kk[i] = kp[4 * i];
#pragma unroll
      for (int c = 0; c < Sh::kVChunks; ++c) {
        const int idx = c * kWave + lane;
        const int row = idx / (D / 8);
        const int col8 = idx % (D / 8);
        const u32x4* vp = (const u32x4*)(vbase + boff + row * kv_row + col8 * 8);
        vv[c] = kStreamV ? __builtin_nontemporal_load(vp) : *vp;
      }
    };

    auto process_block = [&](int j, const u32x4 (&kk)[Sh::kKChunks],
                             const u32x4 (&vv)[Sh::kVChunks]) {
      const int tokb = (b_begin + j) * kBlock;
      // V block into this wave's LDS slice, rows past the sequence zeroed.
#pragma unroll
      for (int c = 0; c < Sh::kVChunks; ++c) {
        const int idx = c * kWave + lane;
        const int row = idx / (D / 8);
        const int col8 = idx % (D / 8);
        const u32x4 z = {0u, 0u, 0u, 0u};
        *(u32x4*)(vl + row * Sh::kLdsRow + col8 * 8) = (tokb + row < L) ? vv[c] : z;
      }
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < Sh::kKChunks; ++i) sacc = mfma_16x16x32(as_bf16x8(kk[i]), qv[i], sacc);
      float sv[4];
      bool over = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tokb + 4 * grp + r;
        sv[r] = tok < tok_end ? sacc[r] * scale_log2 : -INFINITY;
        over |= sv[r] > m + kLazy;
      }
      if (__any(over)) {  // wave-uniform: re-reference the softmax
        float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        bm = max_across_groups(bm);
        const float mn = fmaxf(m, bm);
        const float alpha = fast_exp2(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int mi = 0; mi < Sh::kDTiles; ++mi) o[mi] *= alpha;
        m = mn;
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(sv[r] - m);
        lsum += p[r];
      }
      const u32x2 s01 = split_pack_bf16x2(p[0], p[1]);
      const u32x2 s23 = split_pack_bf16x2(p[2], p[3]);
      const i16x4 phi = __builtin_bit_cast(i16x4, u32x2{s01[0], s23[0]});
      const i16x4 plo = __builtin_bit_cast(i16x4, u32x2{s01[1], s23[1]});
      wave_lds_fence();
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

    u32x4 kb[NBUF][Sh::kKChunks], vb[NBUF][Sh::kVChunks];
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) load_block(u, kb[u], vb[u]);
    for (int j0 = 0; j0 < nblk; j0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int j = j0 + u;
        if (j >= nblk) break;
        load_block(j + NBUF - 1, kb[(u + NBUF - 1) % NBUF], vb[(u + NBUF - 1) % NBUF]);
        process_block(j, kb[u], vb[u]);
      }
    }
    lsum = sum_across_groups(lsum);
  }

  if (nparts == 1) {
    if (!active || hl >= G) return;
    const float inv = 1.0f / lsum;
    uint16_t* op = out + ((int64_t)t0 * Hq + qh) * D + 4 * grp;
#pragma unroll
    for (int mi = 0; mi < Sh::kDTiles; ++mi) {
      u32x2 pr = {pack_bf16x2(o[mi][0] * inv, o[mi][1] * inv),
                  pack_bf16x2(o[mi][2] * inv, o[mi][3] * inv)};
      *(u32x2*)(op + 16 * mi) = pr;
    }
    return;
  }
  if (active && hl < G) {
    const int64_t base = ((int64_t)s * num_parts_max + part) * Hq + qh;
    float* wo = ws_o + base * D + 4 * grp;
    if (fused) {  // read by another workgroup of this kernel, maybe on another XCD
#pragma unroll
      for (int mi = 0; mi < Sh::kDTiles; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e) store_coherent(wo + 16 * mi + e, o[mi][e]);
      if (grp == 0) {
        store_coherent(ws_ml + base * 2 + 0, m);
        store_coherent(ws_ml + base * 2 + 1, lsum);
      }
    } else {  // read by the combine kernel after this one ends
#pragma unroll
      for (int mi = 0; mi < Sh::kDTiles; ++mi) *(f32x4*)(wo + 16 * mi) = o[mi];
      if (grp == 0) {
        ws_ml[base * 2 + 0] = m;
        ws_ml[base * 2 + 1] = lsum;
      }
    }
  }
  if (!fused) return;

  // Last-arriving workgroup of this (row, head group) merges the partitions.
  // The partials went out as coherent stores; waiting for them to complete
  // before the barrier orders them before the arrival count, and the merge
  // reads them with coherent loads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int32_t* ctr = counters + (int64_t)s * gridDim.z + blockIdx.z;
  if (threadIdx.x == 0)
    last_flag = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                nparts - 1;
  __syncthreads();
  if (!last_flag) return;
  if (threadIdx.x == 0)  // ready for the next call
    __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!active) return;
  const int64_t row0 = (int64_t)s * num_parts_max * Hq;  // + p*Hq + head
  for (int idx = lane; idx < G * (D / 4); idx += kWave) {
    const int h = idx / (D / 4);
    const int head = g * G + h;
    merge_head_quad<D>(ws_o, ws_ml, out, row0 + head, Hq, nparts,
                       ((int64_t)t0 * Hq + head) * D, idx % (D / 4));
  }
}

// Separate merge for rows with many partitions: one wave per (row, head),
// lanes across d, partitions in order (deterministic).
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
    // eight partitions per batch, all loads issued before their use
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      float vals[8][kPer];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int kk = min(k0 + k, cnt - 1);
        const float* op = ws_o + (row0 + (int64_t)(p0 + kk) * Hq) * D;
#pragma unroll
        for (int e = 0; e < kPer; ++e) vals[k][e] = op[lane + kWave * e];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float wk = __shfl(wgt, min(k0 + k, kWave - 1));
        if (k0 + k < cnt) {
#pragma unroll
          for (int e = 0; e < kPer; ++e) acc[e] += wk * vals[k][e];
        }
      }
    }
  }
  const float W = wave_sum(wl);
  const float inv = 1.0f / W;
  uint16_t* op = out + ((int64_t)t0 * Hq + qh) * D;
#pragma unroll
  for (int e = 0; e < kPer; ++e) op[lane + kWave * e] = float_to_bf16_bits(acc[e] * inv);
}

template <int D, int NBUF, bool kStreamV>
hipError_t launch_decode_nb(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream) {
  const int waves = a.num_kv_heads < kMaxWavesPerGroup ? a.num_kv_heads : kMaxWavesPerGroup;
  const int groups = (a.num_kv_heads + waves - 1) / waves;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  dim3 grid(p.num_parts_max, a.num_seqs, groups);
  profile_begin(PA_KERNEL_DECODE, stream);
  hipLaunchKernelGGL((decode_partition_kernel<D, NBUF, kStreamV>), grid, dim3(waves * kWave), 0,
                     stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                     (const uint16_t*)a.v_cache, a.block_table, a.seq_lens, a.query_start_loc,
                     (uint16_t*)a.out, p.ws_o, p.ws_ml, p.counters, scale_log2, a.num_q_heads,
                     a.num_kv_heads, a.num_q_heads / a.num_kv_heads, a.max_blocks_per_seq,
                     p.part_tokens, p.num_parts_max, waves, p.fused ? 1 : 0);
  profile_end(PA_KERNEL_DECODE, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.fused || p.num_parts_max <= 1) return e;
  dim3 cgrid((a.num_q_heads + 3) / 4, a.num_seqs);
  profile_begin(PA_KERNEL_COMBINE, stream);
  hipLaunchKernelGGL(decode_combine_kernel<D>, cgrid, dim3(256), 0, stream, a.seq_lens,
                     a.query_start_loc, p.ws_o, p.ws_ml, (uint16_t*)a.out, a.num_q_heads,
                     p.part_tokens, p.num_parts_max);
  profile_end(PA_KERNEL_COMBINE, stream);
  return hipGetLastError();
}

}  // namespace

int32_t decode_groups(int32_t num_kv_heads) {
  const int waves = num_kv_heads < kMaxWavesPerGroup ? num_kv_heads : kMaxWavesPerGroup;
  return (num_kv_heads + waves - 1) / waves;
}

hipError_t launch_decode(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (p.part_tokens <= 0 || p.part_tokens % kBlock || p.part_tokens > kMaxPartTokens)
    return hipErrorInvalidValue;
  const int nbuf = p.prefetch;
  const bool sv = p.stream_v;
#define PA_DECODE_CASE(DD)                                                            \
  if (nbuf <= 2) return sv ? launch_decode_nb<DD, 2, true>(a, p, stream)             \
                           : launch_decode_nb<DD, 2, false>(a, p, stream);           \
  if (nbuf == 3) return sv ? launch_decode_nb<DD, 3, true>(a, p, stream)             \
                           : launch_decode_nb<DD, 3, false>(a, p, stream);           \
  return sv ? launch_decode_nb<DD, 4, true>(a, p, stream)                            \
            : launch_decode_nb<DD, 4, false>(a, p, stream);
  switch (a.head_size) {
    case 64: { PA_DECODE_CASE(64) }
    case 128: { PA_DECODE_CASE(128) }
#undef PA_DECODE_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
