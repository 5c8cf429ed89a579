// Decode rows of the flattened batch (one query token per sequence): paged
// attention over the sequence's whole context, optionally split over the
// context into partitions whose partial softmax states are then merged.
//
// What is computed follows the pages "Inside vLLM: Anatomy of a
// High-Throughput LLM Inference System": section "Scheduler" (decode requests
// attend over all earlier, already cached KV and are bound by memory
// bandwidth; blocks hold 16 tokens) and section "Run forward pass" (block
// tables index the paged KV memory; each sequence sees only its own tokens).
//
// Work decomposition (gfx950): a workgroup is one (sequence, KV head,
// partition of the context) and holds W waves that take the partition's
// 16-token blocks in turn (wave w: blocks w, w+W, ...), so that one CU keeps
// many blocks in flight even when a row is short. Each wave keeps the G query
// heads of the KV head in MFMA operands:
//   S^T[16 tokens x 16 heads] = K[16 x D] . Q^T[D x 16]   (16x16x32 bf16 MFMA,
//                                                          K straight from HBM)
//   O^T[D x 16 heads]       += V^T[D x 16] . P^T[16 x 16] (16x16x16 bf16 MFMA,
//                                                          V transposed via LDS)
// The S^T accumulator layout (lane: head l%16, tokens 4*(l/16)+r) is exactly
// the B operand layout of the second product, so P never leaves registers.
// Blocks stream through a ring of NBUF register buffers whose loads are
// issued unconditionally (indices clamped), so the compiler's wait counts
// only ever wait for the block being consumed. At the end the W partial
// softmax states are merged through LDS.
//
// Softmax: scores are kept in log2 units against a per-head reference max m.
// m is only recomputed (one max across the four 16-lane groups) and the
// accumulators rescaled when some score exceeds m by more than 2^kLazy; in
// between, weights are exp2(s - m) <= 2^kLazy, which bf16 hi+lo parts and the
// fp32 accumulators carry without loss.
//
// Split-K: when rows x KV heads alone would leave CUs idle, rows are split
// into partitions; a partition that is not its row's only one writes its
// merged (m, l, o) to the workspace and a combine kernel merges the
// partitions. (Merging in the last-arriving workgroup instead measured slower
// on this chip: a row's partitions run on several XCDs, whose L2s are not
// coherent with each other, so the hand-over costs three memory round trips
// at the tail, more than the kernel boundary it saves.)
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr float kLazy = 8.0f;  // log2 of the largest unnormalised weight

template <int D>
struct DecodeShape {
  static constexpr int kKChunks = D / 32;  // 16-byte K chunks per lane per block = QK MFMAs
  static constexpr int kVChunks = D / 32;  // 16-byte V chunks per lane per block
  static constexpr int kDTiles = D / 16;   // PV MFMAs per block (per P part)
  // Padded LDS row of V (elements): rows 16B aligned, and consecutive rows 8
  // banks apart so the four rows of one transpose read do not collide.
  static constexpr int kLdsRow = D + 16;
  static constexpr int kLdsWave = kBlock * kLdsRow;  // elements per wave
  // Merge stage (fp32), heads handled per pass: o rows of D + 4 floats.
  // W * 8 * (D + 4) * 4 + W * 8 * 8 bytes fit in the W V slices.
  static constexpr int kMergeHeads = 8;
  static constexpr int kMergeRow = D + 4;
  static_assert(kMergeHeads * (kMergeRow * 4 + 8) <= kLdsWave * 2, "merge stage fits in LDS");
};

// Most waves per decode workgroup: as many as fit on a CU at the kernel's
// register use (<= 128 VGPRs: 4 waves per SIMD; <= 168: 3).
template <int D, int NBUF>
constexpr int max_waves() { return (D == 64 && NBUF == 2) ? 16 : 12; }

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

template <int D, int NBUF, bool kStreamV>
__global__ __launch_bounds__((max_waves<D, NBUF>() * kWave)) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    uint16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    float scale_log2, int32_t Hq, int32_t Hkv, int32_t G, int32_t MB, int32_t part_tokens,
    int32_t num_parts_max) {
  using Sh = DecodeShape<D>;
  // W V slices of kLdsWave elements while streaming; the merge stage after.
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  const int lane = threadIdx.x & (kWave - 1);
  // The wave index is uniform across the wave; saying so keeps the block
  // loop and the table reads on scalar registers.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int W = blockDim.x / kWave;
  // Rows vary fastest in the grid: consecutive workgroups are dealt to the
  // XCDs in turn, so the work of every partition index and head spreads
  // over all XCDs.
  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int part = blockIdx.z;
  // Block ids of this wave (lane k: partition block w + k*W), read before
  // the row's length is known so the loads overlap; the index is kept inside
  // the row, and lanes past the wave's blocks are never used.
  const int bpp = part_tokens / kBlock;
  const int b_begin = part * bpp;
  const int jb = w + lane * W;
  const int my_blk = (jb < bpp && b_begin + jb < MB)
                         ? block_table[(int64_t)s * MB + b_begin + jb] : 0;
  // Workgroup-uniform exits (before any barrier).
  const int t0 = qsl[s];
  if (qsl[s + 1] - t0 != 1) return;  // not a decode row
  const int L = seq_lens[s];
  const int tok_begin = part * part_tokens;
  if (tok_begin >= L) return;
  const int tok_end = min(L, tok_begin + part_tokens);
  const int nparts = (L + part_tokens - 1) / part_tokens;
  const int nblk = (tok_end + kBlock - 1) / kBlock - b_begin;
  const int nmine = nblk > w ? (nblk - 1 - w) / W + 1 : 0;  // blocks of this wave

  const int hl = lane & 15;   // head within the group (MFMA column)
  const int grp = lane >> 4;  // 16-lane group
  const int64_t kv_row = (int64_t)Hkv * D;  // elements between consecutive tokens of a block

  f32x4 o[Sh::kDTiles];
#pragma unroll
  for (int mi = 0; mi < Sh::kDTiles; ++mi) o[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;

  if (nmine > 0) {
    // Q^T as the B operand: lane holds head hl, d = 32*i + 8*grp + e.
    bf16x8 qv[Sh::kKChunks];
    {
      const u32x4* qp = (const u32x4*)(q + ((int64_t)t0 * Hq + g * G + hl) * D) + grp;
#pragma unroll
      for (int i = 0; i < Sh::kKChunks; ++i) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        qv[i] = as_bf16x8(hl < G ? qp[4 * i] : z);
      }
    }
    uint16_t* vl = lds + w * Sh::kLdsWave;
    const uint16_t* kbase = k_cache + (int64_t)g * D + 8 * grp + (int64_t)hl * kv_row;
    const uint16_t* vbase = v_cache + (int64_t)g * D;

    // Loads the wave's block min(k, nmine-1): always issued, so the wait
    // counts stay exact. Unless blocks are shared between rows, V goes
    // through nontemporal (streaming) loads: each V load covers whole rows
    // and is read once, and measured faster that way. K keeps plain loads:
    // two of its loads cover the two halves of one 128-byte line, which
    // streaming loads re-fetch.
    auto load_block = [&](int k, u32x4 (&kk)[Sh::kKChunks], u32x4 (&vv)[Sh::kVChunks]) {
      const int64_t blk = __builtin_amdgcn_readlane(my_blk, min(k, nmine - 1));
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

    auto process_block = [&](int k, const u32x4 (&kk)[Sh::kKChunks],
                             const u32x4 (&vv)[Sh::kVChunks]) {
      const int tokb = (b_begin + w + k * W) * kBlock;
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

    // The main loop runs whole rounds of NBUF blocks with no early exit, so
    // the loads still in flight at its back-edge are always the same NBUF-1
    // ring slots in the same order and every wait is for exactly the block
    // being consumed (an exit inside the round makes the wait at the loop
    // head drain all loads). Block k0 + v of the last partial round already
    // sits in slot v.
    u32x4 kb[NBUF][Sh::kKChunks], vb[NBUF][Sh::kVChunks];
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) load_block(u, kb[u], vb[u]);
    int k0 = 0;
    for (; k0 + NBUF <= nmine; k0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        load_block(k0 + u + NBUF - 1, kb[(u + NBUF - 1) % NBUF], vb[(u + NBUF - 1) % NBUF]);
        process_block(k0 + u, kb[u], vb[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u)
      if (k0 + u < nmine) process_block(k0 + u, kb[u], vb[u]);
    lsum = sum_across_groups(lsum);
  }

  // Merge the W waves' states through LDS (the V slices are free once every
  // wave has passed the barrier), kMergeHeads heads per pass:
  //   M = max_w m_w, l = sum_w 2^(m_w - M) l_w, o = sum_w 2^(m_w - M) o_w,
  // in wave order (deterministic). A wave without blocks holds m = -inf,
  // l = 0, o = 0 and adds nothing; wave 0 always has a block.
  float* mo = (float*)lds;                                       // [W][8][D + 4]
  float* mml = mo + (size_t)W * Sh::kMergeHeads * Sh::kMergeRow;  // [W][8][2]
  for (int hb = 0; hb < G; hb += Sh::kMergeHeads) {
    __syncthreads();
    const int hh = hl - hb;
    if (hl < G && hh >= 0 && hh < Sh::kMergeHeads) {
      float* orow = mo + (w * Sh::kMergeHeads + hh) * Sh::kMergeRow + 4 * grp;
#pragma unroll
      for (int mi = 0; mi < Sh::kDTiles; ++mi) *(f32x4*)(orow + 16 * mi) = o[mi];
      if (grp == 0) {
        mml[(w * Sh::kMergeHeads + hh) * 2 + 0] = m;
        mml[(w * Sh::kMergeHeads + hh) * 2 + 1] = lsum;
      }
    }
    __syncthreads();
    const int nh = min(Sh::kMergeHeads, G - hb);
    for (int idx = threadIdx.x; idx < nh * (D / 2); idx += blockDim.x) {
      const int h = idx / (D / 2);
      const int d = 2 * (idx % (D / 2));
      float M = -INFINITY;
      for (int v = 0; v < W; ++v) M = fmaxf(M, mml[(v * Sh::kMergeHeads + h) * 2]);
      float den = 0.f, n0 = 0.f, n1 = 0.f;
      for (int v = 0; v < W; ++v) {
        const float* ml = mml + (v * Sh::kMergeHeads + h) * 2;
        const float e = fast_exp2(ml[0] - M);
        const float* orow = mo + (v * Sh::kMergeHeads + h) * Sh::kMergeRow + d;
        den += e * ml[1];
        n0 += e * orow[0];
        n1 += e * orow[1];
      }
      const int head = g * G + hb + h;
      if (nparts == 1) {
        const float inv = 1.0f / den;
        *(uint32_t*)(out + ((int64_t)t0 * Hq + head) * D + d) = pack_bf16x2(n0 * inv, n1 * inv);
      } else {  // read by the combine kernel after this one ends
        const int64_t base = ((int64_t)s * num_parts_max + part) * Hq + head;
        *(f32x2*)(ws_o + base * D + d) = f32x2{n0, n1};
        if (d == 0) *(f32x2*)(ws_ml + base * 2) = f32x2{M, den};
      }
    }
  }
}

// Merge of a row's partitions: one wave per (row, head), lanes across d,
// partitions in order (deterministic). Rows vary fastest in the grid.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, uint16_t* __restrict__ out,
    int32_t Hq, int32_t part_tokens, int32_t num_parts_max) {
  constexpr int kPer = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int s = blockIdx.x;
  const int qh = blockIdx.y * (blockDim.x / kWave) + threadIdx.x / kWave;
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
  using Sh = DecodeShape<D>;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  dim3 grid(a.num_seqs, a.num_kv_heads, p.num_parts_max);
  const size_t lds = (size_t)p.waves * Sh::kLdsWave * sizeof(uint16_t);
  profile_begin(PA_KERNEL_DECODE, stream);
  hipLaunchKernelGGL((decode_kernel<D, NBUF, kStreamV>), grid, dim3(p.waves * kWave), lds,
                     stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                     (const uint16_t*)a.v_cache, a.block_table, a.seq_lens, a.query_start_loc,
                     (uint16_t*)a.out, p.ws_o, p.ws_ml, scale_log2, a.num_q_heads,
                     a.num_kv_heads, a.num_q_heads / a.num_kv_heads, a.max_blocks_per_seq,
                     p.part_tokens, p.num_parts_max);
  profile_end(PA_KERNEL_DECODE, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_parts_max <= 1) return e;
  dim3 cgrid(a.num_seqs, (a.num_q_heads + 3) / 4);
  profile_begin(PA_KERNEL_COMBINE, stream);
  hipLaunchKernelGGL(decode_combine_kernel<D>, cgrid, dim3(256), 0, stream, a.seq_lens,
                     a.query_start_loc, p.ws_o, p.ws_ml, (uint16_t*)a.out, a.num_q_heads,
                     p.part_tokens, p.num_parts_max);
  profile_end(PA_KERNEL_COMBINE, stream);
  return hipGetLastError();
}

}  // namespace

int32_t decode_max_waves(int32_t head_size, int32_t prefetch) {
  switch (head_size) {
    case 64: return prefetch >= 3 ? max_waves<64, 3>() : max_waves<64, 2>();
    case 128: return max_waves<128, 2>();
    default: return 0;
  }
}

hipError_t launch_decode(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream) {
  const int maxw = decode_max_waves(a.head_size, p.prefetch);
  if (p.waves < 1 || p.waves > maxw || p.part_tokens <= 0 || p.part_tokens % kBlock ||
      p.part_tokens / kBlock > kWave * p.waves || p.num_parts_max > 65535 ||
      a.num_kv_heads > 65535)
    return hipErrorInvalidValue;
  // Ring depths that fit the register budget of kMaxWaves waves per CU
  // without spills: 2 or 3 blocks at D = 64, 2 at D = 128.
  const bool sv = p.stream_v;
  switch (a.head_size) {
    case 64:
      if (p.prefetch >= 3) return sv ? launch_decode_nb<64, 3, true>(a, p, stream)
                                     : launch_decode_nb<64, 3, false>(a, p, stream);
      return sv ? launch_decode_nb<64, 2, true>(a, p, stream)
                : launch_decode_nb<64, 2, false>(a, p, stream);
    case 128:
      return sv ? launch_decode_nb<128, 2, true>(a, p, stream)
                : launch_decode_nb<128, 2, false>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
