// Decode rows of the flattened batch (one query token per sequence, or a few
// when a step verifies drafted tokens): paged attention over the sequence's
// whole context.
//
// What is computed follows the pages "Inside vLLM: Anatomy of a
// High-Throughput LLM Inference System": section "Scheduler" (decode requests
// attend over all earlier, already cached KV and are bound by memory
// bandwidth; blocks hold 16 tokens) and section "Run forward pass" (block
// tables index the paged KV memory; each sequence sees only its own tokens).
//
// Per wave (gfx950): a wave owns one KV head of one row and streams 16-token
// blocks, keeping the G query heads of that KV head in MFMA operands:
//   S^T[16 tokens x 16 heads] = K[16 x D] . Q^T[D x 16]   (16x16x32 bf16 MFMA,
//                                                          K straight from HBM)
//   O^T[D x 16 heads]       += V^T[D x 16] . P^T[16 x 16] (16x16x16 bf16 MFMA,
//                                                          V transposed via LDS)
// Each K load covers whole 128-byte lines of 8 tokens (a line fetched by two
// instructions that each take half of it measured ~30% slower at low load);
// the QK products take each line as two 32-element rows of the A operand and
// add the pair, which leaves lane group grp with the scores of tokens 2*grp,
// 2*grp+1, 8+2*grp and 9+2*grp. V rows are placed in LDS so that the
// transpose reads give the same group those tokens, so P goes from the score
// registers into the B operand of the second product without moving between
// lanes. Blocks stream through a ring of NBUF register buffers whose loads
// are issued unconditionally (indices clamped), so the compiler's wait counts
// only ever wait for the block being consumed; blocks wholly inside every
// query column's visible range take a path with no masks. Softmax: scores are
// kept in log2 units against a per-head reference max m, re-referenced (one
// max across the four 16-lane groups, accumulators rescaled) only when a
// score exceeds it by more than 2^kLazy; weights stay <= 2^kLazy. Rows of at
// most kSplitKeys keys pass the weights to PV as bf16 hi + lo parts (about
// 2^-17 relative); longer rows as one bf16 part, their weight sums adding the
// same rounded values. Several waves of a workgroup may hold partial states
// of one (row, KV head); they are merged through LDS: M = max m_w, l = sum
// 2^(m_w - M) l_w, o = sum 2^(m_w - M) o_w, in wave order.
//
// Two schedules:
//  * stream (decode_stream_kernel): one persistent workgroup per CU takes an
//    equal, contiguous share of all decode rows' blocks (rows in order, each
//    row's blocks in order), with one wave per KV head (or several per head
//    when there are few heads), so every CU streams the same number of bytes
//    whatever the mix of lengths, and each block is read by all its heads at
//    once. A row whose blocks fall into several shares is merged by the share
//    that finishes last: the others publish their partial state with
//    device-coherent stores and count themselves in on a per-row counter.
//    (Row lengths are read on the device; the host never sees them.)
//  * partitioned (decode_kernel): one workgroup per (row, KV head, fixed-size
//    partition) -- or per (row, partition) holding several KV heads -- with
//    W waves taking the partition's blocks in turn; the last workgroup of a
//    row of several partitions merges their partials (arrival counter), or
//    decode_combine_kernel does after the launch. Used for small batches,
//    whose even shares would be too short to hide their fixed latency, and
//    for batches with too many rows for the stream kernel's row scan.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr float kLazy = 8.0f;  // log2 of the largest unnormalised weight
// Rows of at most this many keys keep the weights to about 2^-17 (bf16 hi +
// lo parts); longer rows take one bf16 part, as the prefill tiles do.
constexpr int kSplitKeys = 128;
// Cache-policy bit of a buffer load that marks it nontemporal (streaming).
constexpr int kBufferNt = 2;

template <int D>
struct DecodeShape {
  static constexpr int kKChunks = D / 32;  // 16-byte K chunks per lane per block = QK MFMAs
  static constexpr int kVChunks = D / 32;  // 16-byte V chunks per lane per block
  static constexpr int kDTiles = D / 16;   // PV MFMAs per block (per P part)
  // Padded LDS row of V (elements): rows 16B aligned, and consecutive rows 8
  // banks apart so the four rows of one transpose read do not collide.
  static constexpr int kLdsRow = D + 16;
  static constexpr int kLdsWave = kBlock * kLdsRow;  // elements per wave
  // Merge stage (fp32): kMergeCols query columns per pass, rows of D + 4
  // floats; W * kMergeCols * (D + 4) * 4 + W * kMergeCols * 8 bytes fit in
  // the W V slices.
  static constexpr int kMergeCols = 8;
  static constexpr int kMergeRow = D + 4;
  static_assert(kMergeCols * (kMergeRow * 4 + 8) <= kLdsWave * 2, "merge stage fits in LDS");
};

// Most waves per partitioned decode workgroup, which sets the kernel's
// register budget (<= 128 VGPRs at 16 waves, 4 per SIMD; <= 168 at 12; <= 256
// at 8). Sweeps of 2..16 waves found four best on every workload.
template <int D, int NBUF, bool kWrite = false>
constexpr int max_waves() { return (D == 64 && NBUF == 2) ? 16 : (kWrite ? 8 : 12); }

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

// Device-coherent store and load of 8 bytes (agent scope, relaxed): they go
// past this XCD's L2, so workgroups on different XCDs can hand data over.
// The order that makes the hand-over correct comes from count_in below.
__device__ __forceinline__ void store_coherent2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 load_coherent2(const float* p) {
  const uint64_t v =
      __hip_atomic_load((uint64_t*)const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x2{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
}

// Hand-over of a split row between workgroups (every thread of the
// workgroup calls it, after storing its partials with store_coherent2).
// Each wave waits for its own stores, the workgroup barrier orders them
// before thread 0's read-modify-write of the arrival counter, which releases
// them at agent scope. The workgroup that arrives last (old value
// ncontrib - 1) has read the value the others' release RMWs left (each RMW
// continues the release sequences of the ones before it); its thread 0 takes
// an agent-scope acquire fence, and the second barrier orders every thread's
// later reads of the partials after it. Only the last arriver acquires, so
// the others pay no cache invalidation. The last arriver resets the counter
// (no other workgroup of this launch touches it again). Returns true in
// every thread of the last workgroup.
__device__ __forceinline__ bool count_in(int32_t* ctr, int ncontrib, int32_t* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == ncontrib - 1;
    if (last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// Online-softmax state of one wave: O^T tiles (lane: d = 16*mi + 4*(l/16) + r,
// query column l%16), the reference max and the running sum of weights.
template <int D>
struct WaveAcc {
  f32x4 o[D / 16];
  float m;
  float lsum;  // the lane's tokens' weights; after finish(), the column's
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int mi = 0; mi < D / 16; ++mi) o[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    lsum = 0.f;
  }
  __device__ __forceinline__ void finish() { lsum = sum_across_groups(lsum); }
};

// Q^T as the B operand: lane holds query column hl (< ncols, else zeros),
// d = 32*i + 8*grp + e. Column hl is head hl % G of token hl / G of the row
// (qrow: the row's first token, its KV head's first query head; Hq heads
// per token).
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qv)[D / 32], const uint16_t* __restrict__ qrow,
                                       int hl, int grp, int ncols, int G, int Hq) {
  // (every lane loads, from a valid column, so no branch guards the loads)
  const int col = hl < ncols ? hl : 0;
  const u32x4* qp = (const u32x4*)(qrow + ((int64_t)(col / G) * Hq + col % G) * D) + grp;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 t = qp[4 * i];
    qv[i] = as_bf16x8(hl < ncols ? t : z);
  }
}

// Where a kernel also writes the step's new tokens into the cache (the fused
// write), it reads the row's newest token from the step's own k and v, not
// from the cache slot being written in the same launch, unless the slot is
// negative (nothing is written and the cache holds the token, as after a
// separate write). The slot sits in lane 0 of `slot`, loaded by a vector
// load at the start and first read when the wave loads its last block, so
// the blocks start streaming before it arrives.
struct NewToken {
  int tok;                          // its position in the row (-1: none)
  const uint16_t* __restrict__ k;   // its K of this KV head (D elements)
  const uint16_t* __restrict__ v;   // its V of this KV head
  int64_t slot;                     // lane 0: its slot_mapping entry
};

// Lane 0's value of a 64-bit register, as a wave-uniform value.
__device__ __forceinline__ int64_t first_lane64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Streams nk (1..64) blocks of one KV head into acc: block k's id sits in lane
// k of `ids`, its first token is tok0 + k * tok_step, and tokens >= tok_end
// are masked (their V rows zeroed). col_lim (per lane: its query column's
// last visible key, >= tok_end - 1 for a single-token row) masks the tail
// of a row with several query tokens causally; full_end (wave-uniform,
// <= tok_end and <= every lane's col_lim + 1) is where masking can start:
// a block wholly below it takes the unmasked path. kbase / vbase point at
// the head's slice of the cache (element g * D of block 0); vl is the
// wave's LDS slice. split_p: the weights enter PV as bf16 hi + lo parts
// (rows with few keys, where each weight carries much of an output), else
// as one bf16 part. With kNew, token nt.tok is read from nt.k / nt.v.
template <int D, int NBUF, bool kStreamV, bool kNew, bool kSplit>
__device__ __forceinline__ void stream_blocks_impl(WaveAcc<D>& acc, const bf16x8 (&qv)[D / 32],
                                                   int ids, int nk, int tok0, int tok_step,
                                                   int tok_end, int full_end,
                                                   const uint16_t* __restrict__ kbase,
                                                   const uint16_t* __restrict__ vbase,
                                                   int64_t kv_row, uint16_t* vl, float scale_log2,
                                                   int lane, NewToken nt, int col_lim) {
  using Sh = DecodeShape<D>;
  const int hl = lane & 15;
  const int grp = lane >> 4;

  // K load j covers 8 tokens' whole 128-byte lines (tokens kt(j) .. +7,
  // elements 64 * kl(j) .. +63 of each): lane (hl, grp) takes token
  // kt(j) + hl/2, elements 64*kl(j) + 32*(hl%2) + 8*grp .. +7, so every line
  // is fetched by one instruction. The lane's 16 bytes are the A operand of
  // a 16x16x32 product whose row hl is half hl%2 of that token's line: the
  // product with q's k-block 2*kl(j) is valid for even rows, with k-block
  // 2*kl(j) + 1 for odd rows, and a token's score is the sum of its two
  // rows. V: 16-byte chunk c*64 + lane of the head's 16 rows, chunk c one
  // fixed stride after chunk 0. A block's loads are buffer loads from a base
  // the wave computes once per block on the scalar unit, so the per-block
  // address work is one lane read, a 32 x 32-bit product and two 64-bit adds.
  const uint32_t blk_bytes = (uint32_t)(kBlock * kv_row * 2);
  const int koff = (int)(((hl / 2) * kv_row + 32 * (hl % 2) + 8 * grp) * 2);
  auto kt = [](int j) { return 8 * (j % 2); };  // first token of K load j
  auto kl = [](int j) { return j / 2; };        // its 64-element line
  const int voff = (int)(((lane / (D / 8)) * kv_row + (lane % (D / 8)) * 8) * 2);
  constexpr int kVRows = kWave / (D / 8);             // rows per V chunk
  const int vstride = (int)(kVRows * kv_row * 2);      // bytes between V chunks
  const int nrec = (int)blk_bytes;  // loads stay inside the block
  // The block (k index) holding the newest token when it is one of ours.
  int knew = -1;
  if constexpr (kNew) {
    const int tb = nt.tok & ~(kBlock - 1);
    if (nt.tok >= 0 && tb >= tok0 && (tb - tok0) % tok_step == 0) {
      const int kk = (tb - tok0) / tok_step;
      knew = kk < nk ? kk : -1;
    }
  }

  // Loads block min(k, nk-1): always issued, so the wait counts stay exact.
  // Unless blocks are shared between rows, K and V go through nontemporal
  // (streaming) loads: every load covers whole 128-byte lines that are read
  // once, and measured faster that way (decode workload 21.8 -> 21.2 us with
  // K streaming too).
  auto load_block = [&](int k, u32x4 (&kk)[Sh::kKChunks], u32x4 (&vv)[Sh::kVChunks]) {
    const int kc = min(k, nk - 1);
    const uint64_t off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(ids, kc) * blk_bytes;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)kbase + off), (short)0, nrec, kBufferWordFlags);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)vbase + off), (short)0, nrec, kBufferWordFlags);
#pragma unroll
    for (int j = 0; j < Sh::kKChunks; ++j)
      kk[j] = __builtin_amdgcn_raw_buffer_load_b128(
          kr, koff, (int)((kt(j) * kv_row + 64 * kl(j)) * 2), kStreamV ? kBufferNt : 0);
#pragma unroll
    for (int c = 0; c < Sh::kVChunks; ++c)
      vv[c] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff, c * vstride,
                                                     kStreamV ? kBufferNt : 0);
    if constexpr (kNew) {
      // One block of the row holds its newest token: the wave that streams
      // it reads the slot here, long after its load returned, and then
      // replaces that token's row with the step's own K and V. Every other
      // block pays one scalar compare.
      if (kc == knew && first_lane64(nt.slot) >= 0) {
        const int r = nt.tok & (kBlock - 1);  // the token's row in the block
#pragma unroll
        for (int j = 0; j < Sh::kKChunks; ++j)
          if (kt(j) + hl / 2 == r)
            kk[j] = *(const u32x4*)(nt.k + 64 * kl(j) + 32 * (hl % 2) + 8 * grp);
#pragma unroll
        for (int c = 0; c < Sh::kVChunks; ++c) {
          const int idx = c * kWave + lane;
          if (idx / (D / 8) == r) vv[c] = *(const u32x4*)(nt.v + (idx % (D / 8)) * 8);
        }
      }
    }
  };

  // One block: V into the wave's LDS slice, S^T = K Q^T, lazy online
  // softmax, O^T += V^T P^T. kFull: every token of the block is visible to
  // every column (no masks, no zeroed rows, no -inf scores).
  auto process_block = [&](int k, const u32x4 (&kk)[Sh::kKChunks],
                           const u32x4 (&vv)[Sh::kVChunks], auto full_tag) {
    constexpr bool kFull = decltype(full_tag)::value;
    const int tokb = tok0 + k * tok_step;
    // V block into this wave's LDS slice (rows past the sequence zeroed),
    // token t at LDS row 4*((t%8)/2) + 2*(t/8) + t%2: the transpose reads
    // of PV then give lane group grp the tokens whose scores it holds.
#pragma unroll
    for (int c = 0; c < Sh::kVChunks; ++c) {
      const int idx = c * kWave + lane;
      const int row = idx / (D / 8);
      const int col8 = idx % (D / 8);
      u32x4 x = vv[c];
      if constexpr (!kFull) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        x = (tokb + row < tok_end) ? x : z;
      }
      const int lrow = 4 * ((row % 8) / 2) + 2 * (row / 8) + row % 2;
      *(u32x4*)(vl + lrow * Sh::kLdsRow + col8 * 8) = x;
    }
    // Scores: product e (valid for even rows) and o (odd rows) per group of
    // 8 tokens; lane (hl, grp) ends with tokens 2*grp, 2*grp + 1, 8 + 2*grp,
    // 9 + 2*grp of the block, in that order.
    f32x4 se[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    f32x4 so[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int j = 0; j < Sh::kKChunks; ++j) {
      se[j % 2] = mfma_16x16x32(as_bf16x8(kk[j]), qv[2 * kl(j)], se[j % 2]);
      so[j % 2] = mfma_16x16x32(as_bf16x8(kk[j]), qv[2 * kl(j) + 1], so[j % 2]);
    }
    const float sacc[4] = {se[0][0] + so[0][1], se[0][2] + so[0][3], se[1][0] + so[1][1],
                           se[1][2] + so[1][3]};
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = sacc[r] * scale_log2;
      if constexpr (!kFull) {
        const int tok = tokb + 2 * grp + (r & 1) + 8 * (r >> 1);
        sv[r] = (tok < tok_end && tok <= col_lim) ? sv[r] : -INFINITY;
      }
    }
    const float bmax = __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(sv[0], sv[1]), __builtin_elementwise_maximum(sv[2], sv[3]));
    if (__any(bmax > acc.m + kLazy)) {  // wave-uniform: re-reference the softmax
      const float mn = fmaxf(acc.m, max_across_groups(bmax));
      // (o and the sums are still zero while m is -inf: a column that has
      // seen no visible key keeps m = -inf without a NaN)
      const float alpha = acc.m == -INFINITY ? 0.f : fast_exp2(acc.m - mn);
      acc.lsum *= alpha;
#pragma unroll
      for (int mi = 0; mi < Sh::kDTiles; ++mi) acc.o[mi] *= alpha;
      acc.m = mn;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (kFull) {
        p[r] = fast_exp2(sv[r] - acc.m);
      } else {
        // (a column of a several-token row can meet a block with none of
        // its keys visible before any visible one: m is still -inf there)
        p[r] = sv[r] == -INFINITY ? 0.f : fast_exp2(sv[r] - acc.m);
      }
    }
    wave_lds_fence();
    // A operand V^T[d = 16*mi + hl][token 4*grp + r] by transpose reads.
    const uint16_t* vrow = vl + (4 * grp + hl / 4) * Sh::kLdsRow + 4 * (hl % 4);
    if constexpr (kSplit) {
      const u32x2 s01 = split_pack_bf16x2(p[0], p[1]);
      const u32x2 s23 = split_pack_bf16x2(p[2], p[3]);
      const i16x4 phi = __builtin_bit_cast(i16x4, u32x2{s01[0], s23[0]});
      const i16x4 plo = __builtin_bit_cast(i16x4, u32x2{s01[1], s23[1]});
#pragma unroll
      for (int mi = 0; mi < Sh::kDTiles; ++mi) {
        const i16x4 a = lds_read_tr16(vrow + 16 * mi);
        acc.o[mi] = mfma_16x16x16(a, phi, acc.o[mi]);
        acc.o[mi] = mfma_16x16x16(a, plo, acc.o[mi]);
      }
      acc.lsum += (p[0] + p[1]) + (p[2] + p[3]);
    } else {
      // one bf16 part; the weight sum adds the same rounded values
      const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
      const i16x4 ph = __builtin_bit_cast(i16x4, u32x2{h01, h23});
#pragma unroll
      for (int mi = 0; mi < Sh::kDTiles; ++mi) {
        const i16x4 a = lds_read_tr16(vrow + 16 * mi);
        acc.o[mi] = mfma_16x16x16(a, ph, acc.o[mi]);
      }
      acc.lsum += (__uint_as_float(h01 << 16) + __uint_as_float(h01 & 0xffff0000u)) +
                  (__uint_as_float(h23 << 16) + __uint_as_float(h23 & 0xffff0000u));
    }
    wave_lds_fence();
  };

  // Blocks wholly below full_end come first (tokb grows with k): nfull of
  // them take the unmasked path, the rest the masked one.
  const int nfull = full_end - kBlock < tok0
                        ? 0 : min(nk, (full_end - kBlock - tok0) / tok_step + 1);

  // The ring: NBUF-1 blocks in flight ahead of the one being consumed, in
  // whole rounds of NBUF so that every slot index is fixed at compile time
  // and every wait is for exactly the block being consumed. The first loop
  // takes rounds of full blocks, the second the rest (loads past the last
  // block re-read it and go unused).
  u32x4 kb[NBUF][Sh::kKChunks], vb[NBUF][Sh::kVChunks];
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) load_block(u, kb[u], vb[u]);
  int k0 = 0;
  for (; k0 + NBUF <= nfull; k0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      load_block(k0 + u + NBUF - 1, kb[(u + NBUF - 1) % NBUF], vb[(u + NBUF - 1) % NBUF]);
      process_block(k0 + u, kb[u], vb[u], std::true_type{});
    }
  }
  for (; k0 < nk; k0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      load_block(k0 + u + NBUF - 1, kb[(u + NBUF - 1) % NBUF], vb[(u + NBUF - 1) % NBUF]);
      if (k0 + u < nk) process_block(k0 + u, kb[u], vb[u], std::false_type{});
    }
  }
}

// stream_blocks_impl with the weights' precision chosen per call (split_p:
// hi + lo parts, for rows of few keys); the rest of the arguments as there.
template <int D, int NBUF, bool kStreamV, bool kNew = false>
__device__ __forceinline__ void stream_blocks(WaveAcc<D>& acc, const bf16x8 (&qv)[D / 32], int ids,
                                              int nk, int tok0, int tok_step, int tok_end,
                                              int full_end, bool split_p,
                                              const uint16_t* __restrict__ kbase,
                                              const uint16_t* __restrict__ vbase, int64_t kv_row,
                                              uint16_t* vl, float scale_log2, int lane,
                                              NewToken nt = NewToken{-1, nullptr, nullptr, -1},
                                              int col_lim = INT32_MAX) {
  if (split_p)  // wave-uniform
    stream_blocks_impl<D, NBUF, kStreamV, kNew, true>(acc, qv, ids, nk, tok0, tok_step, tok_end,
                                                      full_end, kbase, vbase, kv_row, vl,
                                                      scale_log2, lane, nt, col_lim);
  else
    stream_blocks_impl<D, NBUF, kStreamV, kNew, false>(acc, qv, ids, nk, tok0, tok_step,
                                                       tok_end, full_end, kbase, vbase, kv_row,
                                                       vl, scale_log2, lane, nt, col_lim);
}

// Merges the states of waves that share a KV-head slot (slot = w % HG; waves
// slot, slot + HG, ... of the W in the workgroup) through LDS, kMergeCols
// query columns per pass, and calls out(slot, col, d, M, den, n0, n1) for
// every column < ncols and even d: the merged state of d and d+1, summed in
// wave order. A wave that streamed nothing holds m = -inf, l = 0, o = 0 and
// adds nothing. Every wave of the workgroup must call it (it has barriers).
template <int D, class Out>
__device__ __forceinline__ void merge_waves(const WaveAcc<D>& acc, float* stage, int W, int HG,
                                            int ncols, int w, int lane, Out&& out) {
  using Sh = DecodeShape<D>;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int S = W / HG;
  float* mo = stage;                                             // [W][8][D + 4]
  float* mml = stage + (size_t)W * Sh::kMergeCols * Sh::kMergeRow;  // [W][8][2]
  for (int cb = 0; cb < ncols; cb += Sh::kMergeCols) {
    __syncthreads();  // the stage (or the V slices it overlays) is free
    const int hh = hl - cb;
    if (hl < ncols && hh >= 0 && hh < Sh::kMergeCols) {
      float* orow = mo + (w * Sh::kMergeCols + hh) * Sh::kMergeRow + 4 * grp;
#pragma unroll
      for (int mi = 0; mi < Sh::kDTiles; ++mi) *(f32x4*)(orow + 16 * mi) = acc.o[mi];
      if (grp == 0) {
        mml[(w * Sh::kMergeCols + hh) * 2 + 0] = acc.m;
        mml[(w * Sh::kMergeCols + hh) * 2 + 1] = acc.lsum;
      }
    }
    __syncthreads();
    const int nh = min(Sh::kMergeCols, ncols - cb);
    const int per_slot = nh * (D / 2);
    for (int idx = threadIdx.x; idx < HG * per_slot; idx += blockDim.x) {
      const int slot = idx / per_slot;
      const int h = (idx % per_slot) / (D / 2);
      const int d = 2 * (idx % (D / 2));
      float M = -INFINITY;
      for (int sub = 0; sub < S; ++sub)
        M = fmaxf(M, mml[((slot + HG * sub) * Sh::kMergeCols + h) * 2]);
      float den = 0.f, n0 = 0.f, n1 = 0.f;
      for (int sub = 0; sub < S; ++sub) {
        const int v = slot + HG * sub;
        const float* ml = mml + (v * Sh::kMergeCols + h) * 2;
        // a column that saw no visible key (m = -inf) adds nothing, also
        // when no wave saw one (M = -inf)
        const float e = ml[0] == -INFINITY ? 0.f : fast_exp2(ml[0] - M);
        const float* orow = mo + (v * Sh::kMergeCols + h) * Sh::kMergeRow + d;
        den += e * ml[1];
        n0 += e * orow[0];
        n1 += e * orow[1];
      }
      out(slot, cb + h, d, M, den, n0, n1);
    }
  }
}

// ---------------------------------------------------------------------------
// Stream schedule
// ---------------------------------------------------------------------------

// Exclusive prefix sum over the workgroup (any blockDim <= 1024); `tmp`
// holds 17 ints of LDS. Returns the thread's exclusive prefix; *total gets the
// sum of all.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) tmp[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < nw; ++i) {
      const int t = tmp[i];
      tmp[i] = run;
      run += t;
    }
    tmp[16] = run;
  }
  __syncthreads();
  const int r = tmp[w] + x - v;
  *total = tmp[16];
  __syncthreads();  // tmp may be reused
  return r;
}

// Waves of an even-share workgroup: one per KV head of a head group (two
// per head when there are four heads), at most eight.
constexpr int kStreamMaxWaves = 8;

template <int D, int NBUF, bool kStreamV>
__global__ __launch_bounds__(kStreamMaxWaves * kWave) void decode_stream_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    uint16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int32_t* __restrict__ counters, float scale_log2, int32_t Hq, int32_t Hkv, int32_t G,
    int32_t MB, int32_t S, int32_t HG, int32_t QM) {
  using Sh = DecodeShape<D>;
  // LDS: W V slices (the merge stage overlays them), then the row prefix
  // [S + 1], scan scratch [17] and a flag.
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int W = blockDim.x / kWave;
  int32_t* pre = (int32_t*)(lds + (size_t)W * Sh::kLdsWave);
  int32_t* tmp = pre + S + 1;
  int32_t* flag = tmp + 17;

  const int lane = threadIdx.x & (kWave - 1);
  // The wave index is uniform across the wave; saying so keeps the block
  // loop and the table reads on scalar registers.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Ssub = W / HG;
  const int slot = w % HG;
  const int sub = w / HG;
  const int g = blockIdx.y * HG + slot;  // this wave's KV head
  const bool head_ok = g < Hkv;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int64_t kv_row = (int64_t)Hkv * D;

  // 1. Blocks per decode row (rows of 1..QM query tokens; 0 for other rows)
  //    and their exclusive prefix, rows in order: thread t takes rows
  //    [t*R, t*R + R).
  auto row_blocks = [&](int s) {
    const int ql = qsl[s + 1] - qsl[s];
    return (ql >= 1 && ql <= QM) ? (seq_lens[s] + kBlock - 1) / kBlock : 0;
  };
  {
    const int R = (S + blockDim.x - 1) / blockDim.x;
    const int r_lo = min(S, (int)threadIdx.x * R);
    const int r_hi = min(S, r_lo + R);
    int mine = 0;
    for (int s = r_lo; s < r_hi; ++s) mine += row_blocks(s);
    int total;
    int run = block_exclusive_scan(mine, tmp, &total);
    for (int s = r_lo; s < r_hi; ++s) {
      pre[s] = run;
      run += row_blocks(s);
    }
    if (threadIdx.x == 0) pre[S] = total;
    __syncthreads();
  }
  const int64_t T = pre[S];
  const int64_t P = min((int64_t)gridDim.x, T);  // every share holds >= 1 block
  const int p = blockIdx.x;
  if (p >= P) return;  // workgroup-uniform, after the last barrier of the scan
  // Share p: blocks [B(p), B(p+1)) with B(c) = floor(c * T / P).
  auto B = [&](int64_t c) { return c * T / P; };
  const int64_t r0 = B(p), r1 = B(p + 1);
  // First row: the last s with pre[s] <= r0 (rows of no blocks are skipped).
  int s;
  {
    int lo = 0, hi = S;  // pre[lo] <= r0 < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (pre[mid] <= r0) lo = mid; else hi = mid;
    }
    s = lo;
  }

  uint16_t* vl = lds + w * Sh::kLdsWave;
  float* stage = (float*)lds;
  WaveAcc<D> acc;
  for (int64_t pos = r0; pos < r1; ++s) {
    const int64_t a = pre[s], b = pre[s + 1];
    if (b <= pos) continue;  // no blocks in this share (or none at all)
    const int j_lo = (int)(pos - a);
    const int j_hi = (int)(min(b, r1) - a);
    pos = min(b, r1);
    const int t0 = qsl[s];
    const int ql = qsl[s + 1] - t0;
    const int ncols = ql * G;  // query columns: head c % G of token c / G
    const int L = seq_lens[s];
    // Shares that hold blocks of this row: p_first .. p_last.
    const int64_t p_first = ((a + 1) * P + T - 1) / T - 1;
    const int64_t p_last = (b * P + T - 1) / T - 1;
    const int ncontrib = (int)(p_last - p_first + 1);
    // Slot of a share's partial for this row: 1 in the share where the row
    // begins (p_first: the row is its last), 0 in every later share (the
    // row began before the share: it is the share's first).
    auto slot_of = [&](int64_t c) { return c == p_first ? 1 : 0; };

    acc.init();
    const int nk_all = (j_hi - j_lo > sub) ? (j_hi - j_lo - 1 - sub) / Ssub + 1 : 0;
    if (head_ok && nk_all > 0) {
      bf16x8 qv[Sh::kKChunks];
      load_q<D>(qv, q + ((int64_t)t0 * Hq + g * G) * D, hl, grp, ncols, G, Hq);
      const int col_lim = L - ql + min(hl, ncols - 1) / G;  // last key of the lane's column
      const uint16_t* kbase = k_cache + (int64_t)g * D;
      const uint16_t* vbase = v_cache + (int64_t)g * D;
      const int32_t* trow = block_table + (int64_t)s * MB + j_lo + sub;
      for (int kc = 0; kc < nk_all; kc += kWave) {
        const int nk = min(kWave, nk_all - kc);
        const int ids = lane < nk ? trow[(int64_t)(kc + lane) * Ssub] : 0;
        stream_blocks<D, NBUF, kStreamV>(acc, qv, ids, nk, (j_lo + sub + kc * Ssub) * kBlock,
                                         Ssub * kBlock, L, L - ql + 1, L <= kSplitKeys, kbase,
                                         vbase, kv_row, vl, scale_log2, lane,
                                         NewToken{-1, nullptr, nullptr, -1}, col_lim);
      }
      acc.finish();
    }

    const int my_slot = slot_of(p);
    merge_waves<D>(acc, stage, W, HG, ncols, w, lane,
                   [&](int sl, int col, int d, float M, float den, float n0, float n1) {
      const int head = blockIdx.y * HG + sl;
      if (head >= Hkv) return;
      const int tk = col / G;
      const int qh = head * G + col % G;
      if (ncontrib == 1) {
        const float inv = 1.0f / den;
        *(uint32_t*)(out + ((int64_t)(t0 + tk) * Hq + qh) * D + d) =
            pack_bf16x2(n0 * inv, n1 * inv);
      } else {  // read by the share that finishes this row last
        const int64_t row = (((int64_t)p * 2 + my_slot) * QM + tk) * Hq + qh;
        store_coherent2(ws_o + row * D + d, n0, n1);
        if (d == 0) store_coherent2(ws_ml + row * 2, M, den);
      }
    });

    if (ncontrib > 1) {
      // Publish and hand over: see count_in. The last to count in merges
      // every share's partial in share order and leaves the counter at zero
      // for the next call.
      if (count_in(counters + (int64_t)s * gridDim.y + blockIdx.y, ncontrib, flag)) {
        // Online merge in share order, eight shares' loads in flight at a
        // time. A share whose blocks hold no key visible to a column (the
        // few keys past an earlier token of a several-token row) left
        // m = -inf for it and adds nothing.
        const int per_head = ncols * (D / 2);
        for (int idx = threadIdx.x; idx < HG * per_head; idx += blockDim.x) {
          const int head = blockIdx.y * HG + idx / per_head;
          if (head >= Hkv) continue;
          const int col = (idx % per_head) / (D / 2);
          const int tk = col / G;
          const int qh = head * G + col % G;
          const int d = 2 * (idx % (D / 2));
          float M = -INFINITY, den = 0.f, n0 = 0.f, n1 = 0.f;
          for (int64_t c0 = p_first; c0 <= p_last; c0 += 8) {
            f32x2 ml[8], ov[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int64_t c = min(c0 + k, p_last);
              const int64_t row = ((c * 2 + slot_of(c)) * QM + tk) * Hq + qh;
              ml[k] = load_coherent2(ws_ml + row * 2);
              ov[k] = load_coherent2(ws_o + row * D + d);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              if (c0 + k <= p_last && ml[k][0] != -INFINITY) {
                const float mn = fmaxf(M, ml[k][0]);
                const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mn);
                const float e = fast_exp2(ml[k][0] - mn);
                den = den * sc + e * ml[k][1];
                n0 = n0 * sc + e * ov[k][0];
                n1 = n1 * sc + e * ov[k][1];
                M = mn;
              }
            }
          }
          const float inv = 1.0f / den;
          *(uint32_t*)(out + ((int64_t)(t0 + tk) * Hq + qh) * D + d) =
              pack_bf16x2(n0 * inv, n1 * inv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Partitioned schedule
// ---------------------------------------------------------------------------

// kWrite (fused write): the batch is decode rows only and this launch also
// writes each row's new token (token qsl[s], at position seq_lens[s] - 1)
// into the caches at slot_mapping[qsl[s]]: the workgroup of the row's last
// partition writes its KV head's slice, and every workgroup reads that token
// from knew / vnew.
template <int D, int NBUF, bool kStreamV, bool kWrite, bool kHeads>
__global__ __launch_bounds__((max_waves<D, NBUF, kWrite>() * kWave)) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    uint16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    float scale_log2, int32_t Hq, int32_t Hkv, int32_t G, int32_t MB, int32_t part_tokens,
    int32_t num_parts_max, int32_t tok_base, int32_t part_base, int32_t QM, int32_t HG,
    int32_t* __restrict__ counters, const uint16_t* __restrict__ knew,
    const uint16_t* __restrict__ vnew, const int64_t* __restrict__ slot_mapping,
    uint16_t* k_cache_w, uint16_t* v_cache_w) {
  using Sh = DecodeShape<D>;
  // W V slices of kLdsWave elements while streaming; the merge stage after.
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int W = blockDim.x / kWave;
  // Rows vary fastest in the grid: consecutive workgroups are dealt to the
  // XCDs in turn, so the work of every partition index and head spreads
  // over all XCDs. A workgroup holds HG KV heads (HG divides W): wave w
  // takes head w % HG of them and every (W / HG)-th block of the partition
  // from block w / HG on.
  // (kHeads: HG > 1 heads per workgroup; otherwise HG is 1 and the
  // instantiation keeps the index arithmetic free of divisions)
  const int s = blockIdx.x;
  const int sub = kHeads ? w / HG : w;
  const int Wsub = kHeads ? W / HG : W;
  const int g = kHeads ? blockIdx.y * HG + w % HG : blockIdx.y;
  const int part = blockIdx.z;
  // Block ids of this wave (lane k: partition block sub + k*Wsub), read
  // before the row's length is known so the loads overlap; the index is
  // kept inside the row, and lanes past the wave's blocks are never used.
  // Keys from tok_base on (a multiple of 16: after a shared-prefix pass the
  // prefix's partials are already in the workspace).
  const int bpp = part_tokens / kBlock;
  const int b_begin = tok_base / kBlock + part * bpp;
  const int jb = sub + lane * Wsub;
  const int my_blk = (jb < bpp && b_begin + jb < MB)
                         ? block_table[(int64_t)s * MB + b_begin + jb] : 0;
  // Workgroup-uniform exits (before any barrier).
  // Rows of 1..QM query tokens: token i of the row sits at position
  // L - ql + i and sees keys up to it; the row's ql * G (<= 16) query
  // columns share every K/V block.
  // (the row's start, query count and length are loaded together, ahead of
  // any use, so they cost one round trip)
  const int t0 = qsl[s];
  const int t1 = qsl[s + 1];
  const int L = seq_lens[s];
  __builtin_amdgcn_sched_barrier(0);
  const int ql = t1 - t0;
  const int tok_begin = tok_base + part * part_tokens;
  if (ql < 1 || ql > QM || tok_begin >= L) return;  // not a decode row / past its end
  const int ncols = ql * G;
  const int tok_end = min(L, tok_begin + part_tokens);
  const int nparts = (L - tok_base + part_tokens - 1) / part_tokens;
  const int nblk = (tok_end + kBlock - 1) / kBlock - b_begin;
  const int nmine = nblk > sub ? (nblk - 1 - sub) / Wsub + 1 : 0;  // blocks of this wave
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int64_t kv_row = (int64_t)Hkv * D;
  NewToken nt{-1, nullptr, nullptr, -1};
  // The fused write: wave 0 of the row's last partition stores its KV head's
  // slice of the new token after streaming (lanes < 2 * D / 8, 16 bytes
  // each: K, then V). The slot is loaded here by every wave with a vector
  // load (a buffer load, which is never turned into a scalar one), so that
  // nothing waits for it before the blocks start streaming. A negative slot
  // writes nothing. At D = 64 the token's data and q are also loaded here,
  // unconditionally, so the wait for the block ids does not include them;
  // at D = 128 the registers to hold them that long are not there.
  constexpr bool kEarly = D == 64;
  auto new_token_data = [&]() {
    return *(const u32x4*)(((lane % (2 * (D / 8))) >= D / 8 ? nt.v : nt.k) + (lane % (D / 8)) * 8);
  };
  u32x4 wval = {0u, 0u, 0u, 0u};
  if constexpr (kWrite) {
    nt = NewToken{L - 1, knew + ((int64_t)t0 * Hkv + g) * D, vnew + ((int64_t)t0 * Hkv + g) * D,
                  -1};
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(slot_mapping + t0), (short)0, (int)sizeof(int64_t), kBufferWordFlags);
    nt.slot = __builtin_bit_cast(int64_t, __builtin_amdgcn_raw_buffer_load_b64(srs, 0, 0, 0));
    if constexpr (kEarly) wval = new_token_data();
  }
  bf16x8 qv[Sh::kKChunks];
  if constexpr (kEarly) load_q<D>(qv, q + ((int64_t)t0 * Hq + g * G) * D, hl, grp, ncols, G, Hq);

  WaveAcc<D> acc;
  acc.init();
  if (nmine > 0) {
    if constexpr (!kEarly)
      load_q<D>(qv, q + ((int64_t)t0 * Hq + g * G) * D, hl, grp, ncols, G, Hq);
    const int col_lim = L - ql + min(hl, ncols - 1) / G;  // last key of the lane's column
    stream_blocks<D, NBUF, kStreamV, kWrite>(
        acc, qv, my_blk, nmine, (b_begin + sub) * kBlock, Wsub * kBlock, tok_end,
        min(tok_end, L - ql + 1), L <= kSplitKeys, k_cache + (int64_t)g * D,
        v_cache + (int64_t)g * D, kv_row, lds + w * Sh::kLdsWave, scale_log2, lane, nt, col_lim);
    acc.finish();
  }
  if constexpr (kWrite) {
    if (part == nparts - 1 && sub == 0) {  // wave-uniform
      // [NB, 16, Hkv, D]: the slot's row starts at element slot * Hkv * D
      const int64_t slot = first_lane64(nt.slot);
      if constexpr (!kEarly) wval = new_token_data();
      if (slot >= 0 && lane < 2 * (D / 8))
        *(u32x4*)((lane >= D / 8 ? v_cache_w : k_cache_w) + slot * kv_row + (int64_t)g * D +
                  (lane % (D / 8)) * 8) = wval;
    }
  }

  // With counters, the workgroup that finishes a split row last merges its
  // partials (no combine launch): partials go past this XCD's L2. A row
  // whose own keys fit this one partition after partials 0 .. part_base-1
  // left by an earlier launch (the shared-prefix pass) merges those with
  // its state directly, in the same order, with no hand-over.
  const bool split = nparts > 1 || part_base > 0;
  const bool direct = counters && nparts == 1 && part_base > 0;
  const int64_t pstride = (int64_t)QM * Hq;
  // Online merge in partition order of partials c_lo .. c_hi-1 of (token
  // tk, head qh) into (M, den, n0, n1) at d, d+1; eight loads in flight.
  auto merge_partials = [&](int c_lo, int c_hi, int tk, int qh, int d, float& M, float& den,
                            float& n0, float& n1) {
    const int64_t row0 = (int64_t)s * num_parts_max * pstride + (int64_t)tk * Hq + qh;
    for (int c0 = c_lo; c0 < c_hi; c0 += 8) {
      f32x2 ml[8], ov[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t r = row0 + min(c0 + k, c_hi - 1) * pstride;
        ml[k] = load_coherent2(ws_ml + r * 2);
        ov[k] = load_coherent2(ws_o + r * D + d);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // a partition where the column saw no visible key adds nothing
        if (c0 + k < c_hi && ml[k][0] != -INFINITY) {
          const float mn = fmaxf(M, ml[k][0]);
          const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mn);
          const float e = fast_exp2(ml[k][0] - mn);
          den = den * sc + e * ml[k][1];
          n0 = n0 * sc + e * ov[k][0];
          n1 = n1 * sc + e * ov[k][1];
          M = mn;
        }
      }
    }
  };
  auto merged = [&](int sl, int col, int d, float M, float den, float n0, float n1) {
    const int tk = col / G;
    const int qh = (blockIdx.y * HG + sl) * G + col % G;
    if (!split || direct) {
      if (direct) {
        float Mx = -INFINITY, dx = 0.f, x0 = 0.f, x1 = 0.f;
        merge_partials(0, part_base, tk, qh, d, Mx, dx, x0, x1);
        if (M != -INFINITY) {  // this partition's state comes last
          const float mn = fmaxf(Mx, M);
          const float sc = Mx == -INFINITY ? 0.f : fast_exp2(Mx - mn);
          const float e = fast_exp2(M - mn);
          dx = dx * sc + e * den;
          x0 = x0 * sc + e * n0;
          x1 = x1 * sc + e * n1;
        }
        den = dx;
        n0 = x0;
        n1 = x1;
      }
      const float inv = 1.0f / den;
      *(uint32_t*)(out + ((int64_t)(t0 + tk) * Hq + qh) * D + d) =
          pack_bf16x2(n0 * inv, n1 * inv);
    } else {
      const int64_t base =
          (((int64_t)s * num_parts_max + part_base + part) * QM + tk) * Hq + qh;
      if (counters) {
        store_coherent2(ws_o + base * D + d, n0, n1);
        if (d == 0) store_coherent2(ws_ml + base * 2, M, den);
      } else {  // read by the combine kernel after this one ends
        *(f32x2*)(ws_o + base * D + d) = f32x2{n0, n1};
        if (d == 0) *(f32x2*)(ws_ml + base * 2) = f32x2{M, den};
      }
    }
  };
  merge_waves<D>(acc, (float*)lds, W, kHeads ? HG : 1, ncols, w, lane, merged);
  if (!counters || !split || direct) return;
  // Publish and hand over (count_in): the last of the row's nparts
  // workgroups (of these KV heads) merges partials 0 .. part_base + nparts
  // - 1 in order and leaves the counter at zero for the next call.
  // (partitions past the grid do not run: a length past the planned
  // maximum is a caller error, and the counter still returns to zero)
  const int nrun = min(nparts, (int)gridDim.z);
  // (the merge stage's LDS is free again after count_in's first barrier)
  if (!count_in(counters + (int64_t)s * Hkv + blockIdx.y * HG, nrun, (int32_t*)lds)) return;
  const int np = part_base + nrun;
  const int per_head = ncols * (D / 2);
  for (int idx = threadIdx.x; idx < HG * per_head; idx += blockDim.x) {
    const int col = (idx % per_head) / (D / 2);
    const int d = 2 * (idx % (D / 2));
    const int tk = col / G;
    const int qh = (blockIdx.y * HG + idx / per_head) * G + col % G;
    float M = -INFINITY, den = 0.f, n0 = 0.f, n1 = 0.f;
    merge_partials(0, np, tk, qh, d, M, den, n0, n1);
    const float inv = 1.0f / den;
    *(uint32_t*)(out + ((int64_t)(t0 + tk) * Hq + qh) * D + d) = pack_bf16x2(n0 * inv, n1 * inv);
  }
}

// Merge of a row's partitions: one wave per (row, query token, head), lanes
// across d, partitions in order (deterministic). Rows vary fastest in the
// grid. Partial p of token tk sits at ((s * num_parts_max + p) * QM + tk)
// * Hq + head.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, uint16_t* __restrict__ out,
    int32_t Hq, int32_t part_tokens, int32_t num_parts_max, int32_t tok_base,
    int32_t part_base, int32_t QM) {
  constexpr int kPer = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int s = blockIdx.x;
  const int idx = blockIdx.y * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int tk = idx / Hq;
  const int qh = idx - tk * Hq;
  if (tk >= QM) return;
  const int t0 = qsl[s];
  const int ql = qsl[s + 1] - t0;
  if (ql < 1 || ql > QM || tk >= ql) return;
  const int L = seq_lens[s];
  // partials 0 .. part_base-1 come from the shared-prefix pass
  // (clamped to the workspace rows: a length past the planned maximum is a
  // caller error, and reads stay inside the row's partials)
  const int np =
      min(num_parts_max, part_base + max(0, (L - tok_base + part_tokens - 1) / part_tokens));
  if (np <= 1) return;
  const int64_t pstride = (int64_t)QM * Hq;  // partition p at row0 + p * pstride
  const int64_t row0 = (int64_t)s * num_parts_max * pstride + (int64_t)tk * Hq + qh;

  float M = -INFINITY;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    const int p = p0 + lane;
    if (p < np) M = fmaxf(M, ws_ml[(row0 + p * pstride) * 2]);
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
      const int64_t r = row0 + p * pstride;
      wgt = ws_ml[r * 2] == -INFINITY ? 0.f : fast_exp2(ws_ml[r * 2] - M);
      wl += wgt * ws_ml[r * 2 + 1];
    }
    const int cnt = min(kWave, np - p0);
    // eight partitions per batch, all loads issued before their use
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      float vals[8][kPer];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int kk = min(k0 + k, cnt - 1);
        const float* op = ws_o + (row0 + (p0 + kk) * pstride) * D;
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
  uint16_t* op = out + ((int64_t)(t0 + tk) * Hq + qh) * D;
#pragma unroll
  for (int e = 0; e < kPer; ++e) op[lane + kWave * e] = float_to_bf16_bits(acc[e] * inv);
}

template <int D, int NBUF, bool kStreamV>
hipError_t launch_decode_nb(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream) {
  using Sh = DecodeShape<D>;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int G = a.num_q_heads / a.num_kv_heads;
  if (p.stream) {
    const int groups = (a.num_kv_heads + p.stream_heads - 1) / p.stream_heads;
    dim3 grid(p.stream_wgs, groups);
    const size_t lds = (size_t)p.waves * Sh::kLdsWave * sizeof(uint16_t) +
                       ((size_t)a.num_seqs + 1 + 17 + 1) * sizeof(int32_t);
    profile_begin(PA_KERNEL_DECODE, stream);
    hipLaunchKernelGGL((decode_stream_kernel<D, NBUF, kStreamV>), grid, dim3(p.waves * kWave),
                       lds, stream, (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                       (const uint16_t*)a.v_cache, a.block_table, a.seq_lens,
                       a.query_start_loc, (uint16_t*)a.out, p.ws_o, p.ws_ml, p.counters,
                       scale_log2, a.num_q_heads, a.num_kv_heads, G, a.max_blocks_per_seq,
                       a.num_seqs, p.stream_heads, p.qmax);
    profile_end(PA_KERNEL_DECODE, stream);
    return hipGetLastError();
  }
  dim3 grid(a.num_seqs, a.num_kv_heads / p.heads_per_wg, p.num_parts_max - p.part_base);
  const size_t lds = (size_t)p.waves * Sh::kLdsWave * sizeof(uint16_t);
  profile_begin(PA_KERNEL_DECODE, stream);
  if (p.fused_write) {
    hipLaunchKernelGGL((decode_kernel<D, NBUF, kStreamV, true, false>), grid, dim3(p.waves * kWave), lds,
                       stream, (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                       (const uint16_t*)a.v_cache, a.block_table, a.seq_lens, a.query_start_loc,
                       (uint16_t*)a.out, p.ws_o, p.ws_ml, scale_log2, a.num_q_heads,
                       a.num_kv_heads, G, a.max_blocks_per_seq, p.part_tokens, p.num_parts_max,
                       p.tok_base, p.part_base, p.qmax, p.heads_per_wg,
                       p.fused_combine ? p.counters : nullptr, (const uint16_t*)p.knew,
                       (const uint16_t*)p.vnew,
                       p.slot_mapping, (uint16_t*)p.k_cache_w, (uint16_t*)p.v_cache_w);
  } else {
    auto kernel = p.heads_per_wg > 1 ? decode_kernel<D, NBUF, kStreamV, false, true>
                                     : decode_kernel<D, NBUF, kStreamV, false, false>;
    hipLaunchKernelGGL(kernel, grid, dim3(p.waves * kWave),
                       lds, stream, (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                       (const uint16_t*)a.v_cache, a.block_table, a.seq_lens, a.query_start_loc,
                       (uint16_t*)a.out, p.ws_o, p.ws_ml, scale_log2, a.num_q_heads,
                       a.num_kv_heads, G, a.max_blocks_per_seq, p.part_tokens, p.num_parts_max,
                       p.tok_base, p.part_base, p.qmax, p.heads_per_wg,
                       p.fused_combine ? p.counters : nullptr, nullptr, nullptr, nullptr,
                       nullptr, nullptr);
  }
  profile_end(PA_KERNEL_DECODE, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_parts_max <= 1 || p.fused_combine) return e;
  dim3 cgrid(a.num_seqs, (p.qmax * a.num_q_heads + 3) / 4);
  profile_begin(PA_KERNEL_COMBINE, stream);
  hipLaunchKernelGGL(decode_combine_kernel<D>, cgrid, dim3(256), 0, stream, a.seq_lens,
                     a.query_start_loc, p.ws_o, p.ws_ml, (uint16_t*)a.out, a.num_q_heads,
                     p.part_tokens, p.num_parts_max, p.tok_base, p.part_base, p.qmax);
  profile_end(PA_KERNEL_COMBINE, stream);
  return hipGetLastError();
}

}  // namespace

int32_t decode_max_waves(int32_t head_size, int32_t prefetch, bool fused_write) {
  switch (head_size) {
    case 64:
      if (prefetch >= 3) return fused_write ? max_waves<64, 3, true>() : max_waves<64, 3>();
      return fused_write ? max_waves<64, 2, true>() : max_waves<64, 2>();
    case 128: return fused_write ? max_waves<128, 2, true>() : max_waves<128, 2>();
    default: return 0;
  }
}

size_t decode_stream_lds_bytes(int32_t head_size, int32_t waves, int32_t num_seqs) {
  const size_t slice = head_size == 64 ? DecodeShape<64>::kLdsWave : DecodeShape<128>::kLdsWave;
  return (size_t)waves * slice * sizeof(uint16_t) + ((size_t)num_seqs + 1 + 17 + 1) * 4;
}

hipError_t launch_decode(const ForwardArgs& a, const DecodePlan& p, hipStream_t stream) {
  const int maxw = decode_max_waves(a.head_size, p.prefetch, p.fused_write);
  if (p.waves < 1 || p.waves > maxw || a.num_kv_heads > 65535) return hipErrorInvalidValue;
  if (p.fused_write && (p.stream || p.heads_per_wg != 1 || !p.knew || !p.vnew ||
                        !p.slot_mapping || !p.k_cache_w || !p.v_cache_w))
    return hipErrorInvalidValue;
  if (p.tok_base < 0 || p.tok_base % kBlock || p.part_base < 0 ||
      p.num_parts_max - p.part_base < 1 || ((p.tok_base || p.part_base) && p.stream))
    return hipErrorInvalidValue;
  const int G = a.num_q_heads / a.num_kv_heads;
  if (p.qmax < 1 || p.qmax * G > 16 || (p.qmax > 1 && p.fused_write))
    return hipErrorInvalidValue;
  if (p.fused_combine && (p.stream || !p.counters)) return hipErrorInvalidValue;
  if (p.stream) {
    if (p.waves > kStreamMaxWaves || p.stream_heads < 1 || p.waves % p.stream_heads ||
        p.stream_wgs < 1 || !p.counters ||
        decode_stream_lds_bytes(a.head_size, p.waves, a.num_seqs) > 64 * 1024)
      return hipErrorInvalidValue;
  } else if (p.heads_per_wg < 1 || a.num_kv_heads % p.heads_per_wg ||
             p.waves % p.heads_per_wg || p.part_tokens <= 0 || p.part_tokens % kBlock ||
             p.part_tokens / kBlock > kWave * (p.waves / p.heads_per_wg) ||
             p.num_parts_max > 65535) {
    return hipErrorInvalidValue;
  }
  // Ring depths that fit the register budget without spills: 2 or 3 blocks
  // at D = 64, 2 at D = 128.
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
