// Prefill and chunked-prefill rows of the flattened batch (q_len > 1): each
// query row attends to the sequence's earlier cached context and causally to
// the rows of its own chunk, with the key/value tiles gathered block by block
// through the block table.
//
// Pages "Inside vLLM: Anatomy of a High-Throughput LLM Inference System":
// section "Scheduler" (prefill is usually compute bound), section "Chunked
// prefill" (a long prompt is split over several steps; a later chunk sees
// everything cached before it), section "Run forward pass" (flattened
// sequences, per-sequence masks). Query row i of a sequence with c earlier
// tokens sits at position c + i and sees keys 0..c+i.
//
// gfx950 design: one workgroup = one (sequence, tile of query tokens, KV
// head) with NW waves. The tile packs the G query heads that share the KV
// head into the MFMA M dimension: 32*NW rows = (32*NW/G tokens) x (G heads),
// 32 rows per wave, so every K/V tile staged in LDS serves all G heads. Per
// 64-key tile each wave computes S^T = K Q^T (keys x rows) with 16x16x32 bf16
// MFMAs (K rows read from LDS, Q^T held in registers), applies the
// bottom-right causal mask (only on tiles that reach past the first row's
// limit) and an fp32 online softmax with a lazily re-referenced max, and
// accumulates O^T += V^T P^T with 16x16x32 MFMAs whose B operand is the S^T
// accumulator converted to bf16 in place (as hi + lo parts when the tile's
// rows see few keys). K/V tiles move from HBM/L2 straight into a ring of NST
// LDS stages (global_load_lds), NST-1 tiles ahead of the one being computed;
// each tile starts with a wait for that tile's own loads (an explicit
// vmcnt count, so the later tiles' loads stay in flight) and one barrier. A
// single-workgroup planner kernel turns query_start_loc into the lists of
// tiles on the device, so the host never reads lengths.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "kv_write.h"

namespace pa {

namespace {

// List A tiles (rows that see many keys): 8 waves (256 MFMA rows: each K/V
// tile staged in LDS serves twice the rows of a 4-wave tile), two LDS stages
// (a third measured slower). List B tiles (rows that see few keys, P kept as
// hi + lo, which needs more registers): 4 waves (128 rows), two stages.
constexpr int kWavesA = 8, kStagesA = 2;
constexpr int kWavesB = 4, kStagesB = 2;
constexpr int kWavesP = 8;  // shared-prefix pass
// 16-row MFMA tiles per wave (32 rows; 64 rows per wave, which would halve
// the LDS reads per MFMA, needs more than the 512 registers of one wave per
// SIMD in this form): list A, the others.
constexpr int kRowTilesA = 2, kRowTiles = 2;
constexpr int kKeysPerTile = 64;
constexpr float kLazyP = 8.0f;  // log2 of the largest unnormalised weight
constexpr int kSplitKeys = 128;  // workgroups seeing at most this many keys split P
constexpr int kSplitGridMax = 512;  // workgroups walking list B
constexpr int kPlanThreads = 1024;

// Two tile lists, entry = (sequence, first query row), unused entries -1:
// list A holds tiles whose rows see more than kSplitKeys keys, each row's
// heaviest (latest) tiles first; list B the tiles that see at most
// kSplitKeys keys (they keep P as bf16 hi + lo). Rows of at least min_ql
// query tokens are listed: 2 when the decode launch takes the single-token
// rows, 1 when the tiles take every row.
// (one workgroup of kPlanThreads threads builds both lists)
__device__ __forceinline__ void plan_tiles(
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, int32_t S,
    int32_t bq_a, int32_t bq_b, int32_t* __restrict__ tiles_a, int32_t bound_a,
    int32_t* __restrict__ tiles_b, int32_t bound_b, int32_t* __restrict__ counts,
    int32_t min_ql) {
  __shared__ int32_t scan_a[kPlanThreads], scan_b[kPlanThreads];
  __shared__ int32_t carry_a, carry_b;
  const int tid = threadIdx.x;
  if (tid == 0) carry_a = carry_b = 0;
  __syncthreads();
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int na = 0, nb = 0, ql = 0, c = 0, qa = 0;
    if (s < S) {
      ql = qsl[s + 1] - qsl[s];
      c = seq_lens[s] - ql;
      if (ql >= min_ql && ql > 0) {
        const int n = (ql + bq_b - 1) / bq_b;
        // kv_end of B tile t is c + min((t+1)*bq_b, ql): non-decreasing in t
        while (nb < n && c + min((nb + 1) * bq_b, ql) <= kSplitKeys) ++nb;
        qa = min(ql, nb * bq_b);  // A tiles cover queries [qa, ql)
        na = (ql - qa + bq_a - 1) / bq_a;
      }
    }
    scan_a[tid] = na;
    scan_b[tid] = nb;
    __syncthreads();
    for (int d = 1; d < kPlanThreads; d <<= 1) {
      const int add_a = tid >= d ? scan_a[tid - d] : 0;
      const int add_b = tid >= d ? scan_b[tid - d] : 0;
      __syncthreads();
      scan_a[tid] += add_a;
      scan_b[tid] += add_b;
      __syncthreads();
    }
    const int off_a = carry_a + scan_a[tid] - na;
    const int off_b = carry_b + scan_b[tid] - nb;
    for (int k = 0; k < na; ++k) {  // tiles nb .. nb+na-1, latest first
      const int idx = off_a + k;
      if (idx < bound_a) {
        tiles_a[2 * idx] = s;
        tiles_a[2 * idx + 1] = qa + (na - 1 - k) * bq_a;
      }
    }
    for (int k = 0; k < nb; ++k) {
      const int idx = off_b + k;
      if (idx < bound_b) {
        tiles_b[2 * idx] = s;
        tiles_b[2 * idx + 1] = k * bq_b;
      }
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) {
      carry_a += scan_a[tid];
      carry_b += scan_b[tid];
    }
    __syncthreads();
  }
  if (tid == 0) {
    counts[0] = min(carry_a, bound_a);
    counts[1] = min(carry_b, bound_b);
  }
  for (int i = carry_a + tid; i < bound_a; i += kPlanThreads) {
    tiles_a[2 * i] = -1;
    tiles_a[2 * i + 1] = -1;
  }
  for (int i = carry_b + tid; i < bound_b; i += kPlanThreads) {
    tiles_b[2 * i] = -1;
    tiles_b[2 * i + 1] = -1;
  }
}

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, int32_t S,
    int32_t bq_a, int32_t bq_b, int32_t* __restrict__ tiles_a, int32_t bound_a,
    int32_t* __restrict__ tiles_b, int32_t bound_b, int32_t* __restrict__ counts,
    int32_t min_ql) {
  plan_tiles(qsl, seq_lens, S, bq_a, bq_b, tiles_a, bound_a, tiles_b, bound_b, counts, min_ql);
}

// The KV write and the planner in one launch (pa_write_and_forward on a
// batch with prefill rows; one kernel boundary fewer per step): workgroup 0
// plans the tiles, the others write the new tokens, one 16-byte chunk of K
// and of V per thread. The tiles, which read the new tokens through the
// caches, start after this launch has ended, as they did after the two it
// replaces.
__global__ __launch_bounds__(kPlanThreads) void write_plan_kernel(
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, int32_t S,
    int32_t bq_a, int32_t bq_b, int32_t* __restrict__ tiles_a, int32_t bound_a,
    int32_t* __restrict__ tiles_b, int32_t bound_b, int32_t* __restrict__ counts,
    int32_t min_ql, const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, int64_t total_chunks, int32_t chunks_per_token) {
  if (blockIdx.x == 0) {  // workgroup-uniform
    plan_tiles(qsl, seq_lens, S, bq_a, bq_b, tiles_a, bound_a, tiles_b, bound_b, counts, min_ql);
    return;
  }
  const int64_t i = (int64_t)(blockIdx.x - 1) * kPlanThreads + threadIdx.x;
  if (i < total_chunks) write_kv_chunk(k, v, slot_mapping, k_cache, v_cache, i, chunks_per_token);
}

// Waits until at most N vector-memory operations of this wave are in flight
// (its loads into LDS of older tiles have landed; the N most recent stay in
// flight), then joins the workgroup barrier. One asm statement with a memory
// clobber, so the compiler neither adds a full drain nor moves LDS accesses
// across it.
template <int N>
__device__ __forceinline__ void wait_loads_then_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// Waits for this wave's LDS writes, then joins the workgroup barrier.
__device__ __forceinline__ void lds_writes_then_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS chunk swizzles of the K and V tiles: 16-byte chunk c of row r sits at
// chunk c ^ swz(r). gfx950's LDS serves 256 bytes per cycle (64 banks): a
// 16-byte read takes 16 lanes per cycle, an 8-byte transpose read 32. The K
// row reads (lane: row hl of 16, one logical chunk) and the V transpose reads
// (lanes: 8 rows x 2 chunks x 2 halves) then each hit 16 / 32 distinct bank
// slots. Rows are 2*D bytes: at D = 64 two rows share the 256 bytes, so the
// swizzle keys on r / 2.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

// 16 bytes per lane from a buffer into LDS: lane i's bytes land at lds + 16*i.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds,
                                                int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, 0);
}

// Kernel modes: the two prefill tile lists, and the shared-prefix pass.
enum TileMode { kListA = 0, kListB = 1, kPrefix = 2 };

// Shared-prefix pass (PREFIX): the rows of a tile are the single query
// tokens of consecutive decode rows (G heads each), the keys one chunk of
// the prefix that every row's table starts with (read through row 0's
// table); no mask applies (every row sees the whole prefix), and the tile
// leaves unnormalised fp32 partials (numerator, reference max, weight sum)
// as partition `chunk` of each row for the decode combine.
struct PrefixArgs {
  float* ws_o;            // [S][num_parts_max][Hq][D]
  float* ws_ml;           // [S][num_parts_max][Hq][2]
  int32_t num_parts_max;
  int32_t chunk_keys;     // keys per chunk (multiple of 64)
  int32_t prefix_keys;    // 16 * prefix blocks
  int32_t num_seqs;
  int32_t row_tiles;      // ceil(num_seqs / tile rows)
  int32_t chunks;
  int32_t num_tokens;     // q rows (a row's token index is clamped below it)
  // The last tile_grid workgroups take the tiles; those before them write
  // the step's new tokens (write_chunks 16-byte chunks of K and of V, as
  // the cache-write kernel does). The tiles read only the prefix's blocks,
  // which hold no slot being written.
  int32_t tile_grid;
  int32_t chunks_per_token;
  int64_t write_chunks;
  const u32x4* knew;
  const u32x4* vnew;
  const int64_t* slot_mapping;
  u32x4* k_cache_w;
  u32x4* v_cache_w;
};

template <int D, int G, int MODE>
__global__ __launch_bounds__((MODE == kListB ? kWavesB : MODE == kPrefix ? kWavesP : kWavesA) * kWave,
                             1) void prefill_tile_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    uint16_t* __restrict__ out, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, float scale_log2, int32_t Hq, int32_t Hkv,
    int32_t MB, int32_t tile_bound, PrefixArgs pfx) {
  constexpr bool SPLIT = MODE == kListB;
  constexpr bool PREFIX = MODE == kPrefix;
  constexpr int NW = SPLIT ? kWavesB : PREFIX ? kWavesP : kWavesA;  // waves
  constexpr int NST = SPLIT ? kStagesB : kStagesA;  // LDS stages
  constexpr int MT = MODE == kListA ? kRowTilesA : kRowTiles;  // 16-row tiles per wave
  constexpr int RW = 16 * MT;                 // rows per wave
  constexpr int BQ = RW * NW / G;             // query tokens per tile
  constexpr int BN = kKeysPerTile;            // keys per iteration
  constexpr int RB = D * 2;                   // bytes of one K or V row (unpadded)
  constexpr int KC = D / 32;                  // QK MFMAs per 16x16 S tile
  constexpr int DT = D / 16;                  // PV output tiles along d
  constexpr int NS = BN / 16;                 // 16-key sub-tiles per tile
  constexpr int NDMA = BN * RB / 1024 / NW;   // 1 KiB load-to-LDS ops per wave per tile (K; V alike)
  static_assert(NDMA * NW * 1024 == BN * RB, "tile must split evenly");
  static_assert(NST == 2 || NST == 3, "stage count");

  // NST stages (the tile being computed and the ones being filled), rows
  // unpadded; 16-byte chunk c of row r sits at chunk c ^ swz(r) so that both
  // the row reads of the QK operand (8 rows per phase, K) and the transpose
  // reads of the PV operand (4 rows per 16-lane block, V) are bank-conflict
  // free.
  __shared__ __attribute__((aligned(1024))) uint8_t ks[NST][BN * RB];
  __shared__ __attribute__((aligned(1024))) uint8_t vs[NST][BN * RB];

  // One task: (sequence, first query row, KV head) from a tile list, or
  // (first row, prefix chunk, KV head) in the shared-prefix pass.
  auto run_tile = [&](const int s, const int q0, const int g) {
  int tq0, nq, c, kv_end, ktb, first_lim;
  const int32_t* table;
  if constexpr (PREFIX) {
    // rows s .. s+nq-1 (one token each); keys of chunk q0
    tq0 = 0;
    nq = min(BQ, pfx.num_seqs - s);
    c = 0;
    kv_end = min((q0 + 1) * pfx.chunk_keys, pfx.prefix_keys);
    ktb = q0 * (pfx.chunk_keys / BN);
    // every row sees the whole chunk; only keys past its end (in its last
    // tile) are masked
    first_lim = kv_end - 1;
    table = block_table;
  } else {
    tq0 = qsl[s];
    const int ql = qsl[s + 1] - tq0;
    const int L = seq_lens[s];
    c = L - ql;
    nq = min(BQ, ql - q0);
    kv_end = c + q0 + nq;  // keys [0, kv_end) are visible to some row
    ktb = 0;
    // Keys up to first_lim are visible to every row of the tile: key tiles
    // that end at or below it need no mask.
    first_lim = c + q0;
    table = block_table + (int64_t)s * MB;
  }
  // key tiles ktb .. ktb+ntiles-1; below, kt counts from 0 and key tile
  // ktb + kt holds keys (ktb + kt) * 64 ..
  const int ntiles = (kv_end + BN - 1) / BN - ktb;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: scalar table reads
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int64_t kv_row = (int64_t)Hkv * D;

  // Rows of this lane (one per m-tile): row = w*RW + mt*16 + hl = token*G + head.
  bf16x8 qv[MT][KC];
  int lim[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = w * RW + mt * 16 + hl;
    const int tl = row / G;
    const int hh = row % G;
    const bool ok = tl < nq;
    int tok;
    if constexpr (PREFIX) {
      lim[mt] = kv_end - 1;
      tok = min(qsl[s + (ok ? tl : 0)], pfx.num_tokens - 1);
    } else {
      lim[mt] = c + q0 + min(tl, nq - 1);
      tok = tq0 + q0 + (ok ? tl : 0);
    }
    const u32x4* qp = (const u32x4*)(q + ((int64_t)tok * Hq + g * G + hh) * D) + grp;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qv[mt][i] = as_bf16x8(ok ? qp[4 * i] : z);
    }
  }

  f32x4 o[MT][DT];
  float m[MT];  // reference max per row, log2 units
  // Row sums of the weights, accumulated by the matrix core as ones . P^T
  // from the same bf16 P that multiplies V: every element of lsum[mt] holds
  // the running sum of row hl.
  f32x4 lsum[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int mi = 0; mi < DT; ++mi) o[mt][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[mt] = -INFINITY;
    lsum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

  const int last_blk = (kv_end - 1) / kBlock;  // last block any row reads
  constexpr int kTileBlocks = BN / kBlock;     // 16-token blocks per key tile
  // Load op j of wave w fills LDS bytes (j*NW + w)*1024 .. +1024 of a stage:
  // rows of one 16-key block (block kb(j) of the tile), lane l the 16 bytes
  // at l*16. Its table entry is wave-uniform (a scalar load), read one tile
  // ahead and clamped to the last block any row reads.
  auto kb = [&](int j) { return ((j * NW + w) * 1024 / RB) / kBlock; };
  auto tile_ids = [&](int kt, int (&ids)[NDMA]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) ids[j] = table[min((ktb + kt) * kTileBlocks + kb(j), last_blk)];
  };
  // Tile kt straight from HBM/L2 into LDS stage `stage`: lane l of op j
  // covers row r, physical chunk pc, and fetches logical chunk pc ^ swz(r)
  // of key kt*64 + r.
  // The loads are buffer loads into LDS from a base the wave computes per
  // block on the scalar unit (block id * block bytes + the head's offset);
  // the lanes' byte offsets inside the block are fixed.
  const uint32_t blk_bytes = (uint32_t)(kBlock * kv_row * 2);
  auto dma_tile = [&](int stage, const int (&ids)[NDMA]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int p = (j * NW + w) * 1024 + lane * 16;
      const int r = p / RB;
      const int pc = (p % RB) / 16;
      const uint64_t off = (uint64_t)(uint32_t)ids[j] * blk_bytes + (uint64_t)g * D * 2;
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const char*)k_cache + off), (short)0, (int)blk_bytes, kBufferWordFlags);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const char*)v_cache + off), (short)0, (int)blk_bytes, kBufferWordFlags);
      const int rb = (int)((r % kBlock) * kv_row * 2);
      buffer_to_lds16(kr, &ks[stage][(j * NW + w) * 1024], rb + (pc ^ swz_k<D>(r)) * 16);
      buffer_to_lds16(vr, &vs[stage][(j * NW + w) * 1024], rb + (pc ^ swz_v<D>(r)) * 16);
    }
  };
  // Rows of tile kt at or past kv_end came from a clamped or partly used
  // block: zero their V (each thread the bytes it loaded itself, after its
  // own loads completed), so a zero weight never meets a stale value.
  auto zero_tail = [&](int kt, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int p = (j * NW + w) * 1024 + lane * 16;
      if ((ktb + kt) * BN + p / RB >= kv_end) *(u32x4*)(&vs[stage][p]) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // Per-lane LDS byte offsets of the operand reads, so that the rest of each
  // address is a compile-time immediate (the swizzles depend on a row only
  // through its low bits, which the 16- and 32-row steps leave alone).
  // K (QK A operand): lane reads row n*16 + hl, logical chunk 4i + grp.
  int koff[KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) koff[i] = hl * RB + (((4 * i + grp) ^ swz_k<D>(hl)) * 16);
  // V (PV A operand, transpose reads): lane reads row kp*32 + 4*grp + hl/4
  // (and 16 rows on), 8 bytes at half (hl%2) of logical chunk 2*mi + (hl%4)/2.
  int voff[DT];
#pragma unroll
  for (int mi = 0; mi < DT; ++mi) {
    const int r0 = 4 * grp + hl / 4;
    voff[mi] = r0 * RB + (hl & 1) * 8 + (((2 * mi + (hl % 4) / 2) ^ swz_v<D>(r0)) * 16);
  }

  // One 64-key tile: S^T = K Q^T, masked online softmax, O^T += V^T P^T.
  // split: P enters PV as bf16 hi + lo parts (rows with few visible keys).
  auto compute_tile = [&](int kt, int stage, bool masked, auto split_tag)
      __attribute__((always_inline)) {
    constexpr bool kSplit = decltype(split_tag)::value;
    const uint8_t* kst = ks[stage];
    const uint8_t* vst = vs[stage];
    f32x4 st[MT][NS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int n = 0; n < NS; ++n) st[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NS; ++n) {
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)(kst + n * 16 * RB + koff[i]));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) st[mt][n] = mfma_16x16x32(a, qv[mt][i], st[mt][n]);
      }
    }
    if (masked) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int n = 0; n < NS; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = (ktb + kt) * BN + n * 16 + 4 * grp + r;
            st[mt][n][r] = key <= lim[mt] ? st[mt][n][r] : -INFINITY;
          }
    }
    // Lazy reference max (log2 units): re-reference a row only when one of
    // its scores exceeds the current reference by more than 2^kLazyP.
    // NaN-propagating maximum (masked scores are already -inf): needs no
    // canonicalisation of the MFMA results and maps to 3-input maxima.
    float lmax[MT];
    bool over = false;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float va = st[mt][0][0], vb = st[mt][0][1];
#pragma unroll
      for (int i = 2; i < 4 * NS; i += 2) {
        va = __builtin_elementwise_maximum(va, st[mt][i / 4][i % 4]);
        vb = __builtin_elementwise_maximum(vb, st[mt][i / 4][i % 4 + 1]);
      }
      const float v = __builtin_elementwise_maximum(va, vb);
      lmax[mt] = v * scale_log2;
      over |= lmax[mt] > m[mt] + kLazyP;
    }
    if (__any(over)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float mn = fmaxf(m[mt], max_across_groups(lmax[mt]));
        const float alpha = fast_exp2(m[mt] - mn);
        lsum[mt] *= alpha;
#pragma unroll
        for (int mi = 0; mi < DT; ++mi) o[mt][mi] *= alpha;
        m[mt] = mn;
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float negm = -m[mt];
#pragma unroll
      for (int n = 0; n < NS; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st[mt][n][r] = fast_exp2(__builtin_fmaf(st[mt][n][r], scale_log2, negm));
    }
    // O^T += V^T P^T per 32-key pair; the A operand holds keys
    // {4*grp+r, 16+4*grp+r} of the pair for d = 16*mi + hl (two transpose
    // reads), matching the order in which P^T is packed from S^T.
#pragma unroll
    for (int kp = 0; kp < NS / 2; ++kp) {
      bf16x8 pb[MT], pl[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (kSplit) {
          u32x4 hv, lv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32x2 hl2 = split_pack_bf16x2(st[mt][2 * kp + e / 2][2 * (e % 2)],
                                                st[mt][2 * kp + e / 2][2 * (e % 2) + 1]);
            hv[e] = hl2[0];
            lv[e] = hl2[1];
          }
          pb[mt] = as_bf16x8(hv);
          pl[mt] = as_bf16x8(lv);
        } else {
          u32x4 hv = {pack_bf16x2(st[mt][2 * kp][0], st[mt][2 * kp][1]),
                      pack_bf16x2(st[mt][2 * kp][2], st[mt][2 * kp][3]),
                      pack_bf16x2(st[mt][2 * kp + 1][0], st[mt][2 * kp + 1][1]),
                      pack_bf16x2(st[mt][2 * kp + 1][2], st[mt][2 * kp + 1][3])};
          pb[mt] = as_bf16x8(hv);
        }
      }
      const uint8_t* vrow0 = vst + kp * 32 * RB;
#pragma unroll
      for (int mi = 0; mi < DT; ++mi) {
        const uint8_t* va = vrow0 + voff[mi];
        const i16x4 a0 = lds_read_tr16((const uint16_t*)va);
        const i16x4 a1 = lds_read_tr16((const uint16_t*)(va + 16 * RB));
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt][mi] = mfma_16x16x32(av, pb[mt], o[mt][mi]);
        if constexpr (kSplit) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) o[mt][mi] = mfma_16x16x32(av, pl[mt], o[mt][mi]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        lsum[mt] = mfma_16x16x32(ones, pb[mt], lsum[mt]);
        if constexpr (kSplit) lsum[mt] = mfma_16x16x32(ones, pl[mt], lsum[mt]);
      }
    }
  };


  // Tiles 0 .. NST-2 are issued up front; at tile kt the loads of tiles
  // kt .. kt+NST-2 are in flight. Each step waits for tile kt's loads only
  // (2*NDMA operations per later tile in flight stay outstanding), joins the
  // barrier (every wave's part of tile kt has landed, and every wave is done
  // reading tile kt-1, whose stage the next issue overwrites), then issues
  // tile kt+NST-1 and computes tile kt.
  constexpr int kOps = 2 * NDMA;  // vector-memory operations per tile per wave
  int ids[NDMA];
#pragma unroll
  for (int u = 0; u < NST - 1; ++u) {
    if (u < ntiles) {
      tile_ids(u, ids);
      dma_tile(u, ids);
    }
  }
  tile_ids(NST - 1, ids);
  // One step per tile; the loop is unrolled by NST so that every step's
  // stage is a compile-time constant (LDS addresses become immediates).
  auto step = [&](int kt, auto stage_tag) __attribute__((always_inline)) {
    constexpr int stage = decltype(stage_tag)::value;
    const int later = min(NST - 2, ntiles - 1 - kt);  // tiles issued after kt
    if (NST == 3 && later == 1) wait_loads_then_barrier<kOps>();
    else wait_loads_then_barrier<0>();
    if ((ktb + kt + 1) * BN > kv_end) {
      zero_tail(kt, stage);
      lds_writes_then_barrier();
    }
    if (kt + NST - 1 < ntiles) dma_tile((stage + NST - 1) % NST, ids);
    const bool masked = (ktb + kt + 1) * BN - 1 > first_lim;
    // Tiles whose rows see at most kSplitKeys keys (SPLIT) keep P to about
    // 2^-17 (hi + lo): few weights carry each output there, and bf16
    // rounding of P would show in it.
    compute_tile(kt, stage, masked, std::integral_constant<bool, SPLIT>{});
    // The next tile's table entries: scalar loads share a wait counter with
    // LDS reads, so they are issued after this tile's last LDS read (and
    // kept there) and land while the next step waits for its tile.
    __builtin_amdgcn_sched_barrier(0);
    tile_ids(kt + NST, ids);
  };
  for (int kt = 0; kt < ntiles; kt += NST) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < ntiles) step(kt + 1, std::integral_constant<int, 1>{});
    if constexpr (NST == 3) {
      if (kt + 2 < ntiles) step(kt + 2, std::integral_constant<int, 2>{});
    }
  }

  if constexpr (PREFIX) {
    // partition q0 (the chunk) of rows s + tl: unnormalised numerator,
    // reference max (log2 units) and weight sum
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = w * RW + mt * 16 + hl;
      const int tl = row / G;
      const int hh = row % G;
      if (tl >= nq) continue;
      const int64_t base = ((int64_t)(s + tl) * pfx.num_parts_max + q0) * Hq + g * G + hh;
      float* op = pfx.ws_o + base * D + 4 * grp;
#pragma unroll
      for (int mi = 0; mi < DT; ++mi) *(f32x4*)(op + 16 * mi) = o[mt][mi];
      if (grp == 0) *(f32x2*)(pfx.ws_ml + base * 2) = f32x2{m[mt], lsum[mt][0]};
    }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const float ltot = lsum[mt][0];
    const int row = w * RW + mt * 16 + hl;
    const int tl = row / G;
    const int hh = row % G;
    if (tl >= nq) continue;
    const float inv = 1.0f / ltot;
    uint16_t* op = out + ((int64_t)(tq0 + q0 + tl) * Hq + g * G + hh) * D + 4 * grp;
#pragma unroll
    for (int mi = 0; mi < DT; ++mi) {
      u32x2 pr = {pack_bf16x2(o[mt][mi][0] * inv, o[mt][mi][1] * inv),
                  pack_bf16x2(o[mt][mi][2] * inv, o[mt][mi][3] * inv)};
      *(u32x2*)(op + 16 * mi) = pr;
    }
  }
  };  // run_tile

  const int nwg = gridDim.x;
  if (PREFIX) {
    // The writers come first in the grid: they are dispatched first and
    // hold their CUs for one load round trip, so a few tiles start that much
    // later (with the writers after the tiles, they wait for CUs that tiles
    // free and lengthen the launch's tail: 60.2 against 58.4 us per step on
    // the prefix-shared workload, the two-call sequence 61.4).
    const int nwrite = (int)gridDim.x - pfx.tile_grid;
    const int bid = (int)blockIdx.x - nwrite;
    if (bid < 0) {  // workgroup-uniform: the KV write
      const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
      if (i < pfx.write_chunks)
        write_kv_chunk(pfx.knew, pfx.vnew, pfx.slot_mapping, pfx.k_cache_w, pfx.v_cache_w, i,
                       pfx.chunks_per_token);
      return;
    }
    // XCD-aware order: the row tiles of one (KV head, chunk) are
    // consecutive logical tasks, so they share the chunk's K/V in one L2.
    const int logical = (bid % 8) * (pfx.tile_grid / 8) + bid / 8;
    const int rt = logical % pfx.row_tiles;
    const int rest = logical / pfx.row_tiles;
    const int chunk = rest % pfx.chunks;
    const int g = rest / pfx.chunks;
    if (g >= Hkv) return;
    run_tile(rt * BQ, chunk, g);
  } else if (!SPLIT) {
    // XCD-aware order: consecutive logical tiles (same KV head, same
    // sequence) land on the same XCD and share its L2.
    const int logical = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
    const int g = logical / tile_bound;
    const int ti = logical - g * tile_bound;
    if (g >= Hkv) return;
    const int s = tiles[2 * ti];
    if (s < 0) return;
    run_tile(s, tiles[2 * ti + 1], g);
  } else {
    // Few, light tasks: a small grid walks the list the planner counted.
    const int tasks = *tile_count * Hkv;
    for (int task = blockIdx.x; task < tasks; task += nwg) {
      const int ti = task / Hkv;
      run_tile(tiles[2 * ti], tiles[2 * ti + 1], task - ti * Hkv);
      __syncthreads();  // LDS stages are reused by the next task
    }
  }
}


template <int D, int G>
hipError_t launch_tiles(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  if (p.bound_a > 0) {
    const int64_t grid = ((int64_t)p.bound_a * a.num_kv_heads + 7) / 8 * 8;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    profile_begin(PA_KERNEL_PREFILL, stream);
    hipLaunchKernelGGL((prefill_tile_kernel<D, G, kListA>), dim3((unsigned)grid),
                       dim3(kWavesA * kWave), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_table,
                       a.seq_lens, a.query_start_loc, (uint16_t*)a.out, p.tiles_a, p.counts,
                       scale_log2, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                       p.bound_a, PrefixArgs{});
    profile_end(PA_KERNEL_PREFILL, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.bound_b > 0) {
    const int64_t grid =
        std::min<int64_t>((int64_t)p.bound_b * a.num_kv_heads, kSplitGridMax);
    profile_begin(PA_KERNEL_PREFILL_SHORT, stream);
    hipLaunchKernelGGL((prefill_tile_kernel<D, G, kListB>), dim3((unsigned)grid),
                       dim3(kWavesB * kWave), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_table,
                       a.seq_lens, a.query_start_loc, (uint16_t*)a.out, p.tiles_b,
                       p.counts + 1, scale_log2, a.num_q_heads, a.num_kv_heads,
                       a.max_blocks_per_seq, p.bound_b, PrefixArgs{});
    profile_end(PA_KERNEL_PREFILL_SHORT, stream);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_tiles_d(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_tiles<D, 1>(a, p, stream);
    case 2: return launch_tiles<D, 2>(a, p, stream);
    case 4: return launch_tiles<D, 4>(a, p, stream);
    case 8: return launch_tiles<D, 8>(a, p, stream);
    case 16: return launch_tiles<D, 16>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int G>
hipError_t launch_prefix_g(const ForwardArgs& a, const PrefixPlan& p, hipStream_t stream) {
  constexpr int BQ = 16 * kRowTiles * kWavesP / G;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int64_t tasks = (int64_t)((a.num_seqs + BQ - 1) / BQ) * p.chunks * a.num_kv_heads;
  const int64_t tile_grid = (tasks + 7) / 8 * 8;
  const int32_t chunks_per_token = a.num_kv_heads * a.head_size / 8;
  const int64_t write_chunks = p.write_tokens > 0 ? (int64_t)p.write_tokens * chunks_per_token : 0;
  const int64_t grid = tile_grid + (write_chunks + kWavesP * kWave - 1) / (kWavesP * kWave);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  PrefixArgs x{p.ws_o, p.ws_ml, p.num_parts_max, p.chunk_keys, p.prefix_keys, a.num_seqs,
               (a.num_seqs + BQ - 1) / BQ, p.chunks, a.num_tokens, (int32_t)tile_grid,
               chunks_per_token, write_chunks, (const u32x4*)p.knew, (const u32x4*)p.vnew,
               p.slot_mapping, (u32x4*)p.k_cache_w, (u32x4*)p.v_cache_w};
  profile_begin(PA_KERNEL_PREFIX, stream);
  hipLaunchKernelGGL((prefill_tile_kernel<D, G, kPrefix>), dim3((unsigned)grid),
                     dim3(kWavesP * kWave), 0, stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_table,
                     a.seq_lens, a.query_start_loc, (uint16_t*)a.out, nullptr, nullptr,
                     scale_log2, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq, 0, x);
  profile_end(PA_KERNEL_PREFIX, stream);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefix_d(const ForwardArgs& a, const PrefixPlan& p, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefix_g<D, 1>(a, p, stream);
    case 2: return launch_prefix_g<D, 2>(a, p, stream);
    case 4: return launch_prefix_g<D, 4>(a, p, stream);
    case 8: return launch_prefix_g<D, 8>(a, p, stream);
    case 16: return launch_prefix_g<D, 16>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefix(const ForwardArgs& a, const PrefixPlan& p, hipStream_t stream) {
  if (p.chunks < 1 || p.chunk_keys < kKeysPerTile || p.chunk_keys % kKeysPerTile ||
      p.prefix_keys < 1 || (int64_t)p.chunks * p.chunk_keys < p.prefix_keys ||
      p.num_parts_max <= p.chunks || !p.ws_o || !p.ws_ml)
    return hipErrorInvalidValue;
  switch (a.head_size) {
    case 64: return launch_prefix_d<64>(a, p, stream);
    case 128: return launch_prefix_d<128>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

int32_t prefill_tile_queries(int32_t group) { return 16 * kRowTilesA * kWavesA / group; }
int32_t prefill_split_tile_queries(int32_t group) { return 16 * kRowTiles * kWavesB / group; }
int32_t prefix_tile_rows(int32_t group) { return 16 * kRowTiles * kWavesP / group; }

int32_t prefill_split_keys() { return kSplitKeys; }

int32_t prefill_split_tiles_per_row(int32_t group) {
  const int32_t bq = 16 * kRowTiles * kWavesB / group;
  return (kSplitKeys + bq - 1) / bq;
}

hipError_t launch_prefill_plan(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream) {
  if (p.bound_a <= 0 && p.bound_b <= 0) return hipSuccess;
  profile_begin(PA_KERNEL_PLAN, stream);
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream,
                     a.query_start_loc, a.seq_lens, a.num_seqs, p.tile_queries,
                     p.split_tile_queries, p.tiles_a,
                     p.bound_a, p.tiles_b, p.bound_b, p.counts, p.all_rows ? 1 : 2);
  profile_end(PA_KERNEL_PLAN, stream);
  return hipGetLastError();
}

hipError_t launch_write_and_plan(const ForwardArgs& a, const PrefillPlan& p, const void* k,
                                 const void* v, const int64_t* slot_mapping, void* k_cache,
                                 void* v_cache, hipStream_t stream) {
  if (p.bound_a <= 0 && p.bound_b <= 0)
    return launch_cache_write(k, v, slot_mapping, k_cache, v_cache, a.num_tokens,
                              a.num_kv_heads, a.head_size, stream);
  const int32_t chunks_per_token = a.num_kv_heads * a.head_size / 8;
  const int64_t total = (int64_t)a.num_tokens * chunks_per_token;
  const int64_t blocks = 1 + (total + kPlanThreads - 1) / kPlanThreads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  profile_begin(PA_KERNEL_WRITE_PLAN, stream);
  hipLaunchKernelGGL(write_plan_kernel, dim3((unsigned)blocks), dim3(kPlanThreads), 0, stream,
                     a.query_start_loc, a.seq_lens, a.num_seqs, p.tile_queries,
                     p.split_tile_queries, p.tiles_a, p.bound_a, p.tiles_b, p.bound_b, p.counts,
                     p.all_rows ? 1 : 2, (const u32x4*)k, (const u32x4*)v, slot_mapping,
                     (u32x4*)k_cache, (u32x4*)v_cache, total, chunks_per_token);
  profile_end(PA_KERNEL_WRITE_PLAN, stream);
  return hipGetLastError();
}

hipError_t launch_prefill_tiles(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream) {
  if (p.bound_a <= 0 && p.bound_b <= 0) return hipSuccess;
  switch (a.head_size) {
    case 64: return launch_tiles_d<64>(a, p, stream);
    case 128: return launch_tiles_d<128>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
