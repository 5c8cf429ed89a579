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
// head) with 4 waves. The tile packs the G query heads that share the KV head
// into the MFMA M dimension: 128 rows = (128/G tokens) x (G heads), 32 rows
// per wave, so every K/V tile staged in LDS serves all G heads. Per 64-key
// tile each wave computes S^T = K Q^T (keys x rows) with 16x16x32 bf16 MFMAs
// (K rows read from LDS, Q^T held in registers), applies the bottom-right
// causal mask (only on tiles that reach past the first row's limit) and an
// fp32 online softmax with a lazily re-referenced max, and accumulates
// O^T += V^T P^T with 16x16x32 MFMAs whose B operand is the S^T accumulator
// converted to bf16 in place (as hi + lo parts when the tile's rows see few
// keys). K/V tiles are double-buffered in LDS through registers: the global
// loads of tile t+2 are in flight while tile t computes and tile t+1 is
// stored, with one barrier per tile. A single-workgroup planner kernel turns
// query_start_loc into the list of tiles on the device, so the host never
// reads lengths.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kPrefillThreads = 256;
constexpr int kRowsPerWG = 128;
constexpr int kKeysPerTile = 64;
constexpr float kLazyP = 8.0f;  // log2 of the largest unnormalised weight
constexpr int kSplitKeys = 128;  // workgroups seeing at most this many keys split P
constexpr int kSplitGridMax = 512;  // workgroups walking list B
constexpr int kPlanThreads = 1024;

// Two tile lists, entry = (sequence, first query row), unused entries -1:
// list A holds tiles whose rows see more than kSplitKeys keys, each row's
// heaviest (latest) tiles first; list B the tiles that see at most
// kSplitKeys keys (they keep P as bf16 hi + lo).
__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, int32_t S,
    int32_t tile_queries, int32_t* __restrict__ tiles_a, int32_t bound_a,
    int32_t* __restrict__ tiles_b, int32_t bound_b, int32_t* __restrict__ counts) {
  __shared__ int32_t scan_a[kPlanThreads], scan_b[kPlanThreads];
  __shared__ int32_t carry_a, carry_b;
  const int tid = threadIdx.x;
  if (tid == 0) carry_a = carry_b = 0;
  __syncthreads();
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int na = 0, nb = 0, ql = 0, c = 0;
    if (s < S) {
      ql = qsl[s + 1] - qsl[s];
      c = seq_lens[s] - ql;
      if (ql > 1) {
        const int n = (ql + tile_queries - 1) / tile_queries;
        // kv_end of tile t is c + t*BQ + min(BQ, ql - t*BQ): non-decreasing in t
        while (nb < n && c + min((nb + 1) * tile_queries, ql) <= kSplitKeys) ++nb;
        na = n - nb;
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
        tiles_a[2 * idx + 1] = (nb + na - 1 - k) * tile_queries;
      }
    }
    for (int k = 0; k < nb; ++k) {
      const int idx = off_b + k;
      if (idx < bound_b) {
        tiles_b[2 * idx] = s;
        tiles_b[2 * idx + 1] = k * tile_queries;
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

template <int D, int G, bool SPLIT>
__global__ __launch_bounds__(kPrefillThreads, SPLIT ? 1 : 2) void prefill_tile_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    uint16_t* __restrict__ out, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, float scale_log2, int32_t Hq, int32_t Hkv,
    int32_t MB, int32_t tile_bound) {
  constexpr int BQ = kRowsPerWG / G;          // query tokens per tile
  constexpr int BN = kKeysPerTile;            // keys per iteration
  constexpr int RSK = D + 8;                  // padded LDS row of K (elements): row reads
                                              // of 8 lanes hit 8 distinct bank quads
  constexpr int RSV = D + 16;                 // padded LDS row of V: the 4 rows of a
                                              // transpose read sit 8 banks apart
  constexpr int KC = D / 32;                  // QK MFMAs per 16x16 S tile
  constexpr int DT = D / 16;                  // PV output tiles along d
  constexpr int NS = BN / 16;                 // 16-key sub-tiles per tile
  constexpr int CPR = D / 8;                  // 16-byte chunks per K/V row
  constexpr int CPT = BN * CPR / kPrefillThreads;  // chunks per thread per tile
  static_assert(CPT * kPrefillThreads == BN * CPR, "tile must split evenly");

  // Two stages: the tile being computed and the one being filled.
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BN * RSK];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][BN * RSV];

  // One (sequence, query tile, KV head) task.
  auto run_tile = [&](const int s, const int q0, const int g) {
  const int tq0 = qsl[s];
  const int ql = qsl[s + 1] - tq0;
  const int L = seq_lens[s];
  const int c = L - ql;
  const int nq = min(BQ, ql - q0);
  const int kv_end = c + q0 + nq;  // keys [0, kv_end) are visible to some row
  const int ntiles = (kv_end + BN - 1) / BN;
  // Keys up to first_lim are visible to every row of the tile: key tiles
  // that end at or below it need no mask.
  const int first_lim = c + q0;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int64_t kv_row = (int64_t)Hkv * D;

  // Rows of this lane (one per m-tile): row = w*32 + mt*16 + hl = token*G + head.
  bf16x8 qv[2][KC];
  int lim[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = w * 32 + mt * 16 + hl;
    const int tl = row / G;
    const int hh = row % G;
    lim[mt] = c + q0 + min(tl, nq - 1);
    const bool ok = tl < nq;
    const u32x4* qp =
        (const u32x4*)(q + ((int64_t)(tq0 + q0 + (ok ? tl : 0)) * Hq + g * G + hh) * D) + grp;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qv[mt][i] = as_bf16x8(ok ? qp[4 * i] : z);
    }
  }

  f32x4 o[2][DT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int mi = 0; mi < DT; ++mi) o[mt][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};  // reference max per row, log2 units
  float lsum[2] = {0.f, 0.f};

  const int32_t* table = block_table + (int64_t)s * MB;
  u32x4 kr[CPT], vr[CPT];
  // Keys at or past kv_end load key kv_end-1 instead: finite data that the
  // mask removes (a zero weight times a finite value), never a stale slot.
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int cidx = j * kPrefillThreads + tid;
      const int key = min(kt * BN + cidx / CPR, kv_end - 1);
      const int col8 = cidx % CPR;
      const int64_t blk = table[key / kBlock];
      const int64_t off = (blk * kBlock + key % kBlock) * kv_row + (int64_t)g * D + col8 * 8;
      kr[j] = *(const u32x4*)(k_cache + off);
      vr[j] = *(const u32x4*)(v_cache + off);
    }
  };
  auto store_tile = [&](int stage) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int cidx = j * kPrefillThreads + tid;
      const int key = cidx / CPR;
      const int col8 = cidx % CPR;
      *(u32x4*)(&ks[stage][key * RSK + col8 * 8]) = kr[j];
      *(u32x4*)(&vs[stage][key * RSV + col8 * 8]) = vr[j];
    }
  };

  // One 64-key tile: S^T = K Q^T, masked online softmax, O^T += V^T P^T.
  // split: P enters PV as bf16 hi + lo parts (rows with few visible keys).
  auto compute_tile = [&](int kt, int stage, bool masked, auto split_tag) {
    constexpr bool kSplit = decltype(split_tag)::value;
    const uint16_t* kst = ks[stage];
    const uint16_t* vst = vs[stage];
    f32x4 st[2][NS];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int n = 0; n < NS; ++n) st[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NS; ++n) {
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)(kst + (n * 16 + hl) * RSK + 32 * i + 8 * grp));
        st[0][n] = mfma_16x16x32(a, qv[0][i], st[0][n]);
        st[1][n] = mfma_16x16x32(a, qv[1][i], st[1][n]);
      }
    }
    if (masked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int n = 0; n < NS; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kt * BN + n * 16 + 4 * grp + r;
            st[mt][n][r] = key <= lim[mt] ? st[mt][n][r] : -INFINITY;
          }
    }
    // Lazy reference max (log2 units): re-reference a row only when one of
    // its scores exceeds the current reference by more than 2^kLazyP.
    float lmax[2];
    bool over = false;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float v = -INFINITY;
#pragma unroll
      for (int n = 0; n < NS; ++n)
        v = fmaxf(v, fmaxf(fmaxf(st[mt][n][0], st[mt][n][1]), fmaxf(st[mt][n][2], st[mt][n][3])));
      lmax[mt] = v * scale_log2;
      over |= lmax[mt] > m[mt] + kLazyP;
    }
    if (__any(over)) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const float mn = fmaxf(m[mt], max_across_groups(lmax[mt]));
        const float alpha = fast_exp2(m[mt] - mn);
        lsum[mt] *= alpha;
#pragma unroll
        for (int mi = 0; mi < DT; ++mi) o[mt][mi] *= alpha;
        m[mt] = mn;
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const float negm = -m[mt];
      float ps = 0.f;
#pragma unroll
      for (int n = 0; n < NS; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(__builtin_fmaf(st[mt][n][r], scale_log2, negm));
          st[mt][n][r] = p;
          ps += p;
        }
      lsum[mt] += ps;
    }
    // O^T += V^T P^T per 32-key pair; the A operand holds keys
    // {4*grp+r, 16+4*grp+r} of the pair for d = 16*mi + hl (two transpose
    // reads), matching the order in which P^T is packed from S^T.
#pragma unroll
    for (int kp = 0; kp < NS / 2; ++kp) {
      bf16x8 pb[2], pl[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        if constexpr (kSplit) {
          uint16_t h[8], l[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) split_bf16(st[mt][2 * kp + e / 4][e % 4], h[e], l[e]);
          u32x4 hv, lv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hv[e] = (uint32_t)h[2 * e] | ((uint32_t)h[2 * e + 1] << 16);
            lv[e] = (uint32_t)l[2 * e] | ((uint32_t)l[2 * e + 1] << 16);
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
      const uint16_t* vrow = vst + (kp * 32 + 4 * grp + hl / 4) * RSV + 4 * (hl % 4);
#pragma unroll
      for (int mi = 0; mi < DT; ++mi) {
        const i16x4 a0 = lds_read_tr16(vrow + 16 * mi);
        const i16x4 a1 = lds_read_tr16(vrow + 16 * RSV + 16 * mi);
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[0][mi] = mfma_16x16x32(av, pb[0], o[0][mi]);
        o[1][mi] = mfma_16x16x32(av, pb[1], o[1][mi]);
        if constexpr (kSplit) {
          o[0][mi] = mfma_16x16x32(av, pl[0], o[0][mi]);
          o[1][mi] = mfma_16x16x32(av, pl[1], o[1][mi]);
        }
      }
    }
  };


  load_tile(0);
  store_tile(0);
  if (ntiles > 1) load_tile(1);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();  // stage kt%2 is filled; every wave is done with tile kt-1
    if (kt + 1 < ntiles) store_tile((kt + 1) & 1);
    if (kt + 2 < ntiles) load_tile(kt + 2);
    const bool masked = (kt + 1) * BN - 1 > first_lim;
    // Tiles whose rows see at most kSplitKeys keys (SPLIT) keep P to about
    // 2^-17 (hi + lo): few weights carry each output there, and bf16
    // rounding of P would show in it.
    compute_tile(kt, kt & 1, masked, std::integral_constant<bool, SPLIT>{});
  }

#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const float ltot = sum_across_groups(lsum[mt]);
    const int row = w * 32 + mt * 16 + hl;
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
  if (!SPLIT) {
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
    profile_begin(PA_KERNEL_PREFILL, stream);
    hipLaunchKernelGGL((prefill_tile_kernel<D, G, false>), dim3((unsigned)grid),
                       dim3(kPrefillThreads), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_table,
                       a.seq_lens, a.query_start_loc, (uint16_t*)a.out, p.tiles_a, p.counts,
                       scale_log2, a.num_q_heads, a.num_kv_heads, a.max_blocks_per_seq,
                       p.bound_a);
    profile_end(PA_KERNEL_PREFILL, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.bound_b > 0) {
    const int64_t grid =
        std::min<int64_t>((int64_t)p.bound_b * a.num_kv_heads, kSplitGridMax);
    profile_begin(PA_KERNEL_PREFILL_SHORT, stream);
    hipLaunchKernelGGL((prefill_tile_kernel<D, G, true>), dim3((unsigned)grid),
                       dim3(kPrefillThreads), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_table,
                       a.seq_lens, a.query_start_loc, (uint16_t*)a.out, p.tiles_b,
                       p.counts + 1, scale_log2, a.num_q_heads, a.num_kv_heads,
                       a.max_blocks_per_seq, p.bound_b);
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

}  // namespace

int32_t prefill_tile_queries(int32_t group) { return kRowsPerWG / group; }

int32_t prefill_split_tiles_per_row(int32_t group) {
  const int32_t bq = kRowsPerWG / group;
  return (kSplitKeys + bq - 1) / bq;
}

hipError_t launch_prefill(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream) {
  if (p.bound_a <= 0 && p.bound_b <= 0) return hipSuccess;
  profile_begin(PA_KERNEL_PLAN, stream);
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream,
                     a.query_start_loc, a.seq_lens, a.num_seqs, p.tile_queries, p.tiles_a,
                     p.bound_a, p.tiles_b, p.bound_b, p.counts);
  profile_end(PA_KERNEL_PLAN, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.head_size) {
    case 64: return launch_tiles_d<64>(a, p, stream);
    case 128: return launch_tiles_d<128>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
