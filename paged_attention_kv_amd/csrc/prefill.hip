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
// causal mask and an fp32 online softmax, and accumulates O^T += V^T P^T with
// 16x16x32 MFMAs whose B operand is the S^T accumulator converted to bf16
// in place. A single-workgroup planner kernel turns query_start_loc into the
// list of tiles on the device, so the host never reads lengths.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kPrefillThreads = 256;
constexpr int kRowsPerWG = 128;
constexpr int kKeysPerTile = 64;
constexpr int kPlanThreads = 1024;

// tiles[2*i] = sequence, tiles[2*i+1] = first query row of the tile, heaviest
// tiles (latest rows, most keys) of each sequence first; unused entries -1.
__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(
    const int32_t* __restrict__ qsl, int32_t S, int32_t tile_queries, int32_t* __restrict__ tiles,
    int32_t tile_bound) {
  __shared__ int32_t scan[kPlanThreads];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int n = 0;
    if (s < S) {
      const int ql = qsl[s + 1] - qsl[s];
      n = ql > 1 ? (ql + tile_queries - 1) / tile_queries : 0;
    }
    scan[tid] = n;
    __syncthreads();
    for (int d = 1; d < kPlanThreads; d <<= 1) {
      const int add = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int off = carry + scan[tid] - n;
    for (int k = 0; k < n; ++k) {
      const int idx = off + k;
      if (idx < tile_bound) {
        tiles[2 * idx] = s;
        tiles[2 * idx + 1] = (n - 1 - k) * tile_queries;
      }
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) carry += scan[tid];
    __syncthreads();
  }
  for (int i = carry + tid; i < tile_bound; i += kPlanThreads) {
    tiles[2 * i] = -1;
    tiles[2 * i + 1] = -1;
  }
}

template <int D, int G>
__global__ __launch_bounds__(kPrefillThreads) void prefill_tile_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
    uint16_t* __restrict__ out, const int32_t* __restrict__ tiles, float scale_log2, int32_t Hq,
    int32_t Hkv, int32_t MB, int32_t tile_bound) {
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

  __shared__ __attribute__((aligned(16))) uint16_t ks[BN * RSK];
  __shared__ __attribute__((aligned(16))) uint16_t vs[BN * RSV];

  // XCD-aware order: consecutive logical tiles (same KV head, same sequence)
  // land on the same XCD and share its L2.
  const int nwg = gridDim.x;
  const int logical = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  const int g = logical / tile_bound;
  const int ti = logical - g * tile_bound;
  if (g >= Hkv) return;
  const int s = tiles[2 * ti];
  if (s < 0) return;
  const int q0 = tiles[2 * ti + 1];
  const int tq0 = qsl[s];
  const int ql = qsl[s + 1] - tq0;
  const int L = seq_lens[s];
  const int c = L - ql;
  const int nq = min(BQ, ql - q0);
  const int kv_end = c + q0 + nq;  // keys [0, kv_end) are visible to some row
  const int ntiles = (kv_end + BN - 1) / BN;

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
  float m[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};

  const int32_t* table = block_table + (int64_t)s * MB;
  u32x4 kr[CPT], vr[CPT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int cidx = j * kPrefillThreads + tid;
      const int key = kt * BN + cidx / CPR;
      const int col8 = cidx % CPR;
      const u32x4 z = {0u, 0u, 0u, 0u};
      if (key < kv_end) {
        const int64_t blk = table[key / kBlock];
        const int64_t off = (blk * kBlock + key % kBlock) * kv_row + (int64_t)g * D + col8 * 8;
        kr[j] = *(const u32x4*)(k_cache + off);
        vr[j] = *(const u32x4*)(v_cache + off);
      } else {
        kr[j] = z;
        vr[j] = z;
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int cidx = j * kPrefillThreads + tid;
      const int key = cidx / CPR;
      const int col8 = cidx % CPR;
      *(u32x4*)(ks + key * RSK + col8 * 8) = kr[j];
      *(u32x4*)(vs + key * RSV + col8 * 8) = vr[j];
    }
  };

  load_tile(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < ntiles) load_tile(kt + 1);

    // S^T = K Q^T for 4 key sub-tiles x 2 row tiles.
    f32x4 st[2][NS];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int n = 0; n < NS; ++n) st[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NS; ++n) {
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)(ks + (n * 16 + hl) * RSK + 32 * i + 8 * grp));
        st[0][n] = mfma_16x16x32(a, qv[0][i], st[0][n]);
        st[1][n] = mfma_16x16x32(a, qv[1][i], st[1][n]);
      }
    }

    // Mask, online softmax, P^T packed (as bf16 hi + lo parts) as the B
    // operand of the PV product.
    bf16x8 pb[2][NS / 2], pl[2][NS / 2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float rmax = -INFINITY;
#pragma unroll
      for (int n = 0; n < NS; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt * BN + n * 16 + 4 * grp + r;
          const float v = key <= lim[mt] ? st[mt][n][r] * scale_log2 : -INFINITY;
          st[mt][n][r] = v;
          rmax = fmaxf(rmax, v);
        }
      rmax = max_across_groups(rmax);
      const float mn = fmaxf(m[mt], rmax);
      const float alpha = fast_exp2(m[mt] - mn);
      m[mt] = mn;
      float ps = 0.f;
#pragma unroll
      for (int n = 0; n < NS; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(st[mt][n][r] - mn);
          st[mt][n][r] = p;
          ps += p;
        }
      lsum[mt] = lsum[mt] * alpha + ps;
#pragma unroll
      for (int mi = 0; mi < DT; ++mi) o[mt][mi] *= alpha;
#pragma unroll
      for (int kp = 0; kp < NS / 2; ++kp) {
        uint16_t h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(st[mt][2 * kp + e / 4][e % 4], h[e], l[e]);
        u32x4 hv, lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[e] = (uint32_t)h[2 * e] | ((uint32_t)h[2 * e + 1] << 16);
          lv[e] = (uint32_t)l[2 * e] | ((uint32_t)l[2 * e + 1] << 16);
        }
        pb[mt][kp] = as_bf16x8(hv);
        pl[mt][kp] = as_bf16x8(lv);
      }
    }

    // O^T += V^T P^T; the A operand holds keys {4*grp+r, 16+4*grp+r} of each
    // 32-key pair for d = 16*mi + hl (two transpose reads), matching the P^T
    // element order.
#pragma unroll
    for (int kp = 0; kp < NS / 2; ++kp) {
      const uint16_t* vrow = vs + (kp * 32 + 4 * grp + hl / 4) * RSV + 4 * (hl % 4);
#pragma unroll
      for (int mi = 0; mi < DT; ++mi) {
        const i16x4 a0 = lds_read_tr16(vrow + 16 * mi);
        const i16x4 a1 = lds_read_tr16(vrow + 16 * RSV + 16 * mi);
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[0][mi] = mfma_16x16x32(av, pb[0][kp], o[0][mi]);
        o[1][mi] = mfma_16x16x32(av, pb[1][kp], o[1][mi]);
        o[0][mi] = mfma_16x16x32(av, pl[0][kp], o[0][mi]);
        o[1][mi] = mfma_16x16x32(av, pl[1][kp], o[1][mi]);
      }
    }
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
}

template <int D, int G>
hipError_t launch_tiles(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int64_t wgs = (int64_t)p.tile_bound * a.num_kv_heads;
  const int64_t grid = (wgs + 7) / 8 * 8;
  hipLaunchKernelGGL((prefill_tile_kernel<D, G>), dim3((unsigned)grid), dim3(kPrefillThreads), 0,
                     stream, (const uint16_t*)a.q, (const uint16_t*)a.k_cache,
                     (const uint16_t*)a.v_cache, a.block_table, a.seq_lens, a.query_start_loc,
                     (uint16_t*)a.out, p.tiles, scale_log2, a.num_q_heads, a.num_kv_heads,
                     a.max_blocks_per_seq, p.tile_bound);
  return hipGetLastError();
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

hipError_t launch_prefill(const ForwardArgs& a, const PrefillPlan& p, hipStream_t stream) {
  if (p.tile_bound <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream,
                     a.query_start_loc, a.num_seqs, p.tile_queries, p.tiles, p.tile_bound);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.head_size) {
    case 64: return launch_tiles_d<64>(a, p, stream);
    case 128: return launch_tiles_d<128>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
