// C ABI of the paged-attention library: argument checks, workspace planning
// and kernel dispatch. Declarations and the contract of every entry point
// are in include/pa.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "errors.h"
#include "kernels.h"
#include "pa.h"

namespace {

thread_local std::string g_last_error;

__attribute__((format(printf, 2, 3))) int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace

namespace pa {
int record_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}
void clear_error() { g_last_error.clear(); }
}  // namespace pa

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int32_t kMinPartTokens = 128;
// Longest decode partition when rows are split for balance: a single
// workgroup streaming a much longer row would outlast the rest of the grid.
constexpr int32_t kBalancePartTokens = 4096;
constexpr int32_t kComputeUnits = 256;  // MI355X
constexpr size_t kAlign = 256;
constexpr int64_t kMaxGridZ = 65535;  // partitions per row ride on grid z
// Row arrival counters of the stream decode schedule: a region of fixed size
// at the start of every workspace, zero before the first call and left zero
// by every call, so no call of any shape writes other data over them.
constexpr int64_t kCounterSlots = 1 << 16;
// Stream decode schedule: at most this many rows (each workgroup scans them
// all in LDS), this many workgroups, and this many waves per workgroup
// (one per KV head of a head group, or several per head when heads are few).
constexpr int32_t kStreamMaxRows = 4096;
constexpr int32_t kStreamMaxWgs = 512;
constexpr int32_t kStreamWaves = 8;
// The stream schedule pays a fixed latency per workgroup (row scan, first
// loads, hand-over of split rows) while HBM idles; it wins once a share is
// long enough to hide it. Shares are estimated from host bounds (rows x
// blocks of the longest row).
constexpr int64_t kStreamMinBlocksPerWg = 64;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int env_int(const char* name, int lo, int hi, int dflt) {
  const char* e = getenv(name);
  if (!e) return dflt;
  const int v = atoi(e);
  return (v >= lo && v <= hi) ? v : dflt;
}

// (max_blocks_per_seq <= kMaxBlocksPerSeq, checked by the planners)
constexpr int32_t kMaxBlocksPerSeq = INT32_MAX / PA_BLOCK_SIZE;
int32_t resolved_max_seq_len(int32_t max_blocks_per_seq, int32_t hint) {
  const int32_t cap = std::min(max_blocks_per_seq, kMaxBlocksPerSeq) * PA_BLOCK_SIZE;
  return hint > 0 ? std::min(hint, cap) : cap;
}

// Waves per decode workgroup (they take a partition's blocks in turn). Four
// measured best on every decode workload tried (2..16 swept): more waves
// per CU add outstanding misses without adding bandwidth. PA_DECODE_WAVES
// overrides it for tuning sweeps, up to what fits on a CU.
constexpr int32_t kDecodeWaves = 4;
int32_t decode_waves(int32_t head_size, int32_t prefetch) {
  static const int v = env_int("PA_DECODE_WAVES", 1, 16, 0);
  const int32_t maxw = std::max(1, pa::decode_max_waves(head_size, prefetch));
  return std::min(v > 0 ? v : kDecodeWaves, maxw);
}

// Tokens per partition of a decode row. When rows x KV heads already give
// every CU a workgroup, rows stay whole up to kBalancePartTokens (rows of one
// partition skip the combine pass); otherwise rows are split until the
// workgroups cover all CUs. A partition holds at most 64 blocks per wave.
// PA_DECODE_PART_TOKENS overrides it (a multiple of 16) for tuning sweeps.
int32_t choose_part_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t waves,
                           int32_t max_len) {
  const int32_t cap = 64 * waves * PA_BLOCK_SIZE;
  static const int32_t env = [] {
    const int v = env_int("PA_DECODE_PART_TOKENS", kMinPartTokens, 1 << 20, 0);
    return v % PA_BLOCK_SIZE == 0 ? v : 0;
  }();
  if (env) return std::min(env, cap);
  const int64_t items = std::max<int64_t>(1, (int64_t)num_seqs * num_kv_heads);
  int64_t nparts = items >= kComputeUnits ? 1 : (kComputeUnits + items - 1) / items;
  nparts = std::max<int64_t>(nparts, (max_len + kBalancePartTokens - 1) / kBalancePartTokens);
  nparts = std::max<int64_t>(nparts, (max_len + cap - 1) / cap);
  int64_t part = (max_len + nparts - 1) / nparts;
  part = (part + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE * PA_BLOCK_SIZE;
  return (int32_t)std::min<int64_t>(std::max<int64_t>(part, kMinPartTokens), cap);
}

// Partitioned decode with the merge in the kernel: the last workgroup of a
// split row merges its partials, so no combine launch follows. Each
// workgroup that hands a partial over pays an agent-scope release (an L2
// write-back); with partitions of more than kFusedMergeMaxPartTokens keys
// that measured 4-40% slower than leaving the merge to the combine launch
// (2 partitions of 1500 keys at 48 x 4 (row, KV head): 43.3 against
// 31.1 us), with partitions of up to 1024 keys faster (64 of 128 keys at
// 1 x 4: 15.4 against 17.7 us). PA_DECODE_FUSED_COMBINE=0 turns the
// in-kernel merge off, =2 uses it at every partition length (comparisons).
// Splitting rows further for balance on this path measured slower on the
// decode workloads (the split adds workgroups and hand-overs while HBM is
// already the limit), so partitions keep the sizes chosen above.
constexpr int32_t kFusedMergeMaxPartTokens = 1024;
bool decode_counters_fit(int32_t num_seqs, int32_t num_kv_heads) {
  return (int64_t)num_seqs * num_kv_heads <= kCounterSlots;
}
bool decode_fused_combine(int32_t num_seqs, int32_t num_kv_heads, int32_t part_tokens) {
  static const int v = env_int("PA_DECODE_FUSED_COMBINE", 0, 2, 1);
  return v != 0 && decode_counters_fit(num_seqs, num_kv_heads) &&
         (v == 2 || part_tokens <= kFusedMergeMaxPartTokens);
}

bool supported_group(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// Query tokens per row that the decode kernel takes (rows of 1..qmax
// tokens, their qmax * G columns in one 16-column matrix tile): with a host
// bound 1 < max_query_len_hint <= 16 / G every row runs there and no prefill
// launch is made; otherwise single-token rows only.
int32_t decode_qmax(int32_t group, int32_t max_query_len_hint) {
  return (max_query_len_hint > 1 && max_query_len_hint * group <= 16) ? max_query_len_hint : 1;
}

// Decode schedules. Even shares (the stream kernel: equal shares of all
// rows' blocks per workgroup) fit when the batch has few enough rows for the
// per-workgroup row scan; they are the default when shares would be long
// enough, else the partitioned schedule is. PA_DECODE_STREAM=0 / 1 makes the
// default partitioned / even shares (where they fit); PA_DECODE_STREAM_WGS
// sets the even-share workgroups (default one per CU). Per call, flags of
// pa_forward_ex choose.
int32_t decode_stream_wgs() {
  static const int v = env_int("PA_DECODE_STREAM_WGS", 1, kStreamMaxWgs, kComputeUnits);
  return v;
}
bool decode_stream_fits(int32_t num_seqs, int32_t num_kv_heads, int32_t head_size) {
  if (num_seqs > kStreamMaxRows) return false;
  const int32_t heads = std::min(num_kv_heads, kStreamWaves);
  const int64_t groups = (num_kv_heads + heads - 1) / heads;
  return (int64_t)num_seqs * groups <= kCounterSlots &&
         pa::decode_stream_lds_bytes(head_size, kStreamWaves / heads * heads, num_seqs) <=
             64 * 1024;
}
bool decode_stream_default(int32_t num_seqs, int32_t max_len) {
  static const int env = env_int("PA_DECODE_STREAM", 0, 2, 2);  // 2: by size
  if (env != 2) return env == 1;
  const int64_t blocks_bound = (int64_t)num_seqs * ((max_len + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE);
  return blocks_bound >= kStreamMinBlocksPerWg * decode_stream_wgs();
}

// Register ring depth of the decode kernel (blocks in flight per wave);
// PA_DECODE_PREFETCH overrides it for tuning sweeps.
int32_t decode_prefetch(int32_t head_size) {
  static const int v = env_int("PA_DECODE_PREFETCH", 2, 3, 0);
  if (head_size > 64) return 2;
  return v ? v : 2;
}

// Mixed batches: decode rows on even shares are bound by HBM bandwidth and
// prefill rows by the matrix cores, so the two parts run side by side (the
// prefill launches on a second stream). The decode then takes fewer shares
// than CUs, leaving CUs to the prefill tiles; on the mixed 8192-token step
// 160 shares measured best (128..224 swept), and the decode rows alone lose
// only ~10% at 160 shares since ~200 CUs already carry HBM's rate. Batches
// with fewer prefill tokens than kOverlapMinPrefillTokens run one part after
// the other. PA_MIXED_OVERLAP=0 turns the overlap off; PA_MIXED_DECODE_WGS
// sets the decode's shares (for sweeps).
constexpr int32_t kOverlapDecodeWgs = 160;
constexpr int64_t kOverlapMinPrefillTokens = 1024;
bool mixed_overlap_enabled() {
  static const int v = env_int("PA_MIXED_OVERLAP", 0, 1, 1);
  return v == 1;
}
constexpr int64_t kShortBatchMaxTasks = 256;
bool short_batch_tiles_enabled() {
  static const int v = env_int("PA_SHORT_BATCH_TILES", 0, 1, 1);
  return v == 1;
}
int32_t mixed_decode_wgs() {
  static const int v = env_int("PA_MIXED_DECODE_WGS", 1, kStreamMaxWgs, kOverlapDecodeWgs);
  return v;
}

}  // namespace

namespace pa {

bool plan_workspace(int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_size, int32_t max_blocks_per_seq,
                    int32_t max_query_len_hint, int32_t max_seq_len_hint, WorkspaceLayout* out) {
  if (num_tokens < 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_size <= 0 || max_blocks_per_seq <= 0 || max_blocks_per_seq > kMaxBlocksPerSeq ||
      num_q_heads % num_kv_heads)
    return false;
  const int32_t group = num_q_heads / num_kv_heads;
  if (!supported_group(group)) return false;
  const int32_t max_len = resolved_max_seq_len(max_blocks_per_seq, max_seq_len_hint);
  WorkspaceLayout w;
  w.qmax = decode_qmax(group, max_query_len_hint);
  w.prefetch = decode_prefetch(head_size);
  // Both decode schedules' parameters; the partial results region fits
  // either, so a per-call flag may pick one.
  w.stream_ok = decode_stream_fits(num_seqs, num_kv_heads, head_size);
  w.stream_default = w.stream_ok && decode_stream_default(num_seqs, max_len);
  w.stream_heads = std::min(num_kv_heads, kStreamWaves);
  w.stream_waves = kStreamWaves / w.stream_heads * w.stream_heads;
  w.stream_wgs = decode_stream_wgs();
  w.waves = decode_waves(head_size, w.prefetch);
  w.part_tokens = choose_part_tokens(num_seqs, num_kv_heads, w.waves, max_len);
  w.fused_combine = decode_fused_combine(num_seqs, num_kv_heads, w.part_tokens);
  w.num_parts_max = (max_len + w.part_tokens - 1) / w.part_tokens;
  if (w.num_parts_max > kMaxGridZ) return false;
  const size_t stream_rows = w.stream_ok ? (size_t)w.stream_wgs * 2 * w.qmax * num_q_heads : 0;
  const size_t part_rows =
      w.num_parts_max > 1 ? (size_t)num_seqs * w.num_parts_max * w.qmax * num_q_heads : 0;
  // (share, slot, token, head) / (row, part, token, head)
  const size_t rows = std::max(stream_rows, part_rows);
  const size_t dec_o = rows * head_size, dec_ml = rows * 2;
  w.tile_queries = prefill_tile_queries(group);
  const int32_t bq_b = prefill_split_tile_queries(group);
  // Each row adds at most one partial tile per list: sum ceil(ql/BQ) <= T/BQ + S.
  const int64_t bound_a = ((int64_t)num_tokens + w.tile_queries - 1) / w.tile_queries + num_seqs;
  const int64_t bound_b = std::min<int64_t>(((int64_t)num_tokens + bq_b - 1) / bq_b + num_seqs,
                                            (int64_t)num_seqs * prefill_split_tiles_per_row(group));
  if (bound_a > INT32_MAX || bound_b > INT32_MAX) return false;
  w.bound_a = (int32_t)bound_a;
  w.bound_b = (int32_t)bound_b;
  w.off_ctr = 0;
  w.off_o = round_up((size_t)kCounterSlots * sizeof(int32_t), kAlign);
  w.off_ml = round_up(w.off_o + dec_o * sizeof(float), kAlign);
  w.off_counts = round_up(w.off_ml + dec_ml * sizeof(float), kAlign);
  w.off_tiles_a = w.off_counts + kAlign;
  w.off_tiles_b = round_up(w.off_tiles_a + (size_t)w.bound_a * 2 * sizeof(int32_t), kAlign);
  w.total = round_up(w.off_tiles_b + (size_t)w.bound_b * 2 * sizeof(int32_t), kAlign);
  *out = w;
  return true;
}

}  // namespace pa

extern "C" {

int64_t pa_kv_block_bytes(int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                          int32_t dtype_bytes) {
  if (block_size <= 0 || num_kv_heads <= 0 || head_size <= 0 || dtype_bytes <= 0) return -1;
  return (int64_t)2 * block_size * num_kv_heads * head_size * dtype_bytes;
}

int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                   void* v_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                   int64_t num_blocks, int32_t block_size, void* stream) {
  g_last_error.clear();
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_SHAPE, "pa_cache_write: num_tokens=%d num_kv_heads=%d head_size=%d "
                "num_blocks=%lld out of range", num_tokens, num_kv_heads, head_size,
                (long long)num_blocks);
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "pa_cache_write: block_size %d (only %d is built)",
                block_size, PA_BLOCK_SIZE);
  if (head_size % 8)
    return fail(PA_ERR_UNSUPPORTED, "pa_cache_write: head_size %d is not a multiple of 8",
                head_size);
  if (!k_cache || !v_cache) return fail(PA_ERR_NULL, "pa_cache_write: null cache pointer");
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping) return fail(PA_ERR_NULL, "pa_cache_write: null k/v/slot_mapping");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return fail(PA_ERR_ALIGN, "pa_cache_write: k, v and caches must be 16-byte aligned");
  hipError_t e = pa::launch_cache_write(k, v, slot_mapping, k_cache, v_cache, num_tokens,
                                        num_kv_heads, head_size, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pa_cache_write launch");
  return PA_OK;
}

size_t pa_forward_workspace_bytes(int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_size,
                                  int32_t max_blocks_per_seq, int32_t max_query_len_hint,
                                  int32_t max_seq_len_hint) {
  pa::WorkspaceLayout w;
  if (!pa::plan_workspace(num_tokens, num_seqs, num_q_heads, num_kv_heads, head_size,
                          max_blocks_per_seq, max_query_len_hint, max_seq_len_hint, &w))
    return 0;
  return w.total;
}

int pa_forward(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* seq_lens,
               const int32_t* query_start_loc, float scale, void* out, int32_t num_tokens,
               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
               int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
               int32_t max_query_len_hint, int32_t max_seq_len_hint, void* workspace,
               size_t workspace_bytes, void* stream) {
  return pa_forward_ex(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, out,
                       num_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                       max_blocks_per_seq, num_blocks, max_query_len_hint, max_seq_len_hint,
                       workspace, workspace_bytes, 0u, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// pa_write_and_forward_noalloc: the same call with the library's own scratch
// ---------------------------------------------------------------------------

namespace {

// The workspace of pa_write_and_forward_noalloc: one array per device (each
// device that runs the call holds its own copy until the process ends). In
// host code `scratch` names a host-side stand-in, not device memory: host
// code uses only the address hipGetSymbolAddress gives for the current
// device, kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// Zero fill of 32-bit words by a kernel (capture-safe, unlike a memset node).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The current device's scratch address. The first call on a device looks it
// up (the device must be current) and clears the arrival-counter region on
// `stream`, ahead of the forward launches enqueued after it; every later
// call leaves that region zero.
int device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "pa_write_and_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "pa_write_and_forward_noalloc: device %d (at most %d)", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "pa_write_and_forward_noalloc: hipGetSymbolAddress(scratch)");
    const int64_t words = PA_WORKSPACE_COUNTER_BYTES / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                       stream, (uint32_t*)p, words);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pa_write_and_forward_noalloc: clearing scratch");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

namespace {

// The second stream of a device on which a mixed batch's prefill launches
// run beside its decode launch, with the events that fork it from and join
// it back to the caller's stream. Made on the first mixed call on the device
// (default priority, non-blocking); kept until the process ends. Calls hold
// g_side_mu from the fork to the join, so calls from several host threads
// take turns on it.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// The current device's side stream (g_side_mu held), or nullptr when it
// cannot be had, or when the caller's stream `st` belongs to another device
// (the call then runs its parts one after the other on `st`).
SideStream* side_stream_locked(hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (st) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(st, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    if (sdev != dev) return nullptr;
  }
  SideStream& sd = g_side[dev];
  if (!sd.s) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      if (j) (void)hipEventDestroy(j);
      if (f) (void)hipEventDestroy(f);
      if (s) (void)hipStreamDestroy(s);
      return nullptr;
    }
    sd.s = s;
    sd.fork = f;
    sd.join = j;
  }
  return &sd;
}

// True when `st` is being captured into a graph (or its state cannot be
// read): such calls keep every launch on `st`.
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return cs != hipStreamCaptureStatusNone;
}

// The step's KV write when it travels with the forward (pa_write_and_forward,
// pa_write_and_forward_shared_prefix).
struct WriteArgs {
  const void* k;
  const void* v;
  const int64_t* slot_mapping;
  void* k_cache;
  void* v_cache;
};

// pa_forward_ex, optionally preceded by the step's KV write (wr): fused into
// the decode launch when every row is a decode row (max_query_len_hint == 1),
// the rows take the partitioned schedule and its waves fit the fused
// kernel's bound; into the tile planner's launch when the batch has prefill
// rows; else a cache-write launch first.
int forward_impl(const WriteArgs* wr, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_table, const int32_t* seq_lens,
                 const int32_t* query_start_loc, float scale, void* out, int32_t num_tokens,
                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                 int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                 int32_t max_query_len_hint, int32_t max_seq_len_hint, void* workspace,
                 size_t workspace_bytes, uint32_t flags, void* stream,
                 bool static_scratch = false) {
  const uint32_t known = PA_FORWARD_SHARED_BLOCKS | PA_FORWARD_DECODE_EVEN_SHARES |
                         PA_FORWARD_DECODE_PARTITIONED | PA_FORWARD_SERIAL;
  if (flags & ~known)
    return fail(PA_ERR_UNSUPPORTED, "pa_forward_ex: unknown flags 0x%x", flags);
  if ((flags & PA_FORWARD_DECODE_EVEN_SHARES) && (flags & PA_FORWARD_DECODE_PARTITIONED))
    return fail(PA_ERR_UNSUPPORTED, "pa_forward_ex: both decode schedule flags set");
  if (num_tokens < 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PA_ERR_SHAPE, "pa_forward: a size is out of range (T=%d S=%d Hq=%d Hkv=%d D=%d "
                "MB=%d NB=%lld)", num_tokens, num_seqs, num_q_heads, num_kv_heads, head_size,
                max_blocks_per_seq, (long long)num_blocks);
  if (num_q_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "pa_forward: num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (num_tokens > 0 && num_seqs == 0)
    return fail(PA_ERR_SHAPE, "pa_forward: %d tokens but no sequences", num_tokens);
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: block_size %d (only %d is built)", block_size,
                PA_BLOCK_SIZE);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: head_size %d (built: 64, 128)", head_size);
  const int32_t group = num_q_heads / num_kv_heads;
  if (!supported_group(group))
    return fail(PA_ERR_UNSUPPORTED, "pa_forward: %d query heads per KV head (built: 1, 2, 4, 8, "
                "16)", group);
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(PA_ERR_SHAPE, "pa_forward: scale is not finite");
  if (num_tokens == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !query_start_loc || !out)
    return fail(PA_ERR_NULL, "pa_forward: null pointer argument");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(query_start_loc, 4))
    return fail(PA_ERR_ALIGN, "pa_forward: q, caches and out must be 16-byte aligned");
  pa::WorkspaceLayout w;
  if (!pa::plan_workspace(num_tokens, num_seqs, num_q_heads, num_kv_heads, head_size,
                          max_blocks_per_seq, max_query_len_hint, max_seq_len_hint, &w))
    return fail(PA_ERR_SHAPE, "pa_forward: cannot plan the workspace");
  if (static_scratch) {
    // pa_write_and_forward_noalloc: the library's fixed array is the workspace
    if (w.total > kScratchBytes)
      return fail(PA_ERR_WORKSPACE, "pa_write_and_forward_noalloc: these sizes need %zu bytes "
                  "of scratch; its fixed size is %zu bytes (use pa_write_and_forward with a "
                  "workspace)", w.total, kScratchBytes);
    const int rc = device_scratch((hipStream_t)stream, &workspace);
    if (rc != PA_OK) return rc;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < w.total)
    return fail(PA_ERR_WORKSPACE, "pa_forward: workspace of %zu bytes, %zu needed",
                workspace ? workspace_bytes : (size_t)0, w.total);
  if (!aligned(workspace, 16))
    return fail(PA_ERR_ALIGN, "pa_forward: workspace must be 16-byte aligned");

  pa::ForwardArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.out = out;
  a.scale = scale;
  a.num_tokens = num_tokens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = resolved_max_seq_len(max_blocks_per_seq, max_seq_len_hint);
  a.max_query_len = max_query_len_hint > 0 ? std::min(max_query_len_hint, num_tokens)
                                           : num_tokens;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;

  pa::DecodePlan dp;
  dp.stream = (flags & PA_FORWARD_DECODE_EVEN_SHARES)   ? w.stream_ok
              : (flags & PA_FORWARD_DECODE_PARTITIONED) ? false
                                                        : w.stream_default;
  dp.qmax = w.qmax;
  const bool fused = wr && max_query_len_hint == 1 && !dp.stream &&
                     w.waves <= pa::decode_max_waves(head_size, w.prefetch, true);

  // A mixed batch on even shares with enough prefill tokens (num_tokens -
  // num_seqs of them at least) runs its prefill tiles on the side stream,
  // forked after the cache write and the tile planner and joined before the
  // call returns; not under graph capture, and not for the no-allocation
  // entry point (the side stream is made on first use).
  const bool has_prefill = a.max_query_len > w.qmax;
  // A small batch with prefill rows in which no row is longer than the
  // few-key tiles' bound (list A stays empty) runs every row, the
  // single-token ones too, as few-key tiles: the planner and one tile
  // launch, no decode launch. Small: at most kShortBatchMaxTasks (row, KV
  // head) pairs, one tile task per workgroup of the few-key grid; with more,
  // each decode row's tile costs more than the decode launch saves (the
  // decode launch and the tiles against all rows as tiles, D 128 and 8 KV
  // heads: 16 rows 19.5 against 15.0 us, 64 rows 22.3 against 23.0, 256
  // rows 38.1 against 61.5). Not when a flag names the decode schedule;
  // PA_SHORT_BATCH_TILES=0 turns it off (for comparisons).
  const bool all_rows = has_prefill && a.max_seq_len <= pa::prefill_split_keys() &&
                        (int64_t)num_seqs * num_kv_heads <= kShortBatchMaxTasks &&
                        !(flags &
                          (PA_FORWARD_DECODE_EVEN_SHARES | PA_FORWARD_DECODE_PARTITIONED)) &&
                        short_batch_tiles_enabled();
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  SideStream* side = nullptr;
  if (has_prefill && !all_rows && dp.stream && !static_scratch && !(flags & PA_FORWARD_SERIAL) &&
      mixed_overlap_enabled() && (int64_t)num_tokens - num_seqs >= kOverlapMinPrefillTokens &&
      !capturing(st)) {
    side_lock.lock();
    side = side_stream_locked(st);
    if (!side) side_lock.unlock();
  }
  // The new tokens' write (unless the decode launch makes it) and the
  // planner run on the caller's stream (the planner is one workgroup: beside
  // the decode launch it would wait behind the decode's loads), in one
  // launch when both are needed; then the fork.
  pa::PrefillPlan pp{};
  if (has_prefill) {
    pp.tile_queries = w.tile_queries;
    pp.split_tile_queries = pa::prefill_split_tile_queries(num_q_heads / num_kv_heads);
    const int64_t by_hint_a =
        (int64_t)num_seqs * (((int64_t)a.max_query_len + w.tile_queries - 1) / w.tile_queries);
    const int64_t by_hint_b =
        (int64_t)num_seqs *
        (((int64_t)a.max_query_len + pp.split_tile_queries - 1) / pp.split_tile_queries);
    pp.bound_a = (int32_t)std::min<int64_t>(w.bound_a, by_hint_a);
    pp.bound_b = (int32_t)std::min<int64_t>(w.bound_b, by_hint_b);
    pp.tiles_a = (int32_t*)(ws + w.off_tiles_a);
    pp.tiles_b = (int32_t*)(ws + w.off_tiles_b);
    pp.counts = (int32_t*)(ws + w.off_counts);
    // no tile sees more keys than the longest row has: list A stays empty
    if (a.max_seq_len <= pa::prefill_split_keys()) pp.bound_a = 0;
    pp.all_rows = all_rows;
  }
  if (wr && !fused && has_prefill) {
    hipError_t e = pa::launch_write_and_plan(a, pp, wr->k, wr->v, wr->slot_mapping, wr->k_cache,
                                             wr->v_cache, st);
    if (e != hipSuccess) return hip_fail(e, "pa_write_and_forward write and planner launch");
  } else {
    if (wr && !fused) {
      hipError_t e = pa::launch_cache_write(wr->k, wr->v, wr->slot_mapping, wr->k_cache,
                                            wr->v_cache, num_tokens, num_kv_heads, head_size, st);
      if (e != hipSuccess) return hip_fail(e, "pa_write_and_forward cache write launch");
    }
    if (has_prefill) {
      hipError_t e = pa::launch_prefill_plan(a, pp, st);
      if (e != hipSuccess) return hip_fail(e, "pa_forward prefill planner launch");
    }
  }
  hipStream_t pst = st;  // the prefill tiles' stream
  if (side) {
    hipError_t e = hipEventRecord(side->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return hip_fail(e, "pa_forward: forking the prefill stream");
    pst = side->s;
  }
  // Joins the side stream back into the caller's stream (every return after
  // the fork passes through it, so no launch is left unordered).
  auto join = [&](int rc) {
    if (!side) return rc;
    hipError_t e = hipEventRecord(side->join, side->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, side->join, 0);
    if (e != hipSuccess && rc == PA_OK) return hip_fail(e, "pa_forward: joining the prefill stream");
    return rc;
  };
  // With the side stream, its prefill tiles are the longer of the two
  // parts: the short list (tiles that see few keys) follows the decode on
  // the caller's stream instead of the long list on the side stream.
  pa::PrefillPlan pp_side = pp, pp_after = pp;
  if (side) pp_side.bound_b = 0;
  pp_after.bound_a = 0;
  if (has_prefill) {
    hipError_t e = pa::launch_prefill_tiles(a, pp_side, pst);
    if (e != hipSuccess) return join(hip_fail(e, "pa_forward prefill launch"));
  }
  if (all_rows) return join(PA_OK);
  dp.stream_wgs = side ? std::min(w.stream_wgs, mixed_decode_wgs()) : w.stream_wgs;
  dp.stream_heads = w.stream_heads;
  dp.part_tokens = w.part_tokens;
  dp.num_parts_max = w.num_parts_max;
  dp.prefetch = w.prefetch;
  dp.waves = dp.stream ? w.stream_waves : w.waves;
  dp.heads_per_wg = 1;
  dp.stream_v = !(flags & PA_FORWARD_SHARED_BLOCKS);
  dp.ws_o = (float*)(ws + w.off_o);
  dp.ws_ml = (float*)(ws + w.off_ml);
  dp.counters = (int32_t*)(ws + w.off_ctr);
  dp.fused_combine = !dp.stream && w.fused_combine;
  dp.tok_base = 0;
  dp.part_base = 0;
  dp.fused_write = fused;
  dp.knew = fused ? wr->k : nullptr;
  dp.vnew = fused ? wr->v : nullptr;
  dp.slot_mapping = fused ? wr->slot_mapping : nullptr;
  dp.k_cache_w = fused ? wr->k_cache : nullptr;
  dp.v_cache_w = fused ? wr->v_cache : nullptr;
  hipError_t e = pa::launch_decode(a, dp, st);
  if (e != hipSuccess) return join(hip_fail(e, "pa_forward decode launch"));
  if (has_prefill && side) {
    e = pa::launch_prefill_tiles(a, pp_after, st);
    if (e != hipSuccess) return join(hip_fail(e, "pa_forward prefill launch"));
  }
  return join(PA_OK);
}

// pa_write_and_forward with a caller's workspace, or with the library's
// fixed array (static_scratch: pa_write_and_forward_noalloc).
int write_and_forward_impl(const void* k, const void* v, const int64_t* slot_mapping,
                           void* k_cache, void* v_cache, const void* q,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* query_start_loc, float scale, void* out,
                           int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks,
                           int32_t max_query_len_hint, int32_t max_seq_len_hint, void* workspace,
                           size_t workspace_bytes, uint32_t flags, void* stream,
                           bool static_scratch) {
  if (num_tokens > 0) {
    if (!k || !v || !slot_mapping || !k_cache || !v_cache)
      return fail(PA_ERR_NULL, "pa_write_and_forward: null k/v/slot_mapping/cache");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8))
      return fail(PA_ERR_ALIGN, "pa_write_and_forward: k and v must be 16-byte aligned");
  }
  const WriteArgs wr{k, v, slot_mapping, k_cache, v_cache};
  return forward_impl(&wr, q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale,
                      out, num_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                      max_blocks_per_seq, num_blocks, max_query_len_hint, max_seq_len_hint,
                      workspace, workspace_bytes, flags, stream, static_scratch);
}

}  // namespace

extern "C" {

int pa_forward_ex(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* seq_lens,
                  const int32_t* query_start_loc, float scale, void* out, int32_t num_tokens,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                  int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                  int32_t max_query_len_hint, int32_t max_seq_len_hint, void* workspace,
                  size_t workspace_bytes, uint32_t flags, void* stream) {
  g_last_error.clear();
  return forward_impl(nullptr, q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale,
                      out, num_tokens, num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                      max_blocks_per_seq, num_blocks, max_query_len_hint, max_seq_len_hint,
                      workspace, workspace_bytes, flags, stream);
}

int pa_write_and_forward(const void* k, const void* v, const int64_t* slot_mapping,
                         void* k_cache, void* v_cache, const void* q, const int32_t* block_table,
                         const int32_t* seq_lens, const int32_t* query_start_loc, float scale,
                         void* out, int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks,
                         int32_t max_query_len_hint, int32_t max_seq_len_hint, void* workspace,
                         size_t workspace_bytes, uint32_t flags, void* stream) {
  g_last_error.clear();
  return write_and_forward_impl(k, v, slot_mapping, k_cache, v_cache, q, block_table, seq_lens,
                                query_start_loc, scale, out, num_tokens, num_seqs, num_q_heads,
                                num_kv_heads, head_size, block_size, max_blocks_per_seq,
                                num_blocks, max_query_len_hint, max_seq_len_hint, workspace,
                                workspace_bytes, flags, stream, false);
}

// The same call with the library's fixed scratch array as the workspace.
int pa_write_and_forward_noalloc(const void* k, const void* v, const int64_t* slot_mapping,
                                 void* k_cache, void* v_cache, const void* q,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* query_start_loc, float scale, void* out,
                                 int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                 int32_t max_blocks_per_seq, int64_t num_blocks,
                                 int32_t max_query_len_hint, int32_t max_seq_len_hint,
                                 uint32_t flags, void* stream) {
  g_last_error.clear();
  return write_and_forward_impl(k, v, slot_mapping, k_cache, v_cache, q, block_table, seq_lens,
                                query_start_loc, scale, out, num_tokens, num_seqs, num_q_heads,
                                num_kv_heads, head_size, block_size, max_blocks_per_seq,
                                num_blocks, max_query_len_hint, max_seq_len_hint, nullptr, 0,
                                flags, stream, true);
}

}  // extern "C"

namespace {

// Shared-prefix decode: the prefix pass covers the first prefix_blocks
// blocks of every row in chunks; each row's remaining keys run on the
// partitioned decode schedule; the combine merges both.
struct PrefixLayout {
  int32_t chunks, chunk_keys, prefix_keys, waves, prefetch, heads_per_wg, part_tokens,
      suffix_parts, num_parts_max;
  size_t off_o, off_ml, total;
};
// Prefix workgroups aimed for: one per CU; chunks of at least 512 keys.
constexpr int32_t kPrefixMinChunkKeys = 512;

bool plan_prefix(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                 int32_t max_blocks_per_seq, int32_t prefix_blocks, int32_t max_seq_len_hint,
                 PrefixLayout* out) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      max_blocks_per_seq <= 0 || max_blocks_per_seq > kMaxBlocksPerSeq ||
      num_q_heads % num_kv_heads || prefix_blocks <= 0 || prefix_blocks >= max_blocks_per_seq)
    return false;
  const int32_t group = num_q_heads / num_kv_heads;
  if (!supported_group(group)) return false;
  const int32_t max_len = resolved_max_seq_len(max_blocks_per_seq, max_seq_len_hint);
  PrefixLayout p;
  p.prefix_keys = prefix_blocks * PA_BLOCK_SIZE;
  if (max_len <= p.prefix_keys) return false;
  const int32_t rows = pa::prefix_tile_rows(group);
  const int64_t row_tiles = (num_seqs + rows - 1) / rows;
  const int64_t want = std::max<int64_t>(1, (kComputeUnits + row_tiles * num_kv_heads - 1) /
                                                (row_tiles * num_kv_heads));
  const int64_t most = std::max<int64_t>(1, (p.prefix_keys + kPrefixMinChunkKeys - 1) /
                                                kPrefixMinChunkKeys);
  const int64_t chunks = std::min(want, most);
  p.chunk_keys = (int32_t)(((p.prefix_keys + chunks - 1) / chunks + 63) / 64 * 64);
  p.chunks = (p.prefix_keys + p.chunk_keys - 1) / p.chunk_keys;
  p.prefetch = decode_prefetch(head_size);
  // The rows' own blocks after the prefix are few per row: one workgroup
  // per row holds all its KV heads (the largest divisor of Hkv that fits,
  // one wave each), instead of a workgroup per (row, KV head) whose waves
  // would each stream one or two blocks. PA_PREFIX_SUFFIX_HEADS=1 restores
  // a workgroup per KV head with the usual waves (for comparisons).
  static const int one_head = env_int("PA_PREFIX_SUFFIX_HEADS", 0, 1, 0);
  if (one_head) {
    p.heads_per_wg = 1;
    p.waves = decode_waves(head_size, p.prefetch);
  } else {
    const int32_t maxw = std::max(1, pa::decode_max_waves(head_size, p.prefetch));
    int32_t hg = std::min(num_kv_heads, maxw);
    while (num_kv_heads % hg) --hg;
    p.heads_per_wg = hg;
    p.waves = hg;
  }
  const int32_t suffix_len = max_len - p.prefix_keys;
  p.part_tokens = choose_part_tokens(num_seqs, num_kv_heads / p.heads_per_wg,
                                     p.waves / p.heads_per_wg, suffix_len);
  p.suffix_parts = (suffix_len + p.part_tokens - 1) / p.part_tokens;
  p.num_parts_max = p.chunks + p.suffix_parts;
  if (p.suffix_parts > kMaxGridZ) return false;
  const size_t prow = (size_t)num_seqs * p.num_parts_max * num_q_heads;
  p.off_o = round_up((size_t)kCounterSlots * sizeof(int32_t), kAlign);
  p.off_ml = round_up(p.off_o + prow * head_size * sizeof(float), kAlign);
  p.total = round_up(p.off_ml + prow * 2 * sizeof(float), kAlign);
  *out = p;
  return true;
}


// pa_forward_shared_prefix, with the step's KV write in the prefix launch
// when wr is given (pa_write_and_forward_shared_prefix; fn names the entry
// point in errors).
int shared_prefix_impl(const WriteArgs* wr, const char* fn, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* query_start_loc, float scale, void* out, int32_t num_seqs,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                       int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                       int32_t prefix_blocks, int32_t max_seq_len_hint, void* workspace,
                       size_t workspace_bytes, uint32_t flags, void* stream) {
  if (flags & ~PA_FORWARD_SHARED_BLOCKS)
    return fail(PA_ERR_UNSUPPORTED, "%s: unsupported flags 0x%x", fn, flags);
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PA_ERR_SHAPE, "%s: a size is out of range", fn);
  if (num_q_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", fn,
                num_q_heads, num_kv_heads);
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only %d is built)", fn, block_size,
                PA_BLOCK_SIZE);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_size %d (built: 64, 128)", fn, head_size);
  if (!supported_group(num_q_heads / num_kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per KV head", fn,
                num_q_heads / num_kv_heads);
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(PA_ERR_SHAPE, "%s: scale is not finite", fn);
  const int32_t max_len = resolved_max_seq_len(max_blocks_per_seq, max_seq_len_hint);
  if (prefix_blocks <= 0 || (int64_t)prefix_blocks * PA_BLOCK_SIZE >= max_len)
    return fail(PA_ERR_SHAPE, "%s: prefix_blocks %d must be >= 1 and leave every row at least "
                "one key past it (max_seq_len %d)", fn, prefix_blocks, max_len);
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !query_start_loc || !out)
    return fail(PA_ERR_NULL, "%s: null pointer argument", fn);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(query_start_loc, 4))
    return fail(PA_ERR_ALIGN, "%s: q, caches and out must be 16-byte aligned", fn);
  PrefixLayout pl;
  if (!plan_prefix(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq,
                   prefix_blocks, max_seq_len_hint, &pl))
    return fail(PA_ERR_SHAPE, "%s: cannot plan the workspace", fn);
  if (!workspace || workspace_bytes < pl.total)
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, pl.total);
  if (!aligned(workspace, 16))
    return fail(PA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);

  pa::ForwardArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.out = out;
  a.scale = scale;
  a.num_tokens = num_seqs;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = max_len;
  a.max_query_len = 1;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;

  pa::PrefixPlan pp = {};
  pp.chunks = pl.chunks;
  pp.chunk_keys = pl.chunk_keys;
  pp.prefix_keys = pl.prefix_keys;
  pp.num_parts_max = pl.num_parts_max;
  pp.ws_o = (float*)(ws + pl.off_o);
  pp.ws_ml = (float*)(ws + pl.off_ml);
  if (wr) {
    pp.write_tokens = num_seqs;
    pp.knew = wr->k;
    pp.vnew = wr->v;
    pp.slot_mapping = wr->slot_mapping;
    pp.k_cache_w = wr->k_cache;
    pp.v_cache_w = wr->v_cache;
  }
  hipError_t e = pa::launch_prefix(a, pp, st);
  if (e != hipSuccess) return hip_fail(e, "shared-prefix prefix launch");

  pa::DecodePlan dp = {};
  dp.stream = false;
  dp.part_tokens = pl.part_tokens;
  dp.num_parts_max = pl.num_parts_max;
  dp.waves = pl.waves;
  dp.heads_per_wg = pl.heads_per_wg;
  dp.prefetch = pl.prefetch;
  dp.stream_v = !(flags & PA_FORWARD_SHARED_BLOCKS);
  dp.ws_o = pp.ws_o;
  dp.ws_ml = pp.ws_ml;
  dp.tok_base = pl.prefix_keys;
  dp.part_base = pl.chunks;
  dp.qmax = 1;
  // The last workgroup of each (row, KV head) merges the prefix chunks'
  // partials with its own row's, through the counters at the start of the
  // workspace (a row whose own keys fit one partition merges them directly);
  // rows whose own keys are split into partitions longer than the in-kernel
  // merge takes (decode_fused_combine) leave every partial to the combine
  // launch.
  dp.counters = (int32_t*)ws;
  dp.fused_combine = decode_fused_combine(num_seqs, num_kv_heads, pl.part_tokens);
  e = pa::launch_decode(a, dp, st);
  if (e != hipSuccess) return hip_fail(e, "shared-prefix decode launch");
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_size,
                                        int32_t max_blocks_per_seq, int32_t prefix_blocks,
                                        int32_t max_seq_len_hint) {
  PrefixLayout p;
  if (!plan_prefix(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq,
                   prefix_blocks, max_seq_len_hint, &p))
    return 0;
  return p.total;
}

int pa_forward_shared_prefix(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* query_start_loc, float scale, void* out,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_blocks, int32_t prefix_blocks, int32_t max_seq_len_hint,
                             void* workspace, size_t workspace_bytes, uint32_t flags,
                             void* stream) {
  g_last_error.clear();
  return shared_prefix_impl(nullptr, "pa_forward_shared_prefix", q, k_cache, v_cache,
                            block_table, seq_lens, query_start_loc, scale, out, num_seqs,
                            num_q_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                            num_blocks, prefix_blocks, max_seq_len_hint, workspace,
                            workspace_bytes, flags, stream);
}

int pa_write_and_forward_shared_prefix(const void* k, const void* v, const int64_t* slot_mapping,
                                       void* k_cache, void* v_cache, const void* q,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* query_start_loc, float scale, void* out,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_size,
                                       int32_t block_size, int32_t max_blocks_per_seq,
                                       int64_t num_blocks, int32_t prefix_blocks,
                                       int32_t max_seq_len_hint, void* workspace,
                                       size_t workspace_bytes, uint32_t flags, void* stream) {
  g_last_error.clear();
  if (num_seqs > 0) {
    if (!k || !v || !slot_mapping || !k_cache || !v_cache)
      return fail(PA_ERR_NULL, "pa_write_and_forward_shared_prefix: null k/v/slot_mapping/cache");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8))
      return fail(PA_ERR_ALIGN, "pa_write_and_forward_shared_prefix: k and v must be 16-byte "
                  "aligned");
  }
  const WriteArgs wr{k, v, slot_mapping, k_cache, v_cache};
  return shared_prefix_impl(&wr, "pa_write_and_forward_shared_prefix", q, k_cache, v_cache,
                            block_table, seq_lens, query_start_loc, scale, out, num_seqs,
                            num_q_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                            num_blocks, prefix_blocks, max_seq_len_hint, workspace,
                            workspace_bytes, flags, stream);
}

int pa_probe_block_read(const void* k_cache, const void* v_cache, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                        int32_t head_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                        int32_t waves, int32_t blocks_per_workgroup, uint32_t* sink,
                        void* stream) {
  g_last_error.clear();
  if (num_seqs <= 0 || num_kv_heads <= 0 || head_size <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || waves < 1 || waves > 16 || blocks_per_workgroup < 1 ||
      (max_blocks_per_seq + (int64_t)blocks_per_workgroup - 1) / blocks_per_workgroup > 65535)
    return fail(PA_ERR_SHAPE, "pa_probe_block_read: a size is out of range");
  if ((head_size * num_kv_heads) % 8 || (int64_t)16 * num_kv_heads * head_size / 8 > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "pa_probe_block_read: unsupported block shape");
  if (!k_cache || !v_cache || !block_table || !seq_lens || !sink)
    return fail(PA_ERR_NULL, "pa_probe_block_read: null pointer argument");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(sink, 4))
    return fail(PA_ERR_ALIGN, "pa_probe_block_read: caches must be 16-byte aligned");
  hipError_t e = pa::launch_block_read_probe(k_cache, v_cache, block_table, seq_lens, num_seqs,
                                             num_kv_heads, head_size, max_blocks_per_seq,
                                             num_blocks, waves, blocks_per_workgroup, sink,
                                             (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pa_probe_block_read launch");
  return PA_OK;
}

int pa_validate_inputs(const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* query_start_loc, const int64_t* slot_mapping,
                       int32_t num_tokens, int32_t num_seqs, int32_t max_blocks_per_seq,
                       int64_t num_blocks, int32_t block_size, int32_t num_write_tokens,
                       int32_t max_query_len_hint, int32_t max_seq_len_hint, void* stream) {
  g_last_error.clear();
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      num_write_tokens < 0)
    return fail(PA_ERR_SHAPE, "pa_validate_inputs: a size is out of range");
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "pa_validate_inputs: block_size %d", block_size);
  if (!block_table || !seq_lens || !query_start_loc || (num_write_tokens > 0 && !slot_mapping))
    return fail(PA_ERR_NULL, "pa_validate_inputs: null pointer argument");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "pa_validate_inputs sync");
  std::vector<int32_t> qsl(num_seqs + 1), lens(num_seqs),
      table((size_t)num_seqs * max_blocks_per_seq);
  std::vector<int64_t> slots(num_write_tokens);
  if ((e = hipMemcpy(qsl.data(), query_start_loc, qsl.size() * 4, hipMemcpyDeviceToHost)) ||
      (num_seqs && (e = hipMemcpy(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost))) ||
      (num_seqs && (e = hipMemcpy(table.data(), block_table, table.size() * 4,
                                  hipMemcpyDeviceToHost))) ||
      (num_write_tokens && (e = hipMemcpy(slots.data(), slot_mapping, slots.size() * 8,
                                          hipMemcpyDeviceToHost))))
    return hip_fail(e, "pa_validate_inputs copy");
  if (qsl[0] != 0) return fail(PA_ERR_INVALID_DATA, "query_start_loc[0] = %d, not 0", qsl[0]);
  if (qsl[num_seqs] != num_tokens)
    return fail(PA_ERR_INVALID_DATA, "query_start_loc[S] = %d, not num_tokens = %d",
                qsl[num_seqs], num_tokens);
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  int32_t max_q = 0, max_l = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t ql = qsl[s + 1] - qsl[s];
    if (ql < 0) return fail(PA_ERR_INVALID_DATA, "query_start_loc decreases at sequence %d", s);
    if (lens[s] < ql || lens[s] > cap)
      return fail(PA_ERR_INVALID_DATA, "sequence %d: seq_len %d outside [q_len %d, %lld]", s,
                  lens[s], ql, (long long)cap);
    max_q = std::max(max_q, ql);
    max_l = std::max(max_l, lens[s]);
    const int32_t nb = (lens[s] + block_size - 1) / block_size;
    for (int32_t b = 0; b < nb; ++b) {
      const int32_t id = table[(size_t)s * max_blocks_per_seq + b];
      if (id < 0 || id >= num_blocks)
        return fail(PA_ERR_INVALID_DATA, "sequence %d: block_table[%d] = %d outside [0, %lld)", s,
                    b, id, (long long)num_blocks);
    }
  }
  if (max_query_len_hint > 0 && max_query_len_hint < max_q)
    return fail(PA_ERR_INVALID_DATA, "max_query_len_hint %d < longest query %d",
                max_query_len_hint, max_q);
  if (max_seq_len_hint > 0 && max_seq_len_hint < max_l)
    return fail(PA_ERR_INVALID_DATA, "max_seq_len_hint %d < longest sequence %d",
                max_seq_len_hint, max_l);
  std::unordered_set<int64_t> seen;
  for (int32_t t = 0; t < num_write_tokens; ++t) {
    const int64_t sl = slots[t];
    if (sl < 0) continue;
    if (sl >= num_blocks * block_size)
      return fail(PA_ERR_INVALID_DATA, "slot_mapping[%d] = %lld outside the pool", t,
                  (long long)sl);
    if (!seen.insert(sl).second)
      return fail(PA_ERR_INVALID_DATA, "slot %lld is written twice", (long long)sl);
  }
  return PA_OK;
}

int pa_validate_shared_prefix(const int32_t* block_table, const int32_t* seq_lens,
                              const int64_t* slot_mapping, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t prefix_blocks, void* stream) {
  g_last_error.clear();
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_blocks_per_seq > kMaxBlocksPerSeq ||
      prefix_blocks <= 0 || prefix_blocks >= max_blocks_per_seq)
    return fail(PA_ERR_SHAPE, "pa_validate_shared_prefix: a size is out of range");
  if (!block_table || !seq_lens)
    return fail(PA_ERR_NULL, "pa_validate_shared_prefix: null pointer argument");
  if (num_seqs == 0) return PA_OK;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pa_validate_shared_prefix sync");
  std::vector<int32_t> lens(num_seqs), table((size_t)num_seqs * max_blocks_per_seq);
  std::vector<int64_t> slots(slot_mapping ? num_seqs : 0);
  if ((e = hipMemcpy(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost)) ||
      (e = hipMemcpy(table.data(), block_table, table.size() * 4, hipMemcpyDeviceToHost)) ||
      (slot_mapping &&
       (e = hipMemcpy(slots.data(), slot_mapping, slots.size() * 8, hipMemcpyDeviceToHost))))
    return hip_fail(e, "pa_validate_shared_prefix copy");
  const int64_t prefix_keys = (int64_t)prefix_blocks * PA_BLOCK_SIZE;
  const int64_t cap = (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE;
  std::unordered_set<int64_t> prefix(table.begin(), table.begin() + prefix_blocks);
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (lens[s] <= prefix_keys || lens[s] > cap)
      return fail(PA_ERR_INVALID_DATA, "sequence %d: seq_len %d outside (%lld, %lld]", s,
                  lens[s], (long long)prefix_keys, (long long)cap);
    for (int32_t b = 0; b < prefix_blocks; ++b)
      if (table[(size_t)s * max_blocks_per_seq + b] != table[b])
        return fail(PA_ERR_INVALID_DATA, "sequence %d: block_table[%d] = %d, row 0 has %d", s,
                    b, table[(size_t)s * max_blocks_per_seq + b], table[b]);
    if (slot_mapping && slots[s] >= 0 && prefix.count(slots[s] / PA_BLOCK_SIZE))
      return fail(PA_ERR_INVALID_DATA, "sequence %d: slot %lld lies in a prefix block", s,
                  (long long)slots[s]);
  }
  return PA_OK;
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

const char* pa_version(void) { return "paged_attention_kv_amd 0.2.0 (gfx950)"; }

}  // extern "C"
