// Host-side KV-cache block manager and step planner (contract in
// include/pa_sched.h). Page "Inside vLLM: Anatomy of a High-Throughput LLM
// Inference System": section "Scheduler" (decode-first order, token budget,
// allocate_slots: blocks needed, availability check, preemption, blocks
// taken from the left of the free queue), section "Chunked prefill" (new
// tokens per step capped by long_prefill_token_threshold), section "Prefix
// Caching" (per-block hashes chained through the previous block's hash, the
// hash -> block map, reference counts, lazy invalidation when a cached block
// is handed out again) and section "Run forward pass" (slot_mapping, block
// tables, flattened rows).
#include <stdint.h>

#include <algorithm>
#include <array>
#include <deque>
#include <memory>
#include <unordered_map>
#include <vector>

#include "errors.h"
#include "pa.h"
#include "pa_sched.h"

namespace {

constexpr int32_t kBlockTokens = PA_BLOCK_SIZE;

// 64-bit hash of a full block: FNV-1a over the parent hash and the 16 token
// ids, finished with a 64-bit mixer. Lookups check the stored tokens and
// parent, so collisions cost a miss, never a wrong block.
uint64_t block_hash(uint64_t parent, const int32_t* toks) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (v >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  mix(parent);
  for (int i = 0; i < kBlockTokens; ++i) mix((uint32_t)toks[i]);
  h ^= h >> 33;
  h *= 0xff51afd7ed558ccdull;
  h ^= h >> 33;
  return h;
}

struct Block {
  int32_t ref = 0;
  bool hashed = false;  // registered in the hash map under `hash`
  uint64_t hash = 0;
  uint64_t parent = 0;
  std::array<int32_t, kBlockTokens> toks{};
  int32_t prev = -1, next = -1;  // free queue links
  bool in_free = false;
};

class BlockPool {
 public:
  explicit BlockPool(int32_t n) : blocks_(n) {
    for (int32_t b = 0; b < n; ++b) push_back(b);
  }
  int32_t size() const { return (int32_t)blocks_.size(); }
  int64_t num_free() const { return nfree_; }
  size_t num_cached() const { return map_.size(); }
  Block& at(int32_t b) { return blocks_[b]; }
  const Block& at(int32_t b) const { return blocks_[b]; }

  // Leftmost free block, out of the queue with one reference; a hash it
  // still carries is dropped with its map entry (lazy invalidation).
  int32_t take() {
    const int32_t b = head_;
    unlink(b);
    Block& k = blocks_[b];
    if (k.hashed) {
      auto it = map_.find(k.hash);
      if (it != map_.end() && it->second == b) map_.erase(it);
      k.hashed = false;
    }
    k.ref = 1;
    return b;
  }
  // One more reference to a block found in the map; a free one leaves the
  // queue (it keeps its hash).
  void touch(int32_t b) {
    Block& k = blocks_[b];
    if (k.ref == 0) unlink(b);
    ++k.ref;
  }
  void release(int32_t b) {
    Block& k = blocks_[b];
    if (--k.ref == 0) push_back(b);
  }
  // The block holding exactly (parent, toks), or -1.
  int32_t lookup(uint64_t h, uint64_t parent, const int32_t* toks) const {
    auto it = map_.find(h);
    if (it == map_.end()) return -1;
    const Block& k = blocks_[it->second];
    if (k.parent != parent || !std::equal(k.toks.begin(), k.toks.end(), toks)) return -1;
    return it->second;
  }
  // Registers a computed full block (unless the hash is already taken).
  void cache(int32_t b, uint64_t h, uint64_t parent, const int32_t* toks) {
    Block& k = blocks_[b];
    if (k.hashed || map_.count(h)) return;
    k.hashed = true;
    k.hash = h;
    k.parent = parent;
    std::copy(toks, toks + kBlockTokens, k.toks.begin());
    map_.emplace(h, b);
  }

 private:
  void push_back(int32_t b) {
    Block& k = blocks_[b];
    k.prev = tail_;
    k.next = -1;
    if (tail_ >= 0) blocks_[tail_].next = b;
    else head_ = b;
    tail_ = b;
    k.in_free = true;
    ++nfree_;
  }
  void unlink(int32_t b) {
    Block& k = blocks_[b];
    if (k.prev >= 0) blocks_[k.prev].next = k.next;
    else head_ = k.next;
    if (k.next >= 0) blocks_[k.next].prev = k.prev;
    else tail_ = k.prev;
    k.prev = k.next = -1;
    k.in_free = false;
    --nfree_;
  }

  std::vector<Block> blocks_;
  int32_t head_ = -1, tail_ = -1;
  int64_t nfree_ = 0;
  std::unordered_map<uint64_t, int32_t> map_;
};

struct Request {
  int64_t id;
  std::vector<int32_t> tokens;  // prompt, then generated tokens
  int32_t max_new_tokens;
  int32_t generated = 0;
  int32_t computed = 0;         // leading tokens whose K/V are in the cache
  std::vector<int32_t> blocks;
  std::vector<uint64_t> hashes;  // hashes of the full blocks of `tokens`
  int32_t registered = 0;        // leading blocks offered to the map
  bool running = false;
};

struct Row {
  Request* req;
  int32_t start;  // tokens already in the cache
  int32_t count;  // new tokens this step
};

}  // namespace

struct pa_sched {
  BlockPool pool;
  int32_t budget_tokens, max_seqs, threshold;
  bool caching;
  std::unordered_map<int64_t, std::unique_ptr<Request>> live;
  std::deque<Request*> waiting;
  std::vector<Request*> running;  // admission order
  std::vector<Row> rows;
  bool planned = false;
  pa_sched_stats st{};

  pa_sched(int64_t nb, int32_t bt, int32_t ms, int32_t th, bool pc)
      : pool((int32_t)nb), budget_tokens(bt), max_seqs(ms), threshold(th), caching(pc) {}

  // Hashes of every full block of r's known tokens (extends r.hashes).
  void hash_blocks(Request& r) {
    const int32_t full = (int32_t)r.tokens.size() / kBlockTokens;
    for (int32_t k = (int32_t)r.hashes.size(); k < full; ++k) {
      const uint64_t parent = k ? r.hashes[k - 1] : 0;
      r.hashes.push_back(block_hash(parent, r.tokens.data() + (size_t)k * kBlockTokens));
    }
  }

  // Leading blocks of r's tokens found in the map, leaving at least the
  // last token to compute.
  std::vector<int32_t> longest_cache_hit(Request& r) {
    std::vector<int32_t> hit;
    if (!caching) return hit;
    hash_blocks(r);
    const int32_t most = ((int32_t)r.tokens.size() - 1) / kBlockTokens;
    for (int32_t k = 0; k < most && k < (int32_t)r.hashes.size(); ++k) {
      const uint64_t parent = k ? r.hashes[k - 1] : 0;
      const int32_t b = pool.lookup(r.hashes[k], parent, r.tokens.data() + (size_t)k * kBlockTokens);
      if (b < 0) break;
      hit.push_back(b);
    }
    return hit;
  }

  // Blocks for `computed` cached tokens (the hits, if any) plus `count` new
  // ones; false (nothing changed) when the free queue cannot supply them.
  bool allocate_slots(Request& r, int32_t count, const std::vector<int32_t>& hits) {
    const int32_t have = (int32_t)r.blocks.size() + (int32_t)hits.size();
    const int32_t base = hits.empty() ? r.computed : (int32_t)hits.size() * kBlockTokens;
    const int32_t need = (base + count + kBlockTokens - 1) / kBlockTokens - have;
    int64_t hits_free = 0;  // hits sitting in the free queue leave it too
    for (int32_t b : hits) hits_free += pool.at(b).ref == 0;
    if (std::max(need, 0) > pool.num_free() - hits_free) return false;
    for (int32_t b : hits) {
      pool.touch(b);
      r.blocks.push_back(b);
    }
    for (int32_t i = 0; i < need; ++i) r.blocks.push_back(pool.take());
    return true;
  }

  void free_blocks(Request& r) {
    for (auto it = r.blocks.rbegin(); it != r.blocks.rend(); ++it) pool.release(*it);
    r.blocks.clear();
  }

  // Recompute preemption: the request gives back its blocks and waits at the
  // front of the queue; its tokens (prompt and generated) are computed anew.
  void preempt(Request* r) {
    free_blocks(*r);
    r->computed = 0;
    r->registered = 0;
    r->running = false;
    waiting.push_front(r);
    ++st.num_preemptions;
  }

  int32_t cap(int32_t n, int32_t budget) const {
    if (threshold > 0) n = std::min(n, threshold);
    return std::min(n, budget);
  }

  void schedule() {
    rows.clear();
    int32_t budget = budget_tokens;
    // 1. running requests, in admission order (decode rows come first)
    for (size_t i = 0; i < running.size() && budget > 0;) {
      Request* r = running[i];
      const int32_t n = cap((int32_t)r->tokens.size() - r->computed, budget);
      if (n <= 0) {
        ++i;
        continue;
      }
      bool ok = true;
      while (!allocate_slots(*r, n, {})) {
        Request* victim = running.back();
        running.pop_back();
        preempt(victim);
        if (victim == r) {
          ok = false;
          break;
        }
      }
      if (!ok) break;  // r was the last running request and is now waiting
      rows.push_back({r, r->computed, n});
      budget -= n;
      ++i;
    }
    // 2. waiting requests in order, while they fit
    while (!waiting.empty() && budget > 0 && (int32_t)running.size() < max_seqs) {
      Request* r = waiting.front();
      std::vector<int32_t> hits = longest_cache_hit(*r);
      const int32_t start = (int32_t)hits.size() * kBlockTokens;
      const int32_t n = cap((int32_t)r->tokens.size() - start, budget);
      if (!allocate_slots(*r, n, hits)) break;
      waiting.pop_front();
      r->computed = start;
      r->registered = (int32_t)hits.size();
      r->running = true;
      running.push_back(r);
      st.prefix_hit_tokens += start;
      rows.push_back({r, start, n});
      budget -= n;
    }
    planned = true;
    ++st.num_steps;
  }

  void finish(Request* r) {
    free_blocks(*r);
    r->running = false;
    running.erase(std::find(running.begin(), running.end(), r));
    ++st.num_finished;
    live.erase(r->id);
  }

  void update(const int32_t* sampled) {
    std::vector<Request*> done;
    for (size_t i = 0; i < rows.size(); ++i) {
      Request& r = *rows[i].req;
      r.computed = rows[i].start + rows[i].count;
      // full blocks whose keys and values are now written become reusable
      if (caching) {
        hash_blocks(r);
        const int32_t full = r.computed / kBlockTokens;
        for (int32_t k = r.registered; k < full; ++k) {
          const uint64_t parent = k ? r.hashes[k - 1] : 0;
          pool.cache(r.blocks[k], r.hashes[k], parent, r.tokens.data() + (size_t)k * kBlockTokens);
        }
        r.registered = std::max(r.registered, full);
      }
      if (r.computed == (int32_t)r.tokens.size()) {  // the row's last position was computed
        r.tokens.push_back(sampled ? sampled[i] : 0);
        if (++r.generated >= r.max_new_tokens) done.push_back(&r);
      }
    }
    for (Request* r : done) finish(r);
    rows.clear();
    planned = false;
  }
};

extern "C" {

pa_sched* pa_sched_create(int64_t num_blocks, int32_t block_size,
                          int32_t max_num_batched_tokens, int32_t max_num_seqs,
                          int32_t long_prefill_token_threshold, int32_t enable_prefix_caching) {
  pa::clear_error();
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size != kBlockTokens ||
      max_num_batched_tokens <= 0 || max_num_seqs <= 0 ||
      (enable_prefix_caching != 0 && enable_prefix_caching != 1)) {
    pa::record_error(PA_ERR_SHAPE, "pa_sched_create: invalid argument");
    return nullptr;
  }
  return new pa_sched(num_blocks, max_num_batched_tokens, max_num_seqs,
                      long_prefill_token_threshold, enable_prefix_caching == 1);
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int pa_sched_add_request(pa_sched* s, int64_t request_id, const int32_t* prompt,
                         int32_t prompt_len, int32_t max_new_tokens) {
  pa::clear_error();
  if (!s || (!prompt && prompt_len > 0)) return pa::record_error(PA_ERR_NULL, "pa_sched_add_request: null argument");
  if (prompt_len <= 0 || max_new_tokens <= 0)
    return pa::record_error(PA_ERR_SHAPE, "pa_sched_add_request: prompt_len %d, max_new_tokens %d",
                            prompt_len, max_new_tokens);
  if (s->live.count(request_id))
    return pa::record_error(PA_ERR_SHAPE, "pa_sched_add_request: request %lld is live",
                            (long long)request_id);
  auto r = std::make_unique<Request>();
  r->id = request_id;
  r->tokens.assign(prompt, prompt + prompt_len);
  r->max_new_tokens = max_new_tokens;
  s->waiting.push_back(r.get());
  s->live.emplace(request_id, std::move(r));
  return PA_OK;
}

int pa_sched_schedule(pa_sched* s, int32_t* num_seqs, int32_t* num_tokens, int32_t* max_blocks) {
  pa::clear_error();
  if (!s || !num_seqs || !num_tokens || !max_blocks)
    return pa::record_error(PA_ERR_NULL, "pa_sched_schedule: null argument");
  if (s->planned && !s->rows.empty())
    return pa::record_error(PA_ERR_SHAPE, "pa_sched_schedule: the planned step was not updated");
  s->schedule();
  int32_t t = 0, mb = 0;
  for (const Row& row : s->rows) {
    t += row.count;
    mb = std::max(mb, (int32_t)row.req->blocks.size());
  }
  *num_seqs = (int32_t)s->rows.size();
  *num_tokens = t;
  *max_blocks = mb;
  return PA_OK;
}

int pa_sched_step_inputs(const pa_sched* s, int64_t* request_ids, int32_t* query_start_loc,
                         int32_t* seq_lens, int32_t* block_table, int32_t table_cols,
                         int64_t* slot_mapping, int32_t* token_ids, int32_t* positions) {
  pa::clear_error();
  if (!s || !query_start_loc ||
      (!s->rows.empty() && (!request_ids || !seq_lens || !block_table)))
    return pa::record_error(PA_ERR_NULL, "pa_sched_step_inputs: null argument");
  if (!s->planned) return pa::record_error(PA_ERR_SHAPE, "pa_sched_step_inputs: no planned step");
  int32_t t = 0;
  query_start_loc[0] = 0;
  for (size_t i = 0; i < s->rows.size(); ++i) {
    const Row& row = s->rows[i];
    const Request& r = *row.req;
    if ((int32_t)r.blocks.size() > table_cols)
      return pa::record_error(PA_ERR_SHAPE, "pa_sched_step_inputs: table_cols %d < %zu blocks",
                              table_cols, r.blocks.size());
    request_ids[i] = r.id;
    seq_lens[i] = row.start + row.count;
    int32_t* trow = block_table + i * (size_t)table_cols;
    for (int32_t j = 0; j < table_cols; ++j) trow[j] = j < (int32_t)r.blocks.size() ? r.blocks[j] : -1;
    for (int32_t k = 0; k < row.count; ++k, ++t) {
      const int32_t pos = row.start + k;
      if (slot_mapping)
        slot_mapping[t] = (int64_t)r.blocks[pos / kBlockTokens] * kBlockTokens + pos % kBlockTokens;
      if (token_ids) token_ids[t] = r.tokens[pos];
      if (positions) positions[t] = pos;
    }
    query_start_loc[i + 1] = t;
  }
  return PA_OK;
}

int pa_sched_update(pa_sched* s, const int32_t* sampled) {
  pa::clear_error();
  if (!s) return pa::record_error(PA_ERR_NULL, "pa_sched_update: null handle");
  if (!s->planned) return pa::record_error(PA_ERR_SHAPE, "pa_sched_update: no planned step");
  s->update(sampled);
  return PA_OK;
}

int pa_sched_finish_request(pa_sched* s, int64_t request_id) {
  pa::clear_error();
  if (!s) return pa::record_error(PA_ERR_NULL, "pa_sched_finish_request: null handle");
  if (s->planned && !s->rows.empty())
    return pa::record_error(PA_ERR_SHAPE, "pa_sched_finish_request: a planned step is open");
  auto it = s->live.find(request_id);
  if (it == s->live.end())
    return pa::record_error(PA_ERR_SHAPE, "pa_sched_finish_request: unknown request %lld",
                            (long long)request_id);
  Request* r = it->second.get();
  if (r->running) {
    s->finish(r);
  } else {
    s->waiting.erase(std::find(s->waiting.begin(), s->waiting.end(), r));
    s->free_blocks(*r);
    ++s->st.num_finished;
    s->live.erase(it);
  }
  return PA_OK;
}

int pa_sched_get_stats(const pa_sched* s, pa_sched_stats* out) {
  pa::clear_error();
  if (!s || !out) return pa::record_error(PA_ERR_NULL, "pa_sched_get_stats: null argument");
  *out = s->st;
  out->num_free_blocks = s->pool.num_free();
  out->num_cached_blocks = (int64_t)s->pool.num_cached();
  out->num_waiting = (int32_t)s->waiting.size();
  out->num_running = (int32_t)s->running.size();
  return PA_OK;
}

int32_t pa_sched_request_blocks(const pa_sched* s, int64_t request_id, int32_t* blocks,
                                int32_t cap) {
  if (!s) return PA_ERR_NULL;
  auto it = s->live.find(request_id);
  if (it == s->live.end()) return PA_ERR_SHAPE;
  const std::vector<int32_t>& b = it->second->blocks;
  for (int32_t i = 0; i < cap && i < (int32_t)b.size(); ++i) blocks[i] = b[i];
  return (int32_t)b.size();
}

int32_t pa_sched_request_computed(const pa_sched* s, int64_t request_id) {
  if (!s) return PA_ERR_NULL;
  auto it = s->live.find(request_id);
  return it == s->live.end() ? PA_ERR_SHAPE : it->second->computed;
}

int32_t pa_sched_block_ref_count(const pa_sched* s, int32_t block) {
  if (!s || block < 0 || block >= s->pool.size()) return -1;
  return s->pool.at(block).ref;
}

int32_t pa_sched_shared_prefix_blocks(const int32_t* query_start_loc, const int32_t* seq_lens,
                                      const int32_t* block_table, int32_t num_seqs,
                                      int32_t table_cols) {
  if (!query_start_loc || !seq_lens || !block_table || num_seqs <= 0 || table_cols <= 0)
    return 0;
  // every row a decode row; the prefix ends a key before the shortest row
  int64_t p = table_cols;
  for (int32_t r = 0; r < num_seqs; ++r) {
    if (query_start_loc[r + 1] - query_start_loc[r] != 1 || seq_lens[r] < 1) return 0;
    p = std::min<int64_t>(p, (seq_lens[r] - 1) / PA_BLOCK_SIZE);
  }
  // the leading entries every row shares with row 0
  for (int32_t r = 1; r < num_seqs && p > 0; ++r) {
    const int32_t* row = block_table + (size_t)r * table_cols;
    int64_t b = 0;
    while (b < p && row[b] == block_table[b]) ++b;
    p = b;
  }
  return (int32_t)p;
}

}  // extern "C"
