// libpa host runtime: KV block manager, iteration-level scheduler and the
// engine loop that enqueues the pa_* kernels. See include/pa_sched.h for the
// contract; this file only adds how the state is kept.
#include "pa_sched.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <deque>
#include <map>
#include <vector>

#include "pa.h"

namespace {

constexpr int kHeader = 16;

int32_t cdiv(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

// Physical blocks: a stack of free ids and a reference count per block.
class BlockPool {
 public:
  void init(const int32_t* order, int32_t n) {
    free_.assign(order, order + n);
    std::reverse(free_.begin(), free_.end());  // the back is handed out first
    refs_.assign(n, 0);
  }
  int32_t free_count() const { return static_cast<int32_t>(free_.size()); }
  int32_t take() {
    const int32_t b = free_.back();
    free_.pop_back();
    refs_[b] = 1;
    return b;
  }
  void share(int32_t b) { ++refs_[b]; }
  bool shared(int32_t b) const { return refs_[b] > 1; }
  int32_t users(int32_t b) const { return refs_[b]; }
  void drop(int32_t b) {
    if (--refs_[b] == 0) free_.push_back(b);
  }
  void drop_all(const std::vector<int32_t>& table) {
    for (int32_t b : table) drop(b);
  }

 private:
  std::vector<int32_t> free_;
  std::vector<int32_t> refs_;
};

struct Seq {  // one sample after its prompt is cached
  std::vector<int32_t> table;
  std::vector<int32_t> host_table;  // its blocks' host copies while swapped out
  int32_t cached = 0;  // tokens whose KV is in the pool
  int32_t made = 0;    // tokens generated
  int32_t want = 0;
  bool finished = false, released = false;
};

enum class Phase { kQueued, kPrefill, kDecode, kSwapped, kDone };

struct Req {
  int32_t prompt = 0, arrival = 0;
  int32_t prefix_id = -1, prefix_len = 0;  // shared prompt prefix (id -1: none)
  std::vector<int32_t> outs;
  Phase phase = Phase::kQueued;
  int32_t prefilled = 0;
  std::vector<int32_t> prompt_table;             // blocks of the prompt during prefill
  std::vector<std::vector<int32_t>> spare;       // reservations of samples 1..n-1
  std::vector<Seq> seqs;
  int32_t width() const { return static_cast<int32_t>(outs.size()); }
  void restart() {
    phase = Phase::kQueued;
    prefilled = 0;
    prompt_table.clear();
    spare.clear();
    seqs.clear();
  }
};

struct PlanBuf {
  int32_t iteration = 0, generated = 0, longest_chunk = 0;
  std::vector<int32_t> copies, pre_slots, dec_slots;
  std::vector<int32_t> chunk_req, chunk_start, chunk_ctx, chunk_tab;
  std::vector<int32_t> dec_req, dec_sample, dec_ctx, dec_tab;
  std::vector<int32_t> admitted, preempted, finished;
  std::vector<int32_t> swap_out, swap_in;  // (device, host) and (host, device) pairs
  void reset(int32_t it) {
    iteration = it;
    generated = longest_chunk = 0;
    for (auto* v : {&copies, &pre_slots, &dec_slots, &chunk_req, &chunk_start, &chunk_ctx,
                    &chunk_tab, &dec_req, &dec_sample, &dec_ctx, &dec_tab, &admitted,
                    &preempted, &finished, &swap_out, &swap_in})
      v->clear();
  }
};

}  // namespace

struct pa_sched {
  pa_sched_config cfg{};
  int32_t mb = 0;  // table row width
  BlockPool pool;
  std::vector<Req> reqs;
  size_t next_arrival = 0;
  std::deque<int32_t> queue;
  std::vector<int32_t> running;  // admission order
  int32_t slots_used = 0;
  std::vector<int32_t> owed_copies;
  std::vector<int32_t> host_free;  // stack of host blocks for swapped requests
  // Prefix cache: (prefix id, block index) -> block, holding one reference
  // to it; keys in least-recently-used order.
  std::map<int64_t, int32_t> cache;
  std::vector<int64_t> lru;
  int32_t iteration = 0;
  PlanBuf plan;

  static int64_t prefix_key(int32_t id, int32_t j) {
    return (static_cast<int64_t>(id) << 32) | static_cast<uint32_t>(j);
  }
  void touch(int64_t key) {
    auto it = std::find(lru.begin(), lru.end(), key);
    if (it != lru.end()) lru.erase(it);
    lru.push_back(key);
  }
  // A block: the free stack's top, or, with none free, the block of the
  // oldest cache entry that only the cache still holds.
  int32_t alloc() {
    if (pool.free_count() == 0) {
      for (auto it = lru.begin(); it != lru.end(); ++it) {
        const int32_t b = cache.at(*it);
        if (pool.users(b) == 1) {
          cache.erase(*it);
          lru.erase(it);
          pool.drop(b);
          break;
        }
      }
    }
    return pool.take();
  }
  // Blocks an allocation can get: free ones and cached ones only the cache holds.
  int64_t available() const {
    int64_t n = pool.free_count();
    for (const auto& kv : cache) n += pool.users(kv.second) == 1 ? 1 : 0;
    return n;
  }
  // Cached blocks of r's prefix from block 0 up to the first miss.
  std::vector<int32_t> prefix_hits(const Req& r) const {
    std::vector<int32_t> hits;
    if (!cfg.prefix_caching || r.prefix_id < 0) return hits;
    const int32_t limit = std::min(r.prefix_len, r.prompt - 1);
    for (int32_t j = 0; (j + 1) * cfg.block_size <= limit; ++j) {
      auto it = cache.find(prefix_key(r.prefix_id, j));
      if (it == cache.end()) break;
      hits.push_back(it->second);
    }
    return hits;
  }

  bool finished() const {
    return next_arrival == reqs.size() && queue.empty() && running.empty();
  }

  // Slot of logical position `pos` of `table`: a new block when the position
  // opens one, a private copy when the block is shared.
  int32_t slot_for(std::vector<int32_t>& table, int32_t pos) {
    const int32_t j = pos / cfg.block_size;
    if (j == static_cast<int32_t>(table.size())) {
      table.push_back(alloc());
    } else if (pool.shared(table[j])) {
      const int32_t fresh = alloc();
      plan.copies.push_back(table[j]);
      plan.copies.push_back(fresh);
      pool.drop(table[j]);
      table[j] = fresh;
    }
    return table[j] * cfg.block_size + pos % cfg.block_size;
  }

  template <typename F>
  void each_decoding(F&& f) {  // unfinished samples, admission then sample order
    for (int32_t rid : running) {
      Req& r = reqs[rid];
      if (r.phase != Phase::kDecode) continue;
      for (size_t k = 0; k < r.seqs.size(); ++k)
        if (!r.seqs[k].finished && !f(rid, static_cast<int32_t>(k), r.seqs[k])) return;
    }
  }

  int32_t chunk_len(const Req& r, int32_t budget) const {
    return std::min(std::min(r.prompt - r.prefilled, cfg.max_chunk), budget);
  }

  // Upper bound of the blocks the running requests take this iteration.
  int64_t blocks_wanted(int32_t budget) {
    int64_t want = 0;
    int32_t left = budget;
    each_decoding([&](int32_t, int32_t, Seq& q) {
      if (left == 0) return false;
      --left;
      if (q.cached % cfg.block_size == 0 || pool.shared(q.table.back())) ++want;
      return true;
    });
    for (int32_t rid : running) {
      const Req& r = reqs[rid];
      if (r.phase != Phase::kPrefill) continue;
      const int32_t L = chunk_len(r, left);
      if (L <= 0) break;
      want += cdiv(r.prefilled + L, cfg.block_size) - static_cast<int64_t>(r.prompt_table.size());
      left -= L;
    }
    return want;
  }

  // Distinct entries of the tables of the unreleased samples, in sample then
  // table order.
  template <typename Get>
  std::vector<int32_t> distinct(const Req& r, Get get) const {
    std::vector<int32_t> seen;
    for (const Seq& q : r.seqs) {
      if (q.released) continue;
      for (int32_t b : get(q))
        if (std::find(seen.begin(), seen.end(), b) == seen.end()) seen.push_back(b);
    }
    return seen;
  }

  // A decoding request's blocks to host blocks; false if they do not fit.
  bool swap_out(Req& r) {
    const std::vector<int32_t> blocks = distinct(r, [](const Seq& q) { return q.table; });
    if (blocks.size() > host_free.size()) return false;
    std::vector<int32_t> host(blocks.size());
    for (size_t i = 0; i < blocks.size(); ++i) {
      host[i] = host_free.back();
      host_free.pop_back();
      plan.swap_out.push_back(blocks[i]);
      plan.swap_out.push_back(host[i]);
    }
    for (Seq& q : r.seqs) {
      if (q.released) continue;
      q.host_table.clear();
      for (int32_t b : q.table)
        q.host_table.push_back(host[std::find(blocks.begin(), blocks.end(), b) - blocks.begin()]);
      pool.drop_all(q.table);
      q.table.clear();
      --slots_used;
    }
    r.phase = Phase::kSwapped;
    return true;
  }

  // A swapped request back onto the device; false if it does not fit yet.
  bool swap_in(Req& r) {
    int32_t live = 0;
    for (const Seq& q : r.seqs) live += q.released ? 0 : 1;
    const std::vector<int32_t> host = distinct(r, [](const Seq& q) { return q.host_table; });
    if (slots_used + live > cfg.max_seqs || static_cast<int64_t>(host.size()) > available())
      return false;
    std::vector<int32_t> dev(host.size());
    for (size_t i = 0; i < host.size(); ++i) {
      dev[i] = alloc();
      plan.swap_in.push_back(host[i]);
      plan.swap_in.push_back(dev[i]);
    }
    for (Seq& q : r.seqs) {
      if (q.released) continue;
      q.table.clear();
      for (int32_t h : q.host_table)
        q.table.push_back(dev[std::find(host.begin(), host.end(), h) - host.begin()]);
      q.host_table.clear();
    }
    // take() counted one user per block; every further table use adds one
    std::vector<int32_t> uses(host.size(), 0);
    for (const Seq& q : r.seqs) {
      if (q.released) continue;
      for (int32_t b : q.table) ++uses[std::find(dev.begin(), dev.end(), b) - dev.begin()];
    }
    for (size_t i = 0; i < dev.size(); ++i)
      for (int32_t u = 1; u < uses[i]; ++u) pool.share(dev[i]);
    for (int32_t h : host) host_free.push_back(h);
    slots_used += live;
    r.phase = Phase::kDecode;
    return true;
  }

  void evict(int32_t rid) {
    Req& r = reqs[rid];
    if (r.phase == Phase::kDecode && cfg.num_host_blocks > 0 && swap_out(r)) {
      running.erase(std::find(running.begin(), running.end(), rid));
      queue.push_front(rid);
      plan.preempted.push_back(rid);
      return;
    }
    if (r.phase == Phase::kPrefill) {
      pool.drop_all(r.prompt_table);
      for (auto& t : r.spare) pool.drop_all(t);
      slots_used -= r.width();
    } else {
      for (Seq& q : r.seqs)
        if (!q.released) {
          pool.drop_all(q.table);
          --slots_used;
        }
    }
    r.restart();
    running.erase(std::find(running.begin(), running.end(), rid));
    queue.push_front(rid);
    plan.preempted.push_back(rid);
  }

  void put_table(std::vector<int32_t>& dst, const std::vector<int32_t>& table) const {
    dst.insert(dst.end(), table.begin(), table.end());
    dst.insert(dst.end(), mb - table.size(), 0);
  }

  // Next prefill chunk of `rid` (its blocks are known to be available).
  int32_t prefill_chunk(int32_t rid, int32_t budget) {
    Req& r = reqs[rid];
    const int32_t L = chunk_len(r, budget);
    if (L <= 0) return 0;
    plan.chunk_req.push_back(rid);
    plan.chunk_start.push_back(static_cast<int32_t>(plan.pre_slots.size()));
    for (int32_t pos = r.prefilled; pos < r.prefilled + L; ++pos)
      plan.pre_slots.push_back(slot_for(r.prompt_table, pos));
    const int32_t before = r.prefilled;
    r.prefilled += L;
    if (cfg.prefix_caching && r.prefix_id >= 0) {  // full prefix blocks this chunk completed
      for (int32_t j = before / cfg.block_size; j < r.prefilled / cfg.block_size; ++j) {
        const int64_t key = prefix_key(r.prefix_id, j);
        if ((j + 1) * cfg.block_size <= r.prefix_len && !cache.count(key)) {
          cache[key] = r.prompt_table[j];
          pool.share(r.prompt_table[j]);
          touch(key);
        }
      }
    }
    plan.chunk_ctx.push_back(r.prefilled);
    put_table(plan.chunk_tab, r.prompt_table);
    plan.longest_chunk = std::max(plan.longest_chunk, L);
    if (r.prefilled == r.prompt) fork(r);
    return L;
  }

  // The prompt is cached: every sample gets its first token and a table.
  void fork(Req& r) {
    r.phase = Phase::kDecode;
    r.seqs.resize(r.outs.size());
    for (size_t k = 0; k < r.outs.size(); ++k) {
      Seq& q = r.seqs[k];
      if (k == 0) {
        q.table = r.prompt_table;
      } else if (cfg.policy == PA_POLICY_PAGED) {
        q.table = r.prompt_table;
        for (int32_t b : q.table) pool.share(b);
      } else {
        q.table = std::move(r.spare[k - 1]);
        for (int32_t j = 0; j < cdiv(r.prompt, cfg.block_size); ++j) {
          owed_copies.push_back(r.prompt_table[j]);
          owed_copies.push_back(q.table[j]);
        }
      }
      q.cached = r.prompt;
      q.made = 1;
      q.want = r.outs[k];
      q.finished = q.want == 1;
    }
    r.prompt_table.clear();
    r.spare.clear();
    plan.generated += r.width();
  }

  bool admit_head(int32_t budget) {
    const int32_t rid = queue.front();
    Req& r = reqs[rid];
    if (slots_used + r.width() > cfg.max_seqs) return false;
    std::vector<int32_t> hits;
    if (cfg.policy == PA_POLICY_PAGED) {
      hits = prefix_hits(r);
      const int32_t got = static_cast<int32_t>(hits.size()) * cfg.block_size;
      const int32_t first = std::min(std::min(r.prompt - got, cfg.max_chunk), budget);
      int64_t held_by_cache_only = 0;
      for (int32_t b : hits) held_by_cache_only += pool.users(b) == 1 ? 1 : 0;
      if (cdiv(got + first, cfg.block_size) - static_cast<int64_t>(hits.size()) >
          available() - held_by_cache_only)
        return false;
    } else {
      const int32_t per = cdiv(cfg.max_len, cfg.block_size);
      if (static_cast<int64_t>(per) * r.width() > pool.free_count()) return false;
      for (int32_t i = 0; i < per; ++i) r.prompt_table.push_back(alloc());
      r.spare.assign(r.outs.size() - 1, {});
      for (auto& t : r.spare)
        for (int32_t i = 0; i < per; ++i) t.push_back(alloc());
    }
    queue.pop_front();
    running.push_back(rid);
    slots_used += r.width();
    r.phase = Phase::kPrefill;
    plan.admitted.push_back(rid);
    for (size_t j = 0; j < hits.size(); ++j) {  // the cached prefix blocks: no prefill
      pool.share(hits[j]);
      r.prompt_table.push_back(hits[j]);
      touch(prefix_key(r.prefix_id, static_cast<int32_t>(j)));
    }
    r.prefilled = static_cast<int32_t>(hits.size()) * cfg.block_size;
    return true;
  }

  void release_finished() {
    if (cfg.policy == PA_POLICY_STATIC) {
      if (running.empty()) return;
      for (int32_t rid : running) {
        const Req& r = reqs[rid];
        if (r.phase != Phase::kDecode) return;
        for (const Seq& q : r.seqs)
          if (!q.finished) return;
      }
      for (int32_t rid : running) {
        for (Seq& q : reqs[rid].seqs) pool.drop_all(q.table);
        reqs[rid].phase = Phase::kDone;
        plan.finished.push_back(rid);
      }
      running.clear();
      slots_used = 0;
      return;
    }
    std::vector<int32_t> still;
    for (int32_t rid : running) {
      Req& r = reqs[rid];
      bool all = r.phase == Phase::kDecode;
      if (all) {
        for (Seq& q : r.seqs) {
          if (q.finished && !q.released) {
            pool.drop_all(q.table);
            q.released = true;
            --slots_used;
          }
          all = all && q.released;
        }
      }
      if (all) {
        r.phase = Phase::kDone;
        plan.finished.push_back(rid);
      } else {
        still.push_back(rid);
      }
    }
    running.swap(still);
  }

  int step() {
    if (finished()) return PA_SCHED_FINISHED;
    plan.reset(iteration);
    plan.copies.swap(owed_copies);
    owed_copies.clear();
    while (next_arrival < reqs.size() && reqs[next_arrival].arrival <= iteration)
      queue.push_back(static_cast<int32_t>(next_arrival++));
    const bool batch_open = running.empty();
    int32_t budget = cfg.max_tokens;
    if (cfg.policy == PA_POLICY_PAGED) {
      while (blocks_wanted(budget) > available()) {
        if (running.size() <= 1) return PA_ERR_STATE;
        evict(running.back());
      }
    }
    each_decoding([&](int32_t rid, int32_t k, Seq& q) {
      if (budget == 0) return false;
      plan.dec_slots.push_back(slot_for(q.table, q.cached));
      ++q.cached;
      ++q.made;
      q.finished = q.made == q.want;
      plan.dec_req.push_back(rid);
      plan.dec_sample.push_back(k);
      plan.dec_ctx.push_back(q.cached);
      put_table(plan.dec_tab, q.table);
      ++plan.generated;
      --budget;
      return true;
    });
    const std::vector<int32_t> order = running;
    for (int32_t rid : order)
      if (reqs[rid].phase == Phase::kPrefill) budget -= prefill_chunk(rid, budget);
    const bool may_admit =
        plan.preempted.empty() && (cfg.policy != PA_POLICY_STATIC || batch_open);
    // A static batch is formed whole; continuous batching admits only what the
    // budget can start on this iteration.
    const bool whole_batch = cfg.policy == PA_POLICY_STATIC;
    while (may_admit && !queue.empty() && (budget > 0 || whole_batch)) {
      const int32_t head = queue.front();
      if (reqs[head].phase == Phase::kSwapped) {  // back with its progress, no prefill
        if (!swap_in(reqs[head])) break;
        queue.pop_front();
        running.push_back(head);
        plan.admitted.push_back(head);
        continue;
      }
      if (!admit_head(budget)) break;
      budget -= prefill_chunk(running.back(), budget);
    }
    release_finished();
    ++iteration;
    // An iteration with no work while nothing is yet to arrive means the state
    // is broken (a whole pool always admits the head of the queue).
    if (plan.pre_slots.empty() && plan.dec_slots.empty() && plan.copies.empty() &&
        plan.preempted.empty() && plan.finished.empty() && plan.swap_in.empty() &&
        next_arrival == reqs.size())
      return PA_ERR_STATE;
    return PA_OK;
  }

  int64_t capacity() const {
    const int64_t seqs = cfg.max_seqs;
    const int64_t copies = 2 * (seqs * mb + seqs);
    const int64_t swaps = 4 * static_cast<int64_t>(cfg.num_blocks);
    return kHeader + copies + cfg.max_tokens + seqs * (3 + mb) + 1 + seqs * (3 + mb) + 3 * seqs +
           swaps;
  }

  int64_t words() const {
    const PlanBuf& p = plan;
    return kHeader + static_cast<int64_t>(p.copies.size() + p.pre_slots.size() +
                                          p.dec_slots.size() + 3 * p.chunk_req.size() + 1 +
                                          p.chunk_tab.size() + 3 * p.dec_req.size() +
                                          p.dec_tab.size() + p.admitted.size() +
                                          p.preempted.size() + p.finished.size() +
                                          p.swap_out.size() + p.swap_in.size());
  }

  void write(int32_t* buf) const {
    const PlanBuf& p = plan;
    int32_t* h = buf;
    std::fill(h, h + kHeader, 0);
    h[0] = p.iteration;
    h[1] = p.generated;
    h[2] = static_cast<int32_t>(p.copies.size() / 2);
    h[3] = static_cast<int32_t>(p.pre_slots.size() + p.dec_slots.size());
    h[4] = static_cast<int32_t>(p.pre_slots.size());
    h[5] = static_cast<int32_t>(p.chunk_req.size());
    h[6] = static_cast<int32_t>(p.dec_req.size());
    h[7] = static_cast<int32_t>(p.admitted.size());
    h[8] = static_cast<int32_t>(p.preempted.size());
    h[9] = static_cast<int32_t>(p.finished.size());
    h[10] = mb;
    h[11] = p.longest_chunk;
    h[12] = static_cast<int32_t>(p.swap_out.size() / 2);
    h[13] = static_cast<int32_t>(p.swap_in.size() / 2);
    int32_t* w = buf + kHeader;
    auto put = [&w](const std::vector<int32_t>& v) { w = std::copy(v.begin(), v.end(), w); };
    put(p.copies);
    put(p.pre_slots);
    put(p.dec_slots);
    put(p.chunk_req);
    put(p.chunk_start);
    *w++ = static_cast<int32_t>(p.pre_slots.size());
    put(p.chunk_ctx);
    put(p.chunk_tab);
    put(p.dec_req);
    put(p.dec_sample);
    put(p.dec_ctx);
    put(p.dec_tab);
    put(p.admitted);
    put(p.preempted);
    put(p.finished);
    put(p.swap_out);
    put(p.swap_in);
  }
};

// ---------------------------------------------------------------------------
// Engine
// ---------------------------------------------------------------------------
namespace {
constexpr int kRing = 4;
}

struct pa_engine {
  pa_sched* s = nullptr;
  void* pool = nullptr;
  int32_t hkv = 0, hq = 0, d = 0, dtype = 0;
  float scale = 0.f;
  const void *q_prefill = nullptr, *q_decode = nullptr, *k_rows = nullptr, *v_rows = nullptr;
  void *out_prefill = nullptr, *out_decode = nullptr, *ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t stream = nullptr;
  int64_t cap = 0;
  int32_t* host_ring = nullptr;  // pinned, kRing packets
  void* host_pool = nullptr;     // pinned, the scheduler's host blocks for swapping
  int32_t* dev_ring = nullptr;
  hipEvent_t sent[kRing] = {};
  bool used[kRing] = {};
  int next = 0;
  pa_engine_stats stats{};

  ~pa_engine() {
    for (auto& e : sent)
      if (e) (void)hipEventDestroy(e);
    if (host_ring) (void)hipHostFree(host_ring);
    if (host_pool) (void)hipHostFree(host_pool);
    if (dev_ring) (void)hipFree(dev_ring);
  }

  int launch(const int32_t* h, const int32_t* dev) {
    const pa_sched_config& c = s->cfg;
    const int32_t mb = h[10];
    const int32_t n_copies = h[2], n_slots = h[3], n_pre = h[4], n_chunks = h[5], n_dec = h[6];
    const int32_t* copies = dev + kHeader;
    const int32_t* slots = copies + 2 * n_copies;
    const int32_t* chunk_req = slots + n_slots;
    const int32_t* qsl = chunk_req + n_chunks;
    const int32_t* chunk_ctx = qsl + n_chunks + 1;
    const int32_t* chunk_tab = chunk_ctx + n_chunks;
    const int32_t* dec_req = chunk_tab + static_cast<int64_t>(n_chunks) * mb;
    const int32_t* dec_ctx = dec_req + 2 * n_dec;
    const int32_t* dec_tab = dec_ctx + n_dec;
    const int32_t* swap_out = dec_tab + static_cast<int64_t>(n_dec) * mb + h[7] + h[8] + h[9];
    const int32_t* swap_in = swap_out + 2 * h[12];
    // blocks leave before any is reused, and return before anything is written
    if (h[12] > 0)
      if (int st = pa_swap_blocks(pool, host_pool, swap_out, h[12], PA_SWAP_OUT, c.num_blocks,
                                  c.num_host_blocks, hkv, d, c.block_size, dtype, stream))
        return st;
    if (h[13] > 0)
      if (int st = pa_swap_blocks(pool, host_pool, swap_in, h[13], PA_SWAP_IN, c.num_blocks,
                                  c.num_host_blocks, hkv, d, c.block_size, dtype, stream))
        return st;
    for (int32_t i = 0; i < n_copies; i += 65535) {
      const int32_t n = std::min(65535, n_copies - i);
      if (int st = pa_copy_blocks(pool, copies + 2 * i, n, c.num_blocks, hkv, d, c.block_size,
                                  dtype, stream))
        return st;
    }
    // A decode-only iteration appends one token per decoding sequence, rows in
    // decode order: its append and attention go in one launch.
    if (n_chunks == 0 && n_pre == 0 && n_dec > 0 && n_slots == n_dec)
      return pa_decode_append(out_decode, q_decode, pool, dec_tab, dec_ctx, k_rows, v_rows, slots,
                              n_dec, mb, c.max_len, hq, hkv, d, c.block_size, c.num_blocks, scale,
                              dtype, ws, ws_bytes, stream);
    if (int st = pa_append_kv(pool, k_rows, v_rows, slots, n_slots, c.num_blocks, hkv, d,
                              c.block_size, dtype, stream))
      return st;
    if (n_chunks > 0 && n_dec > 0)  // both kinds of work: one fused launch
      return pa_mixed_attention(out_decode, q_decode, dec_tab, dec_ctx, n_dec, mb, c.max_len,
                                out_prefill, q_prefill, chunk_tab, chunk_ctx, qsl, n_chunks,
                                n_pre, h[11], mb, pool, hq, hkv, d, c.block_size, c.num_blocks,
                                scale, dtype, ws, ws_bytes, stream);
    if (n_chunks > 0) {
      if (int st = pa_prefill_chunk(out_prefill, q_prefill, pool, chunk_tab, chunk_ctx, qsl,
                                    n_chunks, n_pre, h[11], mb, hq, hkv, d, c.block_size,
                                    c.num_blocks, scale, dtype, stream))
        return st;
    }
    if (n_dec > 0) {
      if (int st = pa_decode(out_decode, q_decode, pool, dec_tab, dec_ctx, n_dec, mb, c.max_len,
                             hq, hkv, d, c.block_size, c.num_blocks, scale, dtype, ws, ws_bytes,
                             stream))
        return st;
    }
    return PA_OK;
  }

  int step(int32_t* out, int64_t out_cap, int64_t* used_words) {
    using clock = std::chrono::steady_clock;
    const auto t0 = clock::now();
    if (out && out_cap < s->capacity()) return PA_ERR_SHAPE;
    const int st = s->step();
    if (st != PA_OK) return st;
    const int slot = next;
    next = (next + 1) % kRing;
    const auto t1 = clock::now();
    if (used[slot] && hipEventSynchronize(sent[slot]) != hipSuccess) return PA_ERR_LAUNCH;
    const auto t2 = clock::now();
    int32_t* h = host_ring + slot * cap;
    int32_t* dv = dev_ring + slot * cap;
    s->write(h);
    const int64_t words = s->words();
    if (out) std::copy(h, h + words, out);
    if (used_words) *used_words = words;
    if (hipMemcpyAsync(dv, h, words * sizeof(int32_t), hipMemcpyHostToDevice, stream) !=
            hipSuccess ||
        hipEventRecord(sent[slot], stream) != hipSuccess)
      return PA_ERR_LAUNCH;
    used[slot] = true;
    const int ls = launch(h, dv);
    stats.iterations += 1;
    stats.generated += h[1];
    stats.prefill_tokens += h[4];
    stats.decode_tokens += h[6];
    for (int32_t ctx : s->plan.dec_ctx) stats.decode_context_tokens += ctx;
    stats.copies += h[2];
    stats.evictions += h[8];
    stats.swapped_blocks += h[12];
    const auto t3 = clock::now();
    using us = std::chrono::duration<double, std::micro>;
    stats.host_us += us(t1 - t0).count() + us(t3 - t2).count();
    stats.wait_us += us(t2 - t1).count();
    return ls;
  }
};

extern "C" {

int pa_sched_create(const pa_sched_config* cfg, const int32_t* free_order, int32_t num_requests,
                    const int32_t* prompt_lens, const int32_t* arrival,
                    const int32_t* sample_offsets, const int32_t* output_lens,
                    const int32_t* prefix_ids, const int32_t* prefix_lens, pa_sched** out) {
  if (!cfg || !out || !free_order || (num_requests > 0 && (!prompt_lens || !arrival ||
                                                           !sample_offsets || !output_lens)))
    return PA_ERR_NULL;
  *out = nullptr;
  const pa_sched_config& c = *cfg;
  if (c.num_blocks <= 0 || c.block_size <= 0 || c.max_seqs <= 0 || c.max_tokens <= 0 ||
      c.max_chunk <= 0 || c.max_len <= 0 || num_requests < 0 || c.policy < PA_POLICY_PAGED ||
      c.policy > PA_POLICY_STATIC || c.num_host_blocks < 0 ||
      (c.num_host_blocks > 0 && c.policy != PA_POLICY_PAGED) ||
      (c.prefix_caching != 0 && c.policy != PA_POLICY_PAGED))
    return PA_ERR_SHAPE;
  std::vector<char> seen(c.num_blocks, 0);
  for (int32_t i = 0; i < c.num_blocks; ++i) {
    const int32_t b = free_order[i];
    if (b < 0 || b >= c.num_blocks || seen[b]) return PA_ERR_SHAPE;
    seen[b] = 1;
  }
  auto* s = new pa_sched;
  s->cfg = c;
  s->mb = cdiv(c.max_len, c.block_size);
  s->pool.init(free_order, c.num_blocks);
  for (int32_t h = c.num_host_blocks - 1; h >= 0; --h) s->host_free.push_back(h);
  s->reqs.resize(num_requests);
  for (int32_t r = 0; r < num_requests; ++r) {
    Req& q = s->reqs[r];
    q.prompt = prompt_lens[r];
    q.arrival = arrival[r];
    if (prefix_ids && prefix_ids[r] >= 0) {
      q.prefix_id = prefix_ids[r];
      q.prefix_len = prefix_lens ? prefix_lens[r] : 0;
    }
    const int32_t a = sample_offsets[r], b = sample_offsets[r + 1];
    bool ok = q.prompt >= 1 && b > a && (r == 0 || arrival[r] >= arrival[r - 1]) &&
              q.prefix_len >= 0 && q.prefix_len <= q.prompt;
    int32_t longest = 0;
    for (int32_t k = a; ok && k < b; ++k) {
      ok = output_lens[k] >= 1;
      longest = std::max(longest, output_lens[k]);
      q.outs.push_back(output_lens[k]);
    }
    const int64_t reach = static_cast<int64_t>(q.prompt) + longest - 1;
    const int64_t per = c.policy == PA_POLICY_PAGED ? cdiv(reach, c.block_size)
                                                    : cdiv(c.max_len, c.block_size);
    ok = ok && reach <= c.max_len && q.width() <= c.max_seqs &&
         per * q.width() <= c.num_blocks;
    if (!ok) {
      delete s;
      return PA_ERR_SHAPE;
    }
  }
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int64_t pa_sched_plan_capacity(const pa_sched* s) { return s ? s->capacity() : 0; }

int32_t pa_sched_num_free(const pa_sched* s) { return s ? s->pool.free_count() : 0; }

int pa_sched_step(pa_sched* s, int32_t* buf, int64_t cap, int64_t* used) {
  if (!s) return PA_ERR_NULL;
  if (buf && cap < s->capacity()) return PA_ERR_SHAPE;
  const int st = s->step();
  if (st != PA_OK) return st;
  if (buf) s->write(buf);
  if (used) *used = buf ? s->words() : 0;
  return PA_OK;
}

int pa_engine_create(pa_sched* s, void* kv_pool, int32_t num_kv_heads, int32_t num_q_heads,
                     int32_t head_dim, int32_t dtype, float scale, const void* q_prefill,
                     const void* q_decode, const void* k_rows, const void* v_rows,
                     void* out_prefill, void* out_decode, void* workspace,
                     size_t workspace_bytes, void* stream, pa_engine** out) {
  if (!s || !kv_pool || !q_prefill || !q_decode || !k_rows || !v_rows || !out_prefill ||
      !out_decode || !workspace || !out)
    return PA_ERR_NULL;
  *out = nullptr;
  if (num_kv_heads <= 0 || num_q_heads <= 0 || head_dim <= 0) return PA_ERR_SHAPE;
  if (workspace_bytes <
      pa_decode_workspace_size(s->cfg.max_seqs, num_q_heads, head_dim, s->cfg.max_len))
    return PA_ERR_WORKSPACE;
  auto* e = new pa_engine;
  e->s = s;
  e->pool = kv_pool;
  e->hkv = num_kv_heads;
  e->hq = num_q_heads;
  e->d = head_dim;
  e->dtype = dtype;
  e->scale = scale;
  e->q_prefill = q_prefill;
  e->q_decode = q_decode;
  e->k_rows = k_rows;
  e->v_rows = v_rows;
  e->out_prefill = out_prefill;
  e->out_decode = out_decode;
  e->ws = workspace;
  e->ws_bytes = workspace_bytes;
  e->stream = static_cast<hipStream_t>(stream);
  e->cap = (s->capacity() + 63) & ~int64_t(63);  // 256-byte aligned packets
  const size_t bytes = static_cast<size_t>(e->cap) * kRing * sizeof(int32_t);
  bool ok = hipHostMalloc(reinterpret_cast<void**>(&e->host_ring), bytes, hipHostMallocDefault) ==
                hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&e->dev_ring), bytes) == hipSuccess;
  for (auto& ev : e->sent)
    ok = ok && hipEventCreateWithFlags(&ev, hipEventDisableTiming) == hipSuccess;
  if (ok && s->cfg.num_host_blocks > 0) {
    const size_t blk = size_t(2) * num_kv_heads * s->cfg.block_size * head_dim *
                       (dtype == PA_F32 ? 4 : 2);
    ok = hipHostMalloc(&e->host_pool, blk * s->cfg.num_host_blocks, hipHostMallocDefault) ==
         hipSuccess;
  }
  if (!ok) {
    delete e;
    return PA_ERR_LAUNCH;
  }
  *out = e;
  return PA_OK;
}

void pa_engine_destroy(pa_engine* e) {
  if (e && e->stream) (void)hipStreamSynchronize(e->stream);
  delete e;
}

int pa_engine_step(pa_engine* e, int32_t* buf, int64_t cap, int64_t* used) {
  if (!e) return PA_ERR_NULL;
  return e->step(buf, cap, used);
}

int pa_engine_run(pa_engine* e, pa_engine_stats* stats) {
  if (!e) return PA_ERR_NULL;
  int st = PA_OK;
  while ((st = e->step(nullptr, 0, nullptr)) == PA_OK) {
  }
  if (st != PA_SCHED_FINISHED) return st;
  if (hipStreamSynchronize(e->stream) != hipSuccess) return PA_ERR_LAUNCH;
  if (stats) *stats = e->stats;
  return PA_OK;
}

}  // extern "C"
