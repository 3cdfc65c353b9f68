// Host-side block manager and per-step scheduler (pa_block_manager.h).
//
// Plain C++ on the host: the free lists are intrusive doubly linked queues
// over block ids (take the front, give back to the back, unlink a cached
// block that a prompt hits: all O(1)); requests sit in a hash map and, per
// state, in an arrival-ordered map; the prefix cache maps a 128-bit chained
// key to the block that holds that prefix.  A decode step costs O(1) per
// running request plus O(B) for every block that fills.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <limits>
#include <map>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_block_manager.h"
#include "pa_status.h"

static_assert(sizeof(pa_bm_config) == 32 && sizeof(pa_step_plan) == 112 &&
                  sizeof(pa_bm_stats) == 96 && sizeof(pa_request_info) == 48,
              "block manager structs are part of the ABI");

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// prefix keys
// ---------------------------------------------------------------------------

struct Key128 {
  uint64_t hi = 0, lo = 0;
  bool operator==(const Key128& o) const { return hi == o.hi && lo == o.lo; }
};

struct KeyHash {
  size_t operator()(const Key128& k) const { return size_t(k.lo ^ (k.hi * 0x9E3779B97F4A7C15ull)); }
};

// The output function of SplitMix64 (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014): a bijective 64-bit mixer.
inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Key of a block: its own tokens chained with the key of the prefix before it
// (two independently mixed 64-bit lanes).
Key128 chain_key(const Key128& parent, const int32_t* tokens, int32_t n) {
  uint64_t a = parent.lo ^ 0x243F6A8885A308D3ull;
  uint64_t b = parent.hi ^ 0x13198A2E03707344ull;
  for (int32_t i = 0; i < n; ++i) {
    const uint64_t u = uint32_t(tokens[i]);
    a = mix64(a + u + 0x9E3779B97F4A7C15ull);
    b = mix64(b ^ (u * 0xC2B2AE3D27D4EB4Full + 0x165667B19E3779F9ull));
  }
  return Key128{mix64(b + uint64_t(n)), mix64(a ^ uint64_t(n))};
}

// ---------------------------------------------------------------------------
// free lists
// ---------------------------------------------------------------------------

class IdQueue {
 public:
  void init(int64_t n) {
    prev_.assign(size_t(n), -1);
    next_.assign(size_t(n), -1);
    in_.assign(size_t(n), 0);
    head_ = tail_ = -1;
    size_ = 0;
    for (int64_t i = 0; i < n; ++i) push_back(int32_t(i));
  }
  int64_t size() const { return size_; }
  bool contains(int32_t id) const { return in_[size_t(id)] != 0; }
  int32_t pop_front() {
    const int32_t id = head_;
    unlink(id);
    return id;
  }
  void push_back(int32_t id) {
    prev_[size_t(id)] = tail_;
    next_[size_t(id)] = -1;
    if (tail_ >= 0) next_[size_t(tail_)] = id; else head_ = id;
    tail_ = id;
    in_[size_t(id)] = 1;
    ++size_;
  }
  void unlink(int32_t id) {
    const int32_t p = prev_[size_t(id)], n = next_[size_t(id)];
    if (p >= 0) next_[size_t(p)] = n; else head_ = n;
    if (n >= 0) prev_[size_t(n)] = p; else tail_ = p;
    in_[size_t(id)] = 0;
    --size_;
  }
  int64_t copy_out(int32_t* out, int64_t capacity) const {
    int64_t k = 0;
    for (int32_t id = head_; id >= 0; id = next_[size_t(id)], ++k)
      if (k < capacity) out[k] = id;
    return k;
  }

 private:
  std::vector<int32_t> prev_, next_;
  std::vector<uint8_t> in_;
  int32_t head_ = -1, tail_ = -1;
  int64_t size_ = 0;
};

// ---------------------------------------------------------------------------
// requests
// ---------------------------------------------------------------------------

struct Request {
  int64_t rid = 0;
  int64_t arrival = 0;
  int32_t state = PA_REQ_WAITING;
  int64_t computed = 0;
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;      // GPU block table
  std::vector<int32_t> cpu_blocks;  // CPU blocks while swapped
  std::vector<Key128> keys;         // chained key of each leading full block, filled lazily
};

}  // namespace
}  // namespace pa

struct pa_block_manager {
  // configuration
  int32_t B = 0;
  int64_t num_gpu = 0, num_cpu = 0;
  bool prefix_caching = true;
  int32_t mode = PA_PREEMPT_RECOMPUTE;
  int64_t watermark = 0;

  // pools
  pa::IdQueue free_gpu, free_cpu;
  std::vector<int32_t> refcount;
  // prefix cache: key -> block; per keyed block its key, its parent's key and
  // its tokens, compared on every hit
  std::unordered_map<pa::Key128, int32_t, pa::KeyHash> cache;
  std::vector<uint8_t> keyed;
  std::vector<pa::Key128> block_key, block_parent;
  std::vector<int32_t> block_tokens;

  // requests
  std::unordered_map<int64_t, pa::Request> requests;
  std::map<int64_t, pa::Request*> by_state[3];  // arrival -> request
  int64_t arrivals = 0;

  // per step
  std::vector<uint8_t> cow_source;
  std::vector<int32_t> cow_marked, deferred;
  std::vector<pa::Request*> scheduled;
  std::vector<int64_t> p_seq_ids, p_slots, p_cow, p_swap_out, p_swap_in, p_preempted;
  std::vector<int32_t> p_query_start, p_context_lens, p_tables, p_modes;

  pa_bm_stats totals{};
};

namespace pa {
namespace {

using Manager = pa_block_manager;

int64_t blocks_for(const Manager& m, int64_t tokens) { return (tokens + m.B - 1) / m.B; }

void set_state(Manager& m, Request& r, int32_t state) {
  m.by_state[r.state].erase(r.arrival);
  r.state = state;
  m.by_state[state].emplace(r.arrival, &r);
}

const Key128& key_of(Manager& m, Request& r, int64_t j) {
  while (int64_t(r.keys.size()) <= j) {
    const size_t k = r.keys.size();
    const Key128 parent = k ? r.keys[k - 1] : Key128{};
    r.keys.push_back(chain_key(parent, r.tokens.data() + k * size_t(m.B), m.B));
  }
  return r.keys[size_t(j)];
}

Key128 parent_key(Manager& m, Request& r, int64_t j) {
  return j ? key_of(m, r, j - 1) : Key128{};
}

// Block cached under the key of the request's logical block j, or -1.
int32_t lookup(Manager& m, Request& r, int64_t j) {
  auto it = m.cache.find(key_of(m, r, j));
  if (it == m.cache.end()) return -1;
  const int32_t b = it->second;
  const int32_t* want = r.tokens.data() + j * m.B;
  if (!(m.block_parent[size_t(b)] == parent_key(m, r, j)) ||
      std::memcmp(m.block_tokens.data() + size_t(b) * size_t(m.B), want,
                  size_t(m.B) * sizeof(int32_t)) != 0)
    return -1;  // a key collision: treat as a miss
  return b;
}

void register_block(Manager& m, Request& r, int64_t j, int32_t b) {
  if (m.keyed[size_t(b)]) return;
  const Key128 key = key_of(m, r, j);
  if (!m.cache.emplace(key, b).second) return;  // prefix already cached elsewhere
  m.keyed[size_t(b)] = 1;
  m.block_key[size_t(b)] = key;
  m.block_parent[size_t(b)] = parent_key(m, r, j);
  std::memcpy(m.block_tokens.data() + size_t(b) * size_t(m.B), r.tokens.data() + j * m.B,
              size_t(m.B) * sizeof(int32_t));
}

int32_t pop_gpu(Manager& m) {
  const int32_t b = m.free_gpu.pop_front();
  if (m.keyed[size_t(b)]) {  // new content: the old key leaves the cache
    m.cache.erase(m.block_key[size_t(b)]);
    m.keyed[size_t(b)] = 0;
  }
  m.refcount[size_t(b)] = 1;
  return b;
}

void release_gpu(Manager& m, Request& r) {
  for (auto it = r.blocks.rbegin(); it != r.blocks.rend(); ++it) {
    const int32_t b = *it;
    if (--m.refcount[size_t(b)] == 0) {
      if (m.cow_source[size_t(b)]) m.deferred.push_back(b);
      else m.free_gpu.push_back(b);
    }
  }
  r.blocks.clear();
}

void release_cpu(Manager& m, Request& r) {
  for (auto it = r.cpu_blocks.rbegin(); it != r.cpu_blocks.rend(); ++it) m.free_cpu.push_back(*it);
  r.cpu_blocks.clear();
}

bool shared_write_block(const Manager& m, const Request& r) {
  const int64_t c = r.computed;
  return c % m.B != 0 && m.refcount[size_t(r.blocks[size_t(c / m.B)])] > 1;
}

int64_t blocks_to_grow(const Manager& m, const Request& r, int64_t n) {
  return blocks_for(m, r.computed + n) - int64_t(r.blocks.size()) + (shared_write_block(m, r) ? 1 : 0);
}

// allocate_slots for positions computed .. computed+n-1, then record them in the plan.
void schedule_tokens(Manager& m, Request& r, int64_t n) {
  const int64_t c = r.computed;
  if (shared_write_block(m, r)) {
    const size_t j = size_t(c / m.B);
    const int32_t old = r.blocks[j], fresh = pop_gpu(m);
    --m.refcount[size_t(old)];
    r.blocks[j] = fresh;
    m.p_cow.push_back(old);
    m.p_cow.push_back(fresh);
    if (!m.cow_source[size_t(old)]) {
      m.cow_source[size_t(old)] = 1;
      m.cow_marked.push_back(old);
    }
    ++m.totals.cow_copies;
  }
  while (int64_t(r.blocks.size()) < blocks_for(m, c + n)) r.blocks.push_back(pop_gpu(m));
  if (m.prefix_caching)
    for (int64_t j = c / m.B; j < (c + n) / m.B; ++j) register_block(m, r, j, r.blocks[size_t(j)]);
  r.computed = c + n;
  m.p_seq_ids.push_back(r.rid);
  for (int64_t p = c; p < c + n; ++p)
    m.p_slots.push_back(int64_t(r.blocks[size_t(p / m.B)]) * m.B + p % m.B);
  m.p_query_start.push_back(m.p_query_start.back() + int32_t(n));
  m.p_context_lens.push_back(int32_t(r.computed));
  m.scheduled.push_back(&r);
}

void preempt(Manager& m, Request& r) {
  ++m.totals.preemptions;
  m.p_preempted.push_back(r.rid);
  if (m.mode == PA_PREEMPT_SWAP && m.free_cpu.size() >= int64_t(r.blocks.size())) {
    for (int32_t b : r.blocks) {
      const int32_t cb = m.free_cpu.pop_front();
      r.cpu_blocks.push_back(cb);
      m.p_swap_out.push_back(b);
      m.p_swap_out.push_back(cb);
    }
    m.totals.swapped_out_blocks += int64_t(r.blocks.size());
    release_gpu(m, r);
    set_state(m, r, PA_REQ_SWAPPED);
    m.p_modes.push_back(PA_PREEMPT_SWAP);
  } else {
    release_gpu(m, r);
    r.computed = 0;
    set_state(m, r, PA_REQ_WAITING);
    m.p_modes.push_back(PA_PREEMPT_RECOMPUTE);
  }
}

void swap_in(Manager& m, Request& r) {
  for (int32_t cb : r.cpu_blocks) {
    const int32_t b = pop_gpu(m);
    r.blocks.push_back(b);
    m.p_swap_in.push_back(cb);
    m.p_swap_in.push_back(b);
  }
  m.totals.swapped_in_blocks += int64_t(r.cpu_blocks.size());
  release_cpu(m, r);
  set_state(m, r, PA_REQ_RUNNING);
}

std::vector<Request*> snapshot(Manager& m, int32_t state) {
  std::vector<Request*> v;
  v.reserve(m.by_state[state].size());
  for (auto& kv : m.by_state[state]) v.push_back(kv.second);
  return v;
}

void schedule_step(Manager& m, int64_t budget) {
  m.scheduled.clear();
  m.p_seq_ids.clear(); m.p_slots.clear(); m.p_cow.clear(); m.p_swap_out.clear();
  m.p_swap_in.clear(); m.p_preempted.clear(); m.p_modes.clear(); m.p_context_lens.clear();
  m.p_query_start.assign(1, 0);
  m.deferred.clear();

  // 1. running requests, earliest arrival first
  std::vector<Request*> order = snapshot(m, PA_REQ_RUNNING);
  size_t end = order.size();
  for (size_t i = 0; i < end;) {
    Request& r = *order[i];
    const int64_t n = std::min<int64_t>(int64_t(r.tokens.size()) - r.computed, budget);
    if (n == 0) {
      ++i;
      continue;
    }
    bool preempted_self = false;
    while (blocks_to_grow(m, r, n) > m.free_gpu.size()) {
      Request* victim = order[--end];
      preempt(m, *victim);
      if (victim == &r) {
        preempted_self = true;
        break;
      }
    }
    if (preempted_self) break;
    schedule_tokens(m, r, n);
    budget -= n;
    ++i;
  }

  // 2. swapped, then waiting requests, only in a step without preemption
  if (m.p_preempted.empty()) {
    bool stopped = false;
    for (Request* rp : snapshot(m, PA_REQ_SWAPPED)) {
      Request& r = *rp;
      const int64_t n = std::min<int64_t>(int64_t(r.tokens.size()) - r.computed, budget);
      if (budget == 0 || m.free_gpu.size() - blocks_for(m, r.computed + n) < m.watermark) {
        stopped = true;
        break;
      }
      swap_in(m, r);
      if (n) {
        schedule_tokens(m, r, n);
        budget -= n;
      }
    }
    if (!stopped) {
      std::vector<int32_t> hits;
      for (Request* rp : snapshot(m, PA_REQ_WAITING)) {
        Request& r = *rp;
        if (budget == 0) break;
        hits.clear();
        if (m.prefix_caching) {
          const int64_t max_hits = (int64_t(r.tokens.size()) - 1) / m.B;
          for (int64_t j = 0; j < max_hits; ++j) {
            const int32_t b = lookup(m, r, j);
            if (b < 0) break;
            hits.push_back(b);
          }
        }
        const int64_t cached = int64_t(hits.size()) * m.B;
        const int64_t n = std::min<int64_t>(int64_t(r.tokens.size()) - cached, budget);
        int64_t from_free = 0;
        for (int32_t b : hits) from_free += m.refcount[size_t(b)] == 0 ? 1 : 0;
        const int64_t need =
            blocks_for(m, int64_t(r.tokens.size())) - int64_t(hits.size()) + from_free;
        if (m.free_gpu.size() - need < m.watermark) break;
        for (int32_t b : hits) {
          if (m.refcount[size_t(b)] == 0) m.free_gpu.unlink(b);
          ++m.refcount[size_t(b)];
        }
        r.blocks.assign(hits.begin(), hits.end());
        r.computed = cached;
        set_state(m, r, PA_REQ_RUNNING);
        m.totals.prefix_hit_tokens += cached;
        m.totals.admitted_tokens += int64_t(r.tokens.size());
        schedule_tokens(m, r, n);
        budget -= n;
      }
    }
  }

  for (int32_t b : m.deferred) m.free_gpu.push_back(b);
  m.deferred.clear();
  for (int32_t b : m.cow_marked) m.cow_source[size_t(b)] = 0;
  m.cow_marked.clear();

  // block tables of the scheduled requests, as they stand at the end of the step
  size_t width = 1;
  for (Request* r : m.scheduled) width = std::max(width, r->blocks.size());
  m.p_tables.assign(m.scheduled.size() * width, 0);
  for (size_t k = 0; k < m.scheduled.size(); ++k)
    std::copy(m.scheduled[k]->blocks.begin(), m.scheduled[k]->blocks.end(),
              m.p_tables.begin() + k * width);
}

Request* find(Manager* m, int64_t rid) {
  auto it = m->requests.find(rid);
  return it == m->requests.end() ? nullptr : &it->second;
}

const Request* find(const Manager* m, int64_t rid) {
  auto it = m->requests.find(rid);
  return it == m->requests.end() ? nullptr : &it->second;
}

template <class F>
int guarded(const char* fn, F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return fail(PA_ERR_NOMEM, "%s: out of host memory", fn);
  } catch (...) {
    return fail(PA_ERR_NOMEM, "%s: unexpected host exception", fn);
  }
}

}  // namespace
}  // namespace pa

using pa::fail;

static constexpr int64_t kMaxTokens = std::numeric_limits<int32_t>::max();

PA_API int pa_bm_create(const pa_bm_config* cfg, pa_block_manager** out) {
  if (!cfg || !out) return fail(PA_ERR_NULL, "pa_bm_create: config or out is NULL");
  *out = nullptr;
  constexpr int64_t kMaxIds = std::numeric_limits<int32_t>::max();
  if (cfg->num_gpu_blocks < 1 || cfg->num_gpu_blocks > kMaxIds || cfg->num_cpu_blocks < 0 ||
      cfg->num_cpu_blocks > kMaxIds || cfg->block_size < 1 || cfg->watermark_blocks < 0 ||
      (cfg->prefix_caching != 0 && cfg->prefix_caching != 1) ||
      (cfg->preempt_mode != PA_PREEMPT_RECOMPUTE && cfg->preempt_mode != PA_PREEMPT_SWAP))
    return fail(PA_ERR_SHAPE, "pa_bm_create: configuration out of range");
  if (double(cfg->num_gpu_blocks) * cfg->block_size > 9.0e18)
    return fail(PA_ERR_SHAPE, "pa_bm_create: slot ids overflow int64");
  return pa::guarded("pa_bm_create", [&] {
    auto* m = new pa_block_manager();
    try {
      m->B = cfg->block_size;
      m->num_gpu = cfg->num_gpu_blocks;
      m->num_cpu = cfg->num_cpu_blocks;
      m->prefix_caching = cfg->prefix_caching != 0;
      m->mode = cfg->preempt_mode;
      m->watermark = cfg->watermark_blocks;
      m->free_gpu.init(m->num_gpu);
      m->free_cpu.init(m->num_cpu);
      m->refcount.assign(size_t(m->num_gpu), 0);
      m->cow_source.assign(size_t(m->num_gpu), 0);
      m->keyed.assign(size_t(m->num_gpu), 0);
      if (m->prefix_caching) {
        m->block_key.resize(size_t(m->num_gpu));
        m->block_parent.resize(size_t(m->num_gpu));
        m->block_tokens.resize(size_t(m->num_gpu) * size_t(m->B));
      }
      m->p_query_start.assign(1, 0);
    } catch (...) {
      delete m;
      throw;
    }
    *out = m;
    return int(PA_OK);
  });
}

PA_API void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

PA_API int pa_bm_add_request(pa_block_manager* bm, int64_t rid, const int32_t* tokens,
                             int64_t num_tokens) {
  if (!bm || !tokens) return fail(PA_ERR_NULL, "pa_bm_add_request: manager or tokens is NULL");
  if (num_tokens <= 0 || num_tokens > kMaxTokens)
    return fail(PA_ERR_SHAPE, "pa_bm_add_request: prompt length out of [1, 2^31 - 1]");
  if (pa::blocks_for(*bm, num_tokens) > bm->num_gpu - bm->watermark)
    return fail(PA_ERR_SHAPE, "pa_bm_add_request: a %lld-token prompt can never fit the pool",
                (long long)num_tokens);
  if (bm->requests.count(rid)) return fail(PA_ERR_ID, "pa_bm_add_request: request %lld exists", (long long)rid);
  return pa::guarded("pa_bm_add_request", [&] {
    pa::Request r;
    r.rid = rid;
    r.arrival = bm->arrivals;
    r.tokens.assign(tokens, tokens + num_tokens);
    auto& slot = bm->requests.emplace(rid, std::move(r)).first->second;
    bm->by_state[PA_REQ_WAITING].emplace(slot.arrival, &slot);
    ++bm->arrivals;
    return int(PA_OK);
  });
}

PA_API int pa_bm_append_tokens(pa_block_manager* bm, int64_t rid, const int32_t* tokens,
                               int64_t num_tokens) {
  if (!bm) return fail(PA_ERR_NULL, "pa_bm_append_tokens: manager is NULL");
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "pa_bm_append_tokens: num_tokens < 0");
  if (num_tokens > 0 && !tokens) return fail(PA_ERR_NULL, "pa_bm_append_tokens: tokens is NULL");
  pa::Request* r = pa::find(bm, rid);
  if (!r) return fail(PA_ERR_ID, "pa_bm_append_tokens: no request %lld", (long long)rid);
  if (num_tokens > kMaxTokens - int64_t(r->tokens.size()))
    return fail(PA_ERR_SHAPE, "pa_bm_append_tokens: a request holds at most 2^31 - 1 tokens");
  return pa::guarded("pa_bm_append_tokens", [&] {
    r->tokens.insert(r->tokens.end(), tokens, tokens + num_tokens);
    return int(PA_OK);
  });
}

PA_API int pa_bm_append_batch(pa_block_manager* bm, const int64_t* rids, const int32_t* tokens,
                              int64_t n) {
  if (!bm) return fail(PA_ERR_NULL, "pa_bm_append_batch: manager is NULL");
  if (n < 0) return fail(PA_ERR_SHAPE, "pa_bm_append_batch: n < 0");
  if (n == 0) return PA_OK;
  if (!rids || !tokens) return fail(PA_ERR_NULL, "pa_bm_append_batch: rids or tokens is NULL");
  for (int64_t i = 0; i < n; ++i) {
    const pa::Request* r = pa::find(bm, rids[i]);
    if (!r) return fail(PA_ERR_ID, "pa_bm_append_batch: no request %lld", (long long)rids[i]);
    // (a repeated id appends more than once; the bound below is checked per entry)
    if (int64_t(r->tokens.size()) >= kMaxTokens - n)
      return fail(PA_ERR_SHAPE, "pa_bm_append_batch: a request holds at most 2^31 - 1 tokens");
  }
  return pa::guarded("pa_bm_append_batch", [&] {
    for (int64_t i = 0; i < n; ++i) pa::find(bm, rids[i])->tokens.push_back(tokens[i]);
    return int(PA_OK);
  });
}

PA_API int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return fail(PA_ERR_NULL, "pa_bm_fork: manager is NULL");
  pa::Request* p = pa::find(bm, parent);
  if (!p) return fail(PA_ERR_ID, "pa_bm_fork: no request %lld", (long long)parent);
  if (bm->requests.count(child)) return fail(PA_ERR_ID, "pa_bm_fork: request %lld exists", (long long)child);
  if (p->state != PA_REQ_RUNNING) return fail(PA_ERR_STATE, "pa_bm_fork: the parent is not running");
  return pa::guarded("pa_bm_fork", [&] {
    pa::Request c;
    c.rid = child;
    c.arrival = bm->arrivals;
    c.state = PA_REQ_RUNNING;
    c.computed = p->computed;
    c.tokens = p->tokens;
    c.blocks = p->blocks;
    c.keys = p->keys;
    auto& slot = bm->requests.emplace(child, std::move(c)).first->second;
    bm->by_state[PA_REQ_RUNNING].emplace(slot.arrival, &slot);
    ++bm->arrivals;
    for (int32_t b : slot.blocks) ++bm->refcount[size_t(b)];
    return int(PA_OK);
  });
}

PA_API int pa_bm_finish(pa_block_manager* bm, int64_t rid) {
  if (!bm) return fail(PA_ERR_NULL, "pa_bm_finish: manager is NULL");
  pa::Request* r = pa::find(bm, rid);
  if (!r) return fail(PA_ERR_ID, "pa_bm_finish: no request %lld", (long long)rid);
  pa::release_gpu(*bm, *r);
  pa::release_cpu(*bm, *r);
  bm->by_state[r->state].erase(r->arrival);
  bm->requests.erase(rid);
  return PA_OK;
}

PA_API int pa_bm_schedule(pa_block_manager* bm, int64_t token_budget, pa_step_plan* plan) {
  if (!bm || !plan) return fail(PA_ERR_NULL, "pa_bm_schedule: manager or plan is NULL");
  if (token_budget <= 0 || token_budget > std::numeric_limits<int32_t>::max())
    return fail(PA_ERR_SHAPE, "pa_bm_schedule: token_budget must be in [1, 2^31 - 1]");
  const int st = pa::guarded("pa_bm_schedule", [&] {
    pa::schedule_step(*bm, token_budget);
    return int(PA_OK);
  });
  if (st != PA_OK) return st;
  const int32_t S = int32_t(bm->p_seq_ids.size());
  plan->num_seqs = S;
  plan->num_tokens = bm->p_query_start.back();
  plan->max_blocks = S ? int32_t(bm->p_tables.size() / size_t(S)) : 1;
  plan->num_cow = int32_t(bm->p_cow.size() / 2);
  plan->num_swap_out = int32_t(bm->p_swap_out.size() / 2);
  plan->num_swap_in = int32_t(bm->p_swap_in.size() / 2);
  plan->num_preempted = int32_t(bm->p_preempted.size());
  plan->seq_ids = bm->p_seq_ids.data();
  plan->query_start = bm->p_query_start.data();
  plan->context_lens = bm->p_context_lens.data();
  plan->slot_mapping = bm->p_slots.data();
  plan->block_tables = bm->p_tables.data();
  plan->cow_pairs = bm->p_cow.data();
  plan->swap_out_pairs = bm->p_swap_out.data();
  plan->swap_in_pairs = bm->p_swap_in.data();
  plan->preempted_ids = bm->p_preempted.data();
  plan->preempted_modes = bm->p_modes.data();
  return PA_OK;
}

PA_API int pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* out) {
  if (!bm || !out) return fail(PA_ERR_NULL, "pa_bm_get_stats: manager or out is NULL");
  *out = bm->totals;
  out->free_gpu_blocks = bm->free_gpu.size();
  out->free_cpu_blocks = bm->free_cpu.size();
  out->cached_blocks = int64_t(bm->cache.size());
  out->running = int64_t(bm->by_state[PA_REQ_RUNNING].size());
  out->waiting = int64_t(bm->by_state[PA_REQ_WAITING].size());
  out->swapped = int64_t(bm->by_state[PA_REQ_SWAPPED].size());
  return PA_OK;
}

PA_API int pa_bm_request_info(const pa_block_manager* bm, int64_t rid, pa_request_info* out) {
  if (!bm || !out) return fail(PA_ERR_NULL, "pa_bm_request_info: manager or out is NULL");
  const pa::Request* r = pa::find(bm, rid);
  if (!r) return fail(PA_ERR_ID, "pa_bm_request_info: no request %lld", (long long)rid);
  out->state = r->state;
  out->reserved = 0;
  out->arrival = r->arrival;
  out->num_tokens = int64_t(r->tokens.size());
  out->computed = r->computed;
  out->num_blocks = int64_t(r->blocks.size());
  out->num_cpu_blocks = int64_t(r->cpu_blocks.size());
  return PA_OK;
}

PA_API int pa_bm_blocks(const pa_block_manager* bm, int64_t rid, int32_t cpu, int32_t* out,
                        int64_t capacity, int64_t* count) {
  if (!bm || !count || (capacity > 0 && !out))
    return fail(PA_ERR_NULL, "pa_bm_blocks: manager, out or count is NULL");
  const pa::Request* r = pa::find(bm, rid);
  if (!r) return fail(PA_ERR_ID, "pa_bm_blocks: no request %lld", (long long)rid);
  const std::vector<int32_t>& v = cpu ? r->cpu_blocks : r->blocks;
  *count = int64_t(v.size());
  std::copy_n(v.begin(), size_t(std::max<int64_t>(0, std::min<int64_t>(capacity, *count))), out);
  return PA_OK;
}

PA_API int pa_bm_refcounts(const pa_block_manager* bm, int32_t* out, int64_t capacity) {
  if (!bm || !out) return fail(PA_ERR_NULL, "pa_bm_refcounts: manager or out is NULL");
  if (capacity < bm->num_gpu) return fail(PA_ERR_SHAPE, "pa_bm_refcounts: capacity < num_gpu_blocks");
  std::copy(bm->refcount.begin(), bm->refcount.end(), out);
  return PA_OK;
}

PA_API int pa_bm_free_list(const pa_block_manager* bm, int32_t cpu, int32_t* out,
                           int64_t capacity, int64_t* count) {
  if (!bm || !count || (capacity > 0 && !out))
    return fail(PA_ERR_NULL, "pa_bm_free_list: manager, out or count is NULL");
  *count = (cpu ? bm->free_cpu : bm->free_gpu).copy_out(out, capacity);
  return PA_OK;
}
