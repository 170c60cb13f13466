// Host-side KV block manager and step scheduler (C ABI in pagedattn_kvm.h).
//
// The block manager follows the description in the mistral.rs comparison
// page (paged-attention section): a flat pool of fixed-size blocks with an
// LRU free list, reference counts for blocks shared between requests, and
// content-addressed hashing of full blocks so that a new request reuses the
// longest cached chain of blocks matching its leading tokens.  The
// scheduler follows the same page's scheduling section: a step is either
// all prompt (chunks under a token budget) or all decode, with a bound on
// consecutive decode steps.  TensorSharp's Mistral 3 page, section 11,
// reports the same kind of reuse counters for its block-hash prefix cache.
//
// Host memory only; nothing here touches the GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <unordered_map>
#include <vector>

#include "pa_error.h"
#include "pagedattn.h"
#include "pagedattn_kvm.h"

namespace {

// 64-bit mixing of the splitmix64 finaliser; hash of a block = chain of the
// parent block's hash and the block's token ids
uint64_t mix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

uint64_t block_hash(uint64_t parent, const int32_t *tokens, int n) {
  uint64_t h = mix64(parent ^ 0x5a5a5a5a5a5a5a5aull);
  for (int i = 0; i < n; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i]);
  return h ? h : 1;
}

struct Block {
  int32_t ref = 0;
  int32_t prev = -1, next = -1;  // free-list links
  bool in_free = false;
  bool cached = false;
  uint64_t hash = 0, parent = 0;
  std::vector<int32_t> tokens;   // content of a cached block (verified on lookup)
};

struct Request {
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;
  std::vector<uint64_t> hashes;  // hashes of the leading full blocks
  int32_t num_computed = 0;
};

}  // namespace

struct pa_kvm {
  int32_t num_blocks, block_size;
  bool prefix_cache;
  std::vector<Block> blocks;
  int32_t head = -1, tail = -1, free_count = 0;
  std::unordered_map<uint64_t, int32_t> cache;  // hash -> block id
  std::unordered_map<int64_t, Request> requests;
  pa_kvm_stats stats{};

  void push_head(int32_t b) {
    Block &x = blocks[b];
    x.prev = -1;
    x.next = head;
    if (head >= 0) blocks[head].prev = b;
    else tail = b;
    head = b;
    x.in_free = true;
    ++free_count;
  }
  void push_tail(int32_t b) {
    Block &x = blocks[b];
    x.prev = tail;
    x.next = -1;
    if (tail >= 0) blocks[tail].next = b;
    else head = b;
    tail = b;
    x.in_free = true;
    ++free_count;
  }
  void unlink(int32_t b) {
    Block &x = blocks[b];
    if (x.prev >= 0) blocks[x.prev].next = x.next;
    else head = x.next;
    if (x.next >= 0) blocks[x.next].prev = x.prev;
    else tail = x.prev;
    x.prev = x.next = -1;
    x.in_free = false;
    --free_count;
  }
  int32_t pop_head() {
    const int32_t b = head;
    unlink(b);
    Block &x = blocks[b];
    if (x.cached) {  // recycle a cached block: forget its content
      auto it = cache.find(x.hash);
      if (it != cache.end() && it->second == b) cache.erase(it);
      x.cached = false;
      x.tokens.clear();
      ++stats.evictions;
    }
    return b;
  }
};

struct pa_sched {
  enum Phase { kWaiting, kPrefill, kRunning };
  struct SReq {
    int32_t max_new = 0;
    int32_t generated = 0;
    Phase phase = kWaiting;
  };
  pa_kvm *kvm;
  pa_sched_config cfg;
  std::unordered_map<int64_t, SReq> reqs;
  std::deque<int64_t> waiting;   // not admitted, in arrival order (preempted ones first)
  std::vector<int64_t> admitted; // prefilling or decoding, in admission order
  int32_t decode_streak = 0;
  int32_t finished = 0;
};

namespace {

Request *find(pa_kvm *m, int64_t id) {
  auto it = m->requests.find(id);
  return it == m->requests.end() ? nullptr : &it->second;
}
const Request *find(const pa_kvm *m, int64_t id) {
  auto it = m->requests.find(id);
  return it == m->requests.end() ? nullptr : &it->second;
}

int blocks_for(int32_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

}  // namespace

extern "C" {

pa_kvm *pa_kvm_create(int32_t num_blocks, int32_t block_size, int32_t enable_prefix_cache) {
  if (num_blocks <= 0) {
    pa::set_error(PA_ERR_SHAPE, "num_blocks %d must be > 0", num_blocks);
    return nullptr;
  }
  if (block_size != 8 && block_size != 16 && block_size != 32) {
    pa::set_error(PA_ERR_BLOCK_SIZE, "block_size %d not in {8, 16, 32}", block_size);
    return nullptr;
  }
  pa_kvm *m = new pa_kvm;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->prefix_cache = enable_prefix_cache != 0;
  m->blocks.resize(num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) m->push_tail(b);
  m->stats.num_blocks = num_blocks;
  m->stats.block_size = block_size;
  pa::clear_error();
  return m;
}

void pa_kvm_destroy(pa_kvm *m) { delete m; }

int pa_kvm_add_request(pa_kvm *m, int64_t id, const int32_t *tokens, int32_t n) {
  if (!m) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  if (n < 0 || (n > 0 && !tokens)) return pa::set_error(PA_ERR_SHAPE, "num_tokens %d with tokens %p", n, (const void *)tokens);
  if (find(m, id)) return pa::set_error(PA_ERR_REQUEST, "request %lld already exists", (long long)id);
  Request &r = m->requests[id];
  r.tokens.assign(tokens, tokens + n);
  ++m->stats.active_requests;
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_append_tokens(pa_kvm *m, int64_t id, const int32_t *tokens, int32_t n) {
  if (!m) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  Request *r = find(m, id);
  if (!r) return pa::set_error(PA_ERR_REQUEST, "unknown request %lld", (long long)id);
  if (n < 0 || (n > 0 && !tokens)) return pa::set_error(PA_ERR_SHAPE, "num_tokens %d with tokens %p", n, (const void *)tokens);
  r->tokens.insert(r->tokens.end(), tokens, tokens + n);
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_get_computed_blocks(pa_kvm *m, int64_t id, int32_t *num_computed) {
  if (!m || !num_computed) return pa::set_error(PA_ERR_NULL, "manager or output is NULL");
  Request *r = find(m, id);
  if (!r) return pa::set_error(PA_ERR_REQUEST, "unknown request %lld", (long long)id);
  if (!r->blocks.empty()) return pa::set_error(PA_ERR_REQUEST, "request %lld already holds blocks", (long long)id);
  const int32_t bs = m->block_size;
  ++m->stats.prefix_queries;
  if (m->prefix_cache && !r->tokens.empty()) {
    const int32_t max_blocks = ((int32_t)r->tokens.size() - 1) / bs;  // leave one token to compute
    uint64_t parent = 0;
    for (int32_t j = 0; j < max_blocks; ++j) {
      const int32_t *tok = r->tokens.data() + (size_t)j * bs;
      const uint64_t h = block_hash(parent, tok, bs);
      auto it = m->cache.find(h);
      if (it == m->cache.end()) break;
      Block &b = m->blocks[it->second];
      if (!b.cached || b.parent != parent || memcmp(b.tokens.data(), tok, sizeof(int32_t) * bs) != 0) break;
      if (b.ref == 0) m->unlink(it->second);
      ++b.ref;
      r->blocks.push_back(it->second);
      r->hashes.push_back(h);
      parent = h;
    }
    r->num_computed = (int32_t)r->blocks.size() * bs;
    m->stats.prefix_hit_blocks += (int64_t)r->blocks.size();
    m->stats.prefix_hit_tokens += r->num_computed;
  }
  *num_computed = r->num_computed;
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_allocate_slots(pa_kvm *m, int64_t id, int32_t n) {
  if (!m) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  Request *r = find(m, id);
  if (!r) return pa::set_error(PA_ERR_REQUEST, "unknown request %lld", (long long)id);
  if (n < 0) return pa::set_error(PA_ERR_SHAPE, "num_new_tokens %d must be >= 0", n);
  const int32_t need = blocks_for(r->num_computed + n, m->block_size) - (int32_t)r->blocks.size();
  if (need > m->free_count)
    return pa::set_error(PA_ERR_NO_BLOCKS, "request %lld needs %d more blocks, %d free", (long long)id, need,
                         m->free_count);
  for (int32_t i = 0; i < need; ++i) {
    const int32_t b = m->pop_head();
    m->blocks[b].ref = 1;
    r->blocks.push_back(b);
  }
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_commit(pa_kvm *m, int64_t id, int32_t n) {
  if (!m) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  Request *r = find(m, id);
  if (!r) return pa::set_error(PA_ERR_REQUEST, "unknown request %lld", (long long)id);
  const int32_t bs = m->block_size;
  if (n < 0 || r->num_computed + n > (int32_t)r->tokens.size() ||
      r->num_computed + n > (int32_t)r->blocks.size() * bs)
    return pa::set_error(PA_ERR_SHAPE, "commit of %d tokens: %d computed, %zu tokens, %zu blocks", n,
                         r->num_computed, r->tokens.size(), r->blocks.size());
  r->num_computed += n;
  for (int32_t j = (int32_t)r->hashes.size(); (j + 1) * bs <= r->num_computed; ++j) {
    const uint64_t parent = j ? r->hashes[j - 1] : 0;
    const int32_t *tok = r->tokens.data() + (size_t)j * bs;
    const uint64_t h = block_hash(parent, tok, bs);
    r->hashes.push_back(h);
    if (!m->prefix_cache || m->cache.count(h)) continue;  // an equal block is cached already
    Block &b = m->blocks[r->blocks[j]];
    b.cached = true;
    b.hash = h;
    b.parent = parent;
    b.tokens.assign(tok, tok + bs);
    m->cache[h] = r->blocks[j];
  }
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_free(pa_kvm *m, int64_t id) {
  if (!m) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  Request *r = find(m, id);
  if (!r) return pa::set_error(PA_ERR_REQUEST, "unknown request %lld", (long long)id);
  for (auto it = r->blocks.rbegin(); it != r->blocks.rend(); ++it) {
    Block &b = m->blocks[*it];
    if (--b.ref == 0) m->push_tail(*it);
  }
  m->requests.erase(id);
  --m->stats.active_requests;
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_block_table(const pa_kvm *m, int64_t id, int32_t *table, int32_t max_blocks, int32_t *num_blocks) {
  if (!m || !num_blocks) return pa::set_error(PA_ERR_NULL, "manager or output is NULL");
  const Request *r = find(m, id);
  if (!r) return pa::set_error(PA_ERR_REQUEST, "unknown request %lld", (long long)id);
  *num_blocks = (int32_t)r->blocks.size();
  const int32_t k = std::min<int32_t>(max_blocks, (int32_t)r->blocks.size());
  if (k > 0 && !table) return pa::set_error(PA_ERR_NULL, "table is NULL");
  for (int32_t i = 0; i < k; ++i) table[i] = r->blocks[i];
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_slot_mapping(const pa_kvm *m, int64_t id, int32_t first, int32_t count, int64_t *slots) {
  if (!m) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  const Request *r = find(m, id);
  if (!r) return pa::set_error(PA_ERR_REQUEST, "unknown request %lld", (long long)id);
  const int32_t bs = m->block_size;
  if (first < 0 || count < 0 || first + count > (int32_t)r->blocks.size() * bs)
    return pa::set_error(PA_ERR_SHAPE, "positions %d..%d not covered by %zu blocks of %d", first,
                         first + count - 1, r->blocks.size(), bs);
  if (count > 0 && !slots) return pa::set_error(PA_ERR_NULL, "slots is NULL");
  for (int32_t i = 0; i < count; ++i) {
    const int32_t p = first + i;
    slots[i] = (int64_t)r->blocks[p / bs] * bs + p % bs;
  }
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_request_info(const pa_kvm *m, int64_t id, int32_t *num_tokens, int32_t *num_computed,
                        int32_t *num_blocks) {
  if (!m) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  const Request *r = find(m, id);
  if (!r) return pa::set_error(PA_ERR_REQUEST, "unknown request %lld", (long long)id);
  if (num_tokens) *num_tokens = (int32_t)r->tokens.size();
  if (num_computed) *num_computed = r->num_computed;
  if (num_blocks) *num_blocks = (int32_t)r->blocks.size();
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_get_stats(const pa_kvm *m, pa_kvm_stats *s) {
  if (!m || !s) return pa::set_error(PA_ERR_NULL, "manager or output is NULL");
  *s = m->stats;
  s->free_blocks = m->free_count;
  s->cached_blocks = (int64_t)m->cache.size();
  pa::clear_error();
  return PA_OK;
}

int pa_kvm_grow(pa_kvm *m, int32_t new_num_blocks) {
  if (!m) return pa::set_error(PA_ERR_NULL, "manager is NULL");
  if (new_num_blocks < m->num_blocks)
    return pa::set_error(PA_ERR_SHAPE, "new_num_blocks %d below the current %d (a pool only grows)", new_num_blocks,
                         m->num_blocks);
  const int32_t old = m->num_blocks;
  m->blocks.resize(new_num_blocks);
  // fresh blocks in front, lowest id first
  for (int32_t b = new_num_blocks - 1; b >= old; --b) m->push_head(b);
  m->num_blocks = new_num_blocks;
  m->stats.num_blocks = new_num_blocks;
  pa::clear_error();
  return PA_OK;
}

// ------------------------------------------------------------------ scheduler

pa_sched *pa_sched_create(pa_kvm *kvm, const pa_sched_config *cfg) {
  if (!kvm || !cfg) {
    pa::set_error(PA_ERR_NULL, "manager or config is NULL");
    return nullptr;
  }
  if (cfg->max_batched_tokens <= 0 || cfg->max_chunk_tokens <= 0 || cfg->max_decode_steps <= 0 ||
      cfg->min_decode_steps < 0 || cfg->max_seqs <= 0) {
    pa::set_error(PA_ERR_SHAPE, "scheduler limits must be positive (min_decode_steps >= 0)");
    return nullptr;
  }
  pa_sched *s = new pa_sched;
  s->kvm = kvm;
  s->cfg = *cfg;
  pa::clear_error();
  return s;
}

void pa_sched_destroy(pa_sched *s) { delete s; }

int pa_sched_add_request(pa_sched *s, int64_t id, const int32_t *prompt, int32_t prompt_len, int32_t max_new) {
  if (!s) return pa::set_error(PA_ERR_NULL, "scheduler is NULL");
  if (prompt_len <= 0 || !prompt || max_new < 0)
    return pa::set_error(PA_ERR_SHAPE, "prompt_len %d (prompt %p), max_new_tokens %d", prompt_len,
                         (const void *)prompt, max_new);
  if (s->reqs.count(id)) return pa::set_error(PA_ERR_REQUEST, "request %lld already exists", (long long)id);
  const int st = pa_kvm_add_request(s->kvm, id, prompt, prompt_len);
  if (st) return st;
  auto &q = s->reqs[id];
  q.max_new = max_new;
  s->waiting.push_back(id);
  pa::clear_error();
  return PA_OK;
}

}  // extern "C"

namespace {

// Appends one sequence (its block table row, slots and offsets) to a step.
int step_add(pa_step *st, pa_kvm *kvm, int64_t id, int32_t first, int32_t count) {
  const int32_t i = st->num_seqs;
  int32_t *row = st->block_tables + (size_t)i * st->cap_blocks;
  int32_t nb = 0;
  int rc = pa_kvm_block_table(kvm, id, row, st->cap_blocks, &nb);
  if (rc) return rc;
  for (int32_t j = nb; j < st->cap_blocks; ++j) row[j] = 0;
  rc = pa_kvm_slot_mapping(kvm, id, first, count, st->slot_mapping + st->num_tokens);
  if (rc) return rc;
  st->request_ids[i] = id;
  st->query_start_loc[i] = st->num_tokens;
  st->num_tokens += count;
  st->query_start_loc[i + 1] = st->num_tokens;
  st->context_lens[i] = first + count;
  st->max_query_len = std::max(st->max_query_len, count);
  st->max_context_len = std::max(st->max_context_len, first + count);
  st->num_seqs = i + 1;
  return PA_OK;
}

bool in_step(const pa_step *st, int64_t id) {
  return std::find(st->request_ids, st->request_ids + st->num_seqs, id) != st->request_ids + st->num_seqs;
}

// Drops a request's blocks and computed state but keeps its tokens, so that
// it can be admitted again later (recomputation).
void reset_request(pa_kvm *kvm, int64_t id) {
  std::vector<int32_t> tokens = find(kvm, id)->tokens;
  pa_kvm_free(kvm, id);
  pa_kvm_add_request(kvm, id, tokens.data(), (int32_t)tokens.size());
}

// Preempts the most recently admitted request that was admitted after
// `keep` and is not in the step: it goes back to the front of the waiting
// queue (and later recomputes its tokens).
bool preempt_one(pa_sched *s, const pa_step *st, int64_t keep) {
  const size_t pos = (size_t)(std::find(s->admitted.begin(), s->admitted.end(), keep) - s->admitted.begin());
  for (size_t j = s->admitted.size(); j-- > pos + 1;) {
    const int64_t v = s->admitted[j];
    if (in_step(st, v)) continue;
    s->admitted.erase(s->admitted.begin() + (ptrdiff_t)j);
    reset_request(s->kvm, v);
    s->reqs[v].phase = pa_sched::kWaiting;
    s->waiting.push_front(v);
    return true;
  }
  return false;
}

constexpr int kWait = 1;  // not an error: the request waits for a later step

// Allocates slots for an admitted request, preempting later admissions
// while the pool is short.  kWait when blocks are held by earlier requests
// or by this step; PA_ERR_NO_BLOCKS when the request is the oldest and the
// step is empty, so that the whole pool cannot hold it.
int grow_admitted(pa_sched *s, const pa_step *st, int64_t id, int32_t n) {
  while (pa_kvm_allocate_slots(s->kvm, id, n) != PA_OK) {
    if (preempt_one(s, st, id)) continue;
    if (st->num_seqs == 0 && s->admitted.front() == id)
      return pa::set_error(PA_ERR_NO_BLOCKS, "request %lld does not fit in a pool of %d blocks", (long long)id,
                           s->kvm->num_blocks);
    return kWait;
  }
  return PA_OK;
}

}  // namespace

namespace {

// Prompt work of a step under `budget` tokens: partly computed prompts in
// admission order, then waiting requests first come, first served.
int fill_prompts(pa_sched *s, pa_step *st, int32_t &budget, int32_t seq_cap) {
  pa_kvm *kvm = s->kvm;
  const int32_t bs = kvm->block_size;
  const std::vector<int64_t> order = s->admitted;
  for (int64_t id : order) {
    if (budget <= 0 || st->num_seqs >= seq_cap) break;
    if (s->reqs[id].phase != pa_sched::kPrefill) continue;
    if (std::find(s->admitted.begin(), s->admitted.end(), id) == s->admitted.end()) continue;  // preempted
    const Request *r = find(kvm, id);
    const int32_t ntok = (int32_t)r->tokens.size(), done = r->num_computed;
    if (blocks_for(ntok, bs) > st->cap_blocks)
      return pa::set_error(PA_ERR_SHAPE, "request %lld needs %d blocks, step rows hold %d", (long long)id,
                           blocks_for(ntok, bs), st->cap_blocks);
    const int32_t chunk = std::min({ntok - done, s->cfg.max_chunk_tokens, budget});
    const int rc = grow_admitted(s, st, id, chunk);
    if (rc == kWait) break;
    if (rc) return rc;
    step_add(st, kvm, id, done, chunk);
    budget -= chunk;
  }
  while (!s->waiting.empty() && budget > 0 && st->num_seqs < seq_cap) {
    const int64_t id = s->waiting.front();
    const Request *r = find(kvm, id);
    const int32_t ntok = (int32_t)r->tokens.size();
    if (blocks_for(ntok, bs) > st->cap_blocks)
      return pa::set_error(PA_ERR_SHAPE, "request %lld needs %d blocks, step rows hold %d", (long long)id,
                           blocks_for(ntok, bs), st->cap_blocks);
    int32_t done = 0;
    pa_kvm_get_computed_blocks(kvm, id, &done);
    const int32_t chunk = std::min({ntok - done, s->cfg.max_chunk_tokens, budget});
    if (pa_kvm_allocate_slots(kvm, id, chunk) != PA_OK) {
      reset_request(kvm, id);  // give back the prefix blocks it attached
      if (s->admitted.empty() && st->num_seqs == 0)
        return pa::set_error(PA_ERR_NO_BLOCKS, "request %lld does not fit in a pool of %d blocks", (long long)id,
                             kvm->num_blocks);
      break;
    }
    s->waiting.pop_front();
    s->reqs[id].phase = pa_sched::kPrefill;
    s->admitted.push_back(id);
    step_add(st, kvm, id, done, chunk);
    budget -= chunk;
  }
  return PA_OK;
}

// One new token for every decoding sequence, in admission order, while the
// budget and the step's rows last.
int fill_decodes(pa_sched *s, pa_step *st, int32_t &budget, int32_t seq_cap) {
  pa_kvm *kvm = s->kvm;
  const int32_t bs = kvm->block_size;
  const std::vector<int64_t> order = s->admitted;
  for (int64_t id : order) {
    if (st->num_seqs >= seq_cap || budget <= 0) break;
    if (s->reqs[id].phase != pa_sched::kRunning) continue;
    if (std::find(s->admitted.begin(), s->admitted.end(), id) == s->admitted.end()) continue;  // preempted
    const int32_t done = find(kvm, id)->num_computed;
    if (blocks_for(done + 1, bs) > st->cap_blocks)
      return pa::set_error(PA_ERR_SHAPE, "request %lld needs %d blocks, step rows hold %d", (long long)id,
                           blocks_for(done + 1, bs), st->cap_blocks);
    const int rc = grow_admitted(s, st, id, 1);
    if (rc == kWait) continue;
    if (rc) return rc;
    step_add(st, kvm, id, done, 1);
    budget -= 1;
  }
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_sched_next_step(pa_sched *s, pa_step *st) {
  if (!s || !st) return pa::set_error(PA_ERR_NULL, "scheduler or step is NULL");
  if (!st->request_ids || !st->query_start_loc || !st->context_lens || !st->block_tables || !st->slot_mapping ||
      st->cap_seqs <= 0 || st->cap_tokens <= 0 || st->cap_blocks <= 0)
    return pa::set_error(PA_ERR_NULL, "step arrays and capacities must be set");
  st->kind = 0;
  st->num_seqs = st->num_tokens = st->max_query_len = st->max_context_len = 0;
  st->max_blocks_per_seq = st->cap_blocks;
  st->query_start_loc[0] = 0;
  const int32_t seq_cap = std::min(s->cfg.max_seqs, st->cap_seqs);

  if (s->cfg.mixed) {
    // one batch: every decoding sequence's token first, then prompt chunks
    // in the rest of the budget
    int32_t budget = std::min(s->cfg.max_batched_tokens, st->cap_tokens);
    int rc = fill_decodes(s, st, budget, seq_cap);
    if (rc) return rc;
    const int32_t decode_rows = st->num_seqs;
    rc = fill_prompts(s, st, budget, seq_cap);
    if (rc) return rc;
    if (st->num_seqs > 0) st->kind = st->num_seqs == decode_rows ? 2 : (decode_rows == 0 ? 1 : 3);
    pa::clear_error();
    return PA_OK;
  }

  bool has_prefill = false, has_running = false;
  for (int64_t id : s->admitted) (s->reqs[id].phase == pa_sched::kPrefill ? has_prefill : has_running) = true;
  const bool prompt_work = has_prefill || !s->waiting.empty();
  const bool want_prompt = prompt_work && (!has_running || s->decode_streak >= s->cfg.min_decode_steps ||
                                           s->decode_streak >= s->cfg.max_decode_steps);

  if (want_prompt) {
    int32_t budget = std::min(s->cfg.max_batched_tokens, st->cap_tokens);
    const int rc = fill_prompts(s, st, budget, seq_cap);
    if (rc) return rc;
    if (st->num_seqs > 0) {
      st->kind = 1;
      s->decode_streak = 0;
      pa::clear_error();
      return PA_OK;
    }
  }

  // decode step: one new token for every running sequence
  int32_t budget = st->cap_tokens;
  const int rc = fill_decodes(s, st, budget, seq_cap);
  if (rc) return rc;
  if (st->num_seqs > 0) {
    st->kind = 2;
    ++s->decode_streak;
  }
  pa::clear_error();
  return PA_OK;
}

int pa_sched_complete_step(pa_sched *s, const pa_step *st, const int32_t *sampled, int32_t *num_finished) {
  if (!s || !st) return pa::set_error(PA_ERR_NULL, "scheduler or step is NULL");
  int32_t fin = 0;
  for (int32_t i = 0; i < st->num_seqs; ++i) {
    const int64_t id = st->request_ids[i];
    auto it = s->reqs.find(id);
    if (it == s->reqs.end() || it->second.phase == pa_sched::kWaiting)
      return pa::set_error(PA_ERR_REQUEST, "request %lld of the step is not admitted", (long long)id);
    pa_sched::SReq &q = it->second;
    const int rc = pa_kvm_commit(s->kvm, id, st->query_start_loc[i + 1] - st->query_start_loc[i]);
    if (rc) return rc;
    const Request *r = find(s->kvm, id);
    if (r->num_computed < (int32_t)r->tokens.size()) continue;  // prompt not finished: nothing sampled
    q.phase = pa_sched::kRunning;
    if (q.generated >= q.max_new) {
      s->admitted.erase(std::find(s->admitted.begin(), s->admitted.end(), id));
      pa_kvm_free(s->kvm, id);
      s->reqs.erase(it);
      ++fin;
      continue;
    }
    const int32_t tok = sampled ? sampled[i] : 0;
    pa_kvm_append_tokens(s->kvm, id, &tok, 1);
    ++q.generated;
  }
  s->finished += fin;
  if (num_finished) *num_finished = fin;
  pa::clear_error();
  return PA_OK;
}

int pa_sched_counts(const pa_sched *s, int32_t *waiting, int32_t *running, int32_t *finished) {
  if (!s) return pa::set_error(PA_ERR_NULL, "scheduler is NULL");
  if (waiting) *waiting = (int32_t)s->waiting.size();
  if (running) *running = (int32_t)s->admitted.size();
  if (finished) *finished = s->finished;
  pa::clear_error();
  return PA_OK;
}

}  // extern "C"
