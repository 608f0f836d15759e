// Paged KV store and working sets; see kvstore.h.
#include "kvstore.h"

#include <algorithm>

#include "pie.h"

namespace pie {

void PagePool::reset(int64_t n_pages) {
  refcnt_.assign((size_t)n_pages, 0);
  free_.resize((size_t)n_pages);
  for (int64_t i = 0; i < n_pages; ++i) free_[(size_t)i] = (int32_t)(n_pages - 1 - i);
  ever_allocated_ = 0;
}

int32_t PagePool::take() {
  int32_t p = free_.back();
  free_.pop_back();
  refcnt_[p] = 1;
  ++ever_allocated_;
  return p;
}

void PagePool::unref(int32_t page) {
  if (--refcnt_[page] == 0) free_.push_back(page);
}

// splitmix64 finaliser over (state, token) pairs; two seeds give two
// independent chains.
static inline uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

uint64_t prefix_hash(uint64_t prev, const int32_t* toks, int32_t n, uint64_t seed) {
  uint64_t h = mix64(prev ^ seed);
  for (int32_t i = 0; i < n; ++i) h = mix64(h + (uint64_t)(uint32_t)toks[i] + seed);
  return h | 1;  // never 0, which marks "no key"
}

static constexpr uint64_t SEED1 = 0x9e3779b97f4a7c15ull, SEED2 = 0xd1b54a32d192ed03ull;

void KVStore::unref_page(int32_t page) {
  pool_.unref(page);
  if (pool_.refs(page) == 0 && page_key_[page]) {
    auto it = prefix_.find(page_key_[page]);
    if (it != prefix_.end() && it->second.page == page) prefix_.erase(it);
    page_key_[page] = 0;
  }
}

void KVStore::note_tokens(WorkingSet& ws, const int32_t* tokens, const int32_t* positions, int32_t n) {
  if (!ws.hist_ok) return;
  bool ok = tokens != nullptr && (int32_t)ws.toks.size() == ws.len;
  for (int32_t i = 0; ok && positions && i < n; ++i) ok = positions[i] == ws.len + i;
  if (!ok) {
    ws.hist_ok = false;
    ws.toks.clear();
    ws.toks.shrink_to_fit();
    return;
  }
  ws.toks.insert(ws.toks.end(), tokens, tokens + n);
}

void KVStore::commit(WorkingSet& ws) {
  ws.frozen_len = ws.len;
  if (!ws.hist_ok) return;
  // full pages of the frozen prefix, in order, up to the first partial one
  for (size_t k = ws.chain.size(); k < ws.pages.size(); ++k) {
    const PageEntry& e = ws.pages[k];
    if (e.valid != P_ || (int64_t)(k + 1) * P_ > ws.frozen_len) break;
    const int32_t* t = ws.toks.data() + k * P_;
    const uint64_t h = prefix_hash(k ? ws.chain[k - 1] : 0, t, P_, SEED1);
    const uint64_t h2 = prefix_hash(k ? ws.chain2[k - 1] : 0, t, P_, SEED2);
    ws.chain.push_back(h);
    ws.chain2.push_back(h2);
    if (!prefix_.count(h) && !page_key_[e.page]) {
      prefix_[h] = PrefixEntry{e.page, h2, std::vector<int32_t>(t, t + P_)};
      page_key_[e.page] = h;
    }
  }
}

int KVStore::lookup(const int32_t* tokens, int32_t n, uint64_t* out, int32_t* n_shared, std::string* err) {
  if (!tokens || n < 1 || !out || !n_shared) { *err = "prefix lookup: null argument or n < 1"; return PIE_EINVAL; }
  std::vector<int32_t> hit;
  std::vector<uint64_t> ch, ch2;
  for (int32_t k = 0; (int64_t)(k + 1) * P_ <= (int64_t)n - 1; ++k) {
    const int32_t* t = tokens + (size_t)k * P_;
    const uint64_t h = prefix_hash(k ? ch[k - 1] : 0, t, P_, SEED1);
    const uint64_t h2 = prefix_hash(k ? ch2[k - 1] : 0, t, P_, SEED2);
    auto it = prefix_.find(h);
    if (it == prefix_.end() || it->second.h2 != h2 || pool_.refs(it->second.page) == 0 ||
        !std::equal(t, t + P_, it->second.toks.begin()))
      break;
    hit.push_back(it->second.page);
    ch.push_back(h);
    ch2.push_back(h2);
  }
  uint64_t hnd;
  int rc = alloc(&hnd, err);
  if (rc) return rc;
  WorkingSet* w = get(hnd);
  for (int32_t pg : hit) {
    w->pages.push_back({pg, P_});
    pool_.ref(pg);
  }
  w->len = w->frozen_len = (int32_t)hit.size() * P_;
  w->toks.assign(tokens, tokens + w->len);
  w->chain = std::move(ch);
  w->chain2 = std::move(ch2);
  *out = hnd;
  *n_shared = w->len;
  return PIE_OK;
}

static inline uint64_t make_handle(uint32_t gen, uint32_t slot) {
  return ((uint64_t)gen << 32) | (uint64_t)(slot + 1);
}

WorkingSet* KVStore::get(uint64_t h) {
  uint32_t s = (uint32_t)(h & 0xffffffffu);
  if (s == 0 || s > sets_.size()) return nullptr;
  WorkingSet& w = sets_[s - 1];
  if (!w.live || w.gen != (uint32_t)(h >> 32)) return nullptr;
  return &w;
}

const WorkingSet* KVStore::get(uint64_t h) const {
  return const_cast<KVStore*>(this)->get(h);
}

int KVStore::alloc(uint64_t* out, std::string* err) {
  if (!out) { *err = "null output handle"; return PIE_EINVAL; }
  uint32_t slot;
  if (!free_slots_.empty()) {
    slot = free_slots_.back();
    free_slots_.pop_back();
  } else {
    slot = (uint32_t)sets_.size();
    sets_.emplace_back();
  }
  WorkingSet& w = sets_[slot];
  w.live = true;
  w.gen += 1;  // starts at 1, so a handle is never 0
  w.len = w.frozen_len = 0;
  w.pages.clear();
  w.hist_ok = true;
  w.toks.clear();
  w.chain.clear();
  w.chain2.clear();
  *out = make_handle(w.gen, slot);
  return PIE_OK;
}

int KVStore::fork(uint64_t parent, uint64_t* child, std::string* err) {
  if (!child) { *err = "null output handle"; return PIE_EINVAL; }
  if (!get(parent)) { *err = "fork: invalid or stale parent working set"; return PIE_EINVAL; }
  uint64_t h;
  int rc = alloc(&h, err);
  if (rc) return rc;
  WorkingSet* p = get(parent);  // alloc may have moved the vector
  WorkingSet* c = get(h);
  int32_t start = 0;
  for (const PageEntry& e : p->pages) {
    if (start >= p->frozen_len) break;
    int32_t v = std::min(e.valid, p->frozen_len - start);
    c->pages.push_back({e.page, v});
    pool_.ref(e.page);
    start += e.valid;
  }
  c->len = c->frozen_len = p->frozen_len;
  c->hist_ok = p->hist_ok;
  if (c->hist_ok) c->toks.assign(p->toks.begin(), p->toks.begin() + p->frozen_len);
  c->chain = p->chain;  // registered pages all lie in the frozen prefix
  c->chain2 = p->chain2;
  *child = h;
  return PIE_OK;
}

int KVStore::release(uint64_t h, std::string* err) {
  WorkingSet* w = get(h);
  if (!w) { *err = "free: invalid or stale working set"; return PIE_EINVAL; }
  for (const PageEntry& e : w->pages) unref_page(e.page);
  w->pages.clear();
  w->toks.clear();
  w->chain.clear();
  w->chain2.clear();
  w->live = false;
  w->len = w->frozen_len = 0;
  free_slots_.push_back((uint32_t)((h & 0xffffffffu) - 1));
  return PIE_OK;
}

int KVStore::truncate(uint64_t h, int32_t new_len, std::string* err) {
  WorkingSet* w = get(h);
  if (!w) { *err = "truncate: invalid or stale working set"; return PIE_EINVAL; }
  if (new_len < w->frozen_len || new_len > w->len) {
    *err = "truncate: new length must lie in [frozen_len, len]";
    return PIE_EINVAL;
  }
  int32_t drop = w->len - new_len;
  while (drop > 0) {
    PageEntry& e = w->pages.back();
    int32_t d = std::min(drop, e.valid);
    e.valid -= d;
    drop -= d;
    if (e.valid == 0) {
      unref_page(e.page);
      w->pages.pop_back();
    }
  }
  w->len = new_len;
  if (w->hist_ok) w->toks.resize(new_len);
  return PIE_OK;
}

AppendPlan KVStore::plan_append(const WorkingSet& ws, int32_t n) const {
  AppendPlan a;
  if (!ws.pages.empty()) {
    const PageEntry& e = ws.pages.back();
    if (pool_.refs(e.page) == 1 && e.valid < P_) a.room = P_ - e.valid;
  }
  int32_t rest = n > a.room ? n - a.room : 0;
  a.fresh_pages = (rest + P_ - 1) / P_;
  return a;
}

void KVStore::append(WorkingSet& ws, int32_t n, int32_t* slot_out) {
  AppendPlan a = plan_append(ws, n);
  int32_t i = 0;
  if (a.room > 0) {
    PageEntry& e = ws.pages.back();
    for (; i < n && i < a.room; ++i) slot_out[i] = e.page * P_ + e.valid + i;
    e.valid += i;
  }
  while (i < n) {
    int32_t p = pool_.take();
    int32_t k = 0;
    for (; k < P_ && i < n; ++k, ++i) slot_out[i] = p * P_ + k;
    ws.pages.push_back({p, k});
  }
  ws.len += n;
}

size_t KVStore::live_sets() const {
  size_t n = 0;
  for (const auto& w : sets_) n += w.live ? 1 : 0;
  return n;
}

}  // namespace pie
