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
  *child = h;
  return PIE_OK;
}

int KVStore::release(uint64_t h, std::string* err) {
  WorkingSet* w = get(h);
  if (!w) { *err = "free: invalid or stale working set"; return PIE_EINVAL; }
  for (const PageEntry& e : w->pages) pool_.unref(e.page);
  w->pages.clear();
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
      pool_.unref(e.page);
      w->pages.pop_back();
    }
  }
  w->len = new_len;
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
