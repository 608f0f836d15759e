// Paged KV store: a pool of fixed-size KV pages and the working sets that own
// page tables over it ("How Pie thinks", section 4 Working sets).
//
// A working set is a list of page entries {page id, valid slots}.  Its tokens,
// in append order, are the first `valid` slots of each entry in turn.  The
// first frozen_len tokens are committed; the rest are the writable buffer.
// fork() gives a new working set the entries of the parent's frozen prefix
// (page reference counts +1; nothing is copied).  A page whose reference count
// is above 1 is never written: appends go to the last entry only if that page
// is held once and has room, otherwise to fresh pages.  So a partly filled page
// shared by a fork stays partly filled, and its unused slots are skipped.
//
// Frozen prefixes are also shared across requests ("How Pie thinks", section 4:
// fork shares a prefix without copying it; here the same holds between working
// sets that never forked from each other).  Every full page of a frozen
// prefix whose tokens the host knows, at positions 0, 1, 2, ..., is entered in
// a registry under a chained hash of all tokens up to the page's end;
// lookup() walks a new request's tokens page by page and hands back a
// working set that shares the longest registered prefix (reference counts +1,
// nothing is copied or recomputed).  An entry also keeps the page's own tokens
// and a second, independently seeded chain hash, and a match needs all three.
// A page leaves the registry when its last holder lets go of it.
//
// Host-only code: no HIP here.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace pie {

struct PageEntry {
  int32_t page;
  int32_t valid;  // 1 .. page_size
};

class PagePool {
 public:
  void reset(int64_t n_pages);
  int64_t total() const { return (int64_t)refcnt_.size(); }
  int64_t free_count() const { return (int64_t)free_.size(); }
  int64_t ever_allocated() const { return ever_allocated_; }
  int32_t take();            // caller has checked free_count() > 0
  void ref(int32_t page) { ++refcnt_[page]; }
  void unref(int32_t page);  // back to the free list at 0
  int32_t refs(int32_t page) const { return refcnt_[page]; }

 private:
  std::vector<int32_t> free_;   // stack; lowest ids handed out first
  std::vector<int32_t> refcnt_;
  int64_t ever_allocated_ = 0;
};

struct WorkingSet {
  bool live = false;
  uint32_t gen = 0;
  int32_t len = 0;
  int32_t frozen_len = 0;
  std::vector<PageEntry> pages;
  // prefix registry bookkeeping: the tokens in append order while the host
  // knows them and every position equals the token's index (else hist_ok is
  // false for good), and the two chain hashes after each registered page
  bool hist_ok = true;
  std::vector<int32_t> toks;
  std::vector<uint64_t> chain, chain2;
};

// What appending n tokens to a working set needs and where they go.
struct AppendPlan {
  int32_t room = 0;         // slots usable in the current last entry
  int32_t fresh_pages = 0;  // new pages to take from the pool
};

class KVStore {
 public:
  explicit KVStore(int32_t page_size = 16) : P_(page_size) {}
  void reset(int64_t n_pages) {
    pool_.reset(n_pages);
    sets_.clear();
    free_slots_.clear();
    prefix_.clear();
    page_key_.assign((size_t)n_pages, 0);
  }

  int32_t page_size() const { return P_; }
  const PagePool& pool() const { return pool_; }

  // Handles: (gen << 32) | (slot + 1)
  int alloc(uint64_t* out, std::string* err);
  int fork(uint64_t parent, uint64_t* child, std::string* err);
  int release(uint64_t h, std::string* err);
  int truncate(uint64_t h, int32_t new_len, std::string* err);
  WorkingSet* get(uint64_t h);  // nullptr if stale / invalid
  const WorkingSet* get(uint64_t h) const;

  AppendPlan plan_append(const WorkingSet& ws, int32_t n) const;
  // Append n tokens (the pool must hold plan.fresh_pages free pages).  slot_out[i]
  // receives page * page_size + offset of token i.
  void append(WorkingSet& ws, int32_t n, int32_t* slot_out);
  // Freeze everything appended so far and enter its new full pages in the
  // prefix registry.
  void commit(WorkingSet& ws);
  // Record the n tokens about to be appended (tokens: host ids, or nullptr
  // when only the device knows them; positions: nullptr for len + i).
  void note_tokens(WorkingSet& ws, const int32_t* tokens, const int32_t* positions, int32_t n);

  // A new working set sharing the longest registered prefix of tokens[0, n),
  // whole pages only, at most n - 1 tokens (so that a pass remains to read
  // out the last one).  *n_shared = its length (0: a plain empty set).
  int lookup(const int32_t* tokens, int32_t n, uint64_t* out, int32_t* n_shared, std::string* err);
  size_t registered_pages() const { return prefix_.size(); }

  size_t live_sets() const;

 private:
  struct PrefixEntry {
    int32_t page;
    uint64_t h2;
    std::vector<int32_t> toks;
  };
  void unref_page(int32_t page);  // pool unref; a freed page leaves the registry

  int32_t P_;
  PagePool pool_;
  std::vector<WorkingSet> sets_;
  std::vector<uint32_t> free_slots_;
  std::unordered_map<uint64_t, PrefixEntry> prefix_;  // chain hash -> page
  std::vector<uint64_t> page_key_;                     // page -> its registry key, 0 if none
};

// Chain hash of a page of tokens after the hash `prev` of everything before it.
uint64_t prefix_hash(uint64_t prev, const int32_t* toks, int32_t n, uint64_t seed);

}  // namespace pie
