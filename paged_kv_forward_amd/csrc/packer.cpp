// Batch packer; see packer.h.
#include "packer.h"

#include <cmath>
#include <cstdio>
#include <unordered_set>

namespace pie {

static int fail(std::string* err, int code, const char* fmt, long a = 0, long b = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, b);
  *err = buf;
  return code;
}

int pack_batch(KVStore& store, const pie_pass* passes, int32_t n_passes, const PackLimits& lim,
               Plan* plan, std::string* err, bool host_tokens) {
  if (n_passes < 1) return fail(err, PIE_EINVAL, "pie_forward: need at least one pass");
  if (!passes) return fail(err, PIE_EINVAL, "pie_forward: null passes");
  if (n_passes > lim.max_seqs)
    return fail(err, PIE_ENOMEM, "pie_forward: %ld passes exceed max_seqs %ld", n_passes,
                lim.max_seqs);

  // ---- validation (nothing changes) ------------------------------------
  std::unordered_set<uint64_t> seen;
  int64_t rows = 0, readouts = 0, fresh = 0, entries = 0;
  const int32_t P = store.page_size();
  for (int32_t s = 0; s < n_passes; ++s) {
    const pie_pass& p = passes[s];
    const WorkingSet* ws = store.get(p.ws);
    if (!ws) return fail(err, PIE_EINVAL, "pass %ld: invalid or stale working set", s);
    if (!seen.insert(p.ws).second)
      return fail(err, PIE_EINVAL, "pass %ld: working set appears twice in one call", s);
    if (p.n_tokens < 1 || !p.tokens)
      return fail(err, PIE_EINVAL, "pass %ld: needs at least one token", s);
    for (int32_t i = 0; i < p.n_tokens; ++i)
      if (p.tokens[i] < 0 || p.tokens[i] >= lim.vocab)
        return fail(err, PIE_EINVAL, "pass %ld: token id %ld out of range", s, p.tokens[i]);
    if (p.positions)
      for (int32_t i = 0; i < p.n_tokens; ++i)
        if (p.positions[i] < 0)
          return fail(err, PIE_EINVAL, "pass %ld: negative position %ld", s, p.positions[i]);
    if (p.n_readout < 0 || (p.n_readout > 0 && (!p.readout || !p.epi)))
      return fail(err, PIE_EINVAL, "pass %ld: bad readout list", s);
    for (int32_t r = 0; r < p.n_readout; ++r) {
      if (p.readout[r] < 0 || p.readout[r] >= p.n_tokens)
        return fail(err, PIE_EINVAL, "pass %ld: readout index %ld out of range", s, p.readout[r]);
      const pie_epilogue& e = p.epi[r];
      if (e.kind != PIE_EPI_ARGMAX && e.kind != PIE_EPI_GUMBEL_MAX)
        return fail(err, PIE_EINVAL, "pass %ld: unknown epilogue kind %ld", s, e.kind);
      if (e.kind == PIE_EPI_GUMBEL_MAX && !(std::isfinite(e.temperature) && e.temperature > 0.f))
        return fail(err, PIE_EINVAL, "pass %ld: gumbel_max temperature must be finite and > 0", s);
    }
    if ((int64_t)ws->len + p.n_tokens > lim.max_ctx)
      return fail(err, PIE_EINVAL, "pass %ld: sequence would exceed max_ctx (%ld tokens)", s,
                  lim.max_ctx);
    rows += p.n_tokens;
    readouts += p.n_readout;
    AppendPlan a = store.plan_append(*ws, p.n_tokens);
    fresh += a.fresh_pages;
    entries += (int64_t)ws->pages.size() + a.fresh_pages;
  }
  if (rows > lim.max_rows)
    return fail(err, PIE_ENOMEM, "pie_forward: %ld rows exceed max_rows %ld", (long)rows,
                lim.max_rows);
  if (readouts > lim.max_readout)
    return fail(err, PIE_ENOMEM, "pie_forward: %ld readouts exceed max_readout %ld",
                (long)readouts, lim.max_readout);
  if (entries > lim.max_page_entries)
    return fail(err, PIE_ENOMEM, "pie_forward: %ld page-table entries exceed the limit %ld",
                (long)entries, lim.max_page_entries);
  if (fresh > store.pool().free_count())
    return fail(err, PIE_ENOMEM, "pie_forward: KV pool exhausted (%ld pages needed, %ld free)",
                (long)fresh, (long)store.pool().free_count());
  (void)P;

  // ---- apply -------------------------------------------------------------
  Plan& pl = *plan;
  pl.n_rows = (int32_t)rows;
  pl.n_seqs = n_passes;
  pl.n_readout = (int32_t)readouts;
  pl.tok.resize(rows);
  pl.pos.resize(rows);
  pl.row_seq.resize(rows);
  pl.slot.resize(rows);
  pl.seq_row0.assign(n_passes + 1, 0);
  pl.seq_ctx.resize(n_passes);
  pl.seq_len.resize(n_passes);
  pl.seq_pg0.assign(n_passes + 1, 0);
  pl.pg_id.clear();
  pl.pg_valid.clear();
  pl.pg_start.clear();
  pl.ro_row.clear();
  pl.ro_lane.clear();
  pl.ro_kind.clear();
  pl.ro_temp.clear();
  pl.ro_seed_lo.clear();
  pl.ro_seed_hi.clear();
  pl.max_seq_len = 0;
  pl.max_new = 0;

  int32_t row = 0;
  for (int32_t s = 0; s < n_passes; ++s) {
    const pie_pass& p = passes[s];
    WorkingSet* ws = store.get(p.ws);
    pl.seq_row0[s] = row;
    pl.seq_ctx[s] = ws->len;
    for (int32_t i = 0; i < p.n_tokens; ++i) {
      pl.tok[row + i] = p.tokens[i];
      pl.pos[row + i] = p.positions ? p.positions[i] : ws->len + i;
      pl.row_seq[row + i] = s;
    }
    store.note_tokens(*ws, host_tokens ? p.tokens : nullptr, p.positions, p.n_tokens);
    store.append(*ws, p.n_tokens, &pl.slot[row]);
    if (p.commit) store.commit(*ws);
    pl.seq_len[s] = ws->len;
    if (ws->len > pl.max_seq_len) pl.max_seq_len = ws->len;
    if (p.n_tokens > pl.max_new) pl.max_new = p.n_tokens;
    pl.seq_pg0[s] = (int32_t)pl.pg_id.size();
    int32_t start = 0;
    for (const PageEntry& e : ws->pages) {
      pl.pg_id.push_back(e.page);
      pl.pg_valid.push_back(e.valid);
      pl.pg_start.push_back(start);
      start += e.valid;
    }
    for (int32_t r = 0; r < p.n_readout; ++r) {
      pl.ro_row.push_back(row + p.readout[r]);
      pl.ro_lane.push_back(r);
      pl.ro_kind.push_back(p.epi[r].kind);
      pl.ro_temp.push_back(p.epi[r].temperature);
      pl.ro_seed_lo.push_back((uint32_t)(p.epi[r].seed & 0xffffffffu));
      pl.ro_seed_hi.push_back((uint32_t)(p.epi[r].seed >> 32));
    }
    row += p.n_tokens;
  }
  pl.seq_row0[n_passes] = row;
  pl.seq_pg0[n_passes] = (int32_t)pl.pg_id.size();
  pl.n_pe = (int32_t)pl.pg_id.size();
  return PIE_OK;
}

}  // namespace pie
