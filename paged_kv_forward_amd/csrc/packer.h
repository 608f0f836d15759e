// Batch packer: flattens the forward passes of one call into the arrays the
// kernels read ("How Pie thinks", "Batching is still the engine's job": passes
// from many programs are packed into shared launches).
//
// Rows of all passes are concatenated in pass order.  For each pass
// (= launch-local sequence s) the packer records its first row, its length
// before and after the call, and its whole page table after the append, with
// each entry's valid slot count and the logical index of its first slot.
// Every check runs and every page is reserved before any working set changes,
// so a failed call leaves the store as it was.
//
// Host-only code: no HIP here.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "kvstore.h"
#include "pie.h"

namespace pie {

struct Plan {
  int32_t n_rows = 0, n_seqs = 0, n_readout = 0, n_pe = 0;
  std::vector<int32_t> tok, pos, row_seq, slot;                  // [n_rows]
  std::vector<int32_t> seq_row0;                                 // [n_seqs + 1]
  std::vector<int32_t> seq_ctx, seq_len;                         // [n_seqs]
  std::vector<int32_t> seq_pg0;                                  // [n_seqs + 1]
  std::vector<int32_t> pg_id, pg_valid, pg_start;                // [n_pe]
  std::vector<int32_t> ro_row, ro_lane, ro_kind;                 // [n_readout]
  std::vector<float> ro_temp;                                    // [n_readout]
  std::vector<uint32_t> ro_seed_lo, ro_seed_hi;                  // [n_readout]
  int32_t max_seq_len = 0;      // longest sequence after the call
  int32_t max_new = 0;          // most new rows of one sequence
};

struct PackLimits {
  int32_t max_rows, max_seqs, max_readout, max_ctx, max_page_entries;
  int32_t vocab;
};

// Validate, reserve and apply.  With apply == false only validation and the
// reservation check run (nothing changes).  Returns a pie_status.
// host_tokens: false when the passes' token arrays are placeholders and the
// real ids exist only on the device (loop-carried decode); such tokens are
// kept out of the prefix registry.
int pack_batch(KVStore& store, const pie_pass* passes, int32_t n_passes, const PackLimits& lim,
               Plan* plan, std::string* err, bool host_tokens = true);

}  // namespace pie
