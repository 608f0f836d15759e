// Paged grouped-query attention over working-set page tables (ops.attn.attend
// and ops.attn.prefill on the "Poem ops" page; the working sets of "How Pie
// thinks", section 4).
//
// KV page layout, per layer and page (elements of the KV dtype):
//   K: [n_kv_heads][head_dim / 8][page_size][8]   head-dim groups of 8, token
//                                            within a group: the Q*K^T MFMA
//                                            operand of a k-step is one
//                                            contiguous run
//   V: [n_kv_heads][head_dim][page_size]     transposed, so that the P*V
//                                            MFMA reads consecutive tokens
// Per layer the pages follow each other (page_stride elements apart); layers
// follow each other (n_pages * page_stride apart).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pie {

struct AttnArgs {
  const uint16_t* q;   // [rows][nq][hd] bf16 (after RoPE)
  uint16_t* o;         // [rows][nq * hd] bf16
  const void* kv_layer;
  long page_stride;    // elements per page per layer
  int nq, nkv, hd, page_size, kv_e4m3;
  const float* kv_scale;  // [2][nkv] for this layer (e4m3 only)
  float sm_scale;         // 1 / sqrt(hd)
  const int32_t* seq_row0;
  const int32_t* seq_ctx;
  const int32_t* seq_pg0;
  const int32_t* pg_id;
  const int32_t* pg_valid;
  const int32_t* pg_start;
  const int4* items;   // decode: (seq, first entry, end entry, partial slot or -1)
                       // prefill: (seq, first new token, new tokens in item, 0)
  int n_items;
  float* part_o;       // decode partials [slot][nkv][16][hd]
  float* part_ml;      // [slot][nkv][16][2] (running max in log2 units, sum)
  const int4* combine; // (seq, first slot, n slots, 0)
  int n_combine;
};

// Rows handled by one prefill workgroup (tokens x query heads of a group).
constexpr int PREFILL_ROWS = 256;

// Most partials one decode sequence may be split into (the combine kernel
// holds a weight per partial and query head in LDS).
constexpr int DECODE_MAX_SPLITS = 64;

void launch_attn_decode(const AttnArgs& a, hipStream_t st);
void launch_attn_combine(const AttnArgs& a, hipStream_t st);
void launch_attn_prefill(const AttnArgs& a, hipStream_t st);

}  // namespace pie
