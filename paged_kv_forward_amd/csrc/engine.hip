// The C ABI of include/pie.h: contexts, working sets and the batched forward.
//
// pie_forward packs the passes (packer.cpp), stages the packed metadata into
// the device workspace with one host-to-device copy, and launches per call:
//   rope table, embed, then per layer
//     QKV GEMM (RMSNorm prologue; RoPE + KV append epilogue)
//     decode attention (+ split combine) and/or chunked-prefill attention
//     O GEMM (+ residual)
//     gate/up GEMM (RMSNorm prologue; SwiGLU epilogue)
//     down GEMM (+ residual)
//   then the head GEMM (final RMSNorm of the gathered readout rows; fused
//   argmax / Gumbel-max epilogue) and the cross-tile reduce,
// and copies back only the token ids (and logits when asked).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdlib>
#include <map>
#include <mutex>
#include <tuple>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "attention.h"
#include "gemm.h"
#include "kvstore.h"
#include "misc.h"
#include "packer.h"
#include "pie.h"

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

constexpr int GEMM_BN = 128;
constexpr int GEMM_BK = 64;
constexpr int LM_BN = 128;

// Split-K policy for the small-M (decode) tile: enough workgroups to fill the
// chip, each with at least 4 K-steps.
struct SplitK {
  int splits, k_split;
};

SplitK split_of(int K, int s) {
  int ks = (K + s - 1) / s;
  ks = (ks + GEMM_BK - 1) / GEMM_BK * GEMM_BK;  // whole 64-wide chunks
  return {(K + ks - 1) / ks, ks};
}

SplitK choose_split(int M, int n_tiles, int K) {
  if (M > 64) return {1, K};
  // About one 8-wave workgroup per CU (measured best for the decode shapes),
  // and at least 4 chunks of 64 per split.
  const int target = 256;
  int s = (target + n_tiles / 2) / n_tiles;
  s = std::max(1, std::min(s, pie::SK_MAX_SPLITS));
  int max_by_k = std::max(1, K / (4 * GEMM_BK));
  s = std::min(s, max_by_k);
  SplitK sk = split_of(K, s);
  // One split fewer when that still keeps 3/4 of the CUs busy and fills the
  // activation groups (8 chunks) better: the skinny kernel runs whole groups,
  // and a part-empty one costs its MFMAs and LDS reads.  Measured at the 8B
  // shape: QKV 5 -> 4 splits and down 8 -> 7, 0.03 ms per step each.
  auto waste = [](const SplitK& x) {
    const int nc = x.k_split / GEMM_BK;
    return (nc + 7) / 8 * 8 - nc;
  };
  if (sk.splits > 1 && n_tiles * (sk.splits - 1) * 4 >= 3 * target) {
    const SplitK fewer = split_of(K, sk.splits - 1);
    if (waste(fewer) < waste(sk)) sk = fewer;
  }
  return sk;
}

struct Layout {
  // int32 metadata offsets (in int32 units from meta base)
  size_t tok, pos, row_seq, slot, seq_row0, seq_ctx, seq_len, seq_pg0, pg_id, pg_valid, pg_start,
      ro_row, ro_lane, ro_kind, ro_temp, ro_seed_lo, ro_seed_hi, dec_items, comb_items, pre_items,
      tokens_out, meta_ints;
  int32_t max_pe, max_dec_items, max_pre_items;
  // byte offsets into the workspace
  size_t meta, y, ss, x, q, o, h, rope, part_o, part_ml, gpart, tile_best, tile_idx, logits, total;
  size_t gpart_floats;
};

bool desc_ok(const pie_model_desc* d, std::string* why) {
  if (!d) { *why = "null model desc"; return false; }
  if (d->n_layers < 1 || d->d_model < 128 || d->d_model % 128 || d->n_q_heads < 1 ||
      d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads || d->d_ffn < 8 || d->d_ffn % 8 ||
      d->vocab < 2) {
    *why = "model desc: bad dimensions (d_model % 128, d_ffn % 8, heads)";
    return false;
  }
  if (d->head_dim != 64 && d->head_dim != 128) { *why = "model desc: head_dim must be 64 or 128"; return false; }
  if ((d->n_q_heads * d->head_dim) % 128 || (d->n_kv_heads * d->head_dim) % 128) {
    *why = "model desc: q and kv widths must be multiples of 128";
    return false;
  }
  if (d->n_q_heads / d->n_kv_heads > 16) { *why = "model desc: at most 16 query heads per KV head"; return false; }
  if (d->page_size != 16) { *why = "model desc: page_size must be 16"; return false; }
  if (d->kv_dtype != PIE_KV_BF16 && d->kv_dtype != PIE_KV_E4M3) { *why = "model desc: kv_dtype"; return false; }
  if (!(d->rms_eps > 0.f) || !(d->rope_theta > 1.f)) { *why = "model desc: eps / theta"; return false; }
  return true;
}

bool limits_ok(const pie_limits* l, std::string* why) {
  if (!l || l->max_rows < 1 || l->max_seqs < 1 || l->max_readout < 0 || l->max_ctx < 1 ||
      l->max_seqs > l->max_rows) {
    *why = "bad limits (max_rows >= max_seqs >= 1, max_ctx >= 1)";
    return false;
  }
  return true;
}

size_t kv_elem_bytes(const pie_model_desc& d) { return d.kv_dtype == PIE_KV_E4M3 ? 1 : 2; }
long page_stride_elems(const pie_model_desc& d) { return 2L * d.n_kv_heads * d.page_size * d.head_dim; }

Layout make_layout(const pie_model_desc& d, const pie_limits& l) {
  Layout L{};
  const size_t R = (size_t)l.max_rows, S = (size_t)l.max_seqs, RO = (size_t)std::max(l.max_readout, 1);
  L.max_pe = (int32_t)std::min<int64_t>((int64_t)S * ((l.max_ctx + d.page_size - 1) / d.page_size + 4),
                                        (int64_t)1 << 30);
  L.max_dec_items = L.max_pe / 8 + 2 * (int32_t)S;
  L.max_pre_items = (int32_t)(R + S);
  size_t o = 0;
  auto take = [&](size_t n) { size_t at = o; o += (n + 63) / 64 * 64; return at; };
  L.tok = take(R); L.pos = take(R); L.row_seq = take(R); L.slot = take(R);
  L.seq_row0 = take(S + 1); L.seq_ctx = take(S); L.seq_len = take(S); L.seq_pg0 = take(S + 1);
  L.pg_id = take(L.max_pe); L.pg_valid = take(L.max_pe); L.pg_start = take(L.max_pe);
  L.ro_row = take(RO); L.ro_lane = take(RO); L.ro_kind = take(RO); L.ro_temp = take(RO);
  L.ro_seed_lo = take(RO); L.ro_seed_hi = take(RO);
  L.dec_items = take(4 * (size_t)L.max_dec_items); L.comb_items = take(4 * S);
  L.pre_items = take(4 * (size_t)L.max_pre_items);
  L.tokens_out = take(RO);
  L.meta_ints = o;

  const size_t qw = (size_t)d.n_q_heads * d.head_dim;
  const int n_ss = d.d_model / 64;
  size_t b = 0;
  auto take_b = [&](size_t bytes) { size_t at = b; b = align_up(b + bytes); return at; };
  L.meta = take_b(L.meta_ints * 4);
  L.y = take_b(R * d.d_model * 4);
  L.ss = take_b(R * n_ss * 4);
  L.x = take_b(R * d.d_model * 2);
  L.q = take_b(R * qw * 2);
  L.o = take_b(R * qw * 2);
  L.h = take_b(R * (size_t)d.d_ffn * 2);
  L.rope = take_b(R * (size_t)d.head_dim * 4);
  L.part_o = take_b((size_t)L.max_dec_items * d.n_kv_heads * 16 * d.head_dim * 4);
  L.part_ml = take_b((size_t)L.max_dec_items * d.n_kv_heads * 16 * 2 * 4);
  // split-K partials for the worst case over the four layer GEMMs at M <= 64
  const int kvw = d.n_kv_heads * d.head_dim;
  struct G { int n_tiles, K; } gs[4] = {
      {(int)((qw + 2 * kvw + GEMM_BN - 1) / GEMM_BN), d.d_model},
      {(d.d_model + GEMM_BN - 1) / GEMM_BN, (int)qw},
      {pie::gemm_n_tiles(pie::EPI_SWIGLU, d.d_ffn, pie::TILE_SKINNY), d.d_model},
      {(d.d_model + GEMM_BN - 1) / GEMM_BN, d.d_ffn}};
  size_t worst = 0;
  for (auto& g : gs) {
    SplitK sk = choose_split(64, g.n_tiles, g.K);
    worst = std::max(worst, (size_t)g.n_tiles * sk.splits);
  }
  L.gpart_floats = worst * 64 * GEMM_BN;
  L.gpart = take_b(L.gpart_floats * 4);
  const size_t vt = (size_t)(d.vocab + LM_BN - 1) / LM_BN;
  L.tile_best = take_b(vt * RO * 4);
  L.tile_idx = take_b(vt * RO * 4);
  L.logits = take_b(RO * (size_t)d.vocab * 4);
  L.total = b;
  return L;
}

// Events of the timed launches of one call (timed calls are never captured).
struct EventSink {
  std::vector<hipEvent_t> ev;
  struct Mark {
    int k;         // class
    size_t first;  // index of the start event
    int n;         // launches between the two events
  };
  std::vector<Mark> marks;
  size_t used = 0;
};

// What determines the launch sequence of a call (everything else the kernels
// read comes from the metadata staged in device memory).
struct GraphKey {
  int T, R, n_dec, n_comb, n_pre, flags;
  const void* logits;
  bool operator<(const GraphKey& o) const {
    return std::tie(T, R, n_dec, n_comb, n_pre, flags, logits) <
           std::tie(o.T, o.R, o.n_dec, o.n_comb, o.n_pre, o.flags, o.logits);
  }
};

struct GraphEntry {
  int seen = 0;
  hipGraphExec_t exec = nullptr;
};

}  // namespace

// Pinned metadata staging slots: how many calls may be enqueued ahead of the GPU.
constexpr int PIE_STAGING_SLOTS = 4;

// Device scratch of pie_forward_static: everything a call's kernels use
// besides the caller's inputs and outputs (the workspace layout of the
// context), in a file-scope array that every GPU the library runs on holds
// from module load to process end.  Host code never uses the array's name as
// an address: pie_init looks up its device address once per device
// (hipGetSymbolAddress, with that device current) and keeps it per device.
static __device__ __align__(256) uint8_t scratch[PIE_STATIC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::map<int, uint8_t*> g_scratch_addr;  // device -> address of that device's scratch

// Address of the current device's scratch (looked up once per device).
hipError_t scratch_address(int dev, uint8_t** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_addr.find(dev);
  if (it != g_scratch_addr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
  g_scratch_addr[dev] = static_cast<uint8_t*>(p);
  *out = static_cast<uint8_t*>(p);
  return hipSuccess;
}
}  // namespace

struct pie_ctx {
  pie_model_desc d{};
  pie_limits lim{};
  bool host_only = false, poisoned = false;
  const uint16_t *embed = nullptr, *final_norm = nullptr, *lm_head = nullptr;
  std::vector<const uint16_t*> attn_norm, wq, wk, wv, wo, mlp_norm, wg, wu, wd;
  // block-scaled FP8 copies of the projections for the decode GEMMs
  // (pie_attach_fp8_weights), in the order q, k, v, o, gate, up, down
  bool f8 = false;
  std::vector<const uint8_t*> f8w[7];
  std::vector<const float*> f8s[7];
  const uint8_t* f8_head = nullptr;
  const float* f8_head_s = nullptr;
  const float* kv_scale = nullptr;
  uint8_t* kv = nullptr;
  int64_t n_pages = 0;
  long page_stride = 0;
  uint8_t* ws = nullptr;
  Layout lay{};
  hipStream_t stream = nullptr;
  pie::KVStore store{16};
  pie::Plan plan;
  // Pinned metadata staging: a ring of slots, each reused only after the
  // copy out of it (recorded by its event) has run, so calls may be
  // enqueued ahead of the GPU.  `pinned` is the slot of the current call.
  int32_t* pinned = nullptr;
  std::vector<int32_t*> pin_ring;
  std::vector<hipEvent_t> pin_ev;
  int pin_next = 0;
  // loop-carried decode: device token arrays of the call being enqueued
  const int32_t* dev_tok_in = nullptr;
  int32_t* dev_tok_out = nullptr;
  std::vector<pie_pass> async_pass;
  std::vector<int32_t> async_zero;
  std::vector<int32_t> dec, comb, pre;  // int4 items, flattened
  int n_parts = 0;
  // profiling: events bracketing timed launches, recorded into a sink
  uint32_t prof_mask = 0;
  int prof_reps = 1;  // back-to-back runs of each timed decode-attention launch
  EventSink sink;
  hipStream_t cur = nullptr;    // stream launches go to while enqueueing
  double prof_ms[PIE_K_NUM_CLASSES] = {0};
  int64_t prof_n[PIE_K_NUM_CLASSES] = {0};
  // graphs of the per-call launch sequence, by launch shape
  hipStream_t cap_stream = nullptr;
  std::map<GraphKey, GraphEntry> graphs;
  bool use_graphs = false;
  bool capturing = false;
  // this device's static scratch (pie_forward_static), and whether the
  // context has a workspace of its own (pie_forward, pie_decode_async)
  uint8_t* static_ws = nullptr;
  bool has_workspace = true;
  bool in_static = false;  // a pie_forward_static call is running
};

namespace {

int hip_fail(pie_ctx* c, hipError_t e, const char* what) {
  if (c && !c->capturing) c->poisoned = true;
  return set_err(PIE_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define HIP_TRY(c, call)                                   \
  do {                                                     \
    hipError_t e_ = (call);                                \
    if (e_ != hipSuccess) return hip_fail((c), e_, #call); \
  } while (0)

hipEvent_t next_event(EventSink* k) {
  if (k->used == k->ev.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    k->ev.push_back(e);
  }
  return k->ev[k->used++];
}

// Brackets one launch of class k with events when that class is being timed.
struct Timed {
  pie_ctx* c;
  bool on;
  size_t first = 0, mark = 0;
  Timed(pie_ctx* c_, int k) : c(c_), on(((c_->prof_mask >> k) & 1u) && !c_->capturing) {
    if (on) {
      hipEvent_t a = next_event(&c->sink), b = next_event(&c->sink);
      if (!a || !b) { on = false; return; }
      first = c->sink.used - 2;
      c->sink.marks.push_back({k, first, 1});
      mark = c->sink.marks.size() - 1;
      (void)hipEventRecord(a, c->cur);
    }
  }
  void set_launches(int n) {
    if (on) c->sink.marks[mark].n = n;
  }
  ~Timed() {
    if (on) (void)hipEventRecord(c->sink.ev[first + 1], c->cur);
  }
};

void collect_profile(pie_ctx* c, EventSink& k) {
  for (auto& m : k.marks) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, k.ev[m.first], k.ev[m.first + 1]) == hipSuccess) {
      c->prof_ms[m.k] += ms;
      c->prof_n[m.k] += m.n;
    }
  }
  (void)hipGetLastError();  // a failed timing query must not surface in a later call
}

void release_graphs(pie_ctx* c) {
  for (auto& kv : c->graphs) {
    if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
  }
  c->graphs.clear();
}

int check_launch(pie_ctx* c, int flags, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(c, e, what);
  if (flags & PIE_FLAG_SYNC_DEBUG) {
    e = hipStreamSynchronize(c->cur);
    if (e != hipSuccess) return hip_fail(c, e, what);
  }
  return PIE_OK;
}

int build_work(pie_ctx* c) {
  const pie::Plan& p = c->plan;
  const int G = c->d.n_q_heads / c->d.n_kv_heads;
  const int tpw = std::max(1, pie::PREFILL_ROWS / G);
  c->dec.clear();
  c->comb.clear();
  c->pre.clear();
  c->n_parts = 0;
  int n_dec = 0;
  int64_t dec_entries = 0;
  for (int s = 0; s < p.n_seqs; ++s)
    if (p.seq_row0[s + 1] - p.seq_row0[s] == 1) {
      ++n_dec;
      dec_entries += p.seq_pg0[s + 1] - p.seq_pg0[s];
    }
  int pps = 1 << 30;
  if (n_dec) {
    // One workgroup (4 waves) per (item, KV head); sequences are cut into
    // more items only to reach one workgroup per CU (256): every extra cut
    // adds a partial for the combine launch to merge.  At the 70B shape with
    // batch 32 (8 KV heads), one item per sequence (256 workgroups, no
    // combine) ran 2.9% faster per step than two (512 and the combine).
    const int64_t target = std::max<int64_t>(n_dec, (256 + c->d.n_kv_heads - 1) / c->d.n_kv_heads);
    int64_t v = (dec_entries + target - 1) / target;
    v = std::max<int64_t>(v, 8);
    pps = (int)((v + 1) / 2 * 2);
  }
  for (int s = 0; s < p.n_seqs; ++s) {
    const int n_new = p.seq_row0[s + 1] - p.seq_row0[s];
    const int e0 = p.seq_pg0[s], e1 = p.seq_pg0[s + 1];
    if (n_new == 1) {
      // a long sequence in a batch of short ones takes longer runs, so that
      // it never has more partials than the combine kernel merges
      const int cap = ((e1 - e0 + pie::DECODE_MAX_SPLITS - 1) / pie::DECODE_MAX_SPLITS + 1) / 2 * 2;
      const int pps_s = std::max(pps, cap);
      const int ns = std::max(1, (e1 - e0 + pps_s - 1) / pps_s);
      if (ns == 1) {
        c->dec.insert(c->dec.end(), {s, e0, e1, -1});
      } else {
        for (int k = 0; k < ns; ++k)
          c->dec.insert(c->dec.end(), {s, e0 + k * pps_s, std::min(e1, e0 + (k + 1) * pps_s), c->n_parts + k});
        c->comb.insert(c->comb.end(), {s, c->n_parts, ns, 0});
        c->n_parts += ns;
      }
    } else {
      for (int tb = 0; tb < n_new; tb += tpw)
        c->pre.insert(c->pre.end(), {s, tb, std::min(tpw, n_new - tb), 0});
    }
  }
  // decode items longest first (more entries, more bytes); stable, so equal
  // lengths keep sequence order
  std::vector<std::array<int, 4>> dec(c->dec.size() / 4);
  for (size_t i = 0; i < dec.size(); ++i)
    dec[i] = {c->dec[4 * i], c->dec[4 * i + 1], c->dec[4 * i + 2], c->dec[4 * i + 3]};
  std::stable_sort(dec.begin(), dec.end(), [](const std::array<int, 4>& x, const std::array<int, 4>& y) {
    return x[2] - x[1] > y[2] - y[1];
  });
  for (size_t i = 0; i < dec.size(); ++i)
    for (int k = 0; k < 4; ++k) c->dec[4 * i + k] = dec[i][k];
  // longest first: an item's work grows with its last token's position
  std::vector<std::array<int, 4>> pre(c->pre.size() / 4);
  for (size_t i = 0; i < pre.size(); ++i)
    pre[i] = {c->pre[4 * i], c->pre[4 * i + 1], c->pre[4 * i + 2], c->pre[4 * i + 3]};
  std::stable_sort(pre.begin(), pre.end(), [&](const std::array<int, 4>& x, const std::array<int, 4>& y) {
    return p.seq_ctx[x[0]] + x[1] + x[2] > p.seq_ctx[y[0]] + y[1] + y[2];
  });
  for (size_t i = 0; i < pre.size(); ++i)
    for (int k = 0; k < 4; ++k) c->pre[4 * i + k] = pre[i][k];
  for (size_t i = 0; i + 3 < c->comb.size(); i += 4)
    if (c->comb[i + 2] > pie::DECODE_MAX_SPLITS)
      return set_err(PIE_EINVAL, "pie_forward: decode split plan exceeds the combine limit");
  return PIE_OK;
}

template <typename T>
void put(int32_t* base, size_t off, const std::vector<T>& v) {
  if (!v.empty()) std::memcpy(base + off, v.data(), v.size() * sizeof(T));
}

// Pack the plan and the attention work lists into the pinned staging buffer.
int stage(pie_ctx* c) {
  const pie::Plan& p = c->plan;
  const Layout& L = c->lay;
  if (int rc = build_work(c)) return rc;
  if ((int)(c->dec.size() / 4) > L.max_dec_items || (int)(c->pre.size() / 4) > L.max_pre_items)
    return set_err(PIE_ENOMEM, "pie_forward: attention work list exceeds the workspace");
  int32_t* h = c->pinned;
  put(h, L.tok, p.tok); put(h, L.pos, p.pos); put(h, L.row_seq, p.row_seq); put(h, L.slot, p.slot);
  put(h, L.seq_row0, p.seq_row0); put(h, L.seq_ctx, p.seq_ctx); put(h, L.seq_len, p.seq_len);
  put(h, L.seq_pg0, p.seq_pg0); put(h, L.pg_id, p.pg_id); put(h, L.pg_valid, p.pg_valid);
  put(h, L.pg_start, p.pg_start); put(h, L.ro_row, p.ro_row); put(h, L.ro_lane, p.ro_lane);
  put(h, L.ro_kind, p.ro_kind); put(h, L.ro_temp, p.ro_temp); put(h, L.ro_seed_lo, p.ro_seed_lo);
  put(h, L.ro_seed_hi, p.ro_seed_hi); put(h, L.dec_items, c->dec); put(h, L.comb_items, c->comb);
  put(h, L.pre_items, c->pre);
  return PIE_OK;
}

// Take the next staging slot, once the copy last made out of it has run.
int acquire_staging(pie_ctx* c) {
  if (c->pin_ring.empty()) return PIE_OK;  // host-only context: one host buffer
  c->pinned = c->pin_ring[c->pin_next];
  HIP_TRY(c, hipEventSynchronize(c->pin_ev[c->pin_next]));
  return PIE_OK;
}

// Metadata upload (pinned staging -> device), on the caller's stream; the
// slot's event marks when the slot may be packed again.
int upload_meta(pie_ctx* c) {
  int32_t* dmeta = reinterpret_cast<int32_t*>(c->ws + c->lay.meta);
  HIP_TRY(c, hipMemcpyAsync(dmeta, c->pinned, c->lay.tokens_out * 4, hipMemcpyHostToDevice, c->stream));
  if (!c->pin_ring.empty()) {
    HIP_TRY(c, hipEventRecord(c->pin_ev[c->pin_next], c->stream));
    c->pin_next = (c->pin_next + 1) % (int)c->pin_ring.size();
  }
  return PIE_OK;
}

// Token copy-back (device -> pinned staging), on the caller's stream.
int download_tokens(pie_ctx* c) {
  const int R = c->plan.n_readout;
  if (R <= 0) return PIE_OK;
  int32_t* dmeta = reinterpret_cast<int32_t*>(c->ws + c->lay.meta);
  HIP_TRY(c, hipMemcpyAsync(c->pinned + c->lay.tokens_out, dmeta + c->lay.tokens_out, (size_t)R * 4,
                            hipMemcpyDeviceToHost, c->stream));
  return PIE_OK;
}

// Enqueue every kernel of one call on c->cur (and the logits copy to a host
// buffer when asked).  The metadata must already be in device memory; the
// kernels write the token ids to its token slot.
int enqueue(pie_ctx* c, float* out_logits, int flags) {
  const pie::Plan& p = c->plan;
  const pie_model_desc& d = c->d;
  const Layout& L = c->lay;
  hipStream_t st = c->cur;
  int32_t* dmeta = reinterpret_cast<int32_t*>(c->ws + L.meta);
  auto M32 = [&](size_t off) { return dmeta + off; };

  float* y = reinterpret_cast<float*>(c->ws + L.y);
  float* ss = reinterpret_cast<float*>(c->ws + L.ss);
  uint16_t* q = reinterpret_cast<uint16_t*>(c->ws + L.q);
  uint16_t* o = reinterpret_cast<uint16_t*>(c->ws + L.o);
  uint16_t* hb = reinterpret_cast<uint16_t*>(c->ws + L.h);
  float* rope = reinterpret_cast<float*>(c->ws + L.rope);
  const int T = p.n_rows, R = p.n_readout;
  const int qw = d.n_q_heads * d.head_dim, kvw = d.n_kv_heads * d.head_dim;
  const int n_ss = d.d_model / 64;
  int rc;

  pie::launch_rope_table(M32(L.pos), T, d.head_dim, (double)d.rope_theta, rope, st);
  if ((rc = check_launch(c, flags, "rope table"))) return rc;
  {
    Timed tm(c, PIE_K_EMBED);
    pie::launch_embed(c->embed, c->dev_tok_in ? c->dev_tok_in : M32(L.tok), T, d.d_model, d.vocab, y, ss, st);
  }
  if ((rc = check_launch(c, flags, "embed"))) return rc;

  const bool small = T <= 64;  // decode-sized: the weight-streaming skinny GEMM with split-K
  // prefill-sized calls: 256 x 256 tiles once there are enough rows for them
  const int tile = small ? pie::TILE_SKINNY : (T >= 256 ? pie::TILE_256x256 : pie::TILE_128x128);
  const int qkv_tile = tile == pie::TILE_256x256 && (qw % 256 || kvw % 256) ? pie::TILE_128x128 : tile;
  float* gpart = reinterpret_cast<float*>(c->ws + L.gpart);
  uint16_t* xb = reinterpret_cast<uint16_t*>(c->ws + L.x);
  const size_t elem = kv_elem_bytes(d);

  pie::GemmArgs base{};
  base.M = T;
  base.ss = ss;
  base.n_ss = n_ss;
  base.y = y;
  base.ldy = d.d_model;
  base.eps = d.rms_eps;
  base.partial = gpart;
  base.y_out = y;
  base.ss_out = ss;

  auto set_split = [&](pie::GemmArgs& g, int n_tiles) {
    SplitK sk = choose_split(T, n_tiles, g.K);
    // the reduce kernels address the partials with 32-bit byte offsets
    if ((size_t)n_tiles * sk.splits * 64 * GEMM_BN > L.gpart_floats ||
        (size_t)n_tiles * sk.splits * 64 * GEMM_BN * 4 >= ((size_t)1 << 31))
      sk = {1, g.K};
    g.splits = sk.splits;
    g.k_split = sk.k_split;
  };

  pie::AttnArgs at{};
  at.q = q;
  at.o = o;
  at.page_stride = c->page_stride;
  at.nq = d.n_q_heads;
  at.nkv = d.n_kv_heads;
  at.hd = d.head_dim;
  at.page_size = d.page_size;
  at.kv_e4m3 = d.kv_dtype == PIE_KV_E4M3;
  at.sm_scale = 1.0f / std::sqrt((float)d.head_dim);
  at.seq_row0 = M32(L.seq_row0);
  at.seq_ctx = M32(L.seq_ctx);
  at.seq_pg0 = M32(L.seq_pg0);
  at.pg_id = M32(L.pg_id);
  at.pg_valid = M32(L.pg_valid);
  at.pg_start = M32(L.pg_start);
  at.part_o = reinterpret_cast<float*>(c->ws + L.part_o);
  at.part_ml = reinterpret_cast<float*>(c->ws + L.part_ml);

  for (int l = 0; l < d.n_layers; ++l) {
    void* kv_layer = c->kv + (size_t)l * c->n_pages * c->page_stride * elem;
    const float* kvs = c->kv_scale ? c->kv_scale + (size_t)l * 2 * d.n_kv_heads : nullptr;
    // QKV
    {
      pie::GemmArgs g = base;
      g.N = qw + 2 * kvw;
      g.K = d.d_model;
      g.gain = c->attn_norm[l];
      g.w[0] = c->wq[l]; g.w[1] = c->wk[l]; g.w[2] = c->wv[l];
      g.seg_n0[0] = 0; g.seg_n0[1] = qw; g.seg_n0[2] = qw + kvw; g.seg_n0[3] = qw + 2 * kvw;
      if (small && c->f8) {
        for (int i = 0; i < 3; ++i) { g.w8[i] = c->f8w[i][l]; g.s8[i] = c->f8s[i][l]; }
        g.f8 = 1;
      }
      g.q_out = q;
      g.rope_cs = rope;
      g.slot = M32(L.slot);
      g.kv_layer = kv_layer;
      g.page_stride = c->page_stride;
      g.nq = d.n_q_heads; g.nkv = d.n_kv_heads; g.hd = d.head_dim; g.page_size = d.page_size;
      g.kv_e4m3 = d.kv_dtype == PIE_KV_E4M3;
      g.kv_scale = kvs;
      set_split(g, pie::gemm_n_tiles(pie::EPI_QKV, g.N, qkv_tile));
      Timed tm(c, PIE_K_GEMM_QKV);
      // decode-sized calls: the previous layer's down projection already wrote
      // this layer's normed rows (fused into its split-K reduce)
      if (!small || l == 0)
        pie::launch_rmsnorm(y, ss, n_ss, c->attn_norm[l], T, d.d_model, d.rms_eps, nullptr, xb, st);
      g.a = xb;
      g.lda = d.d_model;
      pie::launch_gemm(pie::A_BF16, pie::EPI_QKV, qkv_tile, g, st);
    }
    if ((rc = check_launch(c, flags, "qkv gemm"))) return rc;
    // attention
    at.kv_layer = kv_layer;
    at.kv_scale = kvs;
    if (!c->dec.empty()) {
      at.items = reinterpret_cast<const int4*>(M32(L.dec_items));
      at.n_items = (int)(c->dec.size() / 4);
      at.combine = reinterpret_cast<const int4*>(M32(L.comb_items));
      at.n_combine = (int)(c->comb.size() / 4);
      {
        Timed tm(c, PIE_K_ATTN_DECODE);
        // when timed, the pair may run several times back to back (same
        // inputs, same outputs): the events' fixed cost spreads over them
        const int reps = tm.on ? c->prof_reps : 1;
        for (int r = 0; r < reps; ++r) {
          pie::launch_attn_decode(at, st);
          pie::launch_attn_combine(at, st);
        }
        tm.set_launches(reps);
      }
      if ((rc = check_launch(c, flags, "decode attention"))) return rc;
    }
    if (!c->pre.empty()) {
      at.items = reinterpret_cast<const int4*>(M32(L.pre_items));
      at.n_items = (int)(c->pre.size() / 4);
      {
        Timed tm(c, PIE_K_ATTN_PREFILL);
        pie::launch_attn_prefill(at, st);
      }
      if ((rc = check_launch(c, flags, "prefill attention"))) return rc;
    }
    // O projection + residual
    {
      pie::GemmArgs g = base;
      g.N = d.d_model;
      g.K = qw;
      g.a = o;
      g.lda = qw;
      g.w[0] = g.w[1] = g.w[2] = c->wo[l];
      g.seg_n0[0] = 0; g.seg_n0[1] = g.seg_n0[2] = g.seg_n0[3] = d.d_model;
      if (small && c->f8) {
        g.w8[0] = c->f8w[3][l]; g.s8[0] = c->f8s[3][l];
        g.f8 = 1;
      }
      set_split(g, pie::gemm_n_tiles(pie::EPI_RESID, g.N, tile));
      if (small) {  // and the MLP RMSNorm of the new rows
        g.next_gain = c->mlp_norm[l];
        g.x_out = xb;
      }
      Timed tm(c, PIE_K_GEMM_O);
      pie::launch_gemm(pie::A_BF16, pie::EPI_RESID, tile, g, st);
    }
    if ((rc = check_launch(c, flags, "o gemm"))) return rc;
    // gate/up + SwiGLU
    {
      pie::GemmArgs g = base;
      g.N = d.d_ffn;
      g.K = d.d_model;
      g.gain = c->mlp_norm[l];
      g.w[0] = c->wg[l]; g.w[1] = c->wu[l]; g.w[2] = c->wu[l];
      if (small && c->f8) {
        g.w8[0] = c->f8w[4][l]; g.s8[0] = c->f8s[4][l];
        g.w8[1] = c->f8w[5][l]; g.s8[1] = c->f8s[5][l];
        g.f8 = 1;
      }
      g.h_out = hb;
      set_split(g, pie::gemm_n_tiles(pie::EPI_SWIGLU, g.N, tile));
      Timed tm(c, PIE_K_GEMM_GATEUP);
      if (!small)  // decode-sized: the O projection's reduce wrote the normed rows
        pie::launch_rmsnorm(y, ss, n_ss, c->mlp_norm[l], T, d.d_model, d.rms_eps, nullptr, xb, st);
      g.a = xb;
      g.lda = d.d_model;
      pie::launch_gemm(pie::A_BF16, pie::EPI_SWIGLU, tile, g, st);
    }
    if ((rc = check_launch(c, flags, "gate/up gemm"))) return rc;
    // down + residual
    {
      pie::GemmArgs g = base;
      g.N = d.d_model;
      g.K = d.d_ffn;
      g.a = hb;
      g.lda = d.d_ffn;
      g.w[0] = g.w[1] = g.w[2] = c->wd[l];
      g.seg_n0[0] = 0; g.seg_n0[1] = g.seg_n0[2] = g.seg_n0[3] = d.d_model;
      if (small && c->f8) {
        g.w8[0] = c->f8w[6][l]; g.s8[0] = c->f8s[6][l];
        g.f8 = 1;
      }
      set_split(g, pie::gemm_n_tiles(pie::EPI_RESID, g.N, tile));
      if (small && l + 1 < d.n_layers) {  // and the next layer's attention RMSNorm
        g.next_gain = c->attn_norm[l + 1];
        g.x_out = xb;
      }
      Timed tm(c, PIE_K_GEMM_DOWN);
      pie::launch_gemm(pie::A_BF16, pie::EPI_RESID, tile, g, st);
    }
    if ((rc = check_launch(c, flags, "down gemm"))) return rc;
  }

  int32_t* dtok = c->dev_tok_out ? c->dev_tok_out : M32(L.tokens_out);
  if (R > 0) {
    float* logits = nullptr;
    if (out_logits) logits = (flags & PIE_FLAG_LOGITS_DEVICE) ? out_logits : reinterpret_cast<float*>(c->ws + L.logits);
    pie::GemmArgs g = base;
    g.M = R;
    g.N = d.vocab;
    g.K = d.d_model;
    g.gain = c->final_norm;
    g.a_rows = M32(L.ro_row);
    g.w[0] = g.w[1] = g.w[2] = c->lm_head;
    g.seg_n0[0] = 0; g.seg_n0[1] = g.seg_n0[2] = g.seg_n0[3] = d.vocab;
    g.splits = 1;
    g.k_split = g.K;
    g.logits = logits;
    g.ro_kind = M32(L.ro_kind);
    g.ro_temp = reinterpret_cast<const float*>(M32(L.ro_temp));
    g.ro_seed_lo = reinterpret_cast<const uint32_t*>(M32(L.ro_seed_lo));
    g.ro_seed_hi = reinterpret_cast<const uint32_t*>(M32(L.ro_seed_hi));
    g.ro_lane = M32(L.ro_lane);
    g.tile_best = reinterpret_cast<float*>(c->ws + L.tile_best);
    g.tile_idx = reinterpret_cast<int32_t*>(c->ws + L.tile_idx);
    const int vt = (d.vocab + LM_BN - 1) / LM_BN;
    {
      Timed tm(c, PIE_K_LM_HEAD);
      if (R <= 64) {  // gather + final RMSNorm of the readout rows, then the weight stream
        pie::launch_rmsnorm(y, ss, n_ss, c->final_norm, R, d.d_model, d.rms_eps, g.a_rows, xb, st);
        g.a = xb;
        g.lda = d.d_model;
        if (c->f8 && c->f8_head) {
          g.w8[0] = c->f8_head;
          g.s8[0] = c->f8_head_s;
          g.f8 = 1;
        }
        pie::launch_gemm(pie::A_BF16, pie::EPI_LOGITS, pie::TILE_SKINNY, g, st);
      } else {
        pie::launch_gemm(pie::A_NORM, pie::EPI_LOGITS, pie::TILE_128x128, g, st);
      }
      pie::launch_argmax_reduce(g.tile_best, g.tile_idx, vt, R, dtok, st);
    }
    if ((rc = check_launch(c, flags, "lm_head"))) return rc;
    if (out_logits && !(flags & PIE_FLAG_LOGITS_DEVICE))
      HIP_TRY(c, hipMemcpyAsync(out_logits, logits, (size_t)R * d.vocab * 4, hipMemcpyDeviceToHost, st));
  }
  return PIE_OK;
}

// Run a call: enqueue directly, or replay (after capturing it the second
// time its launch shape comes up) a graph of the whole launch sequence.
// Graphs are captured on an internal stream and launched on the caller's.
int run_forward(pie_ctx* c, int32_t* out_tokens, float* out_logits, int flags) {
  int rc = acquire_staging(c);
  if (rc) return rc;
  rc = stage(c);
  if (rc) return rc;
  const pie::Plan& p = c->plan;
  const bool host_logits = out_logits && !(flags & PIE_FLAG_LOGITS_DEVICE);
  // timed calls launch directly: kernel timing uses events between launches
  const bool graphable = c->use_graphs && c->cap_stream && !host_logits && !c->prof_mask &&
                         !(flags & PIE_FLAG_SYNC_DEBUG) && !c->in_static;
  GraphEntry* ge = nullptr;
  if (graphable) {
    GraphKey key{p.n_rows, p.n_readout, (int)(c->dec.size() / 4), (int)(c->comb.size() / 4),
                 (int)(c->pre.size() / 4), flags, out_logits};
    if (c->graphs.size() >= 64 && !c->graphs.count(key)) release_graphs(c);
    ge = &c->graphs[key];
    if (!ge->exec && ++ge->seen >= 2) {
      // capture; any failure leaves this shape on direct launches
      c->cur = c->cap_stream;
      c->capturing = true;
      hipGraph_t graph = nullptr;
      hipError_t e = hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal);
      if (e == hipSuccess) {
        rc = enqueue(c, out_logits, flags);
        e = hipStreamEndCapture(c->cap_stream, &graph);
        if (rc == PIE_OK && e == hipSuccess && graph)
          e = hipGraphInstantiate(&ge->exec, graph, nullptr, nullptr, 0);
        else if (e == hipSuccess)
          e = hipErrorUnknown;
      }
      if (graph) (void)hipGraphDestroy(graph);
      c->capturing = false;
      if (e != hipSuccess || !ge->exec) {
        (void)hipGetLastError();
        ge->exec = nullptr;
        ge->seen = -(1 << 30);
        g_err.clear();
      }
    }
  }
  if ((rc = upload_meta(c))) return rc;
  if (ge && ge->exec) {
    HIP_TRY(c, hipGraphLaunch(ge->exec, c->stream));
  } else {
    c->cur = c->stream;
    c->sink.used = 0;
    c->sink.marks.clear();
    rc = enqueue(c, out_logits, flags);
    if (rc) return rc;
  }
  if ((rc = download_tokens(c))) return rc;
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  if (c->prof_mask) collect_profile(c, c->sink);
  if (p.n_readout > 0) std::memcpy(out_tokens, c->pinned + c->lay.tokens_out, (size_t)p.n_readout * 4);
  return PIE_OK;
}

// Enqueue one loop-carried decode step: tokens come from and go to device
// arrays, nothing is copied back and nothing waits for the GPU.
int run_decode_async(pie_ctx* c, const int32_t* tokens_in, int32_t* tokens_out, float* logits_dev) {
  int rc = acquire_staging(c);
  if (rc) return rc;
  if ((rc = stage(c))) return rc;
  if ((rc = upload_meta(c))) return rc;
  c->cur = c->stream;
  c->sink.used = 0;
  c->sink.marks.clear();
  c->dev_tok_in = tokens_in;
  c->dev_tok_out = tokens_out;
  rc = enqueue(c, logits_dev, logits_dev ? PIE_FLAG_LOGITS_DEVICE : 0);
  c->dev_tok_in = nullptr;
  c->dev_tok_out = nullptr;
  return rc;
}

}  // namespace

extern "C" {

size_t pie_kv_page_bytes(const pie_model_desc* desc) {
  std::string why;
  if (!desc_ok(desc, &why)) return 0;
  return (size_t)desc->n_layers * page_stride_elems(*desc) * kv_elem_bytes(*desc);
}

size_t pie_workspace_bytes(const pie_model_desc* desc, const pie_limits* limits) {
  std::string why;
  if (!desc_ok(desc, &why) || !limits_ok(limits, &why)) return 0;
  return make_layout(*desc, *limits).total;
}

int pie_init(const pie_model_desc* desc, const pie_weights* w, void* kv_arena, size_t kv_bytes,
             void* workspace, size_t ws_bytes, const pie_limits* limits, void* hip_stream,
             pie_ctx** out) {
  std::string why;
  if (!out) return set_err(PIE_EINVAL, "pie_init: null output");
  *out = nullptr;
  if (!desc_ok(desc, &why) || !limits_ok(limits, &why)) return set_err(PIE_EINVAL, "pie_init: " + why);
  const size_t page_bytes = pie_kv_page_bytes(desc);
  const int64_t n_pages = (int64_t)(kv_bytes / page_bytes);
  if (n_pages < 1) return set_err(PIE_EINVAL, "pie_init: KV arena smaller than one page");
  if (n_pages * desc->page_size >= ((int64_t)1 << 31))
    return set_err(PIE_EINVAL, "pie_init: too many pages for 32-bit slot ids");
  auto* c = new pie_ctx();
  c->d = *desc;
  c->lim = *limits;
  c->store = pie::KVStore(desc->page_size);
  c->store.reset(n_pages);
  c->n_pages = n_pages;
  c->page_stride = page_stride_elems(*desc);
  c->lay = make_layout(*desc, *limits);
  c->host_only = (w == nullptr);
  if (c->host_only) {
    c->pinned = static_cast<int32_t*>(std::malloc(c->lay.meta_ints * 4));
    *out = c;
    return PIE_OK;
  }
  const int L = desc->n_layers;
  if (!w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wq || !w->wk || !w->wv ||
      !w->wo || !w->mlp_norm || !w->w_gate || !w->w_up || !w->w_down) {
    delete c;
    return set_err(PIE_EINVAL, "pie_init: missing weight pointer");
  }
  if (desc->kv_dtype == PIE_KV_E4M3 && !w->kv_scale) {
    delete c;
    return set_err(PIE_EINVAL, "pie_init: e4m3 KV needs kv_scale");
  }
  // no workspace at all (NULL, 0): only pie_forward_static can run, in the
  // library's static scratch, whose size the limits must then fit
  c->has_workspace = !(workspace == nullptr && ws_bytes == 0);
  if (!kv_arena || (c->has_workspace && (!workspace || ws_bytes < c->lay.total))) {
    size_t need = c->lay.total;
    delete c;
    return set_err(PIE_EINVAL, "pie_init: workspace too small (need " + std::to_string(need) + " bytes)");
  }
  if (!c->has_workspace && c->lay.total > PIE_STATIC_SCRATCH_BYTES) {
    size_t need = c->lay.total;
    delete c;
    return set_err(PIE_ENOMEM, "pie_init: no workspace given and these limits need " + std::to_string(need) +
                                   " bytes, more than the static scratch's " +
                                   std::to_string((size_t)PIE_STATIC_SCRATCH_BYTES));
  }
  auto cp = [&](std::vector<const uint16_t*>& dst, const void* const* src, const char* nm) {
    dst.resize(L);
    for (int l = 0; l < L; ++l) {
      if (!src[l]) return std::string("pie_init: null ") + nm + " weight";
      dst[l] = static_cast<const uint16_t*>(src[l]);
    }
    return std::string();
  };
  for (auto& e : {cp(c->attn_norm, w->attn_norm, "attn_norm"), cp(c->wq, w->wq, "q"), cp(c->wk, w->wk, "k"),
                  cp(c->wv, w->wv, "v"), cp(c->wo, w->wo, "o"), cp(c->mlp_norm, w->mlp_norm, "mlp_norm"),
                  cp(c->wg, w->w_gate, "gate"), cp(c->wu, w->w_up, "up"), cp(c->wd, w->w_down, "down")})
    if (!e.empty()) { delete c; return set_err(PIE_EINVAL, e); }
  c->embed = static_cast<const uint16_t*>(w->embed);
  c->final_norm = static_cast<const uint16_t*>(w->final_norm);
  c->lm_head = static_cast<const uint16_t*>(w->lm_head);
  c->kv_scale = desc->kv_dtype == PIE_KV_E4M3 ? w->kv_scale : nullptr;
  c->kv = static_cast<uint8_t*>(kv_arena);
  c->ws = static_cast<uint8_t*>(workspace);
  c->stream = static_cast<hipStream_t>(hip_stream);

  int dev = 0;
  hipDeviceProp_t prop;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) { delete c; return set_err(PIE_EHIP, std::string("pie_init: ") + hipGetErrorString(e)); }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    delete c;
    return set_err(PIE_ESTATE, std::string("pie_init: kernels are built for gfx950, device is ") + prop.gcnArchName);
  }
  // this device's static scratch, for pie_forward_static; without it only a
  // context that has no workspace of its own cannot run
  e = scratch_address(dev, &c->static_ws);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // must not surface in a later launch check
    c->static_ws = nullptr;
    if (!c->has_workspace) {
      delete c;
      return set_err(PIE_EHIP, std::string("pie_init: static scratch address: ") + hipGetErrorString(e));
    }
  }
  for (int i = 0; i < PIE_STAGING_SLOTS; ++i) {
    int32_t* buf = nullptr;
    hipEvent_t ev = nullptr;
    e = hipHostMalloc(reinterpret_cast<void**>(&buf), c->lay.meta_ints * 4, hipHostMallocDefault);
    if (e == hipSuccess) c->pin_ring.push_back(buf);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e == hipSuccess) c->pin_ev.push_back(ev);
    if (e != hipSuccess) {
      for (auto b : c->pin_ring) (void)hipHostFree(b);
      for (auto v : c->pin_ev) (void)hipEventDestroy(v);
      delete c;
      return set_err(PIE_EHIP, std::string("pie_init: staging buffers: ") + hipGetErrorString(e));
    }
  }
  c->pinned = c->pin_ring[0];
  // a default-priority stream of our own, used only to capture launch graphs
  if (hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking) != hipSuccess) c->cap_stream = nullptr;
  // Graph replay is opt-in: on the measured ROCm stack a replay of the
  // ~300-launch decode sequence started later than direct launches did.
  const char* ug = std::getenv("PIE_GRAPHS");
  c->use_graphs = ug && ug[0] && ug[0] != '0';
  c->cur = c->stream;
  *out = c;
  return PIE_OK;
}

int pie_destroy(pie_ctx* c) {
  if (!c) return PIE_OK;
  if (c->host_only) {
    std::free(c->pinned);
  } else {
    (void)hipStreamSynchronize(c->stream);
    release_graphs(c);
    if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
    for (auto b : c->pin_ring) (void)hipHostFree(b);
    for (auto v : c->pin_ev) (void)hipEventDestroy(v);
    for (auto e : c->sink.ev) (void)hipEventDestroy(e);
  }
  delete c;
  return PIE_OK;
}

#define CTX_OK(c)                                                         \
  do {                                                                    \
    if (!(c)) return set_err(PIE_EINVAL, "null context");                 \
    if ((c)->poisoned) return set_err(PIE_ESTATE, "context is poisoned"); \
  } while (0)

int pie_alloc_working_set(pie_ctx* c, pie_ws* out) {
  CTX_OK(c);
  std::string err;
  int rc = c->store.alloc(out, &err);
  return rc ? set_err(rc, err) : PIE_OK;
}

int pie_fork(pie_ctx* c, pie_ws parent, pie_ws* child) {
  CTX_OK(c);
  std::string err;
  int rc = c->store.fork(parent, child, &err);
  return rc ? set_err(rc, err) : PIE_OK;
}

int pie_free_working_set(pie_ctx* c, pie_ws ws) {
  CTX_OK(c);
  std::string err;
  int rc = c->store.release(ws, &err);
  return rc ? set_err(rc, err) : PIE_OK;
}

int pie_truncate(pie_ctx* c, pie_ws ws, int32_t new_len) {
  CTX_OK(c);
  std::string err;
  int rc = c->store.truncate(ws, new_len, &err);
  return rc ? set_err(rc, err) : PIE_OK;
}

int pie_ws_info(pie_ctx* c, pie_ws ws, pie_ws_stats* stats, int32_t* page_ids) {
  CTX_OK(c);
  const pie::WorkingSet* w = c->store.get(ws);
  if (!w) return set_err(PIE_EINVAL, "ws_info: invalid or stale working set");
  if (stats) {
    stats->len = w->len;
    stats->frozen_len = w->frozen_len;
    stats->n_pages = (int32_t)w->pages.size();
  }
  if (page_ids)
    for (size_t i = 0; i < w->pages.size(); ++i) page_ids[i] = w->pages[i].page;
  return PIE_OK;
}

int pie_pool_stats_get(pie_ctx* c, pie_pool_stats* out) {
  CTX_OK(c);
  if (!out) return set_err(PIE_EINVAL, "null output");
  out->pages_total = c->store.pool().total();
  out->pages_free = c->store.pool().free_count();
  out->pages_ever_allocated = c->store.pool().ever_allocated();
  out->kv_bytes_copied = 0;  // no code path copies KV bytes between pages
  return PIE_OK;
}

int pie_forward(pie_ctx* c, const pie_pass* passes, int32_t n_passes, int32_t* out_tokens,
                float* out_logits, int32_t flags) {
  CTX_OK(c);
  if (!(flags & PIE_FLAG_NO_LAUNCH) && c->host_only)
    return set_err(PIE_ESTATE, "pie_forward: a host-only context can only plan (PIE_FLAG_NO_LAUNCH)");
  // planning without computing would commit tokens whose KV no kernel wrote,
  // and the prefix registry could then hand those pages to another request
  if ((flags & PIE_FLAG_NO_LAUNCH) && !c->host_only)
    return set_err(PIE_EINVAL, "pie_forward: PIE_FLAG_NO_LAUNCH is only for host-only contexts");
  if (!c->host_only && !c->has_workspace)
    return set_err(PIE_ESTATE, "pie_forward: the context has no workspace (use pie_forward_static)");
  pie::PackLimits pl{c->lim.max_rows, c->lim.max_seqs, c->lim.max_readout, c->lim.max_ctx,
                     c->lay.max_pe, c->d.vocab};
  int64_t want_ro = 0;
  if (passes && n_passes > 0)
    for (int i = 0; i < n_passes; ++i) want_ro += passes[i].n_readout > 0 ? passes[i].n_readout : 0;
  if (want_ro > 0 && !out_tokens) return set_err(PIE_EINVAL, "pie_forward: null out_tokens");
  std::string err;
  int rc = pie::pack_batch(c->store, passes, n_passes, pl, &c->plan, &err);
  if (rc) return set_err(rc, err);
  if (flags & PIE_FLAG_NO_LAUNCH) {
    for (int i = 0; i < c->plan.n_readout; ++i) out_tokens[i] = -1;
    return PIE_OK;
  }
  return run_forward(c, out_tokens, out_logits, flags);
}

int pie_forward_static(pie_ctx* c, const pie_pass* passes, int32_t n_passes, int32_t* out_tokens,
                       float* out_logits, int32_t flags) {
  CTX_OK(c);
  if (c->host_only) return set_err(PIE_ESTATE, "pie_forward_static: host-only context");
  if (flags & PIE_FLAG_NO_LAUNCH)
    return set_err(PIE_EINVAL, "pie_forward_static: PIE_FLAG_NO_LAUNCH is only for host-only contexts");
  // kernel timing would create events lazily: not in the entry point that allocates nothing
  if (c->prof_mask) return set_err(PIE_EINVAL, "pie_forward_static: kernel timing must be off");
  if (c->lay.total > PIE_STATIC_SCRATCH_BYTES)
    return set_err(PIE_ENOMEM, "pie_forward_static: the context's limits need " + std::to_string(c->lay.total) +
                                   " bytes of scratch, more than the static scratch's " +
                                   std::to_string((size_t)PIE_STATIC_SCRATCH_BYTES));
  if (!c->static_ws) return set_err(PIE_ESTATE, "pie_forward_static: no static scratch on this device");
  pie::PackLimits pl{c->lim.max_rows, c->lim.max_seqs, c->lim.max_readout, c->lim.max_ctx,
                     c->lay.max_pe, c->d.vocab};
  int64_t want_ro = 0;
  if (passes && n_passes > 0)
    for (int i = 0; i < n_passes; ++i) want_ro += passes[i].n_readout > 0 ? passes[i].n_readout : 0;
  if (want_ro > 0 && !out_tokens) return set_err(PIE_EINVAL, "pie_forward_static: null out_tokens");
  std::string err;
  int rc = pie::pack_batch(c->store, passes, n_passes, pl, &c->plan, &err);
  if (rc) return set_err(rc, err);
  // the same launch sequence over the static scratch instead of the workspace
  uint8_t* own = c->ws;
  c->ws = c->static_ws;
  c->in_static = true;
  rc = run_forward(c, out_tokens, out_logits, flags);
  c->in_static = false;
  c->ws = own;
  return rc;
}

int pie_decode_async(pie_ctx* c, const pie_ws* ws, int32_t n, const int32_t* tokens_in, int32_t* tokens_out,
                     const pie_epilogue* epi, float* logits_dev) {
  CTX_OK(c);
  if (c->host_only) return set_err(PIE_ESTATE, "pie_decode_async: host-only context");
  if (!c->has_workspace)
    return set_err(PIE_ESTATE, "pie_decode_async: the context has no workspace (use pie_forward_static)");
  if (!ws || n < 1 || !tokens_in || !tokens_out || !epi)
    return set_err(PIE_EINVAL, "pie_decode_async: null argument or n < 1");
  if (c->prof_mask) return set_err(PIE_EINVAL, "pie_decode_async: kernel timing needs synchronous calls");
  // one committed pass of one token per working set, read out at its row;
  // the host token is a placeholder (the embedding reads tokens_in)
  if ((int)c->async_zero.size() < n) c->async_zero.assign(n, 0);
  c->async_pass.resize(n);
  static const int32_t zero_row = 0;
  for (int i = 0; i < n; ++i) {
    pie_pass& q = c->async_pass[i];
    q = pie_pass{};
    q.ws = ws[i];
    q.tokens = &c->async_zero[i];
    q.n_tokens = 1;
    q.positions = nullptr;
    q.readout = &zero_row;
    q.n_readout = 1;
    q.epi = &epi[i];
    q.commit = 1;
  }
  pie::PackLimits pl{c->lim.max_rows, c->lim.max_seqs, c->lim.max_readout, c->lim.max_ctx,
                     c->lay.max_pe, c->d.vocab};
  std::string err;
  int rc = pie::pack_batch(c->store, c->async_pass.data(), n, pl, &c->plan, &err, /*host_tokens=*/false);
  if (rc) return set_err(rc, err);
  return run_decode_async(c, tokens_in, tokens_out, logits_dev);
}

int pie_prefix_lookup(pie_ctx* c, const int32_t* tokens, int32_t n, pie_ws* out, int32_t* n_shared) {
  CTX_OK(c);
  if (tokens && n > 0)
    for (int32_t i = 0; i < n; ++i)
      if (tokens[i] < 0 || tokens[i] >= c->d.vocab)
        return set_err(PIE_EINVAL, "pie_prefix_lookup: token id out of range");
  std::string err;
  int rc = c->store.lookup(tokens, n, out, n_shared, &err);
  return rc ? set_err(rc, err) : PIE_OK;
}

int pie_sync(pie_ctx* c) {
  CTX_OK(c);
  if (c->host_only) return PIE_OK;
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  HIP_TRY(c, hipGetLastError());
  return PIE_OK;
}

const char* pie_last_error(void) { return g_err.c_str(); }

int pie_profile_enable(pie_ctx* c, uint32_t mask) {
  CTX_OK(c);
  c->prof_mask = mask & ((1u << PIE_K_NUM_CLASSES) - 1);
  for (int k = 0; k < PIE_K_NUM_CLASSES; ++k) {
    c->prof_ms[k] = 0;
    c->prof_n[k] = 0;
  }
  return PIE_OK;
}

int pie_profile_repeat(pie_ctx* c, int32_t reps) {
  CTX_OK(c);
  if (reps < 1 || reps > 64) return set_err(PIE_EINVAL, "pie_profile_repeat: reps must be in [1, 64]");
  c->prof_reps = reps;
  return PIE_OK;
}

int pie_profile_read(pie_ctx* c, double* ms, int64_t* counts) {
  CTX_OK(c);
  if (!c->host_only) {
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "pie_profile_read");
  }
  for (int k = 0; k < PIE_K_NUM_CLASSES; ++k) {
    if (ms) ms[k] = c->prof_ms[k];
    if (counts) counts[k] = c->prof_n[k];
  }
  return PIE_OK;
}

int pie_debug_plan(pie_ctx* c, pie_plan_view* v) {
  CTX_OK(c);
  if (!v) return set_err(PIE_EINVAL, "null output");
  const pie::Plan& p = c->plan;
  v->n_rows = p.n_rows; v->n_seqs = p.n_seqs; v->n_readout = p.n_readout; v->n_page_entries = p.n_pe;
  v->tok = p.tok.data(); v->pos = p.pos.data(); v->row_seq = p.row_seq.data(); v->slot = p.slot.data();
  v->seq_row0 = p.seq_row0.data(); v->seq_ctx = p.seq_ctx.data(); v->seq_len = p.seq_len.data();
  v->seq_pg0 = p.seq_pg0.data(); v->pg_id = p.pg_id.data(); v->pg_valid = p.pg_valid.data();
  v->pg_start = p.pg_start.data(); v->ro_row = p.ro_row.data(); v->ro_lane = p.ro_lane.data();
  return PIE_OK;
}

int pie_debug_philox(pie_ctx* c, uint64_t seed, uint32_t lane, uint32_t v0, int32_t n, uint32_t* out) {
  CTX_OK(c);
  if (c->host_only) return set_err(PIE_ESTATE, "pie_debug_philox: host-only context");
  if (n < 0 || (n > 0 && !out)) return set_err(PIE_EINVAL, "pie_debug_philox: bad arguments");
  pie::launch_philox(seed, lane, v0, n, out, c->stream);
  HIP_TRY(c, hipGetLastError());
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  return PIE_OK;
}

size_t pie_packed_weight_fp8_bytes(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0) return 0;
  return pie::packed_elems(n, k);
}

size_t pie_fp8_scale_count(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0) return 0;
  return (size_t)pie::fp8_scale_blocks(n) * pie::fp8_scale_blocks(k);
}

int pie_pack_weight_fp8(const void* src, void* codes, float* scales, int32_t n, int32_t k, void* hip_stream) {
  if (!src || !codes || !scales || n <= 0 || k <= 0) return set_err(PIE_EINVAL, "pie_pack_weight_fp8: bad arguments");
  const size_t src_bytes = (size_t)n * k * 2, code_bytes = pie::packed_elems(n, k),
               scale_bytes = (size_t)pie::fp8_scale_blocks(n) * pie::fp8_scale_blocks(k) * 4;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(codes),
                  c8 = reinterpret_cast<uintptr_t>(scales);
  if ((a < b + code_bytes && b < a + src_bytes) || (a < c8 + scale_bytes && c8 < a + src_bytes) ||
      (b < c8 + scale_bytes && c8 < b + code_bytes))
    return set_err(PIE_EINVAL, "pie_pack_weight_fp8: src, codes and scales overlap");
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  hipError_t e = hipMemsetAsync(codes, 0, pie::packed_elems(n, k), st);
  if (e == hipSuccess) {
    pie::launch_pack_weight_fp8(static_cast<const uint16_t*>(src), static_cast<uint8_t*>(codes), scales, n, k, st);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_err(PIE_EHIP, std::string("pie_pack_weight_fp8: ") + hipGetErrorString(e));
  return PIE_OK;
}

int pie_attach_fp8_weights(pie_ctx* c, const pie_fp8_weights* w) {
  CTX_OK(c);
  if (!w) return set_err(PIE_EINVAL, "pie_attach_fp8_weights: null weights");
  const int L = c->d.n_layers;
  const void* const* codes[7] = {w->wq, w->wk, w->wv, w->wo, w->w_gate, w->w_up, w->w_down};
  const float* const* sc[7] = {w->sq, w->sk, w->sv, w->so, w->s_gate, w->s_up, w->s_down};
  for (int i = 0; i < 7; ++i) {
    if (!codes[i] || !sc[i]) return set_err(PIE_EINVAL, "pie_attach_fp8_weights: null array");
    for (int l = 0; l < L; ++l)
      if (!codes[i][l] || !sc[i][l]) return set_err(PIE_EINVAL, "pie_attach_fp8_weights: null pointer");
  }
  for (int i = 0; i < 7; ++i) {
    c->f8w[i].assign(L, nullptr);
    c->f8s[i].assign(L, nullptr);
    for (int l = 0; l < L; ++l) {
      c->f8w[i][l] = static_cast<const uint8_t*>(codes[i][l]);
      c->f8s[i][l] = sc[i][l];
    }
  }
  if (!w->lm_head != !w->s_lm_head) return set_err(PIE_EINVAL, "pie_attach_fp8_weights: lm_head without scales");
  c->f8_head = static_cast<const uint8_t*>(w->lm_head);
  c->f8_head_s = w->s_lm_head;
  // captured launches name the bf16 weights: drop them once nothing runs
  if (!c->host_only) HIP_TRY(c, hipStreamSynchronize(c->stream));
  c->f8 = true;
  release_graphs(c);
  return PIE_OK;
}

size_t pie_packed_weight_bytes(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0) return 0;
  return pie::packed_elems(n, k) * 2;
}

int pie_pack_weight(const void* src, void* dst, int32_t n, int32_t k, void* hip_stream) {
  if (!src || !dst || n <= 0 || k <= 0) return set_err(PIE_EINVAL, "pie_pack_weight: bad arguments");
  const size_t src_bytes = (size_t)n * k * 2, dst_bytes = pie::packed_elems(n, k) * 2;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + dst_bytes && b < a + src_bytes) return set_err(PIE_EINVAL, "pie_pack_weight: src and dst overlap");
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  pie::launch_pack_weight(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), n, k, st);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_err(PIE_EHIP, std::string("pie_pack_weight: ") + hipGetErrorString(e));
  return PIE_OK;
}

}  // extern "C"
