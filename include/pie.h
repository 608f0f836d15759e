/*
 * pie.h -- C ABI of the batched paged-KV forward pass for AMD gfx950.
 *
 * One call, pie_forward, runs the Llama-style decoder of the Pie pages
 * ("Write a model in Poem", section 5 Forward pass: embed, per layer
 * RMSNorm -> RoPE'd grouped-query attention over the sequence's KV ->
 * residual add -> RMSNorm -> SwiGLU -> residual add, then final RMSNorm,
 * gather of the readout rows, lm_head) over a batch of forward passes from
 * many sequences at once ("How Pie thinks", "Batching is still the engine's
 * job"), then runs the fused epilogue of each readout row on the device and
 * returns only a token id per row ("How Pie thinks", section 5 Epilogues).
 *
 * Each sequence's KV lives in a working set ("How Pie thinks", section 4
 * Working sets): a page table over a pool of fixed-size KV pages, with a
 * frozen prefix (committed tokens) and a writable buffer (uncommitted
 * tokens).  pie_fork makes a new working set that shares the frozen prefix's
 * pages without copying them.
 *
 * Conventions
 *  - Every function returning int returns PIE_OK (0) or a negative pie_status;
 *    pie_last_error() then gives a message (thread-local, valid until the next
 *    call on the same thread).
 *  - "device" pointers are HIP device memory of the GPU that is current when
 *    pie_init is called; "host" pointers are ordinary process memory.
 *  - The caller owns weights, the KV arena, the workspace and the stream; they
 *    must outlive the context.  The library owns working-set and page-pool
 *    metadata.  Host arrays passed in are read only during the call.
 *  - A context is not thread-safe: one thread at a time per context.
 *  - After PIE_EHIP a context is poisoned: every later call but pie_destroy
 *    returns PIE_ESTATE.
 */
#ifndef PIE_H
#define PIE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PIE_ABI_VERSION 1

typedef struct pie_ctx pie_ctx;

/* Working-set handle: (generation << 32) | (slot + 1).  0 is never valid; a
 * handle whose working set was freed is stale and rejected with PIE_EINVAL. */
typedef uint64_t pie_ws;

enum pie_status {
  PIE_OK = 0,
  PIE_EINVAL = -1, /* bad argument, stale handle, or a batch that breaks a rule */
  PIE_ENOMEM = -2, /* KV page pool exhausted, or a batch beyond the init limits  */
  PIE_EHIP = -3,   /* a HIP runtime call failed (context is poisoned)            */
  PIE_ESTATE = -4  /* context poisoned, or a call the context cannot serve       */
};

/* KV storage formats ("Write a model in Poem", section 2 Deployments). */
enum pie_kv_dtype { PIE_KV_BF16 = 0, PIE_KV_E4M3 = 1 };

/* Fused epilogues ("How Pie thinks", sections 3 and 5). */
enum pie_epilogue_kind { PIE_EPI_ARGMAX = 0, PIE_EPI_GUMBEL_MAX = 1 };

/* pie_forward flags */
enum pie_forward_flags {
  PIE_FLAG_NO_LAUNCH = 1,     /* validate, reserve, pack and update working sets, launch nothing;
                                 out_tokens are set to -1.  The only mode of a host-only context,
                                 and refused (PIE_EINVAL) on a context with weights, whose
                                 committed pages must hold computed KV. */
  PIE_FLAG_LOGITS_DEVICE = 2, /* out_logits is a device pointer (default: host pointer)           */
  PIE_FLAG_SYNC_DEBUG = 4     /* synchronise and check for errors after every kernel              */
};

/* Model shape ("Write a model in Poem", section 1 MODELS, section 4 caches).
 * Constraints: head_dim = 64 or 128; n_q_heads % n_kv_heads == 0;
 * d_model % 128 == 0; page_size = 16. */
typedef struct pie_model_desc {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rms_eps;    /* epsilon inside the RMSNorm square root               */
  float rope_theta; /* RoPE base; rotate-half pairs (j, j + head_dim/2)     */
  int32_t kv_dtype; /* pie_kv_dtype                                          */
  int32_t page_size;
} pie_model_desc;

/* Weights: caller-owned DEVICE pointers to bf16 tensors ("Write a model in
 * Poem", section 3 Weights: the checkpoint layout is [out][in]).
 *  - embed, final_norm and the norm gains: plain row-major, as in the checkpoint.
 *  - the projections wq, wk, wv, wo, w_gate, w_up, w_down and lm_head: the
 *    library's tiled layout, made from the [out][in] tensor by pie_pack_weight
 *    (pie_packed_weight_bytes gives its size).
 * The per-layer members are HOST arrays of n_layers device pointers; the
 * library copies the pointer arrays during pie_init. */
typedef struct pie_weights {
  const void* embed;      /* [vocab][d_model]            */
  const void* final_norm; /* [d_model]                   */
  const void* lm_head;    /* [vocab][d_model]            */
  const void* const* attn_norm; /* [L] -> [d_model]                     */
  const void* const* wq;        /* [L] -> [n_q_heads*head_dim][d_model] */
  const void* const* wk;        /* [L] -> [n_kv_heads*head_dim][d_model]*/
  const void* const* wv;        /* [L] -> [n_kv_heads*head_dim][d_model]*/
  const void* const* wo;        /* [L] -> [d_model][n_q_heads*head_dim] */
  const void* const* mlp_norm;  /* [L] -> [d_model]                     */
  const void* const* w_gate;    /* [L] -> [d_ffn][d_model]              */
  const void* const* w_up;      /* [L] -> [d_ffn][d_model]              */
  const void* const* w_down;    /* [L] -> [d_model][d_ffn]              */
  /* e4m3 KV only: DEVICE float32 [L][2 (K, V)][n_kv_heads] dequantisation
   * scales (stored code * scale = value); NULL for bf16 KV. */
  const float* kv_scale;
} pie_weights;

/* Capacity of one pie_forward call; fixes the workspace size. */
typedef struct pie_limits {
  int32_t max_rows;    /* packed new tokens per call                          */
  int32_t max_seqs;    /* passes (sequences) per call                         */
  int32_t max_readout; /* readout rows per call                               */
  int32_t max_ctx;     /* tokens in one working set, including the new ones  */
} pie_limits;

/* Tiled weight layout of the projections and lm_head.  An [n][k] bf16 matrix
 * (row-major, the checkpoint's [out][in]) is zero-padded to n and k rounded
 * up to 64 and stored as 8 KiB blocks: block (r / 64, c / 64) sits at block
 * index (r / 64) * ceil(k / 64) + c / 64 and holds its 64 x 64 elements as
 * [4 panels of 16 rows][2 halves of 32 columns][4 groups of 8 columns]
 * [16 rows][8 columns].  A decode GEMM then reads every weight tile in
 * address order.  Returns the packed size in bytes (0 if n or k <= 0). */
size_t pie_packed_weight_bytes(int32_t n, int32_t k);

/* Convert one weight matrix ("Write a model in Poem", section 3 Weights: the
 * checkpoint's [out][in] tensor) to the tiled layout: src is DEVICE bf16 [n][k]
 * row-major, dst DEVICE memory of pie_packed_weight_bytes(n, k) bytes; they
 * must not overlap.  Runs on hip_stream (NULL = the null stream) and
 * synchronises it.  Needs no context.  Errors: PIE_EINVAL, PIE_EHIP. */
int pie_pack_weight(const void* src, void* dst, int32_t n, int32_t k, void* hip_stream);

/* Block-scaled FP8 copies of the layer projections for the decode GEMMs
 * ("Write a model in Poem", section 2: weights in dtype.e4m3tile128a8,
 * block-scaled FP8; the pages do not define the blocking).  Reading taken:
 * OCP e4m3 codes with one power-of-two scale per 128 x 128 block of the
 * [out][in] matrix, 2^e with e the least integer for which the block's
 * largest |w| is at most 448 * 2^e.  A code times its scale is exactly a
 * bf16 value, so a bf16 matrix whose every block is e4m3 times its scale
 * converts losslessly; other values are rounded to the nearest code (ties
 * to even, saturating).  Decode-sized calls (at most 64 rows) then stream
 * half the weight bytes and compute exactly what the bf16 weights give;
 * larger calls keep using the bf16 weights of pie_init.
 * pie_packed_weight_fp8_bytes: bytes of the codes of an [n][k] matrix (a
 * tiled layout of 4 KiB blocks of 64 x 64, see gemm.h); pie_fp8_scale_count:
 * floats of its scales, [ceil(n / 128)][ceil(k / 128)]. */
size_t pie_packed_weight_fp8_bytes(int32_t n, int32_t k);
size_t pie_fp8_scale_count(int32_t n, int32_t k);

/* src: DEVICE bf16 [n][k] row-major; codes: DEVICE memory of
 * pie_packed_weight_fp8_bytes(n, k) bytes (cleared here); scales: DEVICE
 * float32 [pie_fp8_scale_count(n, k)]; the three must not overlap.  Runs on
 * hip_stream and synchronises it.  Needs no context.  Errors: PIE_EINVAL
 * (null pointer, n or k <= 0, overlap), PIE_EHIP. */
int pie_pack_weight_fp8(const void* src, void* codes, float* scales, int32_t n, int32_t k, void* hip_stream);

/* Per-layer HOST arrays of n_layers DEVICE pointers: codes and scales of each
 * projection, made by pie_pack_weight_fp8 from the same matrices pie_init
 * was given.  The caller keeps them alive until pie_destroy. */
typedef struct pie_fp8_weights {
  const void* const *wq, *const *wk, *const *wv, *const *wo, *const *w_gate, *const *w_up, *const *w_down;
  const float* const *sq, *const *sk, *const *sv, *const *so, *const *s_gate, *const *s_up, *const *s_down;
  const void* lm_head;    /* DEVICE codes of [vocab][d_model], or NULL: the head stays bf16 */
  const float* s_lm_head; /* its scales (NULL with lm_head NULL) */
} pie_fp8_weights;

/* From the next call on, decode-sized calls stream these FP8 copies instead
 * of the bf16 projections (and of the bf16 lm_head when given, for calls of
 * at most 64 readout rows).  Errors: PIE_EINVAL (null array or pointer),
 * PIE_ESTATE (poisoned context). */
int pie_attach_fp8_weights(pie_ctx* ctx, const pie_fp8_weights* w);

/* Bytes of one KV page over all layers (K and V, every KV head, page_size
 * tokens): the per-layer K and V of the caches declaration ("Write a model in
 * Poem", section 4 State (caches)) for page_size tokens; 0 on a bad desc. */
size_t pie_kv_page_bytes(const pie_model_desc* desc);

/* Device workspace bytes pie_init needs for these limits (0 on bad input):
 * the activations of one batched launch ("How Pie thinks", "Batching is still
 * the engine's job") plus the attention and GEMM partials. */
size_t pie_workspace_bytes(const pie_model_desc* desc, const pie_limits* limits);

/* Create a context over one model ("Write a model in Poem", section 1 MODELS
 * for the shape, section 3 Weights for the tensors, section 4 for the KV
 * space) on one GPU.
 *  kv_arena/kv_bytes: DEVICE memory for the page pool; pages = kv_bytes / pie_kv_page_bytes.
 *  workspace/ws_bytes: DEVICE scratch of at least pie_workspace_bytes(desc, limits),
 *    or NULL and 0 for a context that runs only pie_forward_static.
 *  hip_stream: the hipStream_t every launch goes to (NULL = the null stream).
 * With weights == NULL the context is host-only: it keeps working sets, page
 * pool and batch packing but never touches the GPU (kv_arena and workspace may be
 * NULL, kv_bytes still sizes the pool) and pie_forward needs PIE_FLAG_NO_LAUNCH.
 * Errors: PIE_EINVAL (bad shape, limits or sizes), PIE_EHIP. */
int pie_init(const pie_model_desc* desc, const pie_weights* weights, void* kv_arena,
             size_t kv_bytes, void* workspace, size_t ws_bytes, const pie_limits* limits,
             void* hip_stream, pie_ctx** out);

/* Destroy a context; outstanding working sets are released.  NULL is a no-op.
 * Caller-owned memory (weights, arena, workspace, stream) is not freed. */
int pie_destroy(pie_ctx* ctx);

/* WorkingSet(): a new, empty working set (len = frozen_len = 0). */
int pie_alloc_working_set(pie_ctx* ctx, pie_ws* out);

/* ws.fork() ("How Pie thinks", section 4): a new working set that shares the
 * parent's FROZEN prefix pages (reference counts +1, no KV bytes move) and has
 * an empty writable buffer; the parent's uncommitted tokens are not inherited.
 * A page shared this way is never written again: whoever appends next starts a
 * fresh page, so a partly filled shared page stays partly filled in both. */
int pie_fork(pie_ctx* ctx, pie_ws parent, pie_ws* child);

/* Release a working set; pages whose reference count drops to 0 return to the
 * pool.  ("How Pie thinks", section 4 Working sets: a working set is a
 * sequence's model state, owned by its program until dropped; shared frozen
 * pages outlive the set as long as a fork still holds them.)  Errors:
 * PIE_EINVAL (stale or null handle). */
int pie_free_working_set(pie_ctx* ctx, pie_ws ws);

/* Roll the writable buffer back to new_len tokens (frozen_len <= new_len <= len).
 * ("How Pie thinks", section 4 Working sets: the writable buffer holds
 * uncommitted tokens that may be rolled back, as a speculative draft is;
 * the frozen prefix never changes.)  Pages left empty return to the pool.
 * Errors: PIE_EINVAL (stale handle, new_len outside [frozen_len, len]). */
int pie_truncate(pie_ctx* ctx, pie_ws ws, int32_t new_len);

typedef struct pie_ws_stats {
  int32_t len;        /* tokens in the working set                    */
  int32_t frozen_len; /* committed prefix length                      */
  int32_t n_pages;    /* page-table entries                           */
} pie_ws_stats;

/* Working-set state ("How Pie thinks", section 4 Working sets: the committed
 * prefix length is frozen_len, everything after it is the writable buffer);
 * page_ids (nullable, host, n_pages entries) receives the page table's page
 * ids in order, which shows that a fork shares its parent's pages.
 * Errors: PIE_EINVAL (stale handle or null stats). */
int pie_ws_info(pie_ctx* ctx, pie_ws ws, pie_ws_stats* stats, int32_t* page_ids);

/* Page-pool counters ("How Pie thinks", section 4 Working sets: a fork shares
 * the frozen prefix without copying it, so kv_bytes_copied stays 0 and a
 * fork takes no page from the free list). */
typedef struct pie_pool_stats {
  int64_t pages_total;
  int64_t pages_free;
  int64_t pages_ever_allocated; /* pages taken from the free list since init      */
  int64_t kv_bytes_copied;      /* KV bytes ever copied between pages (always 0)  */
} pie_pool_stats;

/* Errors: PIE_EINVAL (null out). */
int pie_pool_stats_get(pie_ctx* ctx, pie_pool_stats* out);

/* Epilogue of one readout row.  ARGMAX: the lowest index of the largest logit.
 * GUMBEL_MAX: the lowest index of the largest logit/temperature + G, where
 * G = -ln(-ln u), u = ((x >> 9) + 0.5) * 2^-23 and x is word 0 of
 * Philox4x32-10 with counter (vocab index, lane, 0, 0) and key (seed low 32
 * bits, seed high 32 bits); lane is the row's index in its pass's readout list.
 * temperature must be finite and > 0 for GUMBEL_MAX (ignored for ARGMAX). */
typedef struct pie_epilogue {
  int32_t kind;
  float temperature;
  uint64_t seed;
} pie_epilogue;

/* One ForwardPass ("How Pie thinks", section 3): new tokens for one working
 * set, which rows to read out, the epilogue per readout row, and whether the
 * appended tokens are committed (StateGeometry.folding(): append and freeze). */
typedef struct pie_pass {
  pie_ws ws;
  const int32_t* tokens;    /* host [n_tokens]; 0 <= id < vocab                          */
  const int32_t* positions; /* host [n_tokens] RoPE positions, or NULL for len + i      */
  int32_t n_tokens;         /* >= 1                                                      */
  const int32_t* readout;   /* host [n_readout] row indices into this pass's tokens      */
  int32_t n_readout;        /* >= 0                                                      */
  const pie_epilogue* epi;  /* host [n_readout]                                          */
  int32_t commit;           /* 1: freeze everything appended so far; 0: writable buffer */
} pie_pass;

/* Run one batched forward over n_passes passes of distinct working sets.
 *  out_tokens: host [sum n_readout] int32, pass order then readout order.
 *  out_logits: NULL, or [sum n_readout][vocab] float32 (host pointer, or device
 *              pointer with PIE_FLAG_LOGITS_DEVICE).
 * All-or-nothing: every pass is validated and every page reserved before any
 * launch; on an error no working set changes.
 * Errors: PIE_EINVAL (no passes, stale handle, the same working set twice, a
 * pass without tokens, token id out of range, negative position, readout index
 * out of range, unknown epilogue kind, temperature <= 0 or not finite, a
 * sequence beyond max_ctx), PIE_ENOMEM (page pool exhausted, or more
 * rows/passes/readouts/page-table entries than the init limits), PIE_EHIP,
 * PIE_ESTATE (poisoned or host-only context without PIE_FLAG_NO_LAUNCH).
 * Returns after the stream has finished the call's work. */
int pie_forward(pie_ctx* ctx, const pie_pass* passes, int32_t n_passes, int32_t* out_tokens,
                float* out_logits, int32_t flags);

/* Bytes of the library's static device scratch (pie_forward_static), held
 * by every GPU the library runs on from load to process end. */
#define PIE_STATIC_SCRATCH_BYTES (96u * 1024u * 1024u)

/* pie_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same passes, validation, all-or-nothing rule, results and errors as
 * pie_forward, but every buffer the call's kernels use besides the caller's
 * inputs and outputs (activations, packed metadata, split-K and attention
 * partials, per-tile maxima of the epilogue) lives in the library's static
 * device scratch of PIE_STATIC_SCRATCH_BYTES instead of the context's
 * workspace, and the call allocates nothing (no hipMalloc, hipFree or other
 * allocating routine; metadata goes through the pinned staging pie_init made).
 * A context created with workspace == NULL and ws_bytes == 0 serves only
 * this call (its limits must fit the scratch; pie_forward and
 * pie_decode_async then return PIE_ESTATE).
 *  - Every call on one GPU shares that GPU's scratch, which keeps the last
 *    call's contents; nothing in it needs to start at zero (each kernel
 *    writes what it later reads within the call).  Calls that overlap on one
 *    GPU (two contexts on different streams or threads) race: the caller
 *    serialises them.  The call returns after its stream has finished.
 *  - Errors: as pie_forward; PIE_ENOMEM (before any state changes) when the
 *    context's limits need more scratch than PIE_STATIC_SCRATCH_BYTES;
 *    PIE_EINVAL while kernel timing is on. */
int pie_forward_static(pie_ctx* ctx, const pie_pass* passes, int32_t n_passes, int32_t* out_tokens,
                       float* out_logits, int32_t flags);

/* Loop-carried decode, enqueued without waiting ("How Pie thinks", section 3
 * Forward passes: submitting a pass to a Pipeline returns at once and queued
 * passes run in order, so later passes can be submitted before earlier
 * results are back; section 5 Epilogues: only the chosen token leaves the GPU).
 * Here the token does not even leave it: each step's output feeds the next.
 * One committed pass of one token per working set ws[0..n), read out at that
 * token with epi[i] (host [n]), at position = the working set's length.
 *  tokens_in:  DEVICE int32 [n]; pass i's token is tokens_in[i] as the step
 *              reads it on the GPU, so it may be the output of a step still
 *              in flight (tokens_in == tokens_out is allowed).
 *  tokens_out: DEVICE int32 [n]; receives the chosen tokens.
 *  logits_dev: NULL, or DEVICE float32 [n][vocab] for the step's logits.
 * Nothing is copied to the host and the call returns once the step is
 * enqueued on the context's stream; steps run in the order enqueued.  The
 * host bookkeeping (working-set lengths, page reservation) advances at
 * enqueue, with the same validation and all-or-nothing rule as pie_forward
 * (token values are not checked: they are on the device; an id outside
 * [0, vocab), such as the -1 an all-NaN logits row yields, embeds as a zero
 * row rather than reading outside the table).  At most 4 calls
 * are staged ahead of the GPU; a further call waits for the oldest staging
 * copy to run.  The device arrays must stay valid until the step has run
 * (pie_sync).  Kernel timing (pie_profile_enable) must be off: PIE_EINVAL.
 * Errors: as pie_forward; a HIP error of a step may surface at pie_sync. */
int pie_decode_async(pie_ctx* ctx, const pie_ws* ws, int32_t n, const int32_t* tokens_in, int32_t* tokens_out,
                     const pie_epilogue* epi, float* logits_dev);

/* Wait until every enqueued step has run ("How Pie thinks", section 3: the
 * awaited result of a submitted pass); PIE_EHIP (and a poisoned context) if
 * one of them failed. */
int pie_sync(pie_ctx* ctx);

/* Prefix sharing across requests ("How Pie thinks", section 4 Working sets:
 * a fork shares the frozen prefix and copies nothing; this extends that to
 * working sets with no common parent).  Every whole page of a committed
 * prefix whose token ids were given on the host (pie_forward, not
 * pie_decode_async) at the default positions 0, 1, 2, ... is remembered
 * under its token prefix.  This call returns in *out a new working set
 * holding the longest remembered prefix of tokens (host [n]) in whole pages,
 * at most n - 1 tokens, shared with the working sets that computed it
 * (reference counts +1, no KV byte copied or recomputed); *n_shared is its
 * length, 0 when nothing matched (a plain empty working set).  The caller then
 * runs tokens[*n_shared, n) as the set's first pass.  A page is forgotten when
 * its last holder frees it.  Matching compares the page's own token ids and
 * two independent chain hashes of everything before it.
 * Errors: PIE_EINVAL (null argument, n < 1, token id out of range). */
int pie_prefix_lookup(pie_ctx* ctx, const int32_t* tokens, int32_t n, pie_ws* out, int32_t* n_shared);

/* Message of the last failed call on this thread ("" if none). */
const char* pie_last_error(void);

/* ---------------------------------------------------------------------------
 * Measurement hooks.  Not operations of the pages (which publish no
 * measurement of this path): they time the kernel classes of the forward
 * pass so its throughput can be set against the HBM and matrix-core peaks.
 * ------------------------------------------------------------------------- */

/* Kernel classes a context can time with HIP events recorded on its stream. */
enum pie_kernel_class {
  PIE_K_EMBED = 0,      /* embedding gather                                 */
  PIE_K_GEMM_QKV = 1,   /* RMSNorm-fused QKV projection + RoPE + KV append  */
  PIE_K_ATTN_DECODE = 2,/* paged decode attention (split-KV + combine)      */
  PIE_K_ATTN_PREFILL = 3,/* paged chunked-prefill attention                 */
  PIE_K_GEMM_O = 4,     /* output projection + residual                     */
  PIE_K_GEMM_GATEUP = 5,/* RMSNorm-fused gate/up projection + SwiGLU        */
  PIE_K_GEMM_DOWN = 6,  /* down projection + residual                       */
  PIE_K_LM_HEAD = 7,    /* final RMSNorm + gather + lm_head + epilogue      */
  PIE_K_NUM_CLASSES = 8
};

/* Time every launch of the classes in class_mask (bit i = class i) from now on
 * (0 turns timing off and clears totals). */
int pie_profile_enable(pie_ctx* ctx, uint32_t class_mask);

/* While decode attention (PIE_K_ATTN_DECODE) is timed, run each of its
 * launches reps times back to back inside its timed interval (1 <= reps <= 64;
 * 1 until set).  The repeats read the same q and KV and write the same output,
 * so results do not change, and the class's launch count advances by reps.
 * The event records around an interval idle the GPU for several microseconds;
 * over reps launches that cost is shared, and the average per launch comes
 * close to the kernel's own duration.  Errors: PIE_EINVAL. */
int pie_profile_repeat(pie_ctx* ctx, int32_t reps);

/* Per class: total milliseconds and number of launches timed since enabling.
 * Synchronises the stream.  ms and counts are host arrays [PIE_K_NUM_CLASSES]. */
int pie_profile_read(pie_ctx* ctx, double* ms, int64_t* counts);

/* ---------------------------------------------------------------------------
 * Debug views (used by tests).  pie_debug_plan exposes the packed batch of
 * "How Pie thinks" ("Batching is still the engine's job"); pie_debug_philox
 * the noise of the Gumbel-max epilogue (section 5 Epilogues).
 * ------------------------------------------------------------------------- */

/* The metadata the packer built for the last pie_forward of this context
 * (host copies; valid until the next pie_forward or pie_destroy). */
typedef struct pie_plan_view {
  int32_t n_rows, n_seqs, n_readout, n_page_entries;
  const int32_t* tok;      /* [n_rows]                                           */
  const int32_t* pos;      /* [n_rows]                                           */
  const int32_t* row_seq;  /* [n_rows] launch-local sequence of each row        */
  const int32_t* slot;     /* [n_rows] page * page_size + offset the row's K/V goes to */
  const int32_t* seq_row0; /* [n_seqs + 1] first packed row of each sequence    */
  const int32_t* seq_ctx;  /* [n_seqs] tokens before this call                  */
  const int32_t* seq_len;  /* [n_seqs] tokens after this call                   */
  const int32_t* seq_pg0;  /* [n_seqs + 1] first page entry of each sequence    */
  const int32_t* pg_id;    /* [n_page_entries] page id                          */
  const int32_t* pg_valid; /* [n_page_entries] valid slots (1..page_size)       */
  const int32_t* pg_start; /* [n_page_entries] logical index of the first slot  */
  const int32_t* ro_row;   /* [n_readout] packed row of each readout            */
  const int32_t* ro_lane;  /* [n_readout] index in its pass's readout list      */
} pie_plan_view;

int pie_debug_plan(pie_ctx* ctx, pie_plan_view* out);

/* Word 0 of Philox4x32-10 for counters (v0 + i, lane, 0, 0), i in [0, n), key
 * (seed lo, seed hi), computed by the device code the epilogue uses.
 * out: DEVICE uint32 [n].  Runs on the context's stream and synchronises. */
int pie_debug_philox(pie_ctx* ctx, uint64_t seed, uint32_t lane, uint32_t v0, int32_t n,
                     uint32_t* out);

#ifdef __cplusplus
}
#endif
#endif /* PIE_H */
