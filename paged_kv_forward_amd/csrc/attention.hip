// Paged grouped-query attention on MFMA (see attention.h for the page layout).
//
// One wave computes 16 query rows (a query row = one new token x one query
// head of the KV head's group) against the pages of its sequence, two pages
// (32 tokens) at a time:
//   S^T[32 tok x 16 rows] = K[tok x hd] * Q^T      (A = K from the page, B = Q^T)
//   O^T[hd x 16 rows]    += V^T[hd x tok] * P^T    (A = V^T from the page, B = P^T)
// Taking S transposed leaves each lane holding the probabilities of its own
// query row for 8 tokens, exactly the B operand of the P*V MFMA, so P never
// leaves registers.  The 8 k-slots of a lane group are matched between the two
// operands of each MFMA (any fixed assignment of k values to slots gives the
// same sum): in k-step i of Q*K^T group g takes head-dim group 4i + g (8
// values), for P*V group g takes tokens 4g..4g+3 of both pages.
// Softmax is online (running max and sum per row, in log2 units), in fp32.
// In decode, P enters the P*V MFMA as two bf16 parts, hi = bf16(P) and
// lo = bf16(P - hi), so the product sees P to about 16 significant bits; the
// prefill kernels take V in fp16 instead (e4m3 codes convert to it exactly,
// bf16 values as attn_prefill_h_kernel states) and P in fp16 (11 bits), one
// product per V block.
//
// Memory: K and V are read with streaming (non-temporal) loads, each load
// instruction covering whole 128-byte lines (K's page layout makes a k-step's
// operand one contiguous run).  A wave first loads a slice of its sequence's
// page table into lane
// registers (entry base + l in lane l) and reads entries back with readlane,
// so page ids are never a dependent load in the inner loop.  K and V come
// through a wave-uniform buffer descriptor per page (a missing second page of
// a pair gets a zero-size descriptor and reads zeros), and pairs run through a
// two-slot register ring in straight-line code: the loads of the next pair are
// in flight while the current pair is computed.
#include <climits>
#include <type_traits>

#include "attention.h"
#include "common.h"

namespace pie {

constexpr int PS = 16;  // page size

constexpr float LOG2E = 1.4426950408889634f;

// 2^x for the softmax (x <= 0 or -inf): the hardware exp2.  Results below
// 2^-126 flush to zero, which no row sum (at least 1) can register.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Raw K / V fragments of one pair of entries, as loaded.
template <int HD, bool E4M3>
struct PairRaw {
  static constexpr int STEPS = HD / 32, DB = HD / 16;
  // K: per page and k-step, 8 elements (bf16: 16 B; e4m3: 8 B)
  typename std::conditional<E4M3, uint2, uint4>::type k[2][STEPS];
  // V^T: per page and 16-row block, 4 tokens (bf16: 8 B; e4m3: 4 B)
  typename std::conditional<E4M3, uint32_t, uint2>::type v[2][DB];
  int valid0, valid1, start0, start1;
};

// Page-table slice of up to 64 entries in lane registers.
struct PtSlice {
  int base, n;        // entries [base, base + n)
  int pg, valid, start;
};

__device__ __forceinline__ void load_slice(PtSlice& sl, const AttnArgs& a, int base, int end, int lane) {
  sl.base = base;
  sl.n = min(64, end - base);
  const int e = base + lane;
  const bool ok = lane < sl.n;
  sl.pg = ok ? a.pg_id[e] : 0;
  sl.valid = ok ? a.pg_valid[e] : 0;
  sl.start = ok ? a.pg_start[e] : 0;
}

// Issue the loads of entries (e, e+1); entries at or past e_end are absent.
template <int HD, bool E4M3>
__device__ __forceinline__ void load_pair(PairRaw<HD, E4M3>& f, const AttnArgs& a, const PtSlice& sl, int e,
                                          int e_end, uint32_t kofs, uint32_t vofs, int lane) {
  constexpr int STEPS = HD / 32, DB = HD / 16, EB = E4M3 ? 1 : 2;
  const int t = lane & 15, g = lane >> 4;
  const uint32_t page_bytes = (uint32_t)a.page_stride * EB;
  const uint8_t* kv = reinterpret_cast<const uint8_t*>(a.kv_layer);
  __amdgpu_buffer_rsrc_t r[2];
  int vl[2], st[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int ee = e + p;
    const bool live = ee < e_end;
    const int li = live ? ee - sl.base : 0;  // wave-uniform lane index
    const int pg = __builtin_amdgcn_readlane(sl.pg, li);
    vl[p] = live ? __builtin_amdgcn_readlane(sl.valid, li) : 0;
    st[p] = live ? __builtin_amdgcn_readlane(sl.start, li) : 0;
    r[p] = page_rsrc(kv + (size_t)pg * page_bytes, live ? page_bytes : 0u);
  }
  f.valid0 = vl[0]; f.valid1 = vl[1]; f.start0 = st[0]; f.start1 = st[1];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      // head-dim group 4i + g of token t: one contiguous run of 64 x 8 elements per step
      const uint32_t off = kofs + ((uint32_t)i * 64 + (uint32_t)lane) * 8 * EB;
      if constexpr (E4M3)
        f.k[p][i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r[p], off, 0, CPOL_NT));
      else
        f.k[p][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r[p], off, 0, CPOL_NT));
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const uint32_t off = vofs + ((uint32_t)(16 * b + t) * PS + 4 * g) * EB;
      if constexpr (E4M3)
        f.v[p][b] = __builtin_amdgcn_raw_buffer_load_b32(r[p], off, 0, CPOL_NT);
      else
        f.v[p][b] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r[p], off, 0, CPOL_NT));
    }
  }
}

// Two e4m3 codes (bytes 0, 1 of c, or 2, 3 with HI) as two bf16 in one
// gfx950 conversion instruction, unit scale.  Exact: a code has at most 4
// significant bits and its exponent range sits inside bf16's (checked on the
// GPU against the bit-level decode for every code that is not NaN; the KV
// quantiser saturates and never writes a NaN code).  The scales of K and V
// are applied to the scores and the output instead, once per value.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16(uint32_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, HI));
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16h(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// Two floats -> packed fp16 (a in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}

// Two e4m3 codes as two fp16, the same way.  Also exact: every e4m3 value,
// subnormals included, is an fp16 normal or zero.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16(uint32_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, HI));
}

__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 c) {
  return make_uint4(e4m3x2_to_bf16<false>(c.x), e4m3x2_to_bf16<true>(c.x), e4m3x2_to_bf16<false>(c.y),
                    e4m3x2_to_bf16<true>(c.y));
}

// 4 V^T tokens (4g .. 4g+3) as 2 bf16x2 words with slots >= nvalid zeroed
// (slots past a page's valid count may hold another working set's data or
// never-written memory).
template <bool E4M3, typename T>
__device__ __forceinline__ uint2 v4_bf16(T raw, int nvalid) {
  uint32_t w0, w1;
  if constexpr (E4M3) {
    uint32_t c = raw;
    const uint32_t keep = nvalid >= 4 ? 0xffffffffu : (nvalid <= 0 ? 0u : ((1u << (8 * nvalid)) - 1u));
    c &= keep;
    w0 = e4m3x2_to_bf16<false>(c);
    w1 = e4m3x2_to_bf16<true>(c);
  } else {
    w0 = raw.x;
    w1 = raw.y;
    w0 &= nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0xffffu : 0u);
    w1 &= nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0xffffu : 0u);
  }
  return make_uint2(w0, w1);
}

// 4 e4m3 V^T tokens as 2 fp16x2 words, slots >= nvalid zeroed (as v4_bf16).
__device__ __forceinline__ uint2 v4_f16(uint32_t c, int nvalid) {
  c &= nvalid >= 4 ? 0xffffffffu : (nvalid <= 0 ? 0u : ((1u << (8 * nvalid)) - 1u));
  return make_uint2(e4m3x2_to_f16<false>(c), e4m3x2_to_f16<true>(c));
}

// Online-softmax update of RB row blocks with one pair of entries.
// qidx[rb]: logical index of this lane's query row (keys with a larger logical
// index are masked), or -1 for an unused row.
template <int HD, bool E4M3, int RB>
__device__ __forceinline__ void compute_pair(const PairRaw<HD, E4M3>& f, const uint4 (&qf)[RB][HD / 32],
                                             f32x4 (&oacc)[RB][HD / 16], float (&m_run)[RB],
                                             float (&l_run)[RB], const int (&qidx)[RB], float scale_log2,
                                             int lane) {
  constexpr int STEPS = HD / 32, DB = HD / 16;
  const int g = lane >> 4;
  uint4 kf[2][STEPS];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      if constexpr (E4M3) kf[p][i] = e4m3x8_to_bf16(f.k[p][i]);
      else kf[p][i] = f.k[p][i];
    }
  uint4 vf[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    const uint2 a0 = v4_bf16<E4M3>(f.v[0][b], f.valid0 - 4 * g);
    const uint2 a1 = v4_bf16<E4M3>(f.v[1][b], f.valid1 - 4 * g);
    vf[b] = make_uint4(a0.x, a0.y, a1.x, a1.y);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      s0 = mfma16(kf[0][i], qf[rb][i], s0);
      s1 = mfma16(kf[1][i], qf[rb][i], s1);
    }
    float sc[8];
    const int qi = qidx[rb];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = 4 * g + j;
      const bool ok0 = tok < f.valid0 && f.start0 + tok <= qi;
      const bool ok1 = tok < f.valid1 && f.start1 + tok <= qi;
      sc[j] = ok0 ? s0[j] * scale_log2 : -INFINITY;
      sc[4 + j] = ok1 ? s1[j] * scale_log2 : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run[rb], mx);
    const bool any = m_new != -INFINITY;
    const float alpha = any ? exp2f(m_run[rb] - m_new) : 1.f;
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = any ? exp2f(sc[j] - m_new) : 0.f;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ps += p[j];
    l_run[rb] = l_run[rb] * alpha + ps;
    m_run[rb] = m_new;
    // P as the sum of two bf16 values (hi + lo, about 16 significant bits):
    // one bf16 rounding of P would move the 8B-shape logits by up to ~0.04.
    const uint4 ph = make_uint4(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]), pack_bf2(p[4], p[5]),
                                pack_bf2(p[6], p[7]));
    const uint32_t hw[4] = {ph.x, ph.y, ph.z, ph.w};
    float lo[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[2 * j] = p[2 * j] - bf2f(hw[j] & 0xffffu);
      lo[2 * j + 1] = p[2 * j + 1] - bf2f(hw[j] >> 16);
    }
    const uint4 pl = make_uint4(pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(lo[4], lo[5]),
                                pack_bf2(lo[6], lo[7]));
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      oacc[rb][b] *= alpha;
      oacc[rb][b] = mfma16(vf[b], ph, oacc[rb][b]);
      oacc[rb][b] = mfma16(vf[b], pl, oacc[rb][b]);
    }
  }
}

// Entries [sb, se) (at most 64, page-table slice sl loaded), two at a time
// through a two-slot ring.
template <int HD, bool E4M3, int RB>
__device__ __forceinline__ void attend_slice(const AttnArgs& a, const PtSlice& sl, int sb, int se, uint32_t kofs,
                                             uint32_t vofs, const uint4 (&qf)[RB][HD / 32],
                                             f32x4 (&oacc)[RB][HD / 16], float (&m_run)[RB],
                                             float (&l_run)[RB], const int (&qidx)[RB], float scale_log2,
                                             int lane) {
  const int n_pairs = (se - sb + 1) / 2;
  PairRaw<HD, E4M3> s0, s1;
  load_pair<HD, E4M3>(s0, a, sl, sb, se, kofs, vofs, lane);
  load_pair<HD, E4M3>(s1, a, sl, sb + 2, se, kofs, vofs, lane);
  // straight-line pairs of slots; pairs past n_pairs are absent (all masked)
  for (int pp = 0; pp < n_pairs; pp += 2) {
    compute_pair<HD, E4M3, RB>(s0, qf, oacc, m_run, l_run, qidx, scale_log2, lane);
    load_pair<HD, E4M3>(s0, a, sl, sb + 2 * (pp + 2), se, kofs, vofs, lane);
    compute_pair<HD, E4M3, RB>(s1, qf, oacc, m_run, l_run, qidx, scale_log2, lane);
    load_pair<HD, E4M3>(s1, a, sl, sb + 2 * (pp + 3), se, kofs, vofs, lane);
  }
}

// Entries [e_begin, e_end) of sequence s.  sl0 is the page-table slice of
// the first 64 entries, which the caller loads ahead of its other loads.
template <int HD, bool E4M3, int RB>
__device__ __forceinline__ void attend_range(const AttnArgs& a, const PtSlice& sl0, int e_begin, int e_end,
                                             uint32_t kofs, uint32_t vofs, const uint4 (&qf)[RB][HD / 32],
                                             f32x4 (&oacc)[RB][HD / 16], float (&m_run)[RB],
                                             float (&l_run)[RB], const int (&qidx)[RB], float scale_log2,
                                             int lane) {
  if (e_begin < e_end)
    attend_slice<HD, E4M3, RB>(a, sl0, e_begin, min(e_end, e_begin + 64), kofs, vofs, qf, oacc, m_run, l_run, qidx,
                               scale_log2, lane);
  for (int sb = e_begin + 64; sb < e_end; sb += 64) {
    PtSlice sl;
    load_slice(sl, a, sb, min(e_end, sb + 64), lane);
    attend_slice<HD, E4M3, RB>(a, sl, sb, min(e_end, sb + 64), kofs, vofs, qf, oacc, m_run, l_run, qidx, scale_log2,
                               lane);
  }
}

template <int HD>
__device__ __forceinline__ void load_q(uint4 (&qf)[HD / 32], const uint16_t* qrow, bool ok, int g) {
  constexpr int STEPS = HD / 32;
#pragma unroll
  for (int i = 0; i < STEPS; ++i)
    qf[i] = ok ? *reinterpret_cast<const uint4*>(qrow + (4 * i + g) * 8) : make_uint4(0, 0, 0, 0);
}

// The same through a buffer descriptor r over one token's q row: a lane
// whose ok is false reads zeros from an out-of-range offset.  The loads carry
// no branch, so the page loads after them need not wait for them.
template <int HD>
__device__ __forceinline__ void load_q_row(uint4 (&qf)[HD / 32], __amdgpu_buffer_rsrc_t r, uint32_t head_off,
                                           bool ok, int g) {
  constexpr int STEPS = HD / 32;
#pragma unroll
  for (int i = 0; i < STEPS; ++i)
    qf[i] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(r, ok ? head_off + (uint32_t)(4 * i + g) * 16 : 0xFFFFFFF0u, 0, 0));
}

// ---------------------------------------------------------------- decode

// One workgroup (4 waves) per (item, KV head).  The waves split the item's
// entries into 4 contiguous runs of pairs and merge their running
// (max, sum, O) through LDS.  part < 0: the item covers its sequence and the
// workgroup writes o; else it writes an unnormalised partial for the combine.
template <int HD, bool E4M3>
__global__ __launch_bounds__(256, 2) void attn_decode_kernel(AttnArgs a) {
  constexpr int DB = HD / 16, EB = E4M3 ? 1 : 2;
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ float s_o[4][16][HD + 4];
  const int lane = threadIdx.x & 63, wave = wave_id(), n = lane & 15, g = lane >> 4;
  // grid (item, KV head), items longest first.  Decode items are cut to about
  // equal lengths, so the head-major order of prefill (which dispatches all
  // heads of an item together) does not pay here: measured 1-1.5% slower on
  // equal-length batches.
  const int4 it = a.items[blockIdx.x];
  const int kvh = blockIdx.y;
  const int s = it.x, e_begin = it.y, e_end = it.z, part = it.w;
  // this wave's run of entry pairs and the page-table slice it starts with,
  // loaded before the sequence's row (which q's address needs): the two
  // lookups overlap instead of following each other
  const int n_pairs = (e_end - e_begin + 1) / 2;
  const int ppw = (n_pairs + 3) / 4;
  const int wb = e_begin + 2 * min(n_pairs, wave * ppw);
  const int we = min(e_end, e_begin + 2 * min(n_pairs, (wave + 1) * ppw));
  PtSlice sl0;
  load_slice(sl0, a, wb, min(we, wb + 64), lane);
  const int G = a.nq / a.nkv;
  const int row = a.seq_row0[s];

  uint4 qf[1][HD / 32];
  load_q_row<HD>(qf[0], page_rsrc(a.q + (size_t)row * a.nq * HD, (uint32_t)(a.nq * HD * 2)),
                 (uint32_t)((kvh * G + n) * HD * 2), n < G, g);
  const int qidx[1] = {INT_MAX};
  f32x4 oacc[1][DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[0][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[1] = {-INFINITY}, l_run[1] = {0.f};
  const float ks = E4M3 ? a.kv_scale[kvh] : 1.f;
  const float scale_log2 = a.sm_scale * ks * LOG2E;
  const uint32_t kofs = (uint32_t)(kvh * PS * HD) * EB;
  const uint32_t vofs = (uint32_t)(a.nkv * PS * HD + kvh * HD * PS) * EB;

  attend_range<HD, E4M3, 1>(a, sl0, wb, we, kofs, vofs, qf, oacc, m_run, l_run, qidx, scale_log2, lane);

  float l = l_run[0];
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (g == 0) {
    s_m[wave][n] = m_run[0];
    s_l[wave][n] = l;
  }
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][n][16 * b + 4 * g + i] = oacc[0][b][i];
  __syncthreads();

  const float vs = E4M3 ? a.kv_scale[a.nkv + kvh] : 1.f;
  for (int idx = threadIdx.x; idx < G * HD; idx += 256) {
    const int r = idx / HD, d = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][r]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = s_m[w][r] == -INFINITY ? 0.f : exp2f(s_m[w][r] - M);
      num += s_o[w][r][d] * wt;
      den += s_l[w][r] * wt;
    }
    if (part < 0) {
      a.o[((size_t)row * a.nq + kvh * G + r) * HD + d] = f2bf(num * vs / den);
    } else {
      const size_t base = ((size_t)part * a.nkv + kvh) * 16 + r;
      a.part_o[base * HD + d] = num * vs;
      if (d == 0) {
        a.part_ml[base * 2] = M;
        a.part_ml[base * 2 + 1] = den;
      }
    }
  }
}

// Merges the partials of a sequence split over several workgroups.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int MAXP = DECODE_MAX_SPLITS;  // the host never plans more
  __shared__ float s_w[MAXP][16];
  __shared__ float s_den[16];
  const int4 c = a.combine[blockIdx.x];
  const int kvh = blockIdx.y;
  const int s = c.x, p0 = c.y, np = min(c.z, MAXP);
  const int G = a.nq / a.nkv, HD = a.hd;
  const int row = a.seq_row0[s];
  if ((int)threadIdx.x < G) {
    const int n = threadIdx.x;
    float M = -INFINITY;
    for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_ml[(((size_t)(p0 + p) * a.nkv + kvh) * 16 + n) * 2]);
    float den = 0.f;
    for (int p = 0; p < np; ++p) {
      const size_t base = ((size_t)(p0 + p) * a.nkv + kvh) * 16 + n;
      const float m = a.part_ml[base * 2];
      const float w = m == -INFINITY ? 0.f : exp2f(m - M);
      s_w[p][n] = w;
      den += a.part_ml[base * 2 + 1] * w;
    }
    s_den[n] = den;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * HD; idx += 256) {
    const int n = idx / HD, d = idx % HD;
    float num = 0.f;
    for (int p = 0; p < np; ++p)
      num += a.part_o[(((size_t)(p0 + p) * a.nkv + kvh) * 16 + n) * HD + d] * s_w[p][n];
    a.o[((size_t)row * a.nq + kvh * G + n) * HD + d] = f2bf(num / s_den[n]);
  }
}

// ---------------------------------------------------------------- prefill

// Online-softmax update of RB row blocks with a pair of pages whose K and V
// sit in LDS in their memory layout.  Unlike compute_pair it finishes S and P
// for every row block before it reads V, so K and V fragments are never live
// together.
// Byte offset of a bf16 V page block in LDS: the two 16-byte halves of every
// 32-byte row (16 tokens of one head-dim index) trade places in rows whose
// bit 3 is set, so the MFMA operand reads (16 rows x 8 bytes per lane group)
// hit every bank once instead of twice.  e4m3 rows are 16 bytes and need none.
__device__ __forceinline__ int vswz(int o) { return o ^ (((o >> 8) & 1) << 4); }

template <int HD, bool E4M3, int RB, bool FULL>
__device__ __forceinline__ void prefill_pair(const uint8_t* kb0, const uint8_t* kb1, const uint8_t* vb0,
                                             const uint8_t* vb1, int valid0, int valid1, int start0,
                                             int start1, const uint4 (&qf)[RB][HD / 32],
                                             f32x4 (&oacc)[RB][HD / 16], float (&m_run)[RB], float (&l_run)[RB],
                                             const int (&qidx)[RB], float scale_log2, int lane) {
  // FULL: both pages hold 16 tokens and every one of them is visible to every
  // row of the wave, so no score or V slot needs masking.
  constexpr int STEPS = HD / 32, DB = HD / 16, EB = E4M3 ? 1 : 2;
  const int g = lane >> 4, n = lane & 15;
  uint4 ph[RB], pl[RB];
  float alpha[RB];
  bool rescale[RB];
  __builtin_amdgcn_s_setprio(1);  // scores and softmax ahead of the other wave's P*V (+0.8% at the 70B shape)
  {
    uint4 kf[2][STEPS];
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      const int off = ((i * 64 + lane) * 8) * EB;  // the page's own layout
      if constexpr (E4M3) {
        kf[0][i] = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(kb0 + off));
        kf[1][i] = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(kb1 + off));
      } else {
        kf[0][i] = *reinterpret_cast<const uint4*>(kb0 + off);
        kf[1][i] = *reinterpret_cast<const uint4*>(kb1 + off);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        s0 = mfma16(kf[0][i], qf[rb][i], s0);
        s1 = mfma16(kf[1][i], qf[rb][i], s1);
      }
      float sc[8];
      const int qi = qidx[rb];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (FULL) {
          sc[j] = s0[j] * scale_log2;
          sc[4 + j] = s1[j] * scale_log2;
        } else {
          const int tok = 4 * g + j;
          sc[j] = tok < valid0 && start0 + tok <= qi ? s0[j] * scale_log2 : -INFINITY;
          sc[4 + j] = tok < valid1 && start1 + tok <= qi ? s1[j] * scale_log2 : -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[rb], mx);
      float p[8];
      if constexpr (FULL) {
        // m_new is finite: these rows see every key of the pair
        alpha[rb] = exp2_fast(m_run[rb] - m_new);
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = exp2_fast(sc[j] - m_new);
      } else {
        const bool any = m_new != -INFINITY;
        alpha[rb] = any ? exp2_fast(m_run[rb] - m_new) : 1.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = any ? exp2_fast(sc[j] - m_new) : 0.f;
      }
      // O is rescaled only when some row's running max moved (alpha != 1);
      // multiplying by 1 changes nothing, so skipping it is exact
      rescale[rb] = __builtin_amdgcn_ballot_w64(alpha[rb] != 1.f) != 0;
      if constexpr (E4M3) {
        // e4m3 V is exact in fp16, so P enters one fp16 product; the row sum
        // adds the same rounded weights, so each row's output stays a convex
        // combination of its V rows
        ph[rb] = make_uint4(pack_h2(p[0], p[1]), pack_h2(p[2], p[3]), pack_h2(p[4], p[5]), pack_h2(p[6], p[7]));
        const f16x2_t r0 = __builtin_bit_cast(f16x2_t, ph[rb].x), r1 = __builtin_bit_cast(f16x2_t, ph[rb].y);
        const f16x2_t r2 = __builtin_bit_cast(f16x2_t, ph[rb].z), r3 = __builtin_bit_cast(f16x2_t, ph[rb].w);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          p[j] = (float)r0[j];
          p[2 + j] = (float)r1[j];
          p[4 + j] = (float)r2[j];
          p[6 + j] = (float)r3[j];
        }
      }
      const float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      l_run[rb] = l_run[rb] * alpha[rb] + ps;
      m_run[rb] = m_new;
      if constexpr (!E4M3) {
        // bf16 V: P as a bf16 pair (high part and remainder), two products
        ph[rb] = make_uint4(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]), pack_bf2(p[4], p[5]), pack_bf2(p[6], p[7]));
        const uint32_t hw[4] = {ph[rb].x, ph[rb].y, ph[rb].z, ph[rb].w};
        float lo[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo[2 * j] = p[2 * j] - bf2f(hw[j] & 0xffffu);
          lo[2 * j + 1] = p[2 * j + 1] - bf2f(hw[j] >> 16);
        }
        pl[rb] = make_uint4(pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(lo[4], lo[5]),
                            pack_bf2(lo[6], lo[7]));
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    const int off = ((16 * b + n) * PS + 4 * g) * EB;
    uint2 a0, a1;
    if constexpr (E4M3) {
      a0 = v4_f16(*reinterpret_cast<const uint32_t*>(vb0 + off), FULL ? 4 : valid0 - 4 * g);
      a1 = v4_f16(*reinterpret_cast<const uint32_t*>(vb1 + off), FULL ? 4 : valid1 - 4 * g);
    } else if constexpr (FULL) {
      a0 = *reinterpret_cast<const uint2*>(vb0 + vswz(off));
      a1 = *reinterpret_cast<const uint2*>(vb1 + vswz(off));
    } else {
      a0 = v4_bf16<false>(*reinterpret_cast<const uint2*>(vb0 + vswz(off)), valid0 - 4 * g);
      a1 = v4_bf16<false>(*reinterpret_cast<const uint2*>(vb1 + vswz(off)), valid1 - 4 * g);
    }
    const uint4 vf = make_uint4(a0.x, a0.y, a1.x, a1.y);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rescale[rb]) oacc[rb][b] *= alpha[rb];
      if constexpr (E4M3) {
        oacc[rb][b] = mfma16h(vf, ph[rb], oacc[rb][b]);
      } else {
        oacc[rb][b] = mfma16(vf, ph[rb], oacc[rb][b]);
        oacc[rb][b] = mfma16(vf, pl[rb], oacc[rb][b]);
      }
    }
  }
}

// End of a sequence's page entries once the pages that start after logical
// index qmax are dropped (no row of the workgroup sees them).  Page starts
// ascend, so 64 entries are tested per vector load, from the end: one or two
// loads where a walk back one scalar load at a time took one dependent load
// per dropped page (up to 127 for the first rows of a 2048-token prompt).
__device__ __forceinline__ int drop_pages_after(const int* pg_start, int e_begin, int e_end, int qmax, int lane) {
  for (;;) {
    const int e = e_end - 1 - lane;
    const bool past = e >= e_begin && pg_start[e] > qmax;
    const uint64_t keep = __builtin_amdgcn_ballot_w64(!past);
    if (keep) return e_end - (int)__builtin_ctzll(keep);
    e_end -= 64;
  }
}

// One workgroup (8 waves, PREFILL_ROWS query rows: PREFILL_ROWS / G tokens x
// the G query heads of one KV head) per (item, KV head).  The K and V of the
// sequence pass through LDS four pages (64 tokens) at a time, double
// buffered, so every page is read from memory once per workgroup and serves
// all its rows; each wave runs the online softmax over its 32 rows.  Rows see
// entries up to their own logical index (causal in append order); pages past
// the workgroup's last row are skipped.
constexpr int PF_WAVES = 8, PF_NT = 64 * PF_WAVES;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// 16-byte buffer load into LDS (lane l's 16 bytes at voff + soff go to LDS
// bytes [16l, 16l + 16) past `lds`, a wave-uniform address).  Inline
// assembly keeps the compiler from tracking it (it would make every LDS read
// wait for all such loads); the caller waits with s_waitcnt vmcnt.  M0 holds
// the LDS address; the nop covers the M0-write hazard of these loads.
__device__ __forceinline__ void dma16(i32x4_t r, const void* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m = (uint32_t)(size_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m), "v"(voff), "s"(r), "s"(soff) : "memory");
}

__device__ __forceinline__ i32x4_t page_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return i32x4_t{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// s_waitcnt: vector-memory counter at most n, every LDS access and scalar
// load of the wave complete.
#define PF_WAIT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x70)

template <int HD, bool E4M3>
__global__ __launch_bounds__(PF_NT, 1) void attn_prefill_kernel(AttnArgs a) {
  constexpr int RB = PREFILL_ROWS / (16 * PF_WAVES);  // row blocks of 16 per wave
  constexpr int DB = HD / 16, EB = E4M3 ? 1 : 2;
  constexpr int PAGE_B = PS * HD * EB;          // bytes of one page's K (or V) for one KV head
  constexpr int SP = 4;                         // pages per stage
  constexpr int STAGE_B = SP * 2 * PAGE_B;      // K and V of a stage
  constexpr int NS = 3;                         // stages in the LDS ring
  constexpr int PB_L = PAGE_B / 1024;           // 1 KiB loads per page block
  constexpr int LPW = STAGE_B / 1024 / PF_WAVES;  // loads per wave per stage
  static_assert(PAGE_B % 1024 == 0 && LPW >= 1 && (STAGE_B / 1024) % PF_WAVES == 0, "stage split over the waves");
  static_assert(LPW <= PB_L * 2 && (PB_L % LPW == 0 || LPW % PB_L == 0), "a wave's loads of a stage stay in one page");
  __shared__ __attribute__((aligned(1024))) uint8_t skv[NS][STAGE_B];
  const int lane = threadIdx.x & 63, wave = wave_id(), n = lane & 15, g = lane >> 4;
  // grid (KV head, item): workgroups are dispatched in flat order, so every
  // head of the longest item (items are sorted longest first) starts before
  // any shorter item, and the last round holds only the shortest
  const int4 it = a.items[blockIdx.y];
  const int kvh = blockIdx.x;
  const int s = it.x, tb = it.y, nt = it.z;
  const int G = a.nq / a.nkv;
  const int row0 = a.seq_row0[s] + tb;
  const int ctx = a.seq_ctx[s] + tb;  // logical index of the item's first token

  uint4 qf[RB][HD / 32];
  int qidx[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wave * (RB * 16) + rb * 16 + n;
    const int tq = r / G, h = r % G;
    const bool ok = tq < nt;
    qidx[rb] = ok ? ctx + tq : -1;
    load_q<HD>(qf[rb], a.q + ((size_t)(row0 + (ok ? tq : 0)) * a.nq + kvh * G + h) * HD, ok, g);
  }
  const bool wave_live = wave * (RB * 16) / G < nt;
  // logical index of the wave's first (lowest) query token: a page whose
  // last token is at or before it is visible to every row of the wave
  const int q_first = ctx + wave * (RB * 16) / G;
  const int qmax = ctx + nt - 1;

  f32x4 oacc[RB][DB];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float ks = E4M3 ? a.kv_scale[kvh] : 1.f;
  const float scale_log2 = a.sm_scale * ks * LOG2E;
  const uint32_t kofs = (uint32_t)(kvh * PS * HD) * EB;
  const uint32_t vofs = (uint32_t)(a.nkv * PS * HD + kvh * HD * PS) * EB;
  const uint32_t page_bytes = (uint32_t)a.page_stride * EB;
  const uint8_t* kv = reinterpret_cast<const uint8_t*>(a.kv_layer);
  // the page table is read with scalar loads (wave-uniform entries), which
  // the vector-memory counter the ring waits on does not count
  const_i32_t* pg_id = (const_i32_t*)a.pg_id;
  const_i32_t* pg_valid = (const_i32_t*)a.pg_valid;
  const_i32_t* pg_start = (const_i32_t*)a.pg_start;
  const int e_begin = a.seq_pg0[s];
  int e_end = a.seq_pg0[s + 1];
  e_end = drop_pages_after(a.pg_start, e_begin, e_end, qmax, lane);
  const int n_stages = (e_end - e_begin + SP - 1) / SP;
  // everything loaded above has landed before the ring's loads are counted
  __builtin_amdgcn_s_waitcnt(PF_WAIT(0));

  // This wave's loads of a stage: byte range [wave * LPW KiB, + LPW KiB) of
  // the stage, all within one page's K or V block.  Stages past the end use a
  // zero-size descriptor (zeros, no memory access), so every iteration issues
  // the same number of loads and waits on a fixed count.
  const int l0 = wave * LPW, pj = l0 / (2 * PB_L), kvsel = (l0 / PB_L) & 1, part0 = l0 % PB_L;
  auto issue = [&](int st) {
    const int e = e_begin + st * SP + pj;
    const bool live = st < n_stages && e < e_end;
    const int pg = live ? pg_id[e] : 0;
    const i32x4_t r = page_words(kv + (size_t)pg * page_bytes, live ? page_bytes : 0u);
    uint8_t* dst = &skv[st % NS][(pj * 2 + kvsel) * PAGE_B];
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int d = (part0 + k) * 1024 + lane * 16;  // destination byte in the block
      // V rows are stored with their 16-byte halves swizzled (vswz, an involution)
      const int src = kvsel && !E4M3 ? vswz(d) : d;
      dma16(r, dst + (part0 + k) * 1024, (uint32_t)src + (kvsel ? vofs : kofs), 0u);
    }
  };

  if (n_stages > 0) {
    issue(0);
    issue(1);
    for (int st = 0; st < n_stages; ++st) {
      // stage st landed here (only stage st + 1 may be in flight) and
      // everywhere after the barrier, which also frees stage st - 1's slot
      __builtin_amdgcn_s_waitcnt(PF_WAIT(LPW));
      // a plain barrier: a workgroup fence would also wait for the ring's
      // loads in flight; the memory clobber keeps LDS accesses on their side
      asm volatile("s_barrier" ::: "memory");
      issue(st + 2);
      if (wave_live) {
        const int eb = e_begin + st * SP;
        const uint8_t* sb = skv[st % NS];
#pragma unroll
        for (int j0 = 0; j0 < SP; j0 += 2) {
          const int e0 = eb + j0, e1 = eb + j0 + 1;
          const int v0 = e0 < e_end ? pg_valid[e0] : 0, v1 = e1 < e_end ? pg_valid[e1] : 0;
          const int st0 = e0 < e_end ? pg_start[e0] : 0, st1 = e1 < e_end ? pg_start[e1] : 0;
          const uint8_t *k0 = sb + (j0 * 2) * PAGE_B, *k1 = sb + (j0 * 2 + 2) * PAGE_B;
          const uint8_t *vv0 = sb + (j0 * 2 + 1) * PAGE_B, *vv1 = sb + (j0 * 2 + 3) * PAGE_B;
          if (v0 == PS && v1 == PS && max(st0, st1) + PS - 1 <= q_first)
            prefill_pair<HD, E4M3, RB, true>(k0, k1, vv0, vv1, v0, v1, st0, st1, qf, oacc, m_run, l_run, qidx,
                                             scale_log2, lane);
          else
            prefill_pair<HD, E4M3, RB, false>(k0, k1, vv0, vv1, v0, v1, st0, st1, qf, oacc, m_run, l_run, qidx,
                                              scale_log2, lane);
        }
      }
    }
    // no load into this workgroup's LDS may still be in flight when it ends
    __builtin_amdgcn_s_waitcnt(PF_WAIT(0));
  }

  const float vs = E4M3 ? a.kv_scale[a.nkv + kvh] : 1.f;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = l_run[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (qidx[rb] < 0) continue;
    const int r = wave * (RB * 16) + rb * 16 + n;
    const int tq = r / G, h = r % G;
    const float inv = vs / l;
    uint16_t* o = a.o + ((size_t)(row0 + tq) * a.nq + kvh * G + h) * HD;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      uint2 w = make_uint2(pack_bf2(oacc[rb][b][0] * inv, oacc[rb][b][1] * inv),
                           pack_bf2(oacc[rb][b][2] * inv, oacc[rb][b][3] * inv));
      *reinterpret_cast<uint2*>(o + 16 * b + 4 * g) = w;
    }
  }
}

// ---------------------------------------------------------------- prefill, bf16 KV
//
// The bf16-KV prefill kernel, built around the cost of the softmax: a wave64
// VALU instruction holds the 16-lane SIMD for 4 cycles, a quarter of a
// 16x16x32 MFMA, so at 8 waves per CU the vector instructions per score, not
// LDS or memory, set the pace.  Same work split as attn_prefill_kernel (256
// query rows of one KV head per item, 8 waves of two 16-row blocks); what
// differs:
//  - Persistent: one workgroup per compute unit takes items in rounds
//    (snake order over the longest-first list); the next item's tables and
//    q load while the current item's output is written, and the output goes
//    through LDS so that each store covers whole rows.
//  - Pages pass through a four-stage LDS ring: K loaded straight into LDS
//    three stages ahead, V into registers one stage ahead and converted to
//    fp16 into the ring (two waves per page, each with half of its K and
//    half of its V, so the conversion is evenly shared).  Slots past a
//    page's valid count become zeros there.  bf16 -> fp16 is exact for
//    magnitudes in [2^-14, 65504]; smaller ones keep an absolute error below
//    2^-25, and a V entry of 65520 or more would become infinite
//    (activations of this model family stay many orders below).
//  - Per pair of pages (32 keys): P enters P*V in fp16 (11 significant bits;
//    bf16 has 8); the running maximum is a lazy reference checked with a
//    ballot (check_pair), so the cross-lane max and the rescale of O run only
//    when it moves; the scale is folded into the exponent as one FMA per
//    score; row sums come from a ninth P*V block against an all-ones operand.
//  - Software pipeline (pipe_step): the next pair's scores are computed in
//    the same straight-line block as this pair's softmax and P*V, each score
//    MFMA followed by one probability under scheduling fences, with the
//    wave's priority raised for that phase and lowered for P*V, so that the
//    two waves of a SIMD alternate; a stage's last pair is finished after
//    the barrier that opens the next stage, hence the fourth stage.
//  - Page ids come from an LDS table filled once per workgroup, not from
//    scalar loads in the loop.
//  - One pair body serves complete and masked stages (masking behind a
//    wave-uniform flag), and no register spills: see the kernel's notes.
// Max over lanes l, l ^ 16, l ^ 32 and l ^ 48: each lane-swap instruction
// returns its two operands with half of their 16-lane rows exchanged, so the
// pair at lane l holds the values of lanes l and l ^ 32 (then l ^ 16).
// (maximum, not fmaxf: no NaN reaches it, and fmaxf would first quiet every
// operand with an extra instruction)
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// v *= a in place.  Written as assembly so that the registers of v stay the
// same on both sides of the rarely taken branch that rescales: as plain code
// the compiler copied all of O to fresh registers on every pair instead.
__device__ __forceinline__ void scale_in_place(f32x4& v, float a) {
  float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
  asm volatile("v_mul_f32 %0, %4, %0\n\tv_mul_f32 %1, %4, %1\n\tv_mul_f32 %2, %4, %2\n\tv_mul_f32 %3, %4, %3"
               : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3)
               : "v"(a));
  v = f32x4{x0, x1, x2, x3};
}

// Headroom of the lazy reference maximum, in log2 units: P = 2^(s c - m)
// may reach 2^8 (fp16 holds it exactly enough; sums stay far from fp32 range).
constexpr float LAZY_LOG2 = 8.f;

// One pair of pages (32 keys) in four pieces: scores (qk_pair), their check
// against the reference maximum (check_pair, with the rare rescale),
// probabilities (exp_pair) and P*V (pv_pair).  The reference maximum m_ref
// of a row moves only when some score of the wave exceeds it by more than
// 2^LAZY_LOG2 (a ballot, no cross-lane reduction); then it becomes the
// row's true maximum and O is rescaled.  Any reference works for the
// softmax so long as no P overflows: the sums, weighed by the same P,
// cancel it.
// Token order within a pair: the two 16x16 score MFMAs of a pair take their
// 16 rows from both pages, row r of MFMA j being token
// 8 ((r / 4) % 2) + 4 (p ^ j) + r % 4 of page p = r / 8.  Lane group g then
// holds (in MFMA 0, then 1) the scores of tokens 8 (g % 2) .. + 7 of page
// g / 2: in order for the first page, halves swapped (+4 .. +7 first) for
// the second, whose V the conversion stores with the same swap.  So each
// P*V operand is one contiguous 16-byte read (k-slots only need to match
// between operands), and the K reads of one MFMA cover all 64 LDS banks:
// with the same tokens from both pages (8 KiB apart) they hit half of the
// banks twice.
// koff0 / koff1: this lane's K row of MFMA 0 / 1, head-dim group g, from the
// pair's first K block.
__device__ __forceinline__ int pipe_koff(int lane, int page_b, int j) {
  const int t = lane & 15, g = lane >> 4, p = t >> 3;
  return 2 * p * page_b + (g * 16 + 8 * ((t >> 2) & 1) + 4 * (p ^ j) + (t & 3)) * 16;
}

// V operand of this lane, block 0: row n of page g / 2 of the pair, tokens
// 8 (g % 2) .., under the vswz swap of rows with bit 3 set.
__device__ __forceinline__ int pipe_voff(int lane, int page_b) {
  const int n = lane & 15, g = lane >> 4;
  return 2 * (g >> 1) * page_b + n * 32 + ((16 * (g & 1)) ^ (((n >> 3) & 1) << 4));
}

// (The scheduling barriers bound the LDS reads in flight: at four waves per
// SIMD a wave has 128 registers, and left alone the compiler read every
// operand of a pair ahead and spilled.)
template <int HD, int RB, bool PIN = true>
__device__ __forceinline__ void qk_pair(const uint8_t* sb, int kp0, const uint4 (&qf)[RB][HD / 32],
                                        f32x4 (&s)[RB][2], int koff0, int koff1) {
  constexpr int STEPS = HD / 32, PAGE_B = PS * HD * 2;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint4 kf[STEPS];
    const uint8_t* kb = sb + kp0 * PAGE_B + (j ? koff1 : koff0);
#pragma unroll
    for (int i = 0; i < STEPS; ++i) kf[i] = *reinterpret_cast<const uint4*>(kb + i * 1024);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < STEPS; ++i) acc = mfma16(kf[i], qf[rb][i], acc);
      s[rb][j] = acc;
    }
    if (PIN) __builtin_amdgcn_sched_barrier(0);
  }
}

// masked: scores of keys past a page's valid count or after a row's own
// position become -inf (vld, stt: valid count and first position of the
// pair's two pages; qidx: the row's position, -1 for an unused row).  Rows
// that have seen no key yet stay at -inf.  (One code path for every pair,
// the masking behind a wave-uniform branch: with a second copy of the pair
// for masked stages the compiler hoisted the two copies' common LDS reads
// above the branch and spilled.)
template <int HD, int RB>
__device__ __forceinline__ void check_pair(f32x4 (&s)[RB][2], f32x4 (&oacc)[RB][HD / 16 + 1], float (&m_ref)[RB],
                                           float (&t_raw)[RB], float c, bool masked, int vld0, int vld1, int stt0,
                                           int stt1, const int (&qidx)[RB], int lane) {
  constexpr int DB = HD / 16;
  if (masked) {
    // token 8 (g % 2) + k of the lane's page is visible iff k < lim (per-lane
    // limits, so each test is against an inline constant)
    const int g = lane >> 4;
    const int vld = (g >> 1) ? vld1 : vld0, stt = (g >> 1) ? stt1 : stt0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // MFMA j holds tokens 8 (g % 2) + 4 ((g / 2) ^ j) + i
      const int lim = min(vld, qidx[rb] - stt + 1) - 8 * (g & 1);
      const int lim0 = lim - 4 * (g >> 1), lim1 = lim - 4 * ((g >> 1) ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[rb][0][i] = i < lim0 ? s[rb][0][i] : -INFINITY;
        s[rb][1][i] = i < lim1 ? s[rb][1][i] : -INFINITY;
      }
    }
  }
  float mx[RB];
  bool up = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mx[rb] = max3f(max3f(s[rb][0][0], s[rb][0][1], s[rb][0][2]), max3f(s[rb][0][3], s[rb][1][0], s[rb][1][1]),
                   __builtin_elementwise_maximum(s[rb][1][2], s[rb][1][3]));
    // c > 0, so max(s) c = max(s c): the test is on raw scores against
    // t_raw = (m_ref + LAZY_LOG2) / c; a row still at -inf moves on any key
    up = up || mx[rb] > t_raw[rb];
  }
  if (__builtin_amdgcn_ballot_w64(up)) {  // wave-uniform, rare: every row block moves to its true maximum
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float m_new = __builtin_elementwise_maximum(m_ref[rb], max_over_groups(mx[rb]) * c);
      const bool seen = m_new != -INFINITY;
      const float alpha = seen ? exp2_fast(m_ref[rb] - m_new) : 1.f;
      m_ref[rb] = m_new;
      t_raw[rb] = seen ? (m_new + LAZY_LOG2) / c : -INFINITY;
#pragma unroll
      for (int b = 0; b <= DB; ++b) scale_in_place(oacc[rb][b], alpha);
    }
  }
}

template <int HD, int RB>
__device__ __forceinline__ void exp_pair(const f32x4 (&s)[RB][2], const float (&m_ref)[RB], float c,
                                         uint4 (&ph)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // a row that has seen no key (m_ref = -inf) weighs nothing
    const float nm = m_ref[rb] == -INFINITY ? -INFINITY : -m_ref[rb];
    float p[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[j][i] = exp2_fast(fmaf(s[rb][j][i], c, nm));
    // B operand of P*V: lane group g's 8 k-slots are tokens 8 (g % 2) .. + 7
    // of page g / 2 (first page: MFMA 0 gave the first four, MFMA 1 the next;
    // second page: the other way round, as its V is stored)
    ph[rb] = make_uint4(pack_h2(p[0][0], p[0][1]), pack_h2(p[0][2], p[0][3]), pack_h2(p[1][0], p[1][1]),
                        pack_h2(p[1][2], p[1][3]));
  }
}

template <int HD, int RB, bool PIN = true>
__device__ __forceinline__ void pv_pair(const uint8_t* sb, int vp0, const uint4 (&ph)[RB],
                                        f32x4 (&oacc)[RB][HD / 16 + 1], int voff) {
  constexpr int DB = HD / 16, PAGE_B = PS * HD * 2;
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);  // fp16 1.0
  const uint8_t* vb = sb + vp0 * PAGE_B + voff;
  uint4 vf[2];
  vf[0] = *reinterpret_cast<const uint4*>(vb);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) oacc[rb][DB] = mfma16h(ones, ph[rb], oacc[rb][DB]);
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    // operand b + 1 in flight while block b's MFMAs issue
    if (b + 1 < DB) vf[(b + 1) & 1] = *reinterpret_cast<const uint4*>(vb + (b + 1) * 16 * PS * 2);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) oacc[rb][b] = mfma16h(vf[b & 1], ph[rb], oacc[rb][b]);
    if (PIN) __builtin_amdgcn_sched_barrier(0);
  }
}

// One step of the software pipeline: probabilities and P*V of the older
// pair (scores s_old, V blocks ev0 and ev0 + 2 of se) in the same
// straight-line block as the scores and check of the newer one (K blocks
// qk0, qk0 + 2 of sq), so that the matrix core runs one pair's MFMAs while
// the vector unit works on the other's softmax.  Without it a wave's pair is
// MFMAs, then softmax, then MFMAs, and the two waves of a SIMD, in step with
// each other, leave one unit idle while the other works.
template <int HD, int RB, bool HQ>
__device__ __forceinline__ void pipe_step(const uint8_t* sq, int qk0, f32x4 (&s_new)[RB][2], bool masked,
                                          const int (&pv)[2], const int (&ps)[2], const uint8_t* se, int ev0,
                                          const f32x4 (&s_old)[RB][2], const uint4 (&qf)[RB][HD / 32],
                                          f32x4 (&oacc)[RB][HD / 16 + 1], float (&m_ref)[RB], float (&t_raw)[RB],
                                          const int (&qidx)[RB], float c, int koff0, int koff1, int voff,
                                          int lane) {
  constexpr int STEPS = HD / 32, DB = HD / 16, PAGE_B = PS * HD * 2, NE = 8 * RB;
  // Issue order, fixed with scheduling fences: the pair's K reads, then each
  // score MFMA followed by one probability (an FMA and an exponential) of
  // the older pair, so that the vector unit works while the matrix core
  // runs; then the P*V MFMAs with the V reads two blocks ahead.  Consecutive
  // score MFMAs go to different accumulators (i outer), so none waits for
  // the one before.  (Scheduling-group hints were not followed here: the
  // compiler put every exponential ahead of the MFMAs.)
  float nm[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) nm[rb] = m_ref[rb] == -INFINITY ? -INFINITY : -m_ref[rb];
  float p[NE];
  // probability e: row block e / 8, MFMA (e / 4) % 2 of the pair, value e % 4
  auto prob = [&](int e) { p[e] = exp2_fast(fmaf(s_old[e / 8][(e / 4) & 1][e & 3], c, nm[e / 8])); };
  // beside the score MFMAs, each exponential's FMA goes one MFMA earlier, so
  // that the exponential does not wait for it (+1.6%)
  float xs[NE];
  auto pre = [&](int e) { xs[e] = fmaf(s_old[e / 8][(e / 4) & 1][e & 3], c, nm[e / 8]); };
  const uint8_t* vb = se + ev0 * PAGE_B + voff;
  constexpr int VB = 16 * PS * 2;  // bytes between V blocks
  uint4 vf[3];
  if constexpr (HQ) {
    uint4 kf[2][STEPS];  // read in the order the MFMAs use them
    const uint8_t* kb0 = sq + qk0 * PAGE_B + koff0;
    const uint8_t* kb1 = sq + qk0 * PAGE_B + koff1;
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      kf[0][i] = *reinterpret_cast<const uint4*>(kb0 + i * 1024);
      kf[1][i] = *reinterpret_cast<const uint4*>(kb1 + i * 1024);
    }
    f32x4 acc[RB][2];
    __builtin_amdgcn_sched_barrier(0);
    // this wave's issue priority up while its scores and probabilities
    // interleave, down for the P*V MFMAs: the other wave of the SIMD, in
    // its own P*V phase, then fills the matrix core between them (+6%)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < 2 * RB * STEPS; ++m) {
      const int i = m / (2 * RB), j = (m / RB) & 1, rb = m % RB;
      acc[rb][j] = mfma16(kf[j][i], qf[rb][i], i == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[rb][j]);
      if (m == 0) pre(0);
      if (m + 1 < NE) pre(m + 1);
      if (m < NE) p[m] = exp2_fast(xs[m]);
      if (m == 2 * RB * STEPS - 6) vf[0] = *reinterpret_cast<const uint4*>(vb);
      if (m == 2 * RB * STEPS - 3) vf[1] = *reinterpret_cast<const uint4*>(vb + VB);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 2 * RB * STEPS; e < NE; ++e) prob(e);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 2; ++j) s_new[rb][j] = acc[rb][j];
  } else {
#pragma unroll
    for (int e = 0; e < NE; ++e) prob(e);
    vf[0] = *reinterpret_cast<const uint4*>(vb);
    vf[1] = *reinterpret_cast<const uint4*>(vb + VB);
  }
  // B operand of P*V: lane group g's 8 k-slots are tokens 8 (g % 2) .. + 7
  // of page g / 2 (first page: MFMA 0 gave the first four, MFMA 1 the next;
  // second page: the other way round, as its V is stored)
  uint4 ph[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    ph[rb] = make_uint4(pack_h2(p[8 * rb], p[8 * rb + 1]), pack_h2(p[8 * rb + 2], p[8 * rb + 3]),
                        pack_h2(p[8 * rb + 4], p[8 * rb + 5]), pack_h2(p[8 * rb + 6], p[8 * rb + 7]));
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);  // fp16 1.0
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) oacc[rb][DB] = mfma16h(ones, ph[rb], oacc[rb][DB]);
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    // operands b + 1 and b + 2 in flight while block b's MFMAs issue
    if (b + 2 < DB) vf[(b + 2) % 3] = *reinterpret_cast<const uint4*>(vb + (b + 2) * VB);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) oacc[rb][b] = mfma16h(vf[b % 3], ph[rb], oacc[rb][b]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // after P*V of the older pair: a rescale covers it too
  if constexpr (HQ) check_pair<HD, RB>(s_new, oacc, m_ref, t_raw, c, masked, pv[0], pv[1], ps[0], ps[1], qidx, lane);
}

// 8 waves of two 16-row blocks each (at most 256 registers: two waves per
// SIMD; the kernel uses about 240).
// Sixteen waves of one block each measured 8% slower: every wave reads all of
// a stage's K and V from LDS, so that doubles the operand reads.  No
// register may spill here: a reload is a vector memory load, and since the
// compiler does not see the ring's LDS-bound loads it waits for all of them
// before it.
constexpr int PH_WAVES = 8, PH_NT = 64 * PH_WAVES;
// Page ids a prefill workgroup keeps in LDS (8 KiB: sequences of up to
// 32768 tokens at 16 per page; longer ones read their page ids with scalar
// loads).
constexpr int PF_PT_MAX = 2048;

template <int HD>
__global__ __launch_bounds__(PH_NT, 1) void attn_prefill_h_kernel(AttnArgs a) {
  constexpr int RB = PREFILL_ROWS / (16 * PH_WAVES);
  constexpr int DB = HD / 16;
  constexpr int PAGE_B = PS * HD * 2;            // bytes of one page's K (or V) for one KV head
  // pages per stage, stages in the ring: four, since a stage's last pair is
  // finished after the barrier that lets stage + 3 load
  constexpr int SP = 4, NS = 4;
  constexpr int STAGE_B = SP * 2 * PAGE_B;
  constexpr int PB_L = PAGE_B / 1024;            // 1 KiB loads per K (or V) block of a page
  constexpr int HL = PB_L / 2;                   // K loads and V loads per wave per stage
  static_assert(PH_WAVES == 2 * SP && HL >= 1, "two waves per page: half of its K and half of its V each");
  __shared__ __attribute__((aligned(1024))) uint8_t skv[NS][STAGE_B];
  // The sequence's page ids, so that the ring reads them from LDS: a scalar
  // load in the loop makes the next LDS wait wait for it too (scalar loads
  // complete out of order, so such a wait is for everything), and a miss
  // cost about 1600 cycles per stage.  Longer page tables use scalar loads.
  __shared__ int s_pid[PF_PT_MAX];
  const int lane = threadIdx.x & 63, wave = wave_id(), n = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.x;
  const int G = a.nq / a.nkv;
  const int P = gridDim.y;
  auto item_at = [&](int r) { return r * P + ((r & 1) ? P - 1 - (int)blockIdx.y : (int)blockIdx.y); };
  // The first 128 page entries (start, valid count, page id; entry
  // e_begin + 64 k + lane in slot k) and q, loaded in one round trip (loading
  // each table after the previous one was needed took four, about 5 us per
  // item).  For every item after the first they are loaded while the
  // previous item's output is written.  Indexes are clamped into the
  // sequence's entries (an item has at least one page) and the values
  // outside it ignored.
  int t_start[2], t_valid[2], t_id[2];
  uint4 qf[RB][HD / 32];
  auto fetch = [&](int4 itv, int r0, int eb, int ea) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = max(min(eb + 64 * k + lane, ea - 1), 0);
      t_start[k] = a.pg_start[e];
      t_valid[k] = a.pg_valid[e];
      t_id[k] = a.pg_id[e];
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = wave * (RB * 16) + rb * 16 + n;
      const int tq = r / G, h = r % G;
      const bool ok = tq < itv.z;
      load_q<HD>(qf[rb], a.q + ((size_t)(r0 + itv.y + (ok ? tq : 0)) * a.nq + kvh * G + h) * HD, ok, g);
    }
  };
  int4 it = a.items[item_at(0)];  // grid.y <= the item count: round 0 always has an item
  int seq_row0 = a.seq_row0[it.x], seq_ctx = a.seq_ctx[it.x];
  int pg0 = a.seq_pg0[it.x], pg1 = a.seq_pg0[it.x + 1];
  fetch(it, seq_row0, pg0, pg1);
  // Persistent over items: round r takes item r P + y, or r P + P - 1 - y in
  // odd rounds (P = gridDim.y workgroups per KV head, y = blockIdx.y), so
  // that with items sorted longest first every workgroup gets a similar
  // total; no workgroup is launched per item, so none waits for one to be
  // dispatched.  Every wave runs the same rounds (the barriers match).
  for (int round = 0;; ++round) {
    // lane-derived offsets are recomputed each round rather than held in
    // registers across rounds (that spilled)
    int lane_r = lane;
    asm volatile("" : "+v"(lane_r));
    const int lane = lane_r, n = lane & 15, g = lane >> 4;
    const int tb = it.y, nt = it.z;
    const int row0 = seq_row0 + tb;
    const int ctx = seq_ctx + tb;  // logical index of the item's first token
    const int qmax = ctx + nt - 1;
    const int e_begin = pg0, e_all = pg1;
    // the next round's item and sequence (scalars, in registers long before
    // this round's output)
    const int yn = item_at(round + 1);
    const bool more = yn < a.n_items;
    int4 it_n = it;
    int seq_row0_n = 0, seq_ctx_n = 0, pg0_n = 0, pg1_n = 0;
    if (more) {
      it_n = a.items[yn];
      seq_row0_n = a.seq_row0[it_n.x];
      seq_ctx_n = a.seq_ctx[it_n.x];
      pg0_n = a.seq_pg0[it_n.x];
      pg1_n = a.seq_pg0[it_n.x + 1];
    }

    int qidx[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = wave * (RB * 16) + rb * 16 + n;
      qidx[rb] = r / G < nt ? ctx + r / G : -1;
    }
    const bool wave_live = wave * (RB * 16) / G < nt;

    f32x4 oacc[RB][DB + 1];
    float m_ref[RB], t_raw[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m_ref[rb] = t_raw[rb] = -INFINITY;
#pragma unroll
      for (int b = 0; b <= DB; ++b) oacc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float c = a.sm_scale * LOG2E;
    const int koff0 = pipe_koff(lane, PAGE_B, 0), koff1 = pipe_koff(lane, PAGE_B, 1), voff = pipe_voff(lane, PAGE_B);
    const uint32_t kofs = (uint32_t)(kvh * PS * HD) * 2;
    const uint32_t vofs = (uint32_t)(a.nkv * PS * HD + kvh * HD * PS) * 2;
    const uint32_t page_bytes = (uint32_t)a.page_stride * 2;
    const uint8_t* kv = reinterpret_cast<const uint8_t*>(a.kv_layer);
    const_i32_t* pg_id = (const_i32_t*)a.pg_id;
    const_i32_t* pg_valid = (const_i32_t*)a.pg_valid;
    const_i32_t* pg_start = (const_i32_t*)a.pg_start;
    __builtin_amdgcn_s_waitcnt(PF_WAIT(0));  // tables and q
    // Pages that start after qmax serve no row of the workgroup.  Page starts
    // ascend, so the entries kept are a prefix: counted from the tables when
    // it ends inside them, else scanned from the sequence's end.
    int e_end;
    {
      const uint64_t in0 = __builtin_amdgcn_ballot_w64(e_begin + lane < e_all && t_start[0] <= qmax);
      const uint64_t in1 = __builtin_amdgcn_ballot_w64(e_begin + 64 + lane < e_all && t_start[1] <= qmax);
      if (~in0) e_end = e_begin + __builtin_popcountll(in0);
      else if (~in1) e_end = e_begin + 64 + __builtin_popcountll(in1);
      else e_end = drop_pages_after(a.pg_start, e_begin, e_all, qmax, lane);
    }
    const int n_stages = (e_end - e_begin + SP - 1) / SP;
    const bool pt_lds = e_end - e_begin <= PF_PT_MAX;
    if (pt_lds) {
      if (wave == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
          if (64 * k + lane < e_end - e_begin) s_pid[64 * k + lane] = t_id[k];
      }
      for (int i = 128 + threadIdx.x; i < e_end - e_begin; i += PH_NT) s_pid[i] = a.pg_id[e_begin + i];
    }

    // Leading stages whose four pages are complete and precede the item's
    // first token need no masking for any row.  (Pages are checked 64 at a
    // time, one per lane, the first 128 from the tables; the first page that
    // fails ends the run.)
    int n_full = -1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = e_begin + 64 * k + lane;
      const bool ok = e < e_end && t_valid[k] == PS && t_start[k] + PS - 1 <= ctx;
      const uint64_t bad = __builtin_amdgcn_ballot_w64(!ok);
      if (n_full < 0 && bad) n_full = (64 * k + (int)__builtin_ctzll(bad)) / SP;
    }
    for (int e0 = e_begin + 128; n_full < 0; e0 += 64) {
      const int e = e0 + lane;
      const bool ok = e < e_end && a.pg_valid[e] == PS && a.pg_start[e] + PS - 1 <= ctx;
      const uint64_t bad = __builtin_amdgcn_ballot_w64(!ok);
      if (bad) n_full = (e0 - e_begin + (int)__builtin_ctzll(bad)) / SP;
    }
    __builtin_amdgcn_s_waitcnt(PF_WAIT(0));

    // This wave's share of a stage: page wave / 2 of it, 1 KiB blocks
    // part0 .. part0 + HL - 1 of both its K and its V, so that every wave
    // converts the same share of V (with whole blocks per wave, half of the
    // waves converted and the others waited at the barrier).  Stages past the
    // end use a zero-size descriptor (zeros, no memory access).  Page ids and
    // valid counts come in as arguments, read a stage ahead.
    const int pj = wave >> 1, part0 = (wave & 1) * HL;
    auto live_entry = [&](int st) { return st < n_stages && e_begin + st * SP + pj < e_end; };
    auto entry = [&](int st) { return min(e_begin + st * SP + pj, e_end - 1); };  // clamped: always readable
    auto page_id = [&](int st) {
      return pt_lds ? __builtin_amdgcn_readfirstlane(s_pid[entry(st) - e_begin]) : pg_id[entry(st)];
    };
    auto issue = [&](int st, int pg_raw) {
      const bool live = live_entry(st);
      const int pg = live ? pg_raw : 0;
      const i32x4_t r = page_words(kv + (size_t)pg * page_bytes, live ? page_bytes : 0u);
      uint8_t* kd = &skv[st % NS][(2 * pj) * PAGE_B];
#pragma unroll
      for (int k = 0; k < HL; ++k) {
        const int d = (part0 + k) * 1024 + lane * 16;
        dma16(r, kd + (part0 + k) * 1024, kofs + (uint32_t)d, 0u);
      }
    };
    // V comes through registers, one stage ahead: this lane's chunks of its
    // page's V block (the chunk for LDS bytes d is source bytes vswz(d): V
    // rows are stored with their 16-byte halves swizzled, an involution), so
    // that the conversion need not read them back from LDS.
    uint4 vreg[HL];
    auto load_v = [&](int st, int pg_raw) {
      const bool live = live_entry(st);
      const int pg = live ? pg_raw : 0;
      const __amdgpu_buffer_rsrc_t r = page_rsrc(kv + (size_t)pg * page_bytes, live ? page_bytes : 0u);
#pragma unroll
      for (int k = 0; k < HL; ++k) {
        const int d = (part0 + k) * 1024 + lane * 16;
        vreg[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, vofs + (uint32_t)vswz(d), 0, 0));
      }
    };
    // The loaded V chunks from bf16 to fp16 into the stage's LDS V block;
    // token slots at or past the page's valid count become zeros.
    auto convert_v = [&](int st, int nv_raw) {
      const int nv = live_entry(st) ? nv_raw : 0;
      uint8_t* vd = &skv[st % NS][(2 * pj + 1) * PAGE_B];
#pragma unroll
      for (int k = 0; k < HL; ++k) {
        const int d = (part0 + k) * 1024 + lane * 16;
        const int t0 = ((vswz(d) % 32) / 16) * 8;  // first token of the chunk (a V row is 16 tokens)
        const uint4 raw = vreg[k];
        uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        if (nv < PS) {  // wave-uniform: slots past the valid count may hold anything
          // bf16 word q holds tokens t0 + 2q, t0 + 2q + 1: keep the first
          // clamp(nv - t0 - 2q, 0, 2) halves (bf16 zero converts to fp16 zero)
          asm volatile("" ::: "memory");  // a real branch: complete pages skip this
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int keep = min(max(nv - t0 - 2 * q, 0), 2);
            w[q] &= (uint32_t)(0xffffffffull >> (16 * (2 - keep)));
          }
        }
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = pack_h2(__uint_as_float(w[q] << 16), __uint_as_float(w[q] & 0xffff0000u));
        // the second page of a pair holds its 8-token groups halves swapped
        // (see the token order above): two 8-byte stores, their places chosen
        // by the wave's page parity
        const int sw = (pj & 1) * 8;
        *reinterpret_cast<uint2*>(vd + d + sw) = make_uint2(o[0], o[1]);
        *reinterpret_cast<uint2*>(vd + d + (8 - sw)) = make_uint2(o[2], o[3]);
      }
    };

    // valid counts and first positions of a stage's pair q, read only for
    // stages after the run of complete ones
    auto pair_meta = [&](int st, int q, int (&pv)[2], int (&ps)[2]) {
      pv[0] = pv[1] = PS;
      ps[0] = ps[1] = 0;
      if (st >= n_full) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int e = e_begin + st * SP + 2 * q + j;
          pv[j] = e < e_end ? pg_valid[e] : 0;
          ps[j] = e < e_end ? pg_start[e] : 0;
        }
      }
    };

    if (n_stages > 0) {
      // Ring: right after the barrier that opens stage st the wave issues
      // stage st + 2; in the middle of stage st it waits for all but its LPW
      // loads of stage st + 2, so stage st + 1 has landed, and converts its V
      // share; a barrier then opens stage st + 1.
      __syncthreads();  // the page-id table is written (no ring load in flight yet)
      const int pid0 = page_id(0), pid1 = page_id(1);
      issue(0, pid0);
      issue(1, pid1);
      load_v(0, pid0);
      int pid = page_id(2), pidv = pid1;  // next K stage's page, next V stage's page
      const int nv0 = pg_valid[entry(0)];
      int nvn = pg_valid[entry(1)];
      __builtin_amdgcn_s_waitcnt(PF_WAIT(0));
      convert_v(0, nv0);
      __builtin_amdgcn_s_waitcnt(PF_WAIT(63));
      asm volatile("s_barrier" ::: "memory");
      issue(2, pid);
      load_v(1, pidv);
      pidv = pid;
      pid = page_id(3);
      // Pair 2st + 1's scores go with pair 2st's softmax and P*V, pair
      // 2st + 2's (next stage) with pair 2st + 1's, which is why a stage's
      // last pair is finished after the next stage's barrier.  The last stage
      // is peeled so that no branch holds two copies of a step.
      f32x4 sa[RB][2], sb2[RB][2];
      int pv[2], ps[2];
      if (wave_live) {
        pair_meta(0, 0, pv, ps);
        qk_pair<HD, RB>(skv[0], 0, qf, sa, koff0, koff1);
        check_pair<HD, RB>(sa, oacc, m_ref, t_raw, c, n_full == 0, pv[0], pv[1], ps[0], ps[1], qidx, lane);
      }
      for (int st = 0; st < n_stages; ++st) {
        const uint8_t* sb = skv[st % NS];
        const bool last = st + 1 == n_stages;
        if (wave_live) {
          pair_meta(st, 1, pv, ps);
          pipe_step<HD, RB, true>(sb, 4, sb2, st >= n_full, pv, ps, sb, 1, sa, qf, oacc, m_ref, t_raw, qidx, c, koff0,
                                  koff1, voff, lane);
        }
        // V of stage st + 1 (in registers) and K up to stage st + 2 have landed
        __builtin_amdgcn_s_waitcnt(PF_WAIT(0));
        convert_v(st + 1, nvn);  // slot (st + 1) % NS: no wave reads it before the next barrier
        // stages before n_full hold complete pages; later ones need their count
        nvn = st + 2 < n_full ? PS : pg_valid[entry(st + 2)];
        __builtin_amdgcn_s_waitcnt(PF_WAIT(63));
        asm volatile("s_barrier" ::: "memory");
        issue(st + 3, pid);
        load_v(st + 2, pidv);
        pidv = pid;
        pid = page_id(st + 4);
        if (last) break;
        if (wave_live) {
          pair_meta(st + 1, 0, pv, ps);
          pipe_step<HD, RB, true>(skv[(st + 1) % NS], 0, sa, st + 1 >= n_full, pv, ps, sb, 5, sb2, qf, oacc, m_ref,
                                  t_raw, qidx, c, koff0, koff1, voff, lane);
        }
      }
      if (wave_live)  // the last pair: no next one to start
        pipe_step<HD, RB, false>(skv[0], 0, sa, false, pv, ps, skv[(n_stages - 1) % NS], 5, sb2, qf, oacc, m_ref,
                                 t_raw, qidx, c, koff0, koff1, voff, lane);
      // no load into this workgroup's LDS may still be in flight when it ends
      __builtin_amdgcn_s_waitcnt(PF_WAIT(0));
    }

    // Output through LDS: each wave writes its rows (normalised, bf16) to a
    // region of the ring, then stores them as whole 16-byte pieces, lanes in
    // row order.  The rows of one token are the G query heads of this KV head,
    // adjacent in the output, so one store instruction covers whole runs of
    // G x HD x 2 bytes; straight from the MFMA layout each lane held 8 bytes
    // of 16 different rows per store (about 2.4 us per workgroup).
    constexpr int RS = HD * 2 + 16;        // LDS row stride (padded: the 16 rows of a write hit distinct banks)
    constexpr int CH = HD * 2 / 16;        // 16-byte pieces per row
    constexpr int WR = RB * 16;            // rows per wave
    static_assert(PH_WAVES * WR * RS <= NS * STAGE_B, "the output staging fits in the ring");
    if (more) fetch(it_n, seq_row0_n, pg0_n, pg1_n);  // q is no longer needed: the next item's goes in its place
    __syncthreads();  // every wave is done with the ring
    uint8_t* so = &skv[0][0] + wave * WR * RS;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float inv = 1.f / oacc[rb][DB][0];  // unused rows (inf, nan) are never stored
#pragma unroll
      for (int b = 0; b < DB; ++b)
        *reinterpret_cast<uint2*>(so + (rb * 16 + n) * RS + (16 * b + 4 * g) * 2) =
            make_uint2(pack_bf2(oacc[rb][b][0] * inv, oacc[rb][b][1] * inv),
                       pack_bf2(oacc[rb][b][2] * inv, oacc[rb][b][3] * inv));
    }
#pragma unroll
    for (int k = 0; k < WR * CH / 64; ++k) {
      const int rr = k * (64 / CH) + lane / CH, col = lane % CH;
      const uint4 v = *reinterpret_cast<const uint4*>(so + rr * RS + col * 16);
      const int r = wave * WR + rr;
      const int tq = r / G, h = r % G;
      if (tq < nt) *reinterpret_cast<uint4*>(a.o + ((size_t)(row0 + tq) * a.nq + kvh * G + h) * HD + col * 8) = v;
    }
    __syncthreads();  // the staging reads are done before the next round writes LDS
    if (!more) break;
    it = it_n;
    seq_row0 = seq_row0_n;
    seq_ctx = seq_ctx_n;
    pg0 = pg0_n;
    pg1 = pg1_n;
  }
}

void launch_attn_decode(const AttnArgs& a, hipStream_t st) {
  if (a.n_items == 0) return;
  dim3 grid(a.n_items, a.nkv);
  if (a.hd == 128) {
    if (a.kv_e4m3) hipLaunchKernelGGL((attn_decode_kernel<128, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((attn_decode_kernel<128, false>), grid, dim3(256), 0, st, a);
  } else {
    if (a.kv_e4m3) hipLaunchKernelGGL((attn_decode_kernel<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((attn_decode_kernel<64, false>), grid, dim3(256), 0, st, a);
  }
}

void launch_attn_combine(const AttnArgs& a, hipStream_t st) {
  if (a.n_combine == 0) return;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.n_combine, a.nkv), dim3(256), 0, st, a);
}

// Prefill work items sit on grid dimension y (at most 65535 per launch):
// longer lists go out as several launches over consecutive slices.
constexpr int MAX_GRID_Y = 65535;

// Compute units of the current device (cached per device).
static int n_compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

void launch_attn_prefill(const AttnArgs& a0, hipStream_t st) {
  for (int i0 = 0; i0 < a0.n_items; i0 += MAX_GRID_Y) {
    AttnArgs a = a0;
    a.items = a0.items + i0;
    a.n_items = min(MAX_GRID_Y, a0.n_items - i0);
    dim3 grid(a.nkv, a.n_items);
    // the bf16 kernel is persistent: one workgroup per compute unit at most
    // (one fits per unit), each taking several items in turn
    dim3 grid_p(a.nkv, std::max(1, std::min(a.n_items, (n_compute_units() + a.nkv - 1) / a.nkv)));
    if (a.hd == 128) {
      if (a.kv_e4m3) hipLaunchKernelGGL((attn_prefill_kernel<128, true>), grid, dim3(PF_NT), 0, st, a);
      else hipLaunchKernelGGL(attn_prefill_h_kernel<128>, grid_p, dim3(PH_NT), 0, st, a);
    } else {
      if (a.kv_e4m3) hipLaunchKernelGGL((attn_prefill_kernel<64, true>), grid, dim3(PF_NT), 0, st, a);
      else hipLaunchKernelGGL(attn_prefill_h_kernel<64>, grid_p, dim3(PH_NT), 0, st, a);
    }
  }
}

}  // namespace pie
