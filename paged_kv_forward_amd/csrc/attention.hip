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
// same sum): for Q*K^T group g takes head-dim chunks g*STEPS .. g*STEPS+STEPS-1,
// for P*V group g takes tokens 4g..4g+3 of both pages.
// Softmax is online (running max and sum per row, in log2 units), in fp32;
// P enters the MFMA rounded to bf16.
#include <climits>

#include "attention.h"
#include "common.h"

namespace pie {

constexpr int PS = 16;  // page size
constexpr float LOG2E = 1.4426950408889634f;

template <int HD, bool E4M3>
__device__ __forceinline__ uint4 load_k_frag(const void* kv, size_t elem) {
  if constexpr (E4M3) {
    uint2 c = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(kv) + elem);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t src = j < 2 ? c.x : c.y;
      uint32_t b0 = (src >> (16 * (j & 1))) & 0xffu, b1 = (src >> (16 * (j & 1) + 8)) & 0xffu;
      w[j] = e4m3_to_bf16(b0) | (e4m3_to_bf16(b1) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(kv) + elem);
  }
}

// 4 consecutive V^T elements (tokens 4g..4g+3 of one page), slots >= nvalid zeroed; as 2 bf16x2 words.
template <bool E4M3>
__device__ __forceinline__ uint2 load_v4(const void* kv, size_t elem, int nvalid) {
  uint32_t w0, w1;
  if constexpr (E4M3) {
    uint32_t c = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(kv) + elem);
    uint32_t keep = nvalid >= 4 ? 0xffffffffu : (nvalid <= 0 ? 0u : ((1u << (8 * nvalid)) - 1u));
    c &= keep;
    w0 = e4m3_to_bf16(c & 0xffu) | (e4m3_to_bf16((c >> 8) & 0xffu) << 16);
    w1 = e4m3_to_bf16((c >> 16) & 0xffu) | (e4m3_to_bf16(c >> 24) << 16);
  } else {
    uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(kv) + elem);
    w0 = v.x;
    w1 = v.y;
    if (nvalid < 4) {
      w0 &= nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0xffffu : 0u);
      w1 &= nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0xffffu : 0u);
    }
  }
  return make_uint2(w0, w1);
}

// Process entries (p0, p1) of a page table for RB row blocks of 16 query rows.
// qidx[rb]: logical index of this lane's query row (keys with a larger logical
// index are masked), or -1 for an unused row.
template <int HD, bool E4M3, int RB>
__device__ __forceinline__ void attend_pair(const uint4 (&qf)[RB][HD / 32], f32x4 (&oacc)[RB][HD / 16],
                                            float (&m_run)[RB], float (&l_run)[RB],
                                            const void* kv, size_t kbase0, size_t kbase1,
                                            size_t vbase0, size_t vbase1, int valid0, int valid1,
                                            int start0, int start1, const int (&qidx)[RB],
                                            float scale_log2, int lane) {
  constexpr int STEPS = HD / 32, DB = HD / 16;
  const int t = lane & 15, g = lane >> 4;
  const bool has1 = valid1 > 0;
  // K fragments of both pages
  uint4 kf[2][STEPS];
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    size_t off = (size_t)t * HD + (size_t)(g * STEPS + i) * 8;
    kf[0][i] = load_k_frag<HD, E4M3>(kv, kbase0 + off);
    kf[1][i] = has1 ? load_k_frag<HD, E4M3>(kv, kbase1 + off) : make_uint4(0, 0, 0, 0);
  }
  // V^T fragments of both pages
  uint4 vf[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    size_t off = (size_t)(16 * b + t) * PS + 4 * g;
    uint2 a0 = load_v4<E4M3>(kv, vbase0 + off, valid0 - 4 * g);
    uint2 a1 = has1 ? load_v4<E4M3>(kv, vbase1 + off, valid1 - 4 * g) : make_uint2(0, 0);
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
      int tok = 4 * g + j;
      bool ok0 = tok < valid0 && start0 + tok <= qi;
      bool ok1 = tok < valid1 && start1 + tok <= qi;
      sc[j] = ok0 ? s0[j] * scale_log2 : -INFINITY;
      sc[4 + j] = ok1 ? s1[j] * scale_log2 : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run[rb], mx);
    float p[8];
    float alpha = 1.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = 0.f;
    } else {
      alpha = exp2f(m_run[rb] - m_new);
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = exp2f(sc[j] - m_new);
    }
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ps += p[j];
    l_run[rb] = l_run[rb] * alpha + ps;
    m_run[rb] = m_new;
    uint4 pb = make_uint4(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]), pack_bf2(p[4], p[5]),
                          pack_bf2(p[6], p[7]));
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      oacc[rb][b] *= alpha;
      oacc[rb][b] = mfma16(vf[b], pb, oacc[rb][b]);
    }
  }
}

template <int HD>
__device__ __forceinline__ void load_q(uint4 (&qf)[HD / 32], const uint16_t* qrow, bool ok, int g) {
  constexpr int STEPS = HD / 32;
#pragma unroll
  for (int i = 0; i < STEPS; ++i)
    qf[i] = ok ? *reinterpret_cast<const uint4*>(qrow + (g * STEPS + i) * 8) : make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------- decode

template <int HD, bool E4M3>
__global__ __launch_bounds__(64) void attn_decode_kernel(AttnArgs a) {
  constexpr int DB = HD / 16;
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  const int4 it = a.items[blockIdx.x];
  const int kvh = blockIdx.y;
  const int s = it.x, e_begin = it.y, e_end = it.z, part = it.w;
  const int G = a.nq / a.nkv;
  const int row = a.seq_row0[s];

  uint4 qf[1][HD / 32];
  load_q<HD>(qf[0], a.q + ((size_t)row * a.nq + kvh * G + n) * HD, n < G, g);
  const int qidx[1] = {INT_MAX};
  f32x4 oacc[1][DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[0][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[1] = {-INFINITY}, l_run[1] = {0.f};
  const float ks = E4M3 ? a.kv_scale[kvh] : 1.f;
  const float scale_log2 = a.sm_scale * ks * LOG2E;
  const size_t kofs = (size_t)kvh * PS * HD, vofs = (size_t)a.nkv * PS * HD + (size_t)kvh * HD * PS;

  for (int e = e_begin; e < e_end; e += 2) {
    const int pg0 = a.pg_id[e], v0 = a.pg_valid[e];
    const bool two = e + 1 < e_end;
    const int pg1 = two ? a.pg_id[e + 1] : pg0, v1 = two ? a.pg_valid[e + 1] : 0;
    const size_t b0 = (size_t)pg0 * a.page_stride, b1 = (size_t)pg1 * a.page_stride;
    attend_pair<HD, E4M3, 1>(qf, oacc, m_run, l_run, a.kv_layer, b0 + kofs, b1 + kofs, b0 + vofs,
                             b1 + vofs, v0, v1, 0, 0, qidx, scale_log2, lane);
  }
  float l = l_run[0];
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (n >= G) return;
  const float vs = E4M3 ? a.kv_scale[a.nkv + kvh] : 1.f;
  if (part < 0) {
    const float inv = vs / l;
    uint16_t* o = a.o + ((size_t)row * a.nq + kvh * G + n) * HD;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      uint2 w = make_uint2(pack_bf2(oacc[0][b][0] * inv, oacc[0][b][1] * inv),
                           pack_bf2(oacc[0][b][2] * inv, oacc[0][b][3] * inv));
      *reinterpret_cast<uint2*>(o + 16 * b + 4 * g) = w;
    }
  } else {
    float* po = a.part_o + (((size_t)part * a.nkv + kvh) * 16 + n) * HD;
#pragma unroll
    for (int b = 0; b < DB; ++b)
      *reinterpret_cast<float4*>(po + 16 * b + 4 * g) =
          make_float4(oacc[0][b][0] * vs, oacc[0][b][1] * vs, oacc[0][b][2] * vs, oacc[0][b][3] * vs);
    if (g == 0) {
      float* pm = a.part_ml + (((size_t)part * a.nkv + kvh) * 16 + n) * 2;
      pm[0] = m_run[0];
      pm[1] = l;
    }
  }
}

__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  const int4 c = a.combine[blockIdx.x];
  const int kvh = blockIdx.y;
  const int s = c.x, p0 = c.y, np = c.z;
  const int G = a.nq / a.nkv, HD = a.hd;
  const int row = a.seq_row0[s];
  for (int idx = threadIdx.x; idx < G * HD; idx += 64) {
    const int n = idx / HD, d = idx % HD;
    float M = -INFINITY;
    for (int p = 0; p < np; ++p)
      M = fmaxf(M, a.part_ml[(((size_t)(p0 + p) * a.nkv + kvh) * 16 + n) * 2]);
    float num = 0.f, den = 0.f;
    for (int p = 0; p < np; ++p) {
      const size_t base = ((size_t)(p0 + p) * a.nkv + kvh) * 16 + n;
      const float m = a.part_ml[base * 2], l = a.part_ml[base * 2 + 1];
      const float w = m == -INFINITY ? 0.f : exp2f(m - M);
      num += a.part_o[base * HD + d] * w;
      den += l * w;
    }
    a.o[((size_t)row * a.nq + kvh * G + n) * HD + d] = f2bf(num / den);
  }
}

// ---------------------------------------------------------------- prefill

template <int HD, bool E4M3>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnArgs a) {
  constexpr int RB = PREFILL_ROWS / 64;  // row blocks per wave (4 waves)
  constexpr int DB = HD / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
  const int4 it = a.items[blockIdx.x];
  const int kvh = blockIdx.y;
  const int s = it.x, tb = it.y, nt = it.z;
  const int G = a.nq / a.nkv;
  const int row0 = a.seq_row0[s] + tb;
  const int ctx = a.seq_ctx[s] + tb;  // logical index of the item's first token

  uint4 qf[RB][HD / 32];
  int qidx[RB];
  int last_tok = -1;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wave * (RB * 16) + rb * 16 + n;
    const int tq = r / G, h = r % G;
    const bool ok = tq < nt;
    qidx[rb] = ok ? ctx + tq : -1;
    load_q<HD>(qf[rb], a.q + ((size_t)(row0 + (ok ? tq : 0)) * a.nq + kvh * G + h) * HD, ok, g);
    const int wave_last = (wave * (RB * 16) + rb * 16 + 15) / G;
    last_tok = max(last_tok, min(wave_last, nt - 1));
  }
  if (wave * (RB * 16) / G >= nt) return;  // no rows for this wave
  const int qmax = ctx + last_tok;

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
  const size_t kofs = (size_t)kvh * PS * HD, vofs = (size_t)a.nkv * PS * HD + (size_t)kvh * HD * PS;
  const int e_begin = a.seq_pg0[s], e_stop = a.seq_pg0[s + 1];
  for (int e = e_begin; e < e_stop; e += 2) {
    const int st0 = a.pg_start[e];
    if (st0 > qmax) break;
    const int pg0 = a.pg_id[e], v0 = a.pg_valid[e];
    const bool two = e + 1 < e_stop && a.pg_start[e + 1] <= qmax;
    const int pg1 = two ? a.pg_id[e + 1] : pg0, v1 = two ? a.pg_valid[e + 1] : 0;
    const int st1 = two ? a.pg_start[e + 1] : 0;
    const size_t b0 = (size_t)pg0 * a.page_stride, b1 = (size_t)pg1 * a.page_stride;
    attend_pair<HD, E4M3, RB>(qf, oacc, m_run, l_run, a.kv_layer, b0 + kofs, b1 + kofs, b0 + vofs,
                              b1 + vofs, v0, v1, st0, st1, qidx, scale_log2, lane);
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

void launch_attn_decode(const AttnArgs& a, hipStream_t st) {
  if (a.n_items == 0) return;
  dim3 grid(a.n_items, a.nkv);
  if (a.hd == 128) {
    if (a.kv_e4m3) hipLaunchKernelGGL((attn_decode_kernel<128, true>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((attn_decode_kernel<128, false>), grid, dim3(64), 0, st, a);
  } else {
    if (a.kv_e4m3) hipLaunchKernelGGL((attn_decode_kernel<64, true>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((attn_decode_kernel<64, false>), grid, dim3(64), 0, st, a);
  }
}

void launch_attn_combine(const AttnArgs& a, hipStream_t st) {
  if (a.n_combine == 0) return;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.n_combine, a.nkv), dim3(64), 0, st, a);
}

void launch_attn_prefill(const AttnArgs& a, hipStream_t st) {
  if (a.n_items == 0) return;
  dim3 grid(a.n_items, a.nkv);
  if (a.hd == 128) {
    if (a.kv_e4m3) hipLaunchKernelGGL((attn_prefill_kernel<128, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((attn_prefill_kernel<128, false>), grid, dim3(256), 0, st, a);
  } else {
    if (a.kv_e4m3) hipLaunchKernelGGL((attn_prefill_kernel<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((attn_prefill_kernel<64, false>), grid, dim3(256), 0, st, a);
  }
}

}  // namespace pie
