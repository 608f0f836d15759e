// MFMA GEMM with fused RMSNorm prologue, split-K and the decoder's epilogues.
// See gemm.h for the operation.  The tiled kernel (prefill-sized M) stages
// tiles through LDS with double buffering; each of the 4 waves of a workgroup
// owns a WM x WN block of the BM x BN tile and issues 16x16x32 bf16 MFMAs.
// The skinny kernel (decode-sized M) is a weight stream, described below.
//
// Split-K (skinny kernel): every split writes its fp32 partial tile and exits; a second,
// small kernel sums the partials in split order (so the result does not
// depend on scheduling) and runs the epilogue.  The kernel boundary is what
// makes the partials visible: on gfx950 each XCD has its own L2, and an
// in-kernel device-scope fence would write back and invalidate the whole L2
// of the XCD for every workgroup.
#include <climits>
#include <type_traits>

#include "common.h"
#include "gemm.h"

namespace pie {

struct uint4x2 {
  uint4 a, b;
};

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // bf16 elements per LDS row (16 B pad against bank conflicts)

template <int BM, int BN>
struct Cfg {
  static constexpr int WAVES_M = BM >= 128 ? 2 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int FM = WM / 16;
  static constexpr int FN = WN / 16;
  static constexpr int A_CH = BM * BK / 8 / 256;  // 16-byte chunks per thread
  static constexpr int B_CH = BN * BK / 8 / 256;
  static constexpr int LDS_AB = 2 * (BM + BN) * LDK * 2;
  static constexpr int LDC = BN + 4;
  static constexpr int LDS_C = BM * LDC * 4;
  static constexpr int LDS_BYTES = LDS_AB > LDS_C ? LDS_AB : LDS_C;
};

// Epilogue over rows [m0, m0 + rows) of output tile n_tile, whose fp32 values
// are in sC (row stride ldc).  Called by all NTH threads of a workgroup.
// Global loads are issued B units at a time before any of their
// results is used, so a wave waits for memory once per batch rather than
// once per row (tiles run one workgroup, one wave per SIMD, per CU, so
// nothing else hides that latency).
// EPI_QKV part of the epilogue: RoPE on q and k, q to its bf16 buffer, k and
// v to their KV page slots.  Head size HD (64 or 128) and the 16-token page
// are compile-time, so every index is shifts and masks.
constexpr int KV_PAGE = 16;  // tokens per KV page (the only page size the engine accepts)

// Optional LDS copies of what the epilogue would otherwise load per row:
// rope = the rows' RoPE table ([rows][HD / 2] (cos, sin)), slot = their KV
// slots, scale = the layer's e4m3 scales ([2][nkv]).
struct QkvStaged {
  const float2* rope;
  const int* slot;
  const float* scale;
};

template <int HD, int BN, int NTH, int B>
__device__ __forceinline__ void qkv_epilogue(const GemmArgs& g, const float* sC, int ldc, int m0, int rows,
                                             int n_tile, QkvStaged sg) {
  // q and k: a unit is one row's group of 8 consecutive rotation pairs
  // (d0 .. d0 + 7 with their partners d0 + HD/2 ..), so each half goes out
  // as one 16-byte store (8 bf16; 8 bytes for e4m3 K).  v: a unit is one
  // column over 8 consecutive rows; when their slots are 8 consecutive
  // slots of one page (the usual prefill case) they go out as one store,
  // else one element at a time.
  constexpr int HD2 = HD / 2, P = KV_PAGE, GPR = BN / 16, GPH = HD2 / 8;
  const int tid = threadIdx.x;
  const int n0 = n_tile * BN;
  const int qw = g.nq * HD, kw = g.nkv * HD;
  const int kind = n0 < qw ? 0 : (n0 < qw + kw ? 1 : 2);
  auto slot_of = [&](int row, int m) { return sg.slot ? sg.slot[row] : g.slot[m]; };
  if (kind <= 1) {
    const int head0 = kind == 0 ? n0 / HD : (n0 - qw) / HD;
    // k units run along 16 consecutive rows first, so that the stores of
    // consecutive tokens of a page ([kv head][HD / 8][token][8]) are adjacent
    const int units = kind == 0 ? rows * GPR : (rows + 15) / 16 * 16 * GPR;
    for (int u = tid; u < units; u += NTH) {
      const int row = kind == 0 ? u / GPR : (u / (16 * GPR)) * 16 + u % 16;
      const int grp = kind == 0 ? u % GPR : (u / 16) % GPR;
      const int m = m0 + row;
      if (row >= rows || m >= g.M) continue;
      const int hl = grp / GPH, d0 = (grp % GPH) * 8;
      const float* xr = sC + row * ldc + hl * HD + d0;
      const float4* cs4 = reinterpret_cast<const float4*>(
          sg.rope ? sg.rope + row * HD2 + d0 : reinterpret_cast<const float2*>(g.rope_cs) + (size_t)m * HD2 + d0);
      float4 c4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c4[i] = cs4[i];  // (cos, sin) of pairs 2i, 2i + 1
      const float4 a0 = *reinterpret_cast<const float4*>(xr), a1 = *reinterpret_cast<const float4*>(xr + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(xr + HD2), b1 = *reinterpret_cast<const float4*>(xr + HD2 + 4);
      const float x1[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float x2[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float o1[8], o2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float c = (i & 1) ? c4[i >> 1].z : c4[i >> 1].x, sn = (i & 1) ? c4[i >> 1].w : c4[i >> 1].y;
        o1[i] = x1[i] * c - x2[i] * sn;
        o2[i] = x2[i] * c + x1[i] * sn;
      }
      if (kind == 0) {
        uint16_t* q = g.q_out + (size_t)m * qw + (head0 + hl) * HD + d0;
        *reinterpret_cast<uint4*>(q) = make_uint4(pack_bf2(o1[0], o1[1]), pack_bf2(o1[2], o1[3]),
                                                  pack_bf2(o1[4], o1[5]), pack_bf2(o1[6], o1[7]));
        *reinterpret_cast<uint4*>(q + HD2) = make_uint4(pack_bf2(o2[0], o2[1]), pack_bf2(o2[2], o2[3]),
                                                        pack_bf2(o2[4], o2[5]), pack_bf2(o2[6], o2[7]));
        continue;
      }
      const int sl = slot_of(row, m), page = sl / P, off = sl % P;
      const size_t base = (size_t)page * g.page_stride + (size_t)(head0 + hl) * P * HD + (size_t)off * 8;
      const size_t i1 = base + (size_t)(d0 >> 3) * P * 8, i2 = base + (size_t)((d0 + HD2) >> 3) * P * 8;
      if (g.kv_e4m3) {
        const float sc = sg.scale ? sg.scale[head0 + hl] : g.kv_scale[head0 + hl];
        uint32_t w1[2] = {0u, 0u}, w2[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          w1[i >> 2] |= (uint32_t)f2e4m3(o1[i] / sc) << (8 * (i & 3));
          w2[i >> 2] |= (uint32_t)f2e4m3(o2[i] / sc) << (8 * (i & 3));
        }
        uint8_t* kv = reinterpret_cast<uint8_t*>(g.kv_layer);
        *reinterpret_cast<uint2*>(kv + i1) = make_uint2(w1[0], w1[1]);
        *reinterpret_cast<uint2*>(kv + i2) = make_uint2(w2[0], w2[1]);
      } else {
        uint16_t* kv = reinterpret_cast<uint16_t*>(g.kv_layer);
        *reinterpret_cast<uint4*>(kv + i1) = make_uint4(pack_bf2(o1[0], o1[1]), pack_bf2(o1[2], o1[3]),
                                                        pack_bf2(o1[4], o1[5]), pack_bf2(o1[6], o1[7]));
        *reinterpret_cast<uint4*>(kv + i2) = make_uint4(pack_bf2(o2[0], o2[1]), pack_bf2(o2[2], o2[3]),
                                                        pack_bf2(o2[4], o2[5]), pack_bf2(o2[6], o2[7]));
      }
    }
  } else {
    // v: layout [kv head][HD][token]; consecutive threads take consecutive
    // columns (conflict-free reads of sC)
    const int v0 = n0 - qw - kw;
    const int units = (rows + 7) / 8 * BN;
    for (int u = tid; u < units; u += NTH) {
      const int c = u % BN, r0 = (u / BN) * 8;
      const int vc = v0 + c, kvh = vc / HD, dd = vc % HD;
      const size_t col = (size_t)g.nkv * P * HD + (size_t)kvh * HD * P + (size_t)dd * P;
      const float sc = !g.kv_e4m3 ? 1.f : sg.scale ? sg.scale[g.nkv + kvh] : g.kv_scale[g.nkv + kvh];
      int sl[8];
      float x[8];
      bool whole = true;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = r0 + i, m = m0 + row;
        const bool ok = row < rows && m < g.M;
        sl[i] = ok ? slot_of(row, m) : -1;
        x[i] = ok ? sC[row * ldc + c] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) whole = whole && sl[i] == sl[0] + i;
      whole = whole && sl[0] >= 0 && (sl[0] & 7) == 0;  // 8 slots inside one page
      if (whole) {
        const size_t idx = (size_t)(sl[0] / P) * g.page_stride + col + (sl[0] % P);
        if (g.kv_e4m3) {
          uint32_t w[2] = {0u, 0u};
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i >> 2] |= (uint32_t)f2e4m3(x[i] / sc) << (8 * (i & 3));
          *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(g.kv_layer) + idx) = make_uint2(w[0], w[1]);
        } else {
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(g.kv_layer) + idx) =
              make_uint4(pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7]));
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (sl[i] < 0) continue;
        const size_t idx = (size_t)(sl[i] / P) * g.page_stride + col + (sl[i] % P);
        if (g.kv_e4m3) reinterpret_cast<uint8_t*>(g.kv_layer)[idx] = f2e4m3(x[i] / sc);
        else reinterpret_cast<uint16_t*>(g.kv_layer)[idx] = f2bf(x[i]);
      }
    }
  }
}

template <int EPI, int BN, int NTH = 256, int B = 8>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const float* sC, int ldc, int m0, int rows,
                                         int n_tile, QkvStaged sg = QkvStaged{nullptr, nullptr, nullptr}) {
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (EPI == EPI_RESID) {
    // y += C, and the per-64-column sums of squares of the new y for the
    // next RMSNorm.  A wave step covers RPI rows x BN columns, a float4 per
    // lane; the 16 lanes of a 64-column chunk reduce its sum of squares.
    constexpr int F4 = BN / 4, RPI = 64 / F4;
    const int n0 = n_tile * BN, c4 = lane % F4, rs = lane / F4, col = c4 * 4;
    const bool col_ok = n0 + col < g.N;  // N is a multiple of 64
    const int steps = (rows + RPI - 1) / RPI;
    for (int s0 = wave; s0 < steps; s0 += NW * B) {
      float4 v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int row = (s0 + u * NW) * RPI + rs, m = m0 + row;
        const bool ok = s0 + u * NW < steps && row < rows && m < g.M && col_ok;
        v[u] = ok ? *reinterpret_cast<const float4*>(g.y_out + (size_t)m * g.ldy + n0 + col)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int row = (s0 + u * NW) * RPI + rs, m = m0 + row;
        const bool ok = s0 + u * NW < steps && row < rows && m < g.M && col_ok;
        float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) c = *reinterpret_cast<const float4*>(sC + row * ldc + col);
        const float4 nv = make_float4(v[u].x + c.x, v[u].y + c.y, v[u].z + c.z, v[u].w + c.w);
        if (ok) *reinterpret_cast<float4*>(g.y_out + (size_t)m * g.ldy + n0 + col) = nv;
        float sq = nv.x * nv.x + nv.y * nv.y + nv.z * nv.z + nv.w * nv.w;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
        if (ok && (lane & 15) == 0) g.ss_out[(size_t)m * g.n_ss + (n0 + col) / 64] = sq;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // h = bf16(silu(gate) * up), four columns per thread (N is a multiple of 8)
    constexpr int HALF = BN / 2, F4 = HALF / 4;
    const int cw = g.cw ? g.cw : HALF, j0 = n_tile * cw;
    for (int idx = tid; idx < rows * F4; idx += NTH) {
      const int row = idx / F4, j = (idx % F4) * 4, m = m0 + row, n = j0 + j;
      if (m >= g.M || n >= g.N || j >= cw) continue;
      const float4 gt = *reinterpret_cast<const float4*>(sC + row * ldc + j);
      const float4 up = *reinterpret_cast<const float4*>(sC + row * ldc + HALF + j);
      const float h0 = gt.x / (1.0f + expf(-gt.x)) * up.x, h1 = gt.y / (1.0f + expf(-gt.y)) * up.y;
      const float h2 = gt.z / (1.0f + expf(-gt.z)) * up.z, h3 = gt.w / (1.0f + expf(-gt.w)) * up.w;
      *reinterpret_cast<uint2*>(g.h_out + (size_t)m * g.N + n) = make_uint2(pack_bf2(h0, h1), pack_bf2(h2, h3));
    }
  } else if constexpr (EPI == EPI_QKV) {
    if (g.hd == 128) qkv_epilogue<128, BN, NTH, B>(g, sC, ldc, m0, rows, n_tile, sg);
    else qkv_epilogue<64, BN, NTH, B>(g, sC, ldc, m0, rows, n_tile, sg);
  } else if constexpr (EPI == EPI_LOGITS) {
    // one wave per row; the row's readout parameters are loaded a batch of rows at a time
    const int n0 = n_tile * BN;
    for (int r0 = wave; r0 < rows; r0 += NW * B) {
      int kd[B], ln[B];
      float tp[B];
      uint32_t lo[B], hi[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int row = r0 + u * NW, m = m0 + row;
        const bool ok = row < rows && m < g.M;
        kd[u] = ok ? g.ro_kind[m] : 0;
        tp[u] = ok ? g.ro_temp[m] : 1.f;
        lo[u] = ok ? g.ro_seed_lo[m] : 0u;
        hi[u] = ok ? g.ro_seed_hi[m] : 0u;
        ln[u] = ok ? g.ro_lane[m] : 0;
      }
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int row = r0 + u * NW, m = m0 + row;
        if (row >= rows || m >= g.M) continue;
        float best = -INFINITY;
        int bi = INT_MAX;
        for (int c = lane; c < BN; c += 64) {
          const int v = n0 + c;
          if (v >= g.N) break;
          const float l = sC[row * ldc + c];
          if (g.logits) g.logits[(size_t)m * g.N + v] = l;
          const float sv = kd[u] == 0 ? l : l / tp[u] + gumbel((uint32_t)v, (uint32_t)ln[u], lo[u], hi[u]);
          if (sv > best) { best = sv; bi = v; }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ob = __shfl_xor(best, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
        }
        if (lane == 0) {
          const int n_tiles = (g.N + BN - 1) / BN;
          g.tile_best[(size_t)m * n_tiles + n_tile] = best;
          g.tile_idx[(size_t)m * n_tiles + n_tile] = bi;
        }
      }
    }
  }
}

constexpr int GROUP_M = 16;

// Output tiles along N of the tiled kernel (EPI_SWIGLU tiles hold BN/2 gate and BN/2 up columns).
template <int EPI>
__device__ __forceinline__ int tiles_n(const GemmArgs& g, int BN) {
  return EPI == EPI_SWIGLU ? (g.N + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
}

template <int BM, int BN, int AMODE, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  using C = Cfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  __shared__ float s_rstd[BM];
  __shared__ int s_rows[BM];

  uint16_t* sA = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sB = sA + 2 * BM * LDK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // Grouped raster: consecutive workgroups sweep GROUP_M row tiles for each
  // column tile, so the ~256 workgroups in flight share 16 row tiles and 16
  // column tiles and read each from HBM about once per window (row-major
  // order would read every column tile once per row tile).
  int n_tile, m_tile;
  {
    const int n_tiles = tiles_n<EPI>(g, BN), m_tiles = (g.M + BM - 1) / BM;
    const int pid = blockIdx.x, per_group = GROUP_M * n_tiles;
    const int grp = pid / per_group, m0g = grp * GROUP_M, gm = min(GROUP_M, m_tiles - m0g);
    const int r = pid - grp * per_group;
    m_tile = m0g + r % gm;
    n_tile = r / gm;
  }
  const int m0 = m_tile * BM;
  const int kb = 0, ke = g.K;  // the tiled kernel does not split K

  if (AMODE == A_NORM) {
    for (int i = tid; i < BM; i += 256) {
      int m = m0 + i, src = -1;
      float r = 0.f;
      if (m < g.M) {
        src = g.a_rows ? g.a_rows[m] : m;
        const float* p = g.ss + (size_t)src * g.n_ss;
        float s = 0.f;
        for (int c = 0; c < g.n_ss; ++c) s += p[c];
        r = 1.0f / sqrtf(s / (float)g.K + g.eps);
      }
      s_rows[i] = src;
      s_rstd[i] = r;
    }
    __syncthreads();
  }

  // This thread's W pieces: piece c of the BN x 64 tile lies in 64-row block
  // c / 512 (a packed 8 KiB block per K chunk) at element (c % 512) * 8, so a
  // wave's loads are one contiguous KiB.  wblk: block base at K chunk 0
  // (nullptr = rows past N, read as zeros).
  static_assert(BN == 128, "two 64-row packed blocks per tile");
  const int kc = (g.K + 63) / 64;
  const uint16_t* wblk[C::B_CH];
#pragma unroll
  for (int i = 0; i < C::B_CH; ++i) {
    const int c = tid + 256 * i, bsel = c >> 9;
    const uint16_t* p = nullptr;
    if (EPI == EPI_SWIGLU) {
      if (n_tile * 64 < g.N) p = g.w[bsel] + (size_t)n_tile * kc * 4096;
    } else {
      const int n = n_tile * BN + bsel * 64;
      if (n < g.N) {
        const int s = n >= g.seg_n0[1] ? (n >= g.seg_n0[2] ? 2 : 1) : 0;
        p = g.w[s] + (size_t)((n - g.seg_n0[s]) >> 6) * kc * 4096;
      }
    }
    wblk[i] = p ? p + (size_t)(c & 511) * 8 : nullptr;
  }

  uint4 ra[C::A_CH];
  float4 rn[C::A_CH][2];
  uint4 rg[C::A_CH];
  uint4 rb[C::B_CH];

  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      int c = tid + 256 * i, row = c >> 3, k = k0 + (c & 7) * 8;
      if (AMODE == A_BF16) {
        int m = m0 + row;
        ra[i] = (m < g.M && k < ke) ? *reinterpret_cast<const uint4*>(g.a + (size_t)m * g.lda + k)
                                    : make_uint4(0, 0, 0, 0);
      } else {
        int src = s_rows[row];
        if (src >= 0 && k < ke) {
          const float4* p = reinterpret_cast<const float4*>(g.y + (size_t)src * g.ldy + k);
          rn[i][0] = p[0];
          rn[i][1] = p[1];
          rg[i] = *reinterpret_cast<const uint4*>(g.gain + k);
        } else {
          rn[i][0] = rn[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
          rg[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i)
      rb[i] = wblk[i] ? *reinterpret_cast<const uint4*>(wblk[i] + (size_t)(k0 >> 6) * 4096)
                      : make_uint4(0, 0, 0, 0);
  };

  auto store = [&](int buf) {
    uint16_t* A = sA + buf * BM * LDK;
    uint16_t* B = sB + buf * BN * LDK;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      int c = tid + 256 * i, row = c >> 3, kk = (c & 7) * 8;
      uint4 v;
      if (AMODE == A_BF16) {
        v = ra[i];
      } else {
        float r = s_rstd[row];
        const float* x = reinterpret_cast<const float*>(&rn[i][0]);
        const uint32_t* gw = reinterpret_cast<const uint32_t*>(&rg[i]);
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = pack_bf2(x[2 * j] * r * bf2f(gw[j] & 0xffffu), x[2 * j + 1] * r * bf2f(gw[j] >> 16));
        v = make_uint4(o[0], o[1], o[2], o[3]);
      }
      *reinterpret_cast<uint4*>(A + row * LDK + kk) = v;
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int c = tid + 256 * i, q = c & 511;
      const int row = (c >> 9) * 64 + (q >> 7) * 16 + (q & 15), kk = ((q >> 6) & 1) * 32 + ((q >> 4) & 3) * 8;
      *reinterpret_cast<uint4*>(B + row * LDK + kk) = rb[i];
    }
  };

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int a = 0; a < C::FM; ++a)
#pragma unroll
    for (int b = 0; b < C::FN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
  if (nk > 0) {
    load(kb);
    store(0);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
      if (t + 1 < nk) load(kb + (t + 1) * BK);
      const uint16_t* A = sA + (t & 1) * BM * LDK;
      const uint16_t* B = sB + (t & 1) * BN * LDK;
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        int kk = ks * 32 + (lane >> 4) * 8;
        uint4 af[C::FM], bfr[C::FN];
#pragma unroll
        for (int a = 0; a < C::FM; ++a)
          af[a] = *reinterpret_cast<const uint4*>(A + (wm * C::WM + a * 16 + (lane & 15)) * LDK + kk);
#pragma unroll
        for (int b = 0; b < C::FN; ++b)
          bfr[b] = *reinterpret_cast<const uint4*>(B + (wn * C::WN + b * 16 + (lane & 15)) * LDK + kk);
#pragma unroll
        for (int a = 0; a < C::FM; ++a)
#pragma unroll
          for (int b = 0; b < C::FN; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
      }
      if (t + 1 < nk) store((t + 1) & 1);
      lds_barrier();
    }
  }


  float* sC = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int a = 0; a < C::FM; ++a)
#pragma unroll
    for (int b = 0; b < C::FN; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int row = wm * C::WM + a * 16 + 4 * (lane >> 4) + i;
        int col = wn * C::WN + b * 16 + (lane & 15);
        sC[row * C::LDC + col] = acc[a][b][i];
      }
  __syncthreads();
  epilogue<EPI, BN>(g, sC, C::LDC, m0, BM, n_tile);
}

// ---------------------------------------------------------------------------
// Large variant for prefill-sized M: a 256 x 256 output tile per workgroup of
// 8 waves (2 along M x 4 along N), each wave a 128 x 64 block of 4 x 2
// 32x32x16 MFMAs (128 fp32 accumulators per lane), K in stages of 64 staged
// through double-buffered LDS.  Two waves per SIMD hide each other's load
// and LDS latency; the next stage's global loads are in flight while the
// current stage is computed.  The epilogue runs in four passes of 64 rows
// through LDS.
constexpr int BG_BM = 256, BG_BN = 256, BG_BK = 64, BG_NT = 512, BG_LDK = BG_BK + 8, BG_LDC = BG_BN + 4;
constexpr int BG_PIECES = BG_BM * BG_BK / 8 / BG_NT;  // 16-byte pieces per thread per operand per stage (8)
constexpr int BG_LDS = 2 * (BG_BM + BG_BN) * BG_LDK * 2;
static_assert(64 * BG_LDC * 4 <= BG_LDS, "epilogue pass fits in the operand buffers");

template <int EPI>
__device__ __forceinline__ int big_tiles_n(const GemmArgs& g) {
  return EPI == EPI_SWIGLU ? (g.N + BG_BN / 2 - 1) / (BG_BN / 2) : (g.N + BG_BN - 1) / BG_BN;
}

// XCD-aware raster of the 256 x 256 tiles, one workgroup per tile.
// Workgroup i runs on XCD i % 8 (each XCD has its own L2).  The tiles, in
// bands of 4 tile rows walked along N, are cut into 8 contiguous ranges, one
// per XCD, of the sizes that the round-robin hands each XCD, so every XCD
// gets the same share (to one tile) whatever the grid, and the 32 tiles an
// XCD runs at a time form a 4 x 8 block: each A tile is read by 8 and each
// B tile by 4 of them through the same L2.
constexpr int BIG_BAND = 4;

__device__ __forceinline__ void big_tile_of(int pid, int m_tiles, int n_tiles, int& m_tile, int& n_tile) {
  const int T = m_tiles * n_tiles, q = T >> 3, r = T & 7;
  const int x = pid & 7, j = pid >> 3;
  const int t = x * q + min(x, r) + j;  // XCD x's range starts after the q (+1) tiles of each XCD before it
  const int per_band = BIG_BAND * n_tiles, band = t / per_band;
  const int mb = band * BIG_BAND, bm = min(BIG_BAND, m_tiles - mb), u = t - band * per_band;
  m_tile = mb + u % bm;
  n_tile = u / bm;
}

template <int EPI>
__global__ __launch_bounds__(BG_NT, 2) void gemm_big_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[BG_LDS];
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sB = sA + 2 * BG_BM * BG_LDK;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave >> 2, wn = wave & 3, l32 = lane & 31, lh = lane >> 5;

  int n_tile, m_tile;
  big_tile_of(blockIdx.x, (g.M + BG_BM - 1) / BG_BM, big_tiles_n<EPI>(g), m_tile, n_tile);
  const int m0 = m_tile * BG_BM;
  const int kc = (g.K + 63) / 64;
  const int nk = kc;

  // A pieces: row p / 8, columns (p % 8) * 8; B pieces: packed 64-row block p / 512.
  const uint16_t* bblk[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint16_t* p = nullptr;
    if (EPI == EPI_SWIGLU) {
      const int t64 = n_tile * 2 + (b & 1);
      if (t64 * 64 < g.N) p = g.w[b >> 1] + (size_t)t64 * kc * 4096;
    } else {
      const int n = n_tile * BG_BN + b * 64;
      if (n < g.N) {
        const int s = n >= g.seg_n0[1] ? (n >= g.seg_n0[2] ? 2 : 1) : 0;
        p = g.w[s] + (size_t)((n - g.seg_n0[s]) >> 6) * kc * 4096;
      }
    }
    bblk[b] = p;
  }
  uint4 ra[BG_PIECES], rb[BG_PIECES];
  auto load = [&](int c) {
    const int k0 = c * BG_BK;
#pragma unroll
    for (int i = 0; i < BG_PIECES; ++i) {
      const int p = tid + BG_NT * i, row = p >> 3, k = k0 + (p & 7) * 8, m = m0 + row;
      ra[i] = (m < g.M && k < g.K) ? *reinterpret_cast<const uint4*>(g.a + (size_t)m * g.lda + k)
                                   : make_uint4(0, 0, 0, 0);
      const uint16_t* bp = bblk[p >> 9];
      rb[i] = bp ? *reinterpret_cast<const uint4*>(bp + (size_t)c * 4096 + (size_t)(p & 511) * 8)
                 : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
    uint16_t* A = sA + buf * BG_BM * BG_LDK;
    uint16_t* B = sB + buf * BG_BN * BG_LDK;
#pragma unroll
    for (int i = 0; i < BG_PIECES; ++i) {
      const int p = tid + BG_NT * i, q = p & 511;
      *reinterpret_cast<uint4*>(A + (p >> 3) * BG_LDK + (p & 7) * 8) = ra[i];
      const int row = (p >> 9) * 64 + (q >> 7) * 16 + (q & 15), kk = ((q >> 6) & 1) * 32 + ((q >> 4) & 3) * 8;
      *reinterpret_cast<uint4*>(B + row * BG_LDK + kk) = rb[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  if (nk > 0) {
    load(0);
    store(0);
    lds_barrier();
    for (int t = 0; t < nk; ++t) {
      if (t + 1 < nk) load(t + 1);
      const uint16_t* A = sA + (t & 1) * BG_BM * BG_LDK + (wm * 128 + l32) * BG_LDK + lh * 8;
      const uint16_t* B = sB + (t & 1) * BG_BN * BG_LDK + (wn * 64 + l32) * BG_LDK + lh * 8;
#pragma unroll
      for (int ks = 0; ks < BG_BK / 16; ++ks) {
        uint4 af[4], bf[2];
#pragma unroll
        for (int a = 0; a < 4; ++a) af[a] = *reinterpret_cast<const uint4*>(A + a * 32 * BG_LDK + ks * 16);
#pragma unroll
        for (int b = 0; b < 2; ++b) bf[b] = *reinterpret_cast<const uint4*>(B + b * 32 * BG_LDK + ks * 16);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(af[a], bf[b], acc[a][b]);
      }
      if (t + 1 < nk) store((t + 1) & 1);
      lds_barrier();
    }
  }

  // Epilogue in four passes of 64 rows (the four waves owning them write sC).
  float* sC = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (wm == (pass >> 1)) {
#pragma unroll
      for (int ah = 0; ah < 2; ++ah) {
        const int a = (pass & 1) * 2 + ah;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = ah * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            sC[row * BG_LDC + wn * 64 + b * 32 + l32] = acc[a][b][i];
          }
      }
    }
    __syncthreads();
    epilogue<EPI, BG_BN, BG_NT, 2>(g, sC, BG_LDC, m0 + pass * 64, 64, n_tile);
    __syncthreads();
  }
}

// Raw buffer descriptor over [base, base + bytes); loads past the end read zeros.
constexpr uint32_t OOB = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte raw buffer load (out-of-range offsets read zeros).
template <int CPOL = 0>
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL));
}

// ---------------------------------------------------------------------------
// Direct-to-LDS form of the 256 x 256 tile (K a multiple of 64, A rows
// 16-byte aligned).  Operands go from memory straight into LDS with 16-byte
// buffer loads that write LDS (lane l of a load writes bytes [16l, 16l + 16)
// of a 1 KiB block at a wave-uniform address): staging costs no VGPRs and no
// LDS store instructions.  Four waves, one per SIMD, each own a 128 x 128
// block (4 x 4 32x32x16 MFMAs, 256 fp32 accumulators); K advances in stages
// of 64 through two LDS buffers.
//  - A stage: 256 rows of 128 bytes.  Row r's eight 16-byte chunks sit at
//    slots chunk ^ swz(r), so the MFMA operand reads (32 rows at one chunk)
//    hit every bank once both in 8-lane and in 16-lane LDS phases.  One load
//    covers 8 whole rows (whole 128-byte lines); each lane fetches the chunk
//    that belongs in its slot.
//  - B stage: the four 64-row blocks of the tiled weight layout, 8 KiB each,
//    copied as they are; the operand reads are contiguous 256-byte runs.
// The loop is software-pipelined and its order pinned by scheduling
// barriers, because with one wave per SIMD the wave itself must keep the
// matrix core busy: each k-step's 16 MFMAs run while the next k-step's
// operands are read from LDS.  One barrier per stage, between k-steps 2 and
// 3: by then every wave has read all of stage t (k-step 3's operands were
// read during k-step 2) and waited for its own loads of stage t + 1, so
// after it stage t + 1 may be read and stage t + 2 loaded into t's buffer.
// The O, down and gate/up projections use a 1 x 4 arrangement of the same
// loop (DG_FORM) in which only A passes through LDS.
constexpr int DG_BK = 64, DG_NT = 256;
// 0: 2 x 2 waves of 128 x 128, A and B through LDS; 1: 1 x 4 waves of
// 256 x 64, A through LDS, each wave's B straight into registers (half the
// LDS-writing loads, the same bytes into the CU): 1-1.5% faster on the O,
// down and gate/up shapes
constexpr int DG_FORM = 1;
constexpr int DG_STAGE = (BG_BM + BG_BN) * DG_BK * 2;  // 64 KiB
constexpr int DG_LDS = 2 * DG_STAGE;                    // 128 KiB
// Epilogue LDS: one 64-row pass of fp32 results, then (QKV) 64 RoPE rows of
// up to 64 (cos, sin) pairs, 64 slots and up to 2 x 128 e4m3 scales.
constexpr int DG_EPI_C = (64 * BG_LDC * 4 + 1023) / 1024 * 1024, DG_EPI_ROPE = 64 * 64 * 8;
static_assert(DG_EPI_C + DG_EPI_ROPE + 256 + 2 * 128 * 4 <= DG_LDS, "epilogue pass fits in the stage buffers");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor words over [base, base + bytes) (raw, no stride).
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// 16-byte buffer load into LDS: lane l's bytes [voff + soff, + 16) of the
// buffer go to LDS bytes [16l, 16l + 16) past `lds` (wave-uniform).  Written
// as inline assembly so that the compiler does not track it: it would
// otherwise make every LDS read wait for all such loads in flight.  The
// caller waits for them with s_waitcnt vmcnt.  M0 carries the LDS address;
// the nop covers the M0-write hazard of these loads.
__device__ __forceinline__ void dma16(i32x4_t r, const void* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m = (uint32_t)(size_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m), "v"(voff), "s"(r), "s"(soff) : "memory");
}

__device__ __forceinline__ int dg_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt: vector-memory counter at most n and every LDS access of the wave
// complete (expcnt left at its maximum).
#define DG_WAIT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x70)

// Barrier without a memory fence: a workgroup-scope fence would also wait for
// every LDS-writing load in flight, which is what the pipeline keeps in
// flight.  The memory clobber keeps the compiler from moving LDS accesses
// across it; the loads a wave depends on are waited for before it.
__device__ __forceinline__ void dg_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int EPI>
__global__ __launch_bounds__(DG_NT, 1) void gemm_dma_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DG_LDS];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, lh = lane >> 5;

  int n_tile, m_tile;
  big_tile_of(blockIdx.x, (g.M + BG_BM - 1) / BG_BM, big_tiles_n<EPI>(g), m_tile, n_tile);
  const int m0 = m_tile * BG_BM;
  const int nk = g.K / DG_BK;  // = 64-column blocks of the packed weights

  // A: this wave loads rows 64 * wave .. + 63 of every stage (eight 8-row
  // loads).  Rows past M read row M - 1 (their outputs are never stored).
  const i32x4_t ra = rsrc_words(g.a, (uint32_t)((size_t)g.M * g.lda * 2));
  uint32_t a_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = wave * 64 + i * 8 + (lane >> 3);
    const int m = min(m0 + r, g.M - 1);
    a_off[i] = (uint32_t)(((size_t)m * g.lda + (((lane & 7) ^ dg_swz(r)) * 8)) * 2);
  }
  // B: this wave loads the tile's 64-row block `wave` (8 KiB per stage).
  // Blocks past N read the last one (their outputs are never stored).
  i32x4_t rb;
  const uint16_t* base;
  {
    if (EPI == EPI_SWIGLU) {
      const int t64 = min(n_tile * 2 + (wave & 1), (g.N - 1) >> 6);
      base = g.w[wave >> 1] + (size_t)t64 * nk * 4096;
    } else {
      const int n = min(n_tile * BG_BN + wave * 64, g.N - 1);
      const int s = n >= g.seg_n0[1] ? (n >= g.seg_n0[2] ? 2 : 1) : 0;
      base = g.w[s] + (size_t)((n - g.seg_n0[s]) >> 6) * nk * 4096;
    }
    rb = rsrc_words(base, (uint32_t)nk * 8192u);
  }
  // Load i (0..15) of stage t.  Every iteration issues them, also for t >=
  // nk, so that the loop body is one branch-free block: past the end, A
  // lanes use an offset beyond the buffer and B offsets run past the matrix
  // row, both of which read zeros without touching memory, into the buffer
  // of a stage that is no longer read.
  auto issue_one = [&](int t, int i) {
    uint8_t* st = smem + (t & 1) * DG_STAGE;
    if (i < 8) {
      const bool live = t < nk;
      dma16(ra, st + (wave * 8 + i) * 1024, live ? a_off[i] : OOB, live ? (uint32_t)t * (DG_BK * 2) : 0u);
    } else {
      dma16(rb, st + BG_BM * 128 + wave * 8192 + (i - 8) * 1024, (uint32_t)lane * 16u,
            (uint32_t)t * 8192u + (uint32_t)(i - 8) * 1024u);
    }
  };

  // QKV keeps the 2 x 2 form: with its RoPE epilogue the 1 x 4 form spills
  // its accumulators to scratch
  constexpr int FORM = EPI == EPI_QKV ? 0 : DG_FORM;
  constexpr int AM = FORM == 1 ? 8 : 4, AN = FORM == 1 ? 2 : 4;  // 32 x 32 blocks per wave
  f32x16 acc[AM][AN];
#pragma unroll
  for (int a = 0; a < AM; ++a)
#pragma unroll
    for (int b = 0; b < AN; ++b) acc[a][b] = f32x16{};

  if constexpr (FORM == 1) {
    // Wave w owns all 256 rows and the tile's 64-row weight block w: its B
    // operands are no other wave's, so they go straight into registers (one
    // 16-byte load per fragment, the tiled layout's operand order), and only
    // A passes through LDS: half the LDS-writing loads of the 2 x 2 form
    // and no more bytes moved into the CU.
    const __amdgpu_buffer_rsrc_t rbr = make_rsrc(base, (uint32_t)nk * 8192u);
    const uint32_t boff = (uint32_t)((l32 >> 4) * 2048 + lh * 256 + (l32 & 15) * 16);
    auto bload = [&](int t, int ks, int b) -> uint4 {
      const uint32_t off = boff + (uint32_t)(b * 4096 + (ks >> 1) * 1024 + (ks & 1) * 512);
      return bload16(rbr, t < nk ? off + (uint32_t)t * 8192u : OOB);
    };
    const int a_sw = dg_swz(l32);  // swz depends on the row mod 16 only
    auto afrag = [&](int t, int ks, int a) -> uint4 {
      const uint8_t* st = smem + (t & 1) * DG_STAGE;
      return *reinterpret_cast<const uint4*>(st + (a * 32 + l32) * 128 + (((ks * 2 + lh) ^ a_sw) * 16));
    };
    uint4 BR[2][4][2];  // [stage parity][k-step][column block]
    uint4 FA[8], FB[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_one(0, i);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) BR[0][ks][b2] = bload(0, ks, b2);
    __builtin_amdgcn_s_waitcnt(DG_WAIT(0));
    dg_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_one(1, i);
#pragma unroll
    for (int f = 0; f < 8; ++f) FA[f] = afrag(0, 0, f);
    // One stage; P = t & 1 is a template constant so that the B register
    // sets are addressed statically.  B(t + 1) is loaded in k-step 0 into the
    // set stage t - 1 used; A(t + 2) after the barrier, as in the 2 x 2 form.
    auto stage = [&](int t, auto pc) {
      constexpr int P = decltype(pc)::value;
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
        uint4 (&cur)[8] = (ks & 1) ? FB : FA;
        uint4 (&nxt)[8] = (ks & 1) ? FA : FB;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int a = q >> 1, b2 = q & 1;
          acc[a][b2] = mfma32(cur[a], BR[P][ks][b2], acc[a][b2]);
          if (q < 8) nxt[q] = afrag(t, ks + 1, q);
          if (ks == 0 && (q & 1)) BR[P ^ 1][q >> 2][(q >> 1) & 1] = bload(t + 1, q >> 2, (q >> 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // stage t + 1 landed: A in every wave's share of LDS, B in registers
      __builtin_amdgcn_s_waitcnt(DG_WAIT(0));
      dg_barrier();
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int a = q >> 1, b2 = q & 1;
        acc[a][b2] = mfma32(FB[a], BR[P][3][b2], acc[a][b2]);
        if (q < 8) FA[q] = afrag(t + 1, 0, q);
        if (q & 1) issue_one(t + 2, q >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // pairs of stages; an odd stage count runs one stage of zeros at the end
    for (int t = 0; t < nk; t += 2) {
      stage(t, std::integral_constant<int, 0>{});
      stage(t + 1, std::integral_constant<int, 1>{});
    }
  } else {
  // Operand fragment f of k-step ks of stage t: f < 4 the A rows of block f,
    // f >= 4 the B columns of block f - 4.
    const int a_rd = (wm * 128 + l32) * 128;
    const int a_sw = dg_swz(l32);  // swz depends on the row mod 16 only
    const int b_rd = BG_BM * 128 + wn * 2 * 8192 + (l32 >> 4) * 2048 + lh * 256 + (l32 & 15) * 16;
    auto frag = [&](int t, int ks, int f) -> uint4 {
      const uint8_t* st = smem + (t & 1) * DG_STAGE;
      if (f < 4) return *reinterpret_cast<const uint4*>(st + a_rd + f * 4096 + (((ks * 2 + lh) ^ a_sw) * 16));
      const int b = f - 4;  // column block b: 64-row block (wn * 128 + b * 32) / 64, panel offset
      return *reinterpret_cast<const uint4*>(st + b_rd + (b >> 1) * 8192 + (b & 1) * 4096 + (ks >> 1) * 1024 +
                                             (ks & 1) * 512);
    };
  
    uint4 FA[8], FB[8];
  #pragma unroll
    for (int i = 0; i < 16; ++i) issue_one(0, i);
    __builtin_amdgcn_s_waitcnt(DG_WAIT(0));
    dg_barrier();
  #pragma unroll
    for (int i = 0; i < 8; ++i) issue_one(1, i);
  #pragma unroll
    for (int f = 0; f < 8; ++f) FA[f] = frag(0, 0, f);
  
    // A stage's 16 loads are issued half in k-step 3 of the iteration two
    // before it (right after the barrier that frees its buffer) and half in
    // k-step 0 of the next one, so that the loads of a workgroup spread over
    // two k-steps of MFMAs rather than queueing behind one.
    for (int t = 0; t < nk; ++t) {
      // k-steps 0..2: MFMAs on one fragment set while the next is read
  #pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
        uint4 (&cur)[8] = (ks & 1) ? FB : FA;
        uint4 (&nxt)[8] = (ks & 1) ? FA : FB;
  #pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int a = q >> 2, b = q & 3;
          acc[a][b] = mfma32(cur[a], cur[4 + b], acc[a][b]);
          if (q < 8) nxt[q] = frag(t, ks + 1, q);
          if (ks == 0 && (q & 1)) issue_one(t + 1, 8 + (q >> 1));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // stage t + 1 landed everywhere; all of stage t has been read
      __builtin_amdgcn_s_waitcnt(DG_WAIT(0));
      dg_barrier();
      // k-step 3 (FB) while reading k-step 0 of stage t + 1 (FA; unused past
      // the last stage) and loading half of stage t + 2 into stage t's buffer
  #pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int a = q >> 2, b = q & 3;
        acc[a][b] = mfma32(FB[a], FB[4 + b], acc[a][b]);
        if (q < 8) FA[q] = frag(t + 1, 0, q);
        if (q & 1) issue_one(t + 2, q >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(DG_WAIT(0));
  __syncthreads();

  float* sC = reinterpret_cast<float*>(smem);
  // QKV epilogue staging, past the 64-row pass of sC
  uint8_t* s_rope = smem + DG_EPI_C;
  int* s_slot = reinterpret_cast<int*>(smem + DG_EPI_C + DG_EPI_ROPE);
  float* s_scale = reinterpret_cast<float*>(smem + DG_EPI_C + DG_EPI_ROPE + 256);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if constexpr (FORM == 1) {
#pragma unroll
      for (int ah = 0; ah < 2; ++ah) {
        const int a = pass * 2 + ah;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = ah * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            sC[row * BG_LDC + wave * 64 + b * 32 + l32] = acc[a][b][i];
          }
      }
    } else if (wm == (pass >> 1)) {
#pragma unroll
      for (int ah = 0; ah < 2; ++ah) {
        const int a = (pass & 1) * 2 + ah;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = ah * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            sC[row * BG_LDC + wn * 128 + b * 32 + l32] = acc[a][b][i];
          }
      }
    }
    QkvStaged sg{nullptr, nullptr, nullptr};
    if constexpr (EPI == EPI_QKV) {
      // The pass's 64 RoPE rows (contiguous in the table) go to LDS with the
      // same LDS-writing loads, its slots and the e4m3 scales with plain
      // loads, so the epilogue itself makes no global loads.
      const int hd2 = g.hd >> 1, rb = 64 * hd2 * 8;  // bytes of 64 RoPE rows
      const int r0 = m0 + pass * 64;
      const i32x4_t rr = rsrc_words(g.rope_cs, (uint32_t)((size_t)g.M * hd2 * 8));
      for (int i = wave; i < rb / 1024; i += DG_NT / 64)
        dma16(rr, s_rope + i * 1024, (uint32_t)lane * 16u, (uint32_t)((size_t)r0 * hd2 * 8 + i * 1024));
      if (threadIdx.x < 64) s_slot[threadIdx.x] = g.slot[min(r0 + (int)threadIdx.x, g.M - 1)];
      const bool stage_scale = g.kv_e4m3 && g.nkv <= 128;
      if (stage_scale && pass == 0)
        for (int i = threadIdx.x; i < 2 * g.nkv; i += DG_NT) s_scale[i] = g.kv_scale[i];
      __builtin_amdgcn_s_waitcnt(DG_WAIT(0));
      sg = QkvStaged{reinterpret_cast<const float2*>(s_rope), s_slot, stage_scale ? s_scale : nullptr};
    }
    __syncthreads();
    // EPI_RESID: all 16 of a thread's residual loads of the pass in one batch
    epilogue<EPI, BG_BN, DG_NT, EPI == EPI_QKV ? 2 : (EPI == EPI_RESID ? 16 : 8)>(g, sC, BG_LDC, m0 + pass * 64, 64,
                                                                                n_tile, sg);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Skinny variant for M <= 64 (decode): A is bf16 [M][K], at most 64 rows, and
// every weight byte is used by exactly one workgroup, so the kernel is a
// weight stream.  A workgroup of 8 waves computes a 64 x 128 output tile over
// its K range in 64-wide chunks; wave w owns output columns 16w .. 16w+15.
//  - Weights (tiled layout, see packed_index): per chunk a wave reads its
//    16-row panel's two contiguous KiB (the MFMA B operands of the chunk's
//    two k-halves) with streaming loads into a ring of SK_DEPTH chunks, so
//    several chunks are always in flight and each 64-row tile is read in
//    address order.
//  - Activations: staged in LDS a group of SK_DEPTH chunks (64 x 512) at a
//    time, double-buffered.  The next group's pieces are loaded into
//    registers at the start of a group and written to LDS at its end, so
//    there is one barrier per group and waiting for them never drains the
//    weight ring.
//  - All loads are raw buffer loads with wave-uniform descriptors: a masked
//    load uses an out-of-range offset and reads zeros (the hardware bounds
//    check), so the loop has no branches and the compiler waits for exactly
//    the chunk it consumes.
constexpr int SK_BN = 128, SK_NT = 512, SK_KC = 64, SK_DEPTH = 8, SK_LDC = SK_BN + 4;
constexpr int SK_GK = SK_KC * SK_DEPTH;          // K of one activation group (512)
constexpr int SK_LDX = SK_GK + 8;                // bf16 per LDS row (16-byte pad)
constexpr int SK_XP = 64 * SK_GK / 8 / SK_NT;    // 16-byte activation pieces per thread per group (8)
constexpr int SK_LDS = 2 * 64 * SK_LDX * 2 > 64 * SK_LDC * 4 ? 2 * 64 * SK_LDX * 2 : 64 * SK_LDC * 4;

// Four e4m3 codes (one 32-bit word) times a power-of-two scale -> four bf16,
// two per gfx950 scaled conversion instruction.  Exact: a code has at most 4
// significant bits, and with a power-of-two scale the product is a bf16
// value (checked on the GPU against the bit-level decode times 2^e for every
// code that is not NaN and every e in [-40, 20]).
__device__ __forceinline__ uint2 fp8x4_to_bf16(uint32_t w, float s) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, true)));
}

// W2 (FP8 gate/up only, no split-K): each wave owns two 16-row panels, so a
// tile holds up to 128 gate + 128 up columns and every activation fragment
// read from LDS feeds both.
constexpr int SK_LDC_W = 2 * SK_BN + 4;
static_assert(64 * SK_LDC_W * 4 <= SK_LDS, "the wide output tile fits in the activation buffers");
template <int EPI, int WPOL, bool F8, bool W2 = false>
__global__ __launch_bounds__(SK_NT, 2) void gemm_skinny_kernel(GemmArgs g) {
  static_assert(!W2 || (F8 && EPI == EPI_SWIGLU), "two panels per wave: FP8 gate/up only");
  // activation groups (two buffers), later reused for the output tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[SK_LDS];
  uint16_t* sX = reinterpret_cast<uint16_t*>(smem);
  float* sC = reinterpret_cast<float*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), gq = lane >> 4, r16 = lane & 15;
  const int t = blockIdx.x, split = blockIdx.y;
  const int kb = g.splits > 1 ? split * g.k_split : 0;
  const int ke = g.splits > 1 ? min(g.K, kb + g.k_split) : g.K;
  const int nc = ke > kb ? (ke - kb + SK_KC - 1) / SK_KC : 0;

  // The wave's packed weight tensor and the element of this lane's piece in
  // half 0 of K chunk 0 (half 1 is 512 further): B row r16 of the wave's 16
  // output columns, k group gq.
  const int kc = (g.K + 63) / 64;
  const uint16_t* wt;
  const uint8_t* wt8;
  const float* st8;
  int wrows, wrow;  // rows of the wave's weight matrix; this lane's row in it
  uint32_t wbase, wbase8;
  bool wok = true;
  if (EPI == EPI_SWIGLU) {
    // tile t: gated columns [t * cw, t * cw + cw), gate in waves 0-3, up in
    // waves 4-7, 16 columns per wave.  cw is a multiple of 8, so a wave's
    // columns may straddle two 16-row panels: each lane addresses its own row
    // (8 consecutive rows of a k group stay one 128-byte run).
    const int u = wave >= 4 ? 1 : 0;
    wt = g.w[u];
    wt8 = g.w8[u];
    st8 = g.s8[u];
    wrows = g.N;
    const int j = (wave & 3) * 16 + r16, c = t * g.cw + j;
    wok = j < g.cw && c < g.N;
    wrow = c;
    wbase = (uint32_t)(c >> 6) * (uint32_t)kc * 4096u + (uint32_t)((c >> 4) & 3) * 1024u + (uint32_t)gq * 128u +
            (uint32_t)(c & 15) * 8u;
  } else {
    const int n0 = t * SK_BN;  // whole tiles lie in one segment
    const int sg = n0 >= g.seg_n0[1] ? (n0 >= g.seg_n0[2] ? 2 : 1) : 0;
    wt = g.w[sg];
    wt8 = g.w8[sg];
    st8 = g.s8[sg];
    const int wblk = (n0 - g.seg_n0[sg]) / 64 + (wave >> 2);
    wrows = min(g.N, g.seg_n0[sg + 1]) - g.seg_n0[sg];
    wrow = wblk * 64 + (wave & 3) * 16 + r16;
    wbase = (uint32_t)wblk * (uint32_t)kc * 4096u + (uint32_t)(wave & 3) * 1024u + (uint32_t)lane * 8u;
  }
  // FP8: the same 4 KiB block of 64 x 64 codes, panel, and the lane of row
  // wrow (16 bytes: both k halves of its group)
  wbase8 = (uint32_t)(wrow >> 6) * (uint32_t)kc * 4096u + (uint32_t)((wrow >> 4) & 3) * 1024u +
           (uint32_t)(gq * 16 + (wrow & 15)) * 16u;
  const int kb8 = fp8_scale_blocks(g.K);
  const uint32_t srow8 = (uint32_t)(wrow >> 7) * (uint32_t)kb8;
  const __amdgpu_buffer_rsrc_t wrs = F8 ? make_rsrc(wt8, (uint32_t)packed_elems(wrows, g.K))
                                        : make_rsrc(wt, (uint32_t)(packed_elems(wrows, g.K) * 2));
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(F8 ? st8 : nullptr, F8 ? (uint32_t)(fp8_scale_blocks(wrows) * kb8 * 4) : 0u);
  // W2: this lane's rows in the wave's two panels (columns 32 (wave & 3) + 16 p + r16 of the tile's half)
  uint32_t wb2[2] = {0u, 0u}, sr2[2] = {0u, 0u};
  bool ok2[2] = {false, false};
  if constexpr (W2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int j = (wave & 3) * 32 + p * 16 + r16, c = t * g.cw + j;
      ok2[p] = j < g.cw && c < g.N;
      wb2[p] = (uint32_t)(c >> 6) * (uint32_t)kc * 4096u + (uint32_t)((c >> 4) & 3) * 1024u +
               (uint32_t)(gq * 16 + (c & 15)) * 16u;
      sr2[p] = (uint32_t)(c >> 7) * (uint32_t)kb8;
    }
  }
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(g.a, (uint32_t)((size_t)g.M * g.lda * 2));
  const int c0 = kb / SK_KC;
  // this thread's activation pieces of a group: rows xr0 + 8i, columns xk .. xk + 7
  const int xr0 = tid / (SK_GK / 8), xk = (tid % (SK_GK / 8)) * 8;

  // bf16: the two k halves of the chunk as loaded; FP8: w0 holds the 16 codes
  // and s the block's scale (converted to bf16 when the chunk is consumed)
  struct WSlot {
    uint4 w0, w1;
    float s, s1;
  };
  auto load_w = [&](WSlot& sl, int j) {
    // chunks past nc (this split's end) read zeros; a chunk's padding past K is stored as zeros
    if constexpr (W2) {
      const uint32_t kk = (uint32_t)(c0 + j);
      sl.w0 = bload16<WPOL>(wrs, j < nc && ok2[0] ? wb2[0] + kk * 4096u : OOB);
      sl.w1 = bload16<WPOL>(wrs, j < nc && ok2[1] ? wb2[1] + kk * 4096u : OOB);
      sl.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           srs, j < nc && ok2[0] ? (sr2[0] + kk / 2u) * 4u : OOB, 0, 0));
      sl.s1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            srs, j < nc && ok2[1] ? (sr2[1] + kk / 2u) * 4u : OOB, 0, 0));
    } else if constexpr (F8) {
      const uint32_t e = wbase8 + (uint32_t)(c0 + j) * 4096u;
      sl.w0 = bload16<WPOL>(wrs, j < nc && wok ? e : OOB);
      sl.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           srs, j < nc && wok ? (srow8 + (uint32_t)(c0 + j) / 2u) * 4u : OOB, 0, 0));
    } else {
      const uint32_t e = wbase + (uint32_t)(c0 + j) * 4096u;
      sl.w0 = bload16<WPOL>(wrs, j < nc && wok ? e * 2u : OOB);
      sl.w1 = bload16<WPOL>(wrs, j < nc && wok ? (e + 512u) * 2u : OOB);
    }
  };
  auto load_x = [&](uint4 (&xv)[SK_XP], int gi) {
    const int kx = kb + gi * SK_GK + xk;
#pragma unroll
    for (int i = 0; i < SK_XP; ++i) {
      const int r = xr0 + 8 * i;
      xv[i] = bload16(xrs, r < g.M && kx < ke ? (uint32_t)(r * g.lda + kx) * 2u : OOB);
    }
  };
  auto store_x = [&](const uint4 (&xv)[SK_XP], int buf) {
    uint16_t* X = sX + buf * 64 * SK_LDX;
#pragma unroll
    for (int i = 0; i < SK_XP; ++i) *reinterpret_cast<uint4*>(&X[(xr0 + 8 * i) * SK_LDX + xk]) = xv[i];
  };

  f32x4 acc[4], acc2[4];  // acc2: the second panel (W2)
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = acc2[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nc > 0) {
    // Whole groups of SK_DEPTH chunks, with no branches inside a group:
    // chunks past nc load zeros (out-of-range offsets) and add nothing.
    // the first activation group is needed before any MFMA, so its loads
    // (L2 hits) go ahead of the weight stream's in the memory pipeline
    uint4 xv[SK_XP];
    load_x(xv, 0);
    WSlot ring[SK_DEPTH];
#pragma unroll
    for (int j = 0; j < SK_DEPTH; ++j) load_w(ring[j], j);
    store_x(xv, 0);
    const int ngroups = (nc + SK_DEPTH - 1) / SK_DEPTH;
    // a K range of at most two groups is staged whole, into both buffers, so
    // the loop needs no activation loads and no barriers
    const bool whole = ngroups <= 2;
    if (whole && ngroups == 2) {
      load_x(xv, 1);
      store_x(xv, 1);
    }
    lds_barrier();
    // The scheduling barriers pin the issue order: the next group's activation
    // loads first, then each chunk's refill right after the MFMAs that free its
    // ring slot.  Left alone, the compiler sinks all refills to the end of the
    // group, so the ring drains to empty once per group.
    for (int gi = 0; gi < ngroups; ++gi) {
      if (!whole) load_x(xv, gi + 1);  // the next group, in flight during this one
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* X = sX + (gi & 1) * 64 * SK_LDX;
#pragma unroll
      for (int j = 0; j < SK_DEPTH; ++j) {
        uint4 af[2][4];  // all eight A fragments in flight before the first MFMA
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            af[ks][a] = *reinterpret_cast<const uint4*>(&X[(a * 16 + r16) * SK_LDX + j * SK_KC + ks * 32 + gq * 8]);
        uint4 b0, b1;
        if constexpr (W2) {
          const uint4 c = ring[j].w1;  // second panel: converted and multiplied here
          const uint2 p0 = fp8x4_to_bf16(c.x, ring[j].s1), p1 = fp8x4_to_bf16(c.y, ring[j].s1);
          const uint2 p2 = fp8x4_to_bf16(c.z, ring[j].s1), p3 = fp8x4_to_bf16(c.w, ring[j].s1);
          const uint4 e0 = make_uint4(p0.x, p0.y, p1.x, p1.y), e1 = make_uint4(p2.x, p2.y, p3.x, p3.y);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int a = 0; a < 4; ++a) acc2[a] = mfma16(af[ks][a], ks ? e1 : e0, acc2[a]);
        }
        if constexpr (F8) {
          const uint4 c = ring[j].w0;
          const uint2 p0 = fp8x4_to_bf16(c.x, ring[j].s), p1 = fp8x4_to_bf16(c.y, ring[j].s);
          const uint2 p2 = fp8x4_to_bf16(c.z, ring[j].s), p3 = fp8x4_to_bf16(c.w, ring[j].s);
          b0 = make_uint4(p0.x, p0.y, p1.x, p1.y);
          b1 = make_uint4(p2.x, p2.y, p3.x, p3.y);
        } else {
          b0 = ring[j].w0;
          b1 = ring[j].w1;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[a] = mfma16(af[ks][a], ks ? b1 : b0, acc[a]);
        load_w(ring[j], (gi + 1) * SK_DEPTH + j);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!whole) {
        store_x(xv, (gi + 1) & 1);  // that buffer was last read in group gi - 1
        lds_barrier();
      }
    }
    if (whole) lds_barrier();  // every wave is done with the activations before sC reuses them
  }

  // the loop ended with a barrier: the activation buffers are free for sC
  if constexpr (W2) {
    // gate panels in columns 0..127, up panels in 128..255
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sC[(a * 16 + 4 * gq + i) * SK_LDC_W + wave * 32 + r16] = acc[a][i];
        sC[(a * 16 + 4 * gq + i) * SK_LDC_W + wave * 32 + 16 + r16] = acc2[a][i];
      }
    __syncthreads();
    epilogue<EPI, 2 * SK_BN, SK_NT>(g, sC, SK_LDC_W, 0, 64, t);
    return;
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) sC[(a * 16 + 4 * gq + i) * SK_LDC + wave * 16 + r16] = acc[a][i];
  __syncthreads();
  if (g.splits > 1) {
    const size_t ld = (size_t)gridDim.x * SK_BN;
    float* part = g.partial + (size_t)split * 64 * ld + (size_t)t * SK_BN;
    for (int idx = tid; idx < 64 * SK_BN / 4; idx += SK_NT) {
      const int row = idx / (SK_BN / 4), col = (idx % (SK_BN / 4)) * 4;
      *reinterpret_cast<float4*>(&part[(size_t)row * ld + col]) =
          *reinterpret_cast<const float4*>(&sC[row * SK_LDC + col]);
    }
    return;
  }
  epilogue<EPI, SK_BN, SK_NT>(g, sC, SK_LDC, 0, 64, t);
}

// Split-K reduce of the skinny kernel: one workgroup per 8 rows of a 64 x 128
// tile; each thread owns 4 consecutive columns of one row and issues the loads
// of every split before it adds them, in split order; then the epilogue on
// those rows.
constexpr int SK_RED_ROWS = 8;

// Loads the split-K partials of four consecutive columns: split z from byte
// offset off0 + z * zstride of the partial buffer r (which spans less than
// 2^31 bytes).  Splits past n, and every split of a lane whose ok is false,
// read zeros.  The loads carry no branch, so all of them are in flight
// before the first is used (per-lane conditional loads made the compiler
// wait on the first two before issuing the rest).
__device__ __forceinline__ void load_partials(__amdgpu_buffer_rsrc_t r, bool ok, uint32_t off0, uint32_t zstride,
                                              int n, float4 (&x)[SK_MAX_SPLITS]) {
#pragma unroll
  for (int z = 0; z < SK_MAX_SPLITS; ++z) {
    const uint32_t off = ok && z < n ? off0 + (uint32_t)z * zstride : OOB;
    x[z] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}

// Byte size of the split-K partial region of a skinny GEMM with n_tiles
// tiles (rows of 64, SK_BN columns per tile).
__host__ __device__ inline size_t skinny_partial_bytes(int splits, int n_tiles) {
  return (size_t)splits * 64 * n_tiles * SK_BN * 4;
}

template <int EPI>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(GemmArgs g, int n_tiles) {
  __shared__ __attribute__((aligned(16))) float sC[SK_RED_ROWS * SK_LDC];
  // EPI_QKV: the rows' RoPE table and KV slots, loaded with the partials
  __shared__ __attribute__((aligned(16))) float2 s_rope[EPI == EPI_QKV ? SK_RED_ROWS * 64 : 1];
  __shared__ int s_slot[SK_RED_ROWS];
  const int t = blockIdx.x, r0 = blockIdx.y * SK_RED_ROWS, tid = threadIdx.x;
  const int row = tid / (SK_BN / 4), col = (tid % (SK_BN / 4)) * 4;
  const uint32_t ld = (uint32_t)n_tiles * SK_BN;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(g.partial, (uint32_t)skinny_partial_bytes(g.splits, n_tiles));
  float4 x[SK_MAX_SPLITS];
  load_partials(pr, true, ((uint32_t)(r0 + row) * ld + (uint32_t)t * SK_BN + col) * 4, 64 * ld * 4, g.splits, x);
  float4 cs = make_float4(0.f, 0.f, 0.f, 0.f);
  int sl = 0;
  const int hd2 = g.hd / 2, rope_f4 = SK_RED_ROWS * hd2 / 2;
  if constexpr (EPI == EPI_QKV) {
    // rows past M take row M - 1's values, which no store uses
    if (tid < rope_f4) {
      const int m = min(r0 + tid / (hd2 / 2), g.M - 1);
      cs = reinterpret_cast<const float4*>(g.rope_cs)[(size_t)m * (hd2 / 2) + tid % (hd2 / 2)];
    }
    if (tid < SK_RED_ROWS) sl = g.slot[min(r0 + tid, g.M - 1)];
  }
  float4 v = x[0];
#pragma unroll
  for (int z = 1; z < SK_MAX_SPLITS; ++z) {
    v.x += x[z].x;
    v.y += x[z].y;
    v.z += x[z].z;
    v.w += x[z].w;
  }
  *reinterpret_cast<float4*>(&sC[row * SK_LDC + col]) = v;
  if constexpr (EPI == EPI_QKV) {
    if (tid < rope_f4) reinterpret_cast<float4*>(s_rope)[tid] = cs;
    if (tid < SK_RED_ROWS) s_slot[tid] = sl;
  }
  __syncthreads();
  if constexpr (EPI == EPI_QKV)
    epilogue<EPI, SK_BN, 256>(g, sC, SK_LDC, r0, SK_RED_ROWS, t, QkvStaged{s_rope, s_slot, nullptr});
  else
    epilogue<EPI, SK_BN, 256>(g, sC, SK_LDC, r0, SK_RED_ROWS, t);
}

// Split-K reduce of an EPI_RESID skinny GEMM fused with the RMSNorm that
// follows it: one workgroup per row holds the whole new row of y, four
// columns per thread, in registers.  It adds the partials in split order,
// writes y and the per-64-column sums of squares exactly as the EPI_RESID
// epilogue does (four squares per lane, then the 16 lanes of a 64-column
// chunk), sums those partials in column order as rmsnorm_kernel does, and
// writes the normed bf16 row.  N <= RN_NT * 4 * RN_MAXC.
constexpr int RN_NT = 1024, RN_MAXC = 2;
__global__ __launch_bounds__(RN_NT) void skinny_reduce_norm_kernel(GemmArgs g, int n_tiles) {
  __shared__ __attribute__((aligned(16))) float s_ssq[RN_NT * 4 * RN_MAXC / 64];
  __shared__ float s_r;
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int N = g.N, n_grp = N / 64;
  const uint32_t ld = (uint32_t)n_tiles * SK_BN;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(g.partial, (uint32_t)skinny_partial_bytes(g.splits, n_tiles));
  // y and the gain of this thread's columns, before the partials, from
  // addresses kept inside the row (columns past N are not used)
  float4 yo[RN_MAXC];
  uint2 gw[RN_MAXC];
#pragma unroll
  for (int c = 0; c < RN_MAXC; ++c) {
    const int col = (tid + c * RN_NT) * 4, cc = col < N ? col : 0;
    yo[c] = *reinterpret_cast<const float4*>(g.y_out + (size_t)m * g.ldy + cc);
    gw[c] = *reinterpret_cast<const uint2*>(g.next_gain + cc);
  }
  float4 yn[RN_MAXC];
#pragma unroll
  for (int c = 0; c < RN_MAXC; ++c) {
    yn[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c * RN_NT * 4 >= N) continue;  // uniform
    const int col = (tid + c * RN_NT) * 4;
    const bool ok = col < N;
    float4 x[SK_MAX_SPLITS];
    load_partials(pr, ok, ((uint32_t)m * ld + col) * 4, 64 * ld * 4, g.splits, x);
    float4 v = x[0];
#pragma unroll
    for (int z = 1; z < SK_MAX_SPLITS; ++z) {
      v.x += x[z].x;
      v.y += x[z].y;
      v.z += x[z].z;
      v.w += x[z].w;
    }
    yn[c] = make_float4(yo[c].x + v.x, yo[c].y + v.y, yo[c].z + v.z, yo[c].w + v.w);
    if (ok) *reinterpret_cast<float4*>(g.y_out + (size_t)m * g.ldy + col) = yn[c];
    float sq = yn[c].x * yn[c].x + yn[c].y * yn[c].y + yn[c].z * yn[c].z + yn[c].w * yn[c].w;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
    if (ok && (lane & 15) == 0) {
      g.ss_out[(size_t)m * g.n_ss + col / 64] = sq;
      s_ssq[col / 64] = sq;
    }
  }
  __syncthreads();
  if (tid == 0) {
    // column order, four LDS values per read
    float sum = 0.f;
    int c = 0;
#pragma unroll 4
    for (; c + 4 <= n_grp; c += 4) {
      const float4 q = *reinterpret_cast<const float4*>(&s_ssq[c]);
      sum += q.x;
      sum += q.y;
      sum += q.z;
      sum += q.w;
    }
    for (; c < n_grp; ++c) sum += s_ssq[c];
    s_r = 1.0f / sqrtf(sum / (float)N + g.eps);
  }
  __syncthreads();
  const float r = s_r;
#pragma unroll
  for (int c = 0; c < RN_MAXC; ++c) {
    const int col = (tid + c * RN_NT) * 4;
    if (col >= N) continue;
    const float4 a = yn[c];
    *reinterpret_cast<uint2*>(g.x_out + (size_t)m * g.N + col) =
        make_uint2(pack_bf2(a.x * r * bf2f(gw[c].x & 0xffffu), a.y * r * bf2f(gw[c].x >> 16)),
                   pack_bf2(a.z * r * bf2f(gw[c].y & 0xffffu), a.w * r * bf2f(gw[c].y >> 16)));
  }
}

// ---------------------------------------------------------------------------
// Decode QKV projection in one launch: narrow tiles, no split-K.  With
// split-K the projection needs a second kernel to sum the partials, apply
// RoPE and append k and v, and at decode sizes every launch costs a few
// microseconds of ramp and drain on top of its bytes.  Here a workgroup owns
// 32 output columns over the whole K range, chosen so that RoPE needs no
// other workgroup: for q and k, 16 columns of one head and their 16 rotation
// partners half a head further on; for v, 32 consecutive columns (at the
// Llama-3.1-8B shape: 160 + 32 = 192 workgroups).  Every workgroup reads all
// of A (64 rows x K bf16, from L2 after the first reader) besides its 32
// columns of weights.
//  - Eight waves; wave w takes the 64-wide K chunks w, w + 8, ... counted
//    from a per-workgroup starting chunk, and keeps a ring of NQ_DEPTH chunks
//    in registers.  A chunk is 8 loads of A, each 8 whole rows of 128 bytes
//    (lane l: row 8i + l / 8, bytes 16 (l & 7)), and 4 loads of weights (two
//    16-row panels x two 32-k halves, each one contiguous KiB of the tiled
//    layout, already in MFMA operand order).  A then goes through a private
//    8 KiB LDS slot of the wave (rows swizzled as in gemm_dma_kernel) into
//    MFMA fragments; loading the fragments straight from memory (16 rows x
//    64 bytes per load) measured 35% slower.
//  - The eight waves' partial tiles are summed in wave order through LDS;
//    then RoPE, the q stores and the k / v page-slot stores, as the split-K
//    reduce does them.
constexpr int NQ_WAVES = 8, NQ_NT = 64 * NQ_WAVES, NQ_DEPTH = 3;
constexpr int NQ_LDC = 36;  // fp32 per row of a wave's 64 x 32 partial tile (float4-aligned, padded)
constexpr int NQ_LDS = NQ_WAVES * 64 * NQ_LDC * 4 + NQ_WAVES * 8192;

__host__ __device__ inline int qkv_narrow_units(int qw, int kw) { return (qw + kw) / 32 + kw / 32; }

template <bool F8>
__global__ __launch_bounds__(NQ_NT, 1) void gemm_qkv_narrow_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NQ_LDS];
  const int lane = threadIdx.x & 63, wave = wave_id(), r16 = lane & 15, gq = lane >> 4;
  const int HD = g.hd, qw = g.nq * HD, kw = g.nkv * HD;
  const int n_rope = (qw + kw) / 32, u = blockIdx.x;
  const bool rope = u < n_rope;
  // the two 16-column panels of this workgroup (QKV output columns cA.., cB..)
  const int cA = rope ? (u / (HD / 32)) * HD + (u % (HD / 32)) * 16 : qw + kw + (u - n_rope) * 32;
  const int cB = rope ? cA + HD / 2 : cA + 16;
  const int sg = cA < qw ? 0 : (cA < qw + kw ? 1 : 2);
  const int kc = g.K / 64;
  uint32_t pb[2];  // element offset of each panel in K chunk 0 of the segment's packed matrix
  {
    const int a = cA - g.seg_n0[sg], b = cB - g.seg_n0[sg];
    pb[0] = (uint32_t)(a >> 6) * (uint32_t)kc * 4096u + (uint32_t)((a >> 4) & 3) * 1024u;
    pb[1] = (uint32_t)(b >> 6) * (uint32_t)kc * 4096u + (uint32_t)((b >> 4) & 3) * 1024u;
  }
  const int seg_rows = g.seg_n0[sg + 1] - g.seg_n0[sg];
  const __amdgpu_buffer_rsrc_t rw = F8 ? make_rsrc(g.w8[sg], (uint32_t)packed_elems(seg_rows, g.K))
                                       : make_rsrc(g.w[sg], (uint32_t)(packed_elems(seg_rows, g.K) * 2));
  // FP8: the panels' block scales, one per 128 rows x 128 k
  const int kb8 = fp8_scale_blocks(g.K);
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(F8 ? g.s8[sg] : nullptr, F8 ? (uint32_t)(fp8_scale_blocks(seg_rows) * kb8 * 4) : 0u);
  uint32_t srow[2];
  srow[0] = (uint32_t)((cA - g.seg_n0[sg]) >> 7) * (uint32_t)kb8;
  srow[1] = (uint32_t)((cB - g.seg_n0[sg]) >> 7) * (uint32_t)kb8;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, (uint32_t)((size_t)g.M * g.lda * 2));
  // Workgroups start at different K chunks: all of them read the same A, and
  // in step they would all queue on the few L2 channels that hold one chunk
  // (its 64 rows are a row stride apart).  Workgroups are dispatched to the
  // XCDs round robin, so the ones sharing an L2 (equal u mod 8) are spread
  // evenly over the chunks.
  const int per_xcd = (gridDim.x + 7) / 8;
  const int rot = (int)(((u >> 3) * kc) / per_xcd);
  // K chunk of this wave's iteration it (-1 past the end)
  auto chunk = [&](int it) {
    const int jr = wave + it * NQ_WAVES;
    return jr < kc ? (jr + rot < kc ? jr + rot : jr + rot - kc) : -1;
  };
  // A load i covers rows 8i .. 8i + 7; rows past M read row M - 1 (their
  // outputs are never stored)
  uint32_t a_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    a_off[i] = (uint32_t)(min(i * 8 + (lane >> 3), g.M - 1) * g.lda * 2) + (uint32_t)(lane & 7) * 16u;
  // bf16: b[ks][p] the panels' two k halves as loaded; FP8: b[0][p] holds
  // panel p's 16 codes (both halves) and s[p] its block scale, converted to
  // bf16 when the chunk is consumed (exactly: a code times its power-of-two
  // scale is a bf16 value), so both forms add the same products in the same
  // order
  struct Slot {
    uint4 a[8], b[2][2];
    float s[2];
  };
  // Past K every offset is out of range: the loads read zeros.
  auto load = [&](Slot& sl, int it) {
    const int j = chunk(it);
    const bool live = j >= 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) sl.a[i] = bload16(ra, live ? a_off[i] + (uint32_t)j * 128u : OOB);
    if constexpr (F8) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        sl.b[0][p] = bload16(rw, live ? pb[p] + (uint32_t)j * 4096u + (uint32_t)lane * 16u : OOB);
        sl.s[p] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, live ? (srow[p] + (uint32_t)j / 2u) * 4u : OOB, 0, 0));
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          sl.b[ks][p] =
              bload16(rw, live ? (pb[p] + (uint32_t)j * 4096u + (uint32_t)ks * 512u + (uint32_t)lane * 8u) * 2u : OOB);
    }
  };
  uint8_t* xs = smem + NQ_WAVES * 64 * NQ_LDC * 4 + wave * 8192;
  const int a_sw = dg_swz(r16);  // the swizzle depends on the row mod 16 only

  f32x4 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a][0] = acc[a][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Fully unrolled over the most chunks a wave can have (K <= 4096), so that
  // the compiler's waits are exact: in a rolled loop it waited for every
  // load in flight at the top of each pass.  Iterations past the wave's
  // last chunk load zeros and add nothing.
  constexpr int IT_MAX = 64 / NQ_WAVES;
  Slot ring[NQ_DEPTH];
#pragma unroll
  for (int d = 0; d < NQ_DEPTH; ++d) load(ring[d], d);
#pragma unroll
  for (int it = 0; it < IT_MAX; ++it) {
    Slot& sl = ring[it % NQ_DEPTH];
    // A through the wave's LDS slot into fragments (the wave's LDS accesses
    // complete in order, so the next chunk's writes never pass these reads)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 8 + (lane >> 3);
      *reinterpret_cast<uint4*>(xs + r * 128 + (((lane & 7) ^ dg_swz(r)) * 16)) = sl.a[i];
    }
    uint4 af[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        af[ks][a] = *reinterpret_cast<const uint4*>(xs + (a * 16 + r16) * 128 + (((ks * 4 + gq) ^ a_sw) * 16));
    uint4 bf[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if constexpr (F8) {
        const uint4 c = sl.b[0][p];
        const uint2 p0 = fp8x4_to_bf16(c.x, sl.s[p]), p1 = fp8x4_to_bf16(c.y, sl.s[p]);
        const uint2 p2 = fp8x4_to_bf16(c.z, sl.s[p]), p3 = fp8x4_to_bf16(c.w, sl.s[p]);
        bf[0][p] = make_uint4(p0.x, p0.y, p1.x, p1.y);
        bf[1][p] = make_uint4(p2.x, p2.y, p3.x, p3.y);
      } else {
        bf[0][p] = sl.b[0][p];
        bf[1][p] = sl.b[1][p];
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int p = 0; p < 2; ++p) acc[a][p] = mfma16(af[ks][a], bf[ks][p], acc[a][p]);
    if (it + NQ_DEPTH < IT_MAX) load(sl, it + NQ_DEPTH);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  float* sP = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) sP[(wave * 64 + a * 16 + 4 * gq + i) * NQ_LDC + p * 16 + r16] = acc[a][p][i];
  __syncthreads();
  // four consecutive columns of one row, summed over the waves in wave order
  auto col4 = [&](int row, int c) {
    float4 v = *reinterpret_cast<const float4*>(&sP[row * NQ_LDC + c]);
#pragma unroll
    for (int w = 1; w < NQ_WAVES; ++w) {
      const float4 x = *reinterpret_cast<const float4*>(&sP[(w * 64 + row) * NQ_LDC + c]);
      v.x += x.x;
      v.y += x.y;
      v.z += x.z;
      v.w += x.w;
    }
    return v;
  };
  const int tid = threadIdx.x;
  constexpr int P = KV_PAGE;
  if (rope) {
    // a unit is one row's 8 consecutive rotation pairs: columns cA + 8h ..
    // and their partners cB + 8h ..
    if (tid >= 128) return;
    const int row = tid >> 1, h = tid & 1, m = row;
    if (m >= g.M) return;
    const int d = cA % HD + 8 * h;  // rotation index (< HD / 2)
    const float4* cs4 = reinterpret_cast<const float4*>(reinterpret_cast<const float2*>(g.rope_cs) +
                                                        (size_t)m * (HD / 2) + d);
    float4 c4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c4[i] = cs4[i];  // (cos, sin) of pairs 2i, 2i + 1
    const float4 a0 = col4(row, 8 * h), a1 = col4(row, 8 * h + 4);
    const float4 b0 = col4(row, 16 + 8 * h), b1 = col4(row, 16 + 8 * h + 4);
    const float x1[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float x2[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    float o1[8], o2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = (i & 1) ? c4[i >> 1].z : c4[i >> 1].x, sn = (i & 1) ? c4[i >> 1].w : c4[i >> 1].y;
      o1[i] = x1[i] * c - x2[i] * sn;
      o2[i] = x2[i] * c + x1[i] * sn;
    }
    if (sg == 0) {
      uint16_t* q = g.q_out + (size_t)m * qw;
      *reinterpret_cast<uint4*>(q + cA + 8 * h) = make_uint4(pack_bf2(o1[0], o1[1]), pack_bf2(o1[2], o1[3]),
                                                             pack_bf2(o1[4], o1[5]), pack_bf2(o1[6], o1[7]));
      *reinterpret_cast<uint4*>(q + cB + 8 * h) = make_uint4(pack_bf2(o2[0], o2[1]), pack_bf2(o2[2], o2[3]),
                                                             pack_bf2(o2[4], o2[5]), pack_bf2(o2[6], o2[7]));
      return;
    }
    const int kh = (cA - qw) / HD, sl = g.slot[m];
    const size_t base = (size_t)(sl / P) * g.page_stride + (size_t)kh * P * HD + (size_t)(sl % P) * 8;
    const size_t i1 = base + (size_t)(d >> 3) * P * 8, i2 = base + (size_t)((d + HD / 2) >> 3) * P * 8;
    if (g.kv_e4m3) {
      const float sc = g.kv_scale[kh];
      uint32_t w1[2] = {0u, 0u}, w2[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w1[i >> 2] |= (uint32_t)f2e4m3(o1[i] / sc) << (8 * (i & 3));
        w2[i >> 2] |= (uint32_t)f2e4m3(o2[i] / sc) << (8 * (i & 3));
      }
      uint8_t* kv = reinterpret_cast<uint8_t*>(g.kv_layer);
      *reinterpret_cast<uint2*>(kv + i1) = make_uint2(w1[0], w1[1]);
      *reinterpret_cast<uint2*>(kv + i2) = make_uint2(w2[0], w2[1]);
    } else {
      uint16_t* kv = reinterpret_cast<uint16_t*>(g.kv_layer);
      *reinterpret_cast<uint4*>(kv + i1) = make_uint4(pack_bf2(o1[0], o1[1]), pack_bf2(o1[2], o1[3]),
                                                      pack_bf2(o1[4], o1[5]), pack_bf2(o1[6], o1[7]));
      *reinterpret_cast<uint4*>(kv + i2) = make_uint4(pack_bf2(o2[0], o2[1]), pack_bf2(o2[2], o2[3]),
                                                      pack_bf2(o2[4], o2[5]), pack_bf2(o2[6], o2[7]));
    }
    return;
  }
  // v, layout [kv head][HD][token] in a page: one element per row (the rows
  // of a decode step belong to different sequences)
  const int c = tid & 31, vc = cA - qw - kw + c, kvh = vc / HD, dd = vc % HD;
  const size_t col = (size_t)g.nkv * P * HD + (size_t)kvh * HD * P + (size_t)dd * P;
  const float sc = g.kv_e4m3 ? g.kv_scale[g.nkv + kvh] : 1.f;
  for (int row = tid >> 5; row < g.M; row += NQ_NT / 32) {
    float v = sP[row * NQ_LDC + c];
#pragma unroll
    for (int w = 1; w < NQ_WAVES; ++w) v += sP[(w * 64 + row) * NQ_LDC + c];
    const int sl = g.slot[row];
    const size_t idx = (size_t)(sl / P) * g.page_stride + col + (sl % P);
    if (g.kv_e4m3) reinterpret_cast<uint8_t*>(g.kv_layer)[idx] = f2e4m3(v / sc);
    else reinterpret_cast<uint16_t*>(g.kv_layer)[idx] = f2bf(v);
  }
}

// x[m, :] = bf16(y[m, :] * rsqrt(sum_sq[m] / d + eps) * gain), one workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ y, const float* __restrict__ ss,
                                                      int n_ss, const uint16_t* __restrict__ gain, int d,
                                                      float eps, const int32_t* __restrict__ rows,
                                                      uint16_t* __restrict__ x) {
  const int m = blockIdx.x;
  const int src = rows ? rows[m] : m;
  __shared__ float s_r, s_part[256];
  // the per-64-column sums go through LDS 256 at a time (one coalesced load
  // per thread), then thread 0 adds them in column order; from global memory
  // one at a time, every add waited for its own load
  float s = 0.f;
  for (int c0 = 0; c0 < n_ss; c0 += 256) {
    if (c0 + (int)threadIdx.x < n_ss) s_part[threadIdx.x] = ss[(size_t)src * n_ss + c0 + threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 0) {
      const int n = min(256, n_ss - c0);
#pragma unroll 8
      for (int c = 0; c < n; ++c) s += s_part[c];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) s_r = 1.0f / sqrtf(s / (float)d + eps);
  __syncthreads();
  const float r = s_r;
  for (int k = threadIdx.x * 8; k < d; k += 256 * 8) {
    const float4* p = reinterpret_cast<const float4*>(y + (size_t)src * d + k);
    float4 a = p[0], b = p[1];
    uint4 gw = *reinterpret_cast<const uint4*>(gain + k);
    uint4 o;
    o.x = pack_bf2(a.x * r * bf2f(gw.x & 0xffffu), a.y * r * bf2f(gw.x >> 16));
    o.y = pack_bf2(a.z * r * bf2f(gw.y & 0xffffu), a.w * r * bf2f(gw.y >> 16));
    o.z = pack_bf2(b.x * r * bf2f(gw.z & 0xffffu), b.y * r * bf2f(gw.z >> 16));
    o.w = pack_bf2(b.z * r * bf2f(gw.w & 0xffffu), b.w * r * bf2f(gw.w >> 16));
    *reinterpret_cast<uint4*>(x + (size_t)m * d + k) = o;
  }
}

__global__ __launch_bounds__(64) void argmax_reduce_kernel(const float* tile_best, const int32_t* tile_idx,
                                                           int n_tiles, int M, int32_t* tokens) {
  const int m = blockIdx.x, lane = threadIdx.x;
  float best = -INFINITY;
  int bi = INT_MAX;
  for (int t = lane; t < n_tiles; t += 64) {
    float s = tile_best[(size_t)m * n_tiles + t];
    int i = tile_idx[(size_t)m * n_tiles + t];
    if (s > best || (s == best && i < bi)) { best = s; bi = i; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ob = __shfl_xor(best, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  if (lane == 0) tokens[m] = bi == INT_MAX ? -1 : bi;
}

int gemm_tile_bm(int tile) { return tile == TILE_64x128 ? 64 : (tile >= TILE_256x256 ? 256 : 128); }
int gemm_tile_bn(int tile) { return tile >= TILE_256x256 ? 256 : 128; }

int gemm_n_tiles(int epi, int N, int tile) {
  if (epi == EPI_SWIGLU && tile == TILE_SKINNY) {
    const int cw = skinny_swiglu_cols(N);
    return (N + cw - 1) / cw;
  }
  const int bn = gemm_tile_bn(tile);
  return epi == EPI_SWIGLU ? (N + bn / 2 - 1) / (bn / 2) : (N + bn - 1) / bn;
}

template <int EPI, bool DMA>
static void launch_big(const GemmArgs& g, hipStream_t st) {
  const int tiles = ((g.M + BG_BM - 1) / BG_BM) * gemm_n_tiles(EPI, g.N, TILE_256x256);
  if (DMA) hipLaunchKernelGGL((gemm_dma_kernel<EPI>), dim3(tiles), dim3(DG_NT), 0, st, g);
  else hipLaunchKernelGGL((gemm_big_kernel<EPI>), dim3(tiles), dim3(BG_NT), 0, st, g);
}

// Large tiles (prefill-sized M) never split K: there are enough output tiles.
template <int BM, int BN, int AMODE, int EPI>
static void launch_t(const GemmArgs& g0, hipStream_t st) {
  GemmArgs g = g0;
  g.splits = 1;
  g.k_split = g.K;
  const int n_tiles = EPI == EPI_SWIGLU ? (g.N + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
  dim3 grid(n_tiles * ((g.M + BM - 1) / BM), 1, 1);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AMODE, EPI>), grid, dim3(256), 0, st, g);
}

// Weights stream with non-temporal loads, except the QKV projection's: at its
// size (50 MB at the 8B shape) plain loads measured slightly faster.
// The narrow QKV kernel replaces split-K + reduce when every workgroup's
// copy of A stays small (at most 64 x 4096 bf16) and its grid fits one round
// of the 256 compute units.
static bool qkv_narrow_fits(const GemmArgs& g) {
  const int qw = g.nq * g.hd, kw = g.nkv * g.hd;
  return g.M >= 1 && g.M <= 64 && g.K % 64 == 0 && g.K <= 4096 && (g.hd == 64 || g.hd == 128) &&
         g.page_size == KV_PAGE && g.lda % 8 == 0 && ((uintptr_t)g.a & 15) == 0 &&
         (size_t)g.M * g.lda * 2 < ((size_t)1 << 32) && qkv_narrow_units(qw, kw) <= 256;
}

template <int EPI>
static void launch_skinny(const GemmArgs& g0, hipStream_t st) {
  GemmArgs g = g0;
  if (EPI == EPI_QKV && qkv_narrow_fits(g)) {
    const dim3 grid(qkv_narrow_units(g.nq * g.hd, g.nkv * g.hd));
    if (g.f8) hipLaunchKernelGGL(gemm_qkv_narrow_kernel<true>, grid, dim3(NQ_NT), 0, st, g);
    else hipLaunchKernelGGL(gemm_qkv_narrow_kernel<false>, grid, dim3(NQ_NT), 0, st, g);
    return;
  }
  if (EPI == EPI_SWIGLU && g.f8 && g.splits <= 1 && skinny_swiglu_cols_wide(g.N) > 64) {
    g.cw = skinny_swiglu_cols_wide(g.N);
    const dim3 gw((g.N + g.cw - 1) / g.cw);
    hipLaunchKernelGGL((gemm_skinny_kernel<EPI_SWIGLU, CPOL_NT, true, true>), gw, dim3(SK_NT), 0, st, g);
    return;
  }
  if (EPI == EPI_SWIGLU) g.cw = skinny_swiglu_cols(g.N);
  const int n_tiles = gemm_n_tiles(EPI, g.N, TILE_SKINNY);
  const dim3 grid(n_tiles, g.splits > 1 ? g.splits : 1);
  if (g.f8) {
    if (EPI == EPI_QKV) hipLaunchKernelGGL((gemm_skinny_kernel<EPI, 0, true>), grid, dim3(SK_NT), 0, st, g);
    else hipLaunchKernelGGL((gemm_skinny_kernel<EPI, CPOL_NT, true>), grid, dim3(SK_NT), 0, st, g);
  } else {
    if (EPI == EPI_QKV) hipLaunchKernelGGL((gemm_skinny_kernel<EPI, 0, false>), grid, dim3(SK_NT), 0, st, g);
    else hipLaunchKernelGGL((gemm_skinny_kernel<EPI, CPOL_NT, false>), grid, dim3(SK_NT), 0, st, g);
  }
  const bool norm = EPI == EPI_RESID && g.x_out;
  const bool fused_norm = g.splits > 1 && norm && g.N <= RN_NT * 4 * RN_MAXC;
  if (fused_norm) {
    hipLaunchKernelGGL(skinny_reduce_norm_kernel, dim3(g.M), dim3(RN_NT), 0, st, g, n_tiles);
  } else if (g.splits > 1) {
    hipLaunchKernelGGL((skinny_reduce_kernel<EPI>), dim3(n_tiles, (g.M + SK_RED_ROWS - 1) / SK_RED_ROWS),
                       dim3(256), 0, st, g, n_tiles);
  }
  if (norm && !fused_norm)
    launch_rmsnorm(g.y_out, g.ss_out, g.n_ss, g.next_gain, g.M, g.N, g.eps, nullptr, g.x_out, st);
}

template <int BM, int BN>
static void launch_tile(int amode, int epi, const GemmArgs& g, hipStream_t st) {
  if (amode == A_NORM) {
    switch (epi) {
      case EPI_QKV: return launch_t<BM, BN, A_NORM, EPI_QKV>(g, st);
      case EPI_SWIGLU: return launch_t<BM, BN, A_NORM, EPI_SWIGLU>(g, st);
      case EPI_LOGITS: return launch_t<BM, BN, A_NORM, EPI_LOGITS>(g, st);
      default: return;
    }
  }
  switch (epi) {
    case EPI_QKV: return launch_t<BM, BN, A_BF16, EPI_QKV>(g, st);
    case EPI_SWIGLU: return launch_t<BM, BN, A_BF16, EPI_SWIGLU>(g, st);
    case EPI_RESID: return launch_t<BM, BN, A_BF16, EPI_RESID>(g, st);
    default: return;
  }
}

void launch_gemm(int amode, int epi, int tile, const GemmArgs& g, hipStream_t st) {
  if (tile == TILE_SKINNY) {
    switch (epi) {
      case EPI_QKV: return launch_skinny<EPI_QKV>(g, st);
      case EPI_RESID: return launch_skinny<EPI_RESID>(g, st);
      case EPI_SWIGLU: return launch_skinny<EPI_SWIGLU>(g, st);
      case EPI_LOGITS: return launch_skinny<EPI_LOGITS>(g, st);
    }
    return;
  }
  if (tile == TILE_256x256 || tile == TILE_256x256_STAGED) {
    if (amode != A_BF16) return;
    const bool dma = tile == TILE_256x256 && g.K % DG_BK == 0 && g.lda % 8 == 0 &&
                     ((uintptr_t)g.a & 15) == 0 && (size_t)g.M * g.lda * 2 < ((size_t)1 << 32);
    switch (epi) {
      case EPI_QKV: return dma ? launch_big<EPI_QKV, true>(g, st) : launch_big<EPI_QKV, false>(g, st);
      case EPI_RESID: return dma ? launch_big<EPI_RESID, true>(g, st) : launch_big<EPI_RESID, false>(g, st);
      case EPI_SWIGLU: return dma ? launch_big<EPI_SWIGLU, true>(g, st) : launch_big<EPI_SWIGLU, false>(g, st);
      default: return;
    }
  }
  if (tile == TILE_64x128) launch_tile<64, 128>(amode, epi, g, st);
  else launch_tile<128, 128>(amode, epi, g, st);
}

// One thread per 16-byte piece of the packed matrix (see packed_index).
__global__ void pack_weight_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int N, int K,
                                   size_t n_pieces) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_pieces) return;
  const int kc = (K + 63) / 64;
  const size_t blk = q >> 9;
  const int w = (int)(q & 511);
  const int n = (int)(blk / kc) * 64 + (w >> 7) * 16 + (w & 15);
  const int k = (int)(blk % kc) * 64 + ((w >> 6) & 1) * 32 + ((w >> 4) & 3) * 8;
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (n < N && k + e < K) ? src[(size_t)n * K + k + e] : (uint16_t)0;
  uint4 o;
  o.x = v[0] | ((uint32_t)v[1] << 16);
  o.y = v[2] | ((uint32_t)v[3] << 16);
  o.z = v[4] | ((uint32_t)v[5] << 16);
  o.w = v[6] | ((uint32_t)v[7] << 16);
  *reinterpret_cast<uint4*>(dst + q * 8) = o;
}

void launch_pack_weight(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t st) {
  const size_t pieces = packed_elems(N, K) / 8;
  if (pieces == 0) return;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st, src, dst, N, K,
                     pieces);
}

// One workgroup per 128 x 128 block: the block's largest finite |w|,
// its power-of-two scale 2^e -- e the least integer with max |w| <= 448 * 2^e,
// but at least FP8_MIN_EXP so that every code times the scale is a bf16 value
// -- then every code at its place in the FP8 tiled layout.  The codes are
// w * 2^-e rounded to e4m3 (exact scaling by ldexp, so no factor overflows);
// an infinite w saturates to +-448 and NaN keeps the NaN code.
constexpr int FP8_MIN_EXP = -124;
__global__ __launch_bounds__(256) void pack_weight_fp8_kernel(const uint16_t* __restrict__ src,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales, int N, int K) {
  __shared__ float s_max[4];
  const int bk = blockIdx.x, bn = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kc = (K + 63) / 64;
  float amax = 0.f;
  for (int i = tid; i < 128 * 128; i += 256) {
    const int n = bn * 128 + i / 128, k = bk * 128 + i % 128;
    const float v = n < N && k < K ? fabsf(bf2f(src[(size_t)n * K + k])) : 0.f;
    if (v < INFINITY) amax = fmaxf(amax, v);  // NaN and infinities left out
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  // least e with amax <= 448 * 2^e: amax / 448 = f * 2^x with 0.5 <= f < 1,
  // so amax <= 448 * 2^x and, unless f is exactly 0.5, not <= 448 * 2^(x-1).
  // 448 * 2^k is exact in float, or infinite past its range (which no
  // finite amax exceeds), so the comparisons are exact.
  int e = FP8_MIN_EXP;
  if (amax > 0.f) {
    int x;
    frexpf(amax / 448.f, &x);
    while (amax > ldexpf(448.f, x)) ++x;
    while (amax <= ldexpf(448.f, x - 1)) --x;
    e = max(x, FP8_MIN_EXP);
  }
  if (tid == 0) scales[(size_t)bn * ((K + 127) / 128) + bk] = ldexpf(1.f, e);
  for (int i = tid; i < 128 * 128; i += 256) {
    const int n = bn * 128 + i / 128, k = bk * 128 + i % 128;
    if (n < N && k < K) codes[packed_index_fp8(n, k, kc)] = f2e4m3(ldexpf(bf2f(src[(size_t)n * K + k]), -e));
  }
}

void launch_pack_weight_fp8(const uint16_t* src, uint8_t* codes, float* scales, int N, int K, hipStream_t st) {
  if (N <= 0 || K <= 0) return;
  hipLaunchKernelGGL(pack_weight_fp8_kernel, dim3(fp8_scale_blocks(K), fp8_scale_blocks(N)), dim3(256), 0, st, src,
                     codes, scales, N, K);
}

void launch_rmsnorm(const float* y, const float* ss, int n_ss, const uint16_t* gain, int M, int d,
                    float eps, const int32_t* rows, uint16_t* x, hipStream_t st) {
  if (M <= 0) return;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, st, y, ss, n_ss, gain, d, eps, rows, x);
}

void launch_argmax_reduce(const float* tile_best, const int32_t* tile_idx, int n_tiles, int M,
                          int32_t* tokens, hipStream_t st) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(M), dim3(64), 0, st, tile_best, tile_idx, n_tiles,
                     M, tokens);
}

}  // namespace pie
