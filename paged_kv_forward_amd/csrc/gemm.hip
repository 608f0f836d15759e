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
// are in sC (row stride ldc).  Called by all 256 threads of a workgroup.
template <int EPI, int BN, int NTH = 256>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const float* sC, int ldc, int m0, int rows,
                                         int n_tile) {
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (EPI == EPI_RESID) {
    // y += C; per-64-column sums of squares of the new y for the next RMSNorm
    const int n0 = n_tile * BN;
    constexpr int CH = BN / 64;
    for (int p = wave; p < rows * CH; p += NW) {
      int row = p / CH, ch = p % CH, m = m0 + row;
      if (m >= g.M) continue;
      const int col = ch * 64 + lane;
      const size_t off = (size_t)m * g.ldy + n0 + col;
      const float v = g.y_out[off] + sC[row * ldc + col];
      g.y_out[off] = v;
      const float s = wave_sum(v * v);
      if (lane == 0) g.ss_out[(size_t)m * g.n_ss + n0 / 64 + ch] = s;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    constexpr int HALF = BN / 2;
    const int j0 = n_tile * HALF;
    for (int idx = tid; idx < rows * HALF; idx += NTH) {
      int row = idx / HALF, j = idx % HALF, m = m0 + row, n = j0 + j;
      if (m < g.M && n < g.N) {
        float gt = sC[row * ldc + j], up = sC[row * ldc + HALF + j];
        float h = gt / (1.0f + expf(-gt)) * up;
        g.h_out[(size_t)m * g.N + n] = f2bf(h);
      }
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int n0 = n_tile * BN;
    const int hd = g.hd, hd2 = hd >> 1, P = g.page_size;
    const int qw = g.nq * hd, kw = g.nkv * hd;
    const int kind = n0 < qw ? 0 : (n0 < qw + kw ? 1 : 2);
    if (kind < 2) {
      for (int idx = tid; idx < rows * (BN / 2); idx += NTH) {
        int row = idx / (BN / 2), pr = idx % (BN / 2), m = m0 + row;
        if (m >= g.M) continue;
        int hl = pr / hd2, dd = pr % hd2;
        int c1 = hl * hd + dd, c2 = c1 + hd2;
        float cs = g.rope_cs[((size_t)m * hd2 + dd) * 2], sn = g.rope_cs[((size_t)m * hd2 + dd) * 2 + 1];
        float x1 = sC[row * ldc + c1], x2 = sC[row * ldc + c2];
        float o1 = x1 * cs - x2 * sn, o2 = x2 * cs + x1 * sn;
        if (kind == 0) {
          int head = (n0 + c1) / hd;
          uint16_t* q = g.q_out + (size_t)m * qw + head * hd;
          q[dd] = f2bf(o1);
          q[dd + hd2] = f2bf(o2);
        } else {
          int kvh = (n0 - qw + c1) / hd;
          int sl = g.slot[m], page = sl / P, off = sl % P;
          // K page layout [kv head][hd / 8][token][8]
          size_t base = (size_t)page * g.page_stride + (size_t)kvh * P * hd + (size_t)off * 8;
          const size_t i1 = base + (size_t)(dd >> 3) * P * 8 + (dd & 7);
          const size_t i2 = base + (size_t)((dd + hd2) >> 3) * P * 8 + ((dd + hd2) & 7);
          if (g.kv_e4m3) {
            float s = g.kv_scale[kvh];
            uint8_t* kv = reinterpret_cast<uint8_t*>(g.kv_layer);
            kv[i1] = f2e4m3(o1 / s);
            kv[i2] = f2e4m3(o2 / s);
          } else {
            uint16_t* kv = reinterpret_cast<uint16_t*>(g.kv_layer);
            kv[i1] = f2bf(o1);
            kv[i2] = f2bf(o2);
          }
        }
      }
    } else {
      for (int idx = tid; idx < rows * BN; idx += NTH) {
        int row = idx / BN, c = idx % BN, m = m0 + row;
        if (m >= g.M) continue;
        int vc = n0 - qw - kw + c, kvh = vc / hd, dd = vc % hd;
        int sl = g.slot[m], page = sl / P, off = sl % P;
        size_t idx_v = (size_t)page * g.page_stride + (size_t)g.nkv * P * hd + (size_t)kvh * hd * P +
                       (size_t)dd * P + off;
        float x = sC[row * ldc + c];
        if (g.kv_e4m3) {
          reinterpret_cast<uint8_t*>(g.kv_layer)[idx_v] = f2e4m3(x / g.kv_scale[g.nkv + kvh]);
        } else {
          reinterpret_cast<uint16_t*>(g.kv_layer)[idx_v] = f2bf(x);
        }
      }
    }
  } else if constexpr (EPI == EPI_LOGITS) {
    const int n0 = n_tile * BN;
    for (int row = wave; row < rows; row += NW) {
      int m = m0 + row;
      if (m >= g.M) continue;
      const int kind = g.ro_kind[m];
      const float T = g.ro_temp[m];
      const uint32_t lo = g.ro_seed_lo[m], hi = g.ro_seed_hi[m], ln = (uint32_t)g.ro_lane[m];
      float best = -INFINITY;
      int bi = INT_MAX;
      for (int c = lane; c < BN; c += 64) {
        int v = n0 + c;
        if (v >= g.N) break;
        float l = sC[row * ldc + c];
        if (g.logits) g.logits[(size_t)m * g.N + v] = l;
        float s = kind == 0 ? l : l / T + gumbel((uint32_t)v, ln, lo, hi);
        if (s > best) { best = s; bi = v; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ob = __shfl_xor(best, o, 64);
        int oi = __shfl_xor(bi, o, 64);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (lane == 0) {
        g.tile_best[(size_t)n_tile * g.M + m] = best;
        g.tile_idx[(size_t)n_tile * g.M + m] = bi;
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

template <int EPI>
__global__ __launch_bounds__(BG_NT, 2) void gemm_big_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[BG_LDS];
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sB = sA + 2 * BG_BM * BG_LDK;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave >> 2, wn = wave & 3, l32 = lane & 31, lh = lane >> 5;

  // XCD-aware raster: workgroup i runs on XCD i % 8 (each XCD has its own
  // L2).  A window of 256 workgroups covers 16 x 16 tiles, and the 32 that
  // share an XCD form a 4 x 8 block of it, so each A tile is read by 8 and
  // each B tile by 4 workgroups of the same XCD.  Windows advance along M
  // first.  Workgroups of a partial window past the edge exit at once.
  int n_tile, m_tile;
  {
    const int n_tiles = big_tiles_n<EPI>(g), m_tiles = (g.M + BG_BM - 1) / BG_BM;
    const int m_win = (m_tiles + 15) / 16;
    const int pid = blockIdx.x, win = pid >> 8, x = pid & 7, j = (pid & 255) >> 3;
    m_tile = (win % m_win) * 16 + (x & 3) * 4 + (j & 3);
    n_tile = (win / m_win) * 16 + (x >> 2) * 8 + (j >> 2);
    if (m_tile >= m_tiles || n_tile >= n_tiles) return;
  }
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
    epilogue<EPI, BG_BN, BG_NT>(g, sC, BG_LDC, m0 + pass * 64, 64, n_tile);
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
constexpr uint32_t OOB = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int CPOL = 0>
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL));
}

template <int EPI>
__global__ __launch_bounds__(SK_NT, 2) void gemm_skinny_kernel(GemmArgs g) {
  // activation groups (two buffers), later reused for the output tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[SK_LDS];
  uint16_t* sX = reinterpret_cast<uint16_t*>(smem);
  float* sC = reinterpret_cast<float*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), gq = lane >> 4, r16 = lane & 15;
  const int t = blockIdx.x, split = blockIdx.y;
  const int kb = g.splits > 1 ? split * g.k_split : 0;
  const int ke = g.splits > 1 ? min(g.K, kb + g.k_split) : g.K;
  const int nc = ke > kb ? (ke - kb + SK_KC - 1) / SK_KC : 0;

  // The wave's packed weight tensor, its 64-row block and 16-row panel.
  const uint16_t* wt;
  int wblk, wrows;
  if (EPI == EPI_SWIGLU) {
    const bool up = wave >= 4;
    wt = up ? g.w[1] : g.w[0];
    wblk = t;
    wrows = g.N;
  } else {
    const int n0 = t * SK_BN;  // whole tiles lie in one segment
    const int sg = n0 >= g.seg_n0[1] ? (n0 >= g.seg_n0[2] ? 2 : 1) : 0;
    wt = g.w[sg];
    wblk = (n0 - g.seg_n0[sg]) / 64 + (wave >> 2);
    wrows = min(g.N, g.seg_n0[sg + 1]) - g.seg_n0[sg];
  }
  const int kc = (g.K + 63) / 64;
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wt, (uint32_t)(packed_elems(wrows, g.K) * 2));
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(g.a, (uint32_t)((size_t)g.M * g.lda * 2));
  // element of this lane's piece in half 0 of K chunk 0 (half 1 is 512 further)
  const uint32_t wbase = (uint32_t)wblk * (uint32_t)kc * 4096u + (uint32_t)(wave & 3) * 1024u + (uint32_t)lane * 8u;
  const int c0 = kb / SK_KC;
  // this thread's activation pieces of a group: rows xr0 + 8i, columns xk .. xk + 7
  const int xr0 = tid / (SK_GK / 8), xk = (tid % (SK_GK / 8)) * 8;

  struct WSlot {
    uint4 w0, w1;
  };
  auto load_w = [&](WSlot& sl, int j) {
    // chunks past nc (this split's end) read zeros; a chunk's padding past K is stored as zeros
    const uint32_t e = wbase + (uint32_t)(c0 + j) * 4096u;
    sl.w0 = bload16<CPOL_NT>(wrs, j < nc ? e * 2u : OOB);
    sl.w1 = bload16<CPOL_NT>(wrs, j < nc ? (e + 512u) * 2u : OOB);
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

  f32x4 acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nc > 0) {
    // Whole groups of SK_DEPTH chunks, with no branches inside a group:
    // chunks past nc load zeros (out-of-range offsets) and add nothing.
    WSlot ring[SK_DEPTH];
#pragma unroll
    for (int j = 0; j < SK_DEPTH; ++j) load_w(ring[j], j);
    uint4 xv[SK_XP];
    load_x(xv, 0);
    store_x(xv, 0);
    lds_barrier();
    const int ngroups = (nc + SK_DEPTH - 1) / SK_DEPTH;
    for (int gi = 0; gi < ngroups; ++gi) {
      load_x(xv, gi + 1);  // the next group, in flight during this one
      const uint16_t* X = sX + (gi & 1) * 64 * SK_LDX;
#pragma unroll
      for (int j = 0; j < SK_DEPTH; ++j) {
        uint4 af[2][4];  // all eight A fragments in flight before the first MFMA
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            af[ks][a] = *reinterpret_cast<const uint4*>(&X[(a * 16 + r16) * SK_LDX + j * SK_KC + ks * 32 + gq * 8]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[a] = mfma16(af[ks][a], ks ? ring[j].w1 : ring[j].w0, acc[a]);
        load_w(ring[j], (gi + 1) * SK_DEPTH + j);
      }
      store_x(xv, (gi + 1) & 1);  // that buffer was last read in group gi - 1
      lds_barrier();
    }
  }

  // the loop ended with a barrier: the activation buffers are free for sC
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
template <int EPI>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(GemmArgs g, int n_tiles) {
  __shared__ __attribute__((aligned(16))) float sC[SK_RED_ROWS * SK_LDC];
  const int t = blockIdx.x, r0 = blockIdx.y * SK_RED_ROWS;
  const int row = threadIdx.x / (SK_BN / 4), col = (threadIdx.x % (SK_BN / 4)) * 4;
  const size_t ld = (size_t)n_tiles * SK_BN, zs = 64 * ld;
  const float* base = g.partial + (size_t)(r0 + row) * ld + (size_t)t * SK_BN + col;
  float4 x[SK_MAX_SPLITS];
#pragma unroll
  for (int z = 0; z < SK_MAX_SPLITS; ++z)
    x[z] = z < g.splits ? *reinterpret_cast<const float4*>(base + z * zs) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 v = x[0];
#pragma unroll
  for (int z = 1; z < SK_MAX_SPLITS; ++z) {
    v.x += x[z].x;
    v.y += x[z].y;
    v.z += x[z].z;
    v.w += x[z].w;
  }
  *reinterpret_cast<float4*>(&sC[row * SK_LDC + col]) = v;
  __syncthreads();
  epilogue<EPI, SK_BN, 256>(g, sC, SK_LDC, r0, SK_RED_ROWS, t);
}

// Split-K reduce of an EPI_RESID skinny GEMM fused with the RMSNorm that
// follows it: one workgroup per row holds the whole new row of y.  It adds
// the partials in split order, writes y and the per-64-column sums of
// squares exactly as the EPI_RESID epilogue does, sums those partials in
// column order as rmsnorm_kernel does, and writes the normed bf16 row.
constexpr int RN_NT = 1024;
__global__ __launch_bounds__(RN_NT) void skinny_reduce_norm_kernel(GemmArgs g, int n_tiles) {
  extern __shared__ __attribute__((aligned(16))) float s_row[];  // [N] new y, then [N / 64] sums
  __shared__ float s_r;
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int N = g.N, n_grp = N / 64;
  float* s_ssq = s_row + N;
  const size_t ld = (size_t)n_tiles * SK_BN, zs = 64 * ld;
  for (int c = tid * 4; c < N; c += RN_NT * 4) {
    const float* p = g.partial + (size_t)m * ld + c;
    float4 x[SK_MAX_SPLITS];
#pragma unroll
    for (int z = 0; z < SK_MAX_SPLITS; ++z)
      x[z] = z < g.splits ? *reinterpret_cast<const float4*>(p + z * zs) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 v = x[0];
#pragma unroll
    for (int z = 1; z < SK_MAX_SPLITS; ++z) {
      v.x += x[z].x;
      v.y += x[z].y;
      v.z += x[z].z;
      v.w += x[z].w;
    }
    float4* yp = reinterpret_cast<float4*>(g.y_out + (size_t)m * g.ldy + c);
    const float4 yo = *yp;
    const float4 yn = make_float4(yo.x + v.x, yo.y + v.y, yo.z + v.z, yo.w + v.w);
    *yp = yn;
    *reinterpret_cast<float4*>(&s_row[c]) = yn;
  }
  __syncthreads();
  for (int grp = wave; grp < n_grp; grp += RN_NT / 64) {
    const float v = s_row[grp * 64 + lane];
    const float sq = wave_sum(v * v);
    if (lane == 0) {
      g.ss_out[(size_t)m * g.n_ss + grp] = sq;
      s_ssq[grp] = sq;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
    for (int c = 0; c < n_grp; ++c) sum += s_ssq[c];
    s_r = 1.0f / sqrtf(sum / (float)N + g.eps);
  }
  __syncthreads();
  const float r = s_r;
  for (int k = tid * 8; k < N; k += RN_NT * 8) {
    const float4 a = *reinterpret_cast<const float4*>(&s_row[k]);
    const float4 b = *reinterpret_cast<const float4*>(&s_row[k + 4]);
    const uint4 gw = *reinterpret_cast<const uint4*>(g.next_gain + k);
    uint4 o;
    o.x = pack_bf2(a.x * r * bf2f(gw.x & 0xffffu), a.y * r * bf2f(gw.x >> 16));
    o.y = pack_bf2(a.z * r * bf2f(gw.y & 0xffffu), a.w * r * bf2f(gw.y >> 16));
    o.z = pack_bf2(b.x * r * bf2f(gw.z & 0xffffu), b.y * r * bf2f(gw.z >> 16));
    o.w = pack_bf2(b.z * r * bf2f(gw.w & 0xffffu), b.w * r * bf2f(gw.w >> 16));
    *reinterpret_cast<uint4*>(g.x_out + (size_t)m * g.N + k) = o;
  }
}

// x[m, :] = bf16(y[m, :] * rsqrt(sum_sq[m] / d + eps) * gain), one workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ y, const float* __restrict__ ss,
                                                      int n_ss, const uint16_t* __restrict__ gain, int d,
                                                      float eps, const int32_t* __restrict__ rows,
                                                      uint16_t* __restrict__ x) {
  const int m = blockIdx.x;
  const int src = rows ? rows[m] : m;
  __shared__ float s_r;
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int c = 0; c < n_ss; ++c) s += ss[(size_t)src * n_ss + c];
    s_r = 1.0f / sqrtf(s / (float)d + eps);
  }
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
    float s = tile_best[(size_t)t * M + m];
    int i = tile_idx[(size_t)t * M + m];
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

int gemm_tile_bm(int tile) { return tile == TILE_64x128 ? 64 : (tile == TILE_256x256 ? 256 : 128); }
int gemm_tile_bn(int tile) { return tile == TILE_256x256 ? 256 : 128; }

int gemm_n_tiles(int epi, int N, int tile) {
  const int bn = gemm_tile_bn(tile);
  return epi == EPI_SWIGLU ? (N + bn / 2 - 1) / (bn / 2) : (N + bn - 1) / bn;
}

template <int EPI>
static void launch_big(const GemmArgs& g, hipStream_t st) {
  const int m_win = ((g.M + BG_BM - 1) / BG_BM + 15) / 16, n_win = (gemm_n_tiles(EPI, g.N, TILE_256x256) + 15) / 16;
  hipLaunchKernelGGL((gemm_big_kernel<EPI>), dim3(m_win * n_win * 256), dim3(BG_NT), 0, st, g);
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

template <int EPI>
static void launch_skinny(const GemmArgs& g, hipStream_t st) {
  const int n_tiles = gemm_n_tiles(EPI, g.N, TILE_SKINNY);
  hipLaunchKernelGGL((gemm_skinny_kernel<EPI>), dim3(n_tiles, g.splits > 1 ? g.splits : 1), dim3(SK_NT), 0,
                     st, g);
  const bool norm = EPI == EPI_RESID && g.x_out;
  if (g.splits > 1 && norm) {
    const size_t lds = ((size_t)g.N + g.N / 64) * 4;
    hipLaunchKernelGGL(skinny_reduce_norm_kernel, dim3(g.M), dim3(RN_NT), lds, st, g, n_tiles);
  } else if (g.splits > 1) {
    hipLaunchKernelGGL((skinny_reduce_kernel<EPI>), dim3(n_tiles, (g.M + SK_RED_ROWS - 1) / SK_RED_ROWS),
                       dim3(256), 0, st, g, n_tiles);
  }
  if (g.splits <= 1 && norm)
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
  if (tile == TILE_256x256) {
    if (amode != A_BF16) return;
    switch (epi) {
      case EPI_QKV: return launch_big<EPI_QKV>(g, st);
      case EPI_RESID: return launch_big<EPI_RESID>(g, st);
      case EPI_SWIGLU: return launch_big<EPI_SWIGLU>(g, st);
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
