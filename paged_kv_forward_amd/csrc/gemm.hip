// MFMA GEMM with fused RMSNorm prologue, split-K and the decoder's epilogues.
// See gemm.h for the operation.  Tiles are staged through LDS with double
// buffering; each of the 4 waves of a workgroup owns a WM x WN block of the
// BM x BN tile and issues 16x16x32 bf16 MFMAs.  With split-K, every split
// writes its fp32 partial tile, and the last split to finish (counted with a
// device-scope atomic) sums all partials in split order -- so the result does
// not depend on which split finishes last -- and runs the epilogue.
#include <climits>

#include "common.h"
#include "gemm.h"

namespace pie {

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

template <int BM, int BN, int AMODE, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  using C = Cfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  __shared__ float s_rstd[BM];
  __shared__ int s_rows[BM];
  __shared__ int s_last;

  uint16_t* sA = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sB = sA + 2 * BM * LDK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int n_tile = blockIdx.x, m_tile = blockIdx.y, split = blockIdx.z;
  const int m0 = m_tile * BM;
  const int kb = g.splits > 1 ? split * g.k_split : 0;
  const int ke = g.splits > 1 ? min(g.K, kb + g.k_split) : g.K;

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

  // Row pointers of this thread's W chunks (nullptr = zero row).
  const uint16_t* wrow[C::B_CH];
#pragma unroll
  for (int i = 0; i < C::B_CH; ++i) {
    int r = (tid + 256 * i) >> 3;
    const uint16_t* p = nullptr;
    if (EPI == EPI_SWIGLU) {
      int j = n_tile * (BN / 2) + (r % (BN / 2));
      if (j < g.N) p = (r < BN / 2 ? g.w[0] : g.w[1]) + (size_t)j * g.K;
    } else {
      int n = n_tile * BN + r;
      if (n < g.N) {
        int s = n >= g.seg_n0[1] ? (n >= g.seg_n0[2] ? 2 : 1) : 0;
        p = g.w[s] + (size_t)(n - g.seg_n0[s]) * g.K;
      }
    }
    wrow[i] = p;
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
    for (int i = 0; i < C::B_CH; ++i) {
      int c = tid + 256 * i, k = k0 + (c & 7) * 8;
      rb[i] = (wrow[i] && k < ke) ? *reinterpret_cast<const uint4*>(wrow[i] + k)
                                  : make_uint4(0, 0, 0, 0);
    }
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
      int c = tid + 256 * i, row = c >> 3, kk = (c & 7) * 8;
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
      __syncthreads();
    }
  }

  // ---- split-K: publish the partial; the last split sums them in order ----
  if (g.splits > 1) {
    const int tile_id = m_tile * gridDim.x + n_tile;
    constexpr int PER = C::FM * C::FN * 4;
    float* part = g.partial + (size_t)tile_id * g.splits * (BM * BN);
    float* mine = part + (size_t)split * (BM * BN);
#pragma unroll
    for (int a = 0; a < C::FM; ++a)
#pragma unroll
      for (int b = 0; b < C::FN; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[((a * C::FN + b) * 4 + i) * 256 + tid] = acc[a][b][i];
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&g.counters[tile_id], 1) == g.splits - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int a = 0; a < C::FM; ++a)
#pragma unroll
      for (int b = 0; b < C::FN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < g.splits; ++z) {
      const float* pz = part + (size_t)z * (BM * BN);
#pragma unroll
      for (int a = 0; a < C::FM; ++a)
#pragma unroll
        for (int b = 0; b < C::FN; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[a][b][i] += __builtin_nontemporal_load(pz + ((a * C::FN + b) * 4 + i) * 256 + tid);
    }
    (void)PER;
    if (tid == 0) g.counters[tile_id] = 0;
  }

  // ---- stage the fp32 tile in LDS ----
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

  if constexpr (EPI == EPI_RESID) {
    const int n0 = n_tile * BN;
    constexpr int CH = BN / 128;
    for (int p = wave; p < BM * CH; p += 4) {
      int row = p / CH, ch = p % CH, m = m0 + row;
      if (m >= g.M) continue;
      float s = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int col = ch * 128 + lane + 64 * h;
        size_t off = (size_t)m * g.ldy + n0 + col;
        float v = g.y_out[off] + sC[row * C::LDC + col];
        g.y_out[off] = v;
        s += v * v;
      }
      s = wave_sum(s);
      if (lane == 0) g.ss_out[(size_t)m * g.n_ss + n0 / 128 + ch] = s;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    constexpr int HALF = BN / 2;
    const int j0 = n_tile * HALF;
    for (int idx = tid; idx < BM * HALF; idx += 256) {
      int row = idx / HALF, j = idx % HALF, m = m0 + row, n = j0 + j;
      if (m < g.M && n < g.N) {
        float gt = sC[row * C::LDC + j], up = sC[row * C::LDC + HALF + j];
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
      for (int idx = tid; idx < BM * (BN / 2); idx += 256) {
        int row = idx / (BN / 2), pr = idx % (BN / 2), m = m0 + row;
        if (m >= g.M) continue;
        int hl = pr / hd2, dd = pr % hd2;
        int c1 = hl * hd + dd, c2 = c1 + hd2;
        float cs = g.rope_cs[((size_t)m * hd2 + dd) * 2], sn = g.rope_cs[((size_t)m * hd2 + dd) * 2 + 1];
        float x1 = sC[row * C::LDC + c1], x2 = sC[row * C::LDC + c2];
        float o1 = x1 * cs - x2 * sn, o2 = x2 * cs + x1 * sn;
        if (kind == 0) {
          int head = (n0 + c1) / hd;
          uint16_t* q = g.q_out + (size_t)m * qw + head * hd;
          q[dd] = f2bf(o1);
          q[dd + hd2] = f2bf(o2);
        } else {
          int kvh = (n0 - qw + c1) / hd;
          int sl = g.slot[m], page = sl / P, off = sl % P;
          size_t base = (size_t)page * g.page_stride + (size_t)kvh * P * hd + (size_t)off * hd;
          if (g.kv_e4m3) {
            float s = g.kv_scale[kvh];
            uint8_t* kv = reinterpret_cast<uint8_t*>(g.kv_layer);
            kv[base + dd] = f2e4m3(o1 / s);
            kv[base + dd + hd2] = f2e4m3(o2 / s);
          } else {
            uint16_t* kv = reinterpret_cast<uint16_t*>(g.kv_layer);
            kv[base + dd] = f2bf(o1);
            kv[base + dd + hd2] = f2bf(o2);
          }
        }
      }
    } else {
      for (int idx = tid; idx < BM * BN; idx += 256) {
        int row = idx / BN, c = idx % BN, m = m0 + row;
        if (m >= g.M) continue;
        int vc = n0 - qw - kw + c, kvh = vc / hd, dd = vc % hd;
        int sl = g.slot[m], page = sl / P, off = sl % P;
        size_t idx_v = (size_t)page * g.page_stride + (size_t)g.nkv * P * hd + (size_t)kvh * hd * P +
                       (size_t)dd * P + off;
        float x = sC[row * C::LDC + c];
        if (g.kv_e4m3) {
          reinterpret_cast<uint8_t*>(g.kv_layer)[idx_v] = f2e4m3(x / g.kv_scale[g.nkv + kvh]);
        } else {
          reinterpret_cast<uint16_t*>(g.kv_layer)[idx_v] = f2bf(x);
        }
      }
    }
  } else if constexpr (EPI == EPI_LOGITS) {
    const int n0 = n_tile * BN;
    for (int row = wave; row < BM; row += 4) {
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
        float l = sC[row * C::LDC + c];
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

int gemm_tile_bm(int tile) { return tile == TILE_64x128 ? 64 : 128; }
int gemm_tile_bn(int) { return 128; }

template <int BM, int BN, int AMODE, int EPI>
static void launch_t(const GemmArgs& g, hipStream_t st) {
  int n_tiles = EPI == EPI_SWIGLU ? (g.N + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
  dim3 grid(n_tiles, (g.M + BM - 1) / BM, g.splits > 1 ? g.splits : 1);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AMODE, EPI>), grid, dim3(256), 0, st, g);
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
  if (epi == EPI_RESID) return launch_t<BM, BN, A_BF16, EPI_RESID>(g, st);
}

void launch_gemm(int amode, int epi, int tile, const GemmArgs& g, hipStream_t st) {
  if (tile == TILE_64x128) launch_tile<64, 128>(amode, epi, g, st);
  else launch_tile<128, 128>(amode, epi, g, st);
}

void launch_argmax_reduce(const float* tile_best, const int32_t* tile_idx, int n_tiles, int M,
                          int32_t* tokens, hipStream_t st) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(M), dim3(64), 0, st, tile_best, tile_idx, n_tiles,
                     M, tokens);
}

}  // namespace pie
