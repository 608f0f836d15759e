// Small kernels of the path: the embedding gather (ops.gather.embed, "Write a
// model in Poem", section 5 Forward pass), the RoPE angle table, a fill kernel
// and the Philox debug view.
#include "common.h"
#include "misc.h"

namespace pie {

// y[t, :] = float(E[tok[t], :]); ss[t, c] = sum of y[t, 64c : 64c + 64]^2.
// One workgroup (4 waves) per row; each wave takes 64-column chunks.  Token
// ids that only exist on the device (loop-carried decode) are not validated
// by the host: an id outside [0, vocab) embeds as a zero row instead of
// reading outside the table.
__global__ __launch_bounds__(256) void embed_kernel(const uint16_t* __restrict__ E,
                                                    const int32_t* __restrict__ tok, int d, int vocab,
                                                    float* __restrict__ y, float* __restrict__ ss,
                                                    int n_ss) {
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int id = tok[t];
  float* dst = y + (size_t)t * d;
  if (id < 0 || id >= vocab) {  // whole workgroup: a zero row
    for (int c = wave; c < n_ss; c += 4) {
      dst[c * 64 + lane] = 0.f;
      if (lane == 0) ss[(size_t)t * n_ss + c] = 0.f;
    }
    return;
  }
  const uint16_t* src = E + (size_t)id * d;
  // the loads of U chunks go out before the first is used (a chunk at a
  // time made every chunk a full memory round trip)
  constexpr int U = 8;
  for (int c0 = wave; c0 < n_ss; c0 += 4 * U) {
    float a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + 4 * u, n_ss - 1);  // past the row: a valid chunk, not used
      a[u] = bf2f(src[c * 64 + lane]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
      if (c >= n_ss) break;
      dst[c * 64 + lane] = a[u];
      const float s = wave_sum(a[u] * a[u]);
      if (lane == 0) ss[(size_t)t * n_ss + c] = s;
    }
  }
}

// cs[t, j] = (cos, sin)(pos[t] * theta^(-2j/hd)), angles in double precision.
__global__ void rope_table_kernel(const int32_t* __restrict__ pos, int n_rows, int hd2, double theta,
                                  float* __restrict__ cs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows * hd2) return;
  const int t = i / hd2, j = i % hd2;
  const double w = pow(theta, -2.0 * (double)j / (double)(2 * hd2));
  double s, c;
  sincos((double)pos[t] * w, &s, &c);
  cs[2 * (size_t)i] = (float)c;
  cs[2 * (size_t)i + 1] = (float)s;
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void philox_kernel(uint32_t seed_lo, uint32_t seed_hi, uint32_t lane, uint32_t v0, int n,
                              uint32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = philox_w0(v0 + (uint32_t)i, lane, seed_lo, seed_hi);
}

void launch_embed(const uint16_t* E, const int32_t* tok, int n_rows, int d, int vocab, float* y, float* ss,
                  hipStream_t st) {
  if (n_rows <= 0) return;
  hipLaunchKernelGGL(embed_kernel, dim3(n_rows), dim3(256), 0, st, E, tok, d, vocab, y, ss, d / 64);
}

void launch_rope_table(const int32_t* pos, int n_rows, int hd, double theta, float* cs,
                       hipStream_t st) {
  const int n = n_rows * (hd / 2);
  if (n <= 0) return;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, pos, n_rows, hd / 2,
                     theta, cs);
}

void launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
}

void launch_philox(uint64_t seed, uint32_t lane, uint32_t v0, int n, uint32_t* out, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(philox_kernel, dim3((n + 255) / 256), dim3(256), 0, st, (uint32_t)seed,
                     (uint32_t)(seed >> 32), lane, v0, n, out);
}

}  // namespace pie
