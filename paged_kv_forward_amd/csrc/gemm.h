// Dense projections of the decoder (ops.linear.matmul / glu / lm_head on the
// "Poem ops" page) as one MFMA GEMM kernel with fused prologues and epilogues:
//   C[M, N] = A[M, K] * W[N, K]^T,  W in checkpoint layout [out][in], bf16.
// Prologue A_NORM computes the RMSNorm of the residual stream on the fly:
//   A[m, k] = bf16(y[m, k] * rsqrt(sum_sq[m] / K + eps) * gain[k]),
// with sum_sq[m] summed from per-64-column partials that the producer of y
// wrote; with a_rows it also gathers rows (the readout rows of the head).
// Epilogues:
//   EPI_QKV     RoPE on q and k, q -> bf16 buffer, k and v -> KV page slots
//   EPI_RESID   y += C, and the per-64-column sums of squares of the new y
//   EPI_SWIGLU  h = bf16(silu(gate) * up), gate/up tiles interleaved
//   EPI_LOGITS  logits (optional) and the per-tile maximum of the epilogue's
//               decision value (argmax, or logit/T + Gumbel noise)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pie {

enum { A_BF16 = 0, A_NORM = 1 };

// Tiled ("packed") layout of the projection and lm_head weights.  An [N][K]
// bf16 matrix is zero-padded to Np = N rounded up to 64 and Kp = K rounded up
// to 64 and stored as 8 KiB blocks, block (n / 64, k / 64) at index
// (n / 64) * (Kp / 64) + k / 64, each block laid out
//   [4 panels of 16 rows][2 halves of 32 k][4 groups of 8 k][16 rows][8 k].
// One MFMA B-operand load of a 16-row panel over 32 k (lane = group * 16 +
// row) is then one contiguous KiB, and a 64-row tile streams through memory
// in order as its K loop advances.
__host__ __device__ inline size_t packed_index(int n, int k, int kc) {
  const int r = n & 63, kk = k & 63;
  return ((size_t)(n >> 6) * kc + (k >> 6)) * 4096 + (size_t)(r >> 4) * 1024 + (size_t)(kk >> 5) * 512 +
         (size_t)((kk >> 3) & 3) * 128 + (size_t)(r & 15) * 8 + (kk & 7);
}
__host__ __device__ inline size_t packed_elems(int N, int K) { return (size_t)((N + 63) / 64) * 64 * (size_t)((K + 63) / 64) * 64; }

// dst (packed, packed_elems(N, K) bf16) <- src ([N][K] row-major bf16).
void launch_pack_weight(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t stream);

// Block-scaled FP8 copy of a projection for the decode GEMMs: OCP e4m3 codes
// with one power-of-two scale per 128 x 128 block, scale = 2^e with e the
// least integer for which the block's largest |w| is at most 448 * 2^e.  A
// code times its scale is exactly a bf16 value, so when every block of the
// bf16 matrix is already e4m3 times its scale the copy is lossless (else each
// value is rounded to the nearest e4m3 code, ties to even, saturating).
// Codes use the tiled layout with 1-byte elements: 4 KiB blocks of 64 x 64
// at the same block index as packed_index, each [4 panels of 16 rows][64
// lanes][16 bytes], lane = group * 16 + row of a 16-row panel, its 16 bytes
// = the 8 k of that group in the block's first 32 columns, then the 8 in the
// last 32: one 16-byte load is a lane's MFMA B operands of a 64-wide chunk.
__host__ __device__ inline size_t packed_index_fp8(int n, int k, int kc) {
  const int r = n & 63, kk = k & 63;
  return ((size_t)(n >> 6) * kc + (k >> 6)) * 4096 + (size_t)(r >> 4) * 1024 +
         (size_t)(((kk & 31) >> 3) * 16 + (r & 15)) * 16 + (size_t)(kk >> 5) * 8 + (kk & 7);
}
__host__ __device__ inline int fp8_scale_blocks(int n) { return (n + 127) / 128; }
// codes (packed_elems(N, K) bytes, zero-initialised by the caller),
// scales ([ceil(N/128)][ceil(K/128)] fp32) <- src ([N][K] row-major bf16).
void launch_pack_weight_fp8(const uint16_t* src, uint8_t* codes, float* scales, int N, int K, hipStream_t stream);
enum { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

struct GemmArgs {
  int M, N, K;  // N: output columns (EPI_SWIGLU: d_ffn, the gated width)
  // A operand
  const uint16_t* a;    // A_BF16: [M][lda] bf16
  int lda;
  const float* y;       // A_NORM: residual stream [rows][ldy] fp32
  int ldy;
  const float* ss;      // A_NORM: sum-of-squares partials [rows][n_ss]
  int n_ss;
  const uint16_t* gain; // A_NORM: [K] bf16
  const int32_t* a_rows;// A_NORM: optional row gather (A row m = y row a_rows[m])
  float eps;
  // W segments, each a packed [rows][K] matrix: output column n in
  // [seg_n0[s], seg_n0[s+1]) reads row n - seg_n0[s] of w[s]; segment sizes
  // are multiples of 64.  EPI_SWIGLU: w[0] = gate, w[1] = up, both [N][K].
  const uint16_t* w[3];
  int seg_n0[4];
  // TILE_SKINNY only: when f8 is set the weights stream as block-scaled FP8
  // (w8[s] codes in the FP8 tiled layout, s8[s] the [ceil(rows/128)][ceil(K/128)]
  // scales of segment s) instead of w[s]
  const uint8_t* w8[3];
  const float* s8[3];
  int f8;
  // split-K (splits > 1): K range of split z is [z*k_split, min(K, (z+1)*k_split));
  // split partials go to partial[split][BM][n_tiles * BN] and a reduce kernel
  // runs the epilogue (only with a single M tile).
  int splits, k_split;
  float* partial;
  // EPI_RESID
  float* y_out;     // [rows][ldy]
  float* ss_out;    // [rows][n_ss]
  // EPI_RESID with TILE_SKINNY only: when x_out is set, also the RMSNorm that
  // follows, x_out[m][:] = bf16(rmsnorm(y[m][:]) * next_gain) (N = d_model)
  const uint16_t* next_gain;
  uint16_t* x_out;
  // EPI_SWIGLU
  uint16_t* h_out;  // [M][N] bf16
  int cw;           // TILE_SKINNY: gate (and up) columns per tile, a multiple of 8 (0: BN / 2)
  // EPI_QKV
  uint16_t* q_out;  // [M][nq*hd] bf16
  const float* rope_cs;  // [M][hd/2][2] (cos, sin)
  const int32_t* slot;   // [M] page * page_size + offset
  void* kv_layer;        // base of this layer's pages
  long page_stride;      // elements per page per layer (2 * nkv * P * hd)
  int nq, nkv, hd, page_size, kv_e4m3;
  const float* kv_scale; // [2][nkv] for this layer (e4m3)
  // EPI_LOGITS
  float* logits;         // [M][N] or NULL
  const int32_t* ro_kind;
  const float* ro_temp;
  const uint32_t* ro_seed_lo;
  const uint32_t* ro_seed_hi;
  const int32_t* ro_lane;
  float* tile_best;      // [M][n_tiles] decision value (a row's tiles contiguous for the final reduce)
  int32_t* tile_idx;     // [M][n_tiles] its index
};

// Tile configurations.  TILE_SKINNY: M <= 64 with a bf16 A operand, 128 output
// columns per workgroup, weights streamed through registers (decode).
// TILE_256x256: prefill-sized M with a bf16 A operand and EPI_QKV, EPI_RESID
// or EPI_SWIGLU (for EPI_QKV the q and k/v widths must be multiples of 256);
// operands are loaded straight into LDS when K is a multiple of 32 and A rows
// are 16-byte aligned, else staged through registers.  TILE_256x256_STAGED
// always stages through registers (same results, bit for bit).
enum GemmTile { TILE_64x128 = 0, TILE_128x128 = 1, TILE_SKINNY = 2, TILE_256x256 = 3, TILE_256x256_STAGED = 4 };

// Gate/up columns per TILE_SKINNY EPI_SWIGLU tile: the gated width is cut into
// whole rounds of 256 tiles (one per compute unit of the MI355X) of at most 64
// columns each, in units of 8 columns, so every unit streams about the same
// number of weight bytes (d_ffn 14336: 256 tiles of 56).
inline int skinny_swiglu_cols(int N) {
  const int units = (N + 7) / 8, tiles = 256 * ((N + 64 * 256 - 1) / (64 * 256));
  return 8 * ((units + tiles - 1) / tiles);
}
// The same for the FP8 tiles whose waves own two 16-row panels (at most 128
// gate + 128 up columns): used when it gives more than 64 columns a tile
// (d_ffn 28672: 256 tiles of 112).
inline int skinny_swiglu_cols_wide(int N) {
  const int units = (N + 7) / 8, tiles = 256 * ((N + 128 * 256 - 1) / (128 * 256));
  return 8 * ((units + tiles - 1) / tiles);
}

// Most K splits of one skinny GEMM.
constexpr int SK_MAX_SPLITS = 16;

void launch_gemm(int amode, int epi, int tile, const GemmArgs& g, hipStream_t stream);

// x[m] = bf16(rmsnorm(y[rows ? rows[m] : m]) * gain) for M rows.
void launch_rmsnorm(const float* y, const float* ss, int n_ss, const uint16_t* gain, int M, int d,
                    float eps, const int32_t* rows, uint16_t* x, hipStream_t stream);

// Output tiles of a GEMM along N (EPI_SWIGLU tiles hold half gate, half up columns).
int gemm_n_tiles(int epi, int N, int tile);

// Reduce the per-tile maxima of EPI_LOGITS into one token per row.
void launch_argmax_reduce(const float* tile_best, const int32_t* tile_idx, int n_tiles, int M,
                          int32_t* tokens, hipStream_t stream);

int gemm_tile_bm(int tile);
int gemm_tile_bn(int tile);

}  // namespace pie
