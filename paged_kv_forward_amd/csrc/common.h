// Device helpers shared by the gfx950 kernels: number formats, the bf16 MFMA
// tile op, wave reductions and the Philox generator of the sampling epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pie {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of the raw buffer loads: non-temporal (streaming).
// Data read once per call (weights of the decode GEMMs, KV pages) bypasses
// the normal L2 retention; a plain streaming read measured ~7.0 TB/s with it
// against ~6.2 TB/s without.  It only pays when each load instruction covers
// whole 128-byte lines (the tiled weight layout, the K page layout): with
// half-line accesses it was slower than plain loads.
constexpr int CPOL_NT = 2;

// ---------------------------------------------------------------- formats

// float32 -> bf16 bits, round to nearest even (NaN stays NaN).  Written as a
// select, not a branch: it sits in the innermost loops.
__device__ __forceinline__ uint16_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return (uint16_t)((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
}

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 (a in the low half): one v_cvt_pk_bf16_f32, whose
// rounding (nearest even, NaN kept) matches f2bf bit for bit (checked on
// every class of input: ties, denormals, infinities, NaNs).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// OCP E4M3FN code of x, saturating: clamp to +-448, round to nearest even on
// the grid of 3 stored mantissa bits (binades 2^-6 .. 2^8; quantum 2^-9 below 2^-6).
__device__ __forceinline__ uint8_t f2e4m3(float x) {
  uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  if (!(x == x)) return (uint8_t)(sign | 0x7fu);  // NaN stays NaN (before the clamp, which would drop it)
  float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {               // below 2^-6: subnormal grid, quantum 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8 (8 = smallest normal)
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;  // -6 .. 8
    float m = __builtin_rintf(__builtin_ldexpf(a, 3 - e));   // 8 .. 16
    uint32_t mi = (uint32_t)m;
    if (mi == 16) { mi = 8; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | (mi - 8);
  }
  return (uint8_t)(sign | code);
}


// ---------------------------------------------------------------- MFMA

// D = A * B + C for one 16x16x32 bf16 tile (wave-wide).  Lane l holds, for
// A, row (l % 16) and 8 k-values of group (l / 16); for B, column (l % 16)
// and the same 8 k-values; D gives lane l column (l % 16), rows 4*(l/16)+i.
typedef float f32x16 __attribute__((ext_vector_type(16)));

// D[32x32] += A[32x16] * B[16x32], bf16 in, fp32 accumulate.  Lane l holds A
// row l % 32 and B column l % 32, k values 8 * (l / 32) .. + 7; D value i of
// lane l is row 8 * (i / 4) + 4 * (l / 32) + i % 4, column l % 32.
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- sync

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global
// memory, which makes the compiler wait for every outstanding global load
// (s_waitcnt vmcnt(0)) at each barrier and drains software prefetch rings.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Index of the calling wave in its workgroup, as a wave-uniform value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------- Philox

// Philox4x32-10 (Salmon et al., SC'11), word 0 only is returned: counter
// (c0, c1, 0, 0), key (k0, k1).
__device__ __forceinline__ uint32_t philox_w0(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
  uint32_t c2 = 0, c3 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}

// Gumbel noise of vocabulary entry v for (seed, lane): -ln(-ln u),
// u = ((x >> 9) + 0.5) * 2^-23, x = word 0 of Philox((v, lane, 0, 0), seed).
__device__ __forceinline__ float gumbel(uint32_t v, uint32_t lane, uint32_t seed_lo, uint32_t seed_hi) {
  uint32_t x = philox_w0(v, lane, seed_lo, seed_hi);
  float u = ((float)(x >> 9) + 0.5f) * 1.1920928955078125e-07f;  // 2^-23
  return -logf(-logf(u));
}

}  // namespace pie
