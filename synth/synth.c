/*
 * Seeded synthetic inputs shared by the HIP path's harness and the oracle.
 *
 * This file holds no arithmetic of the forward pass: it only turns a 64-bit
 * key and an element index into numbers.  Every stream is counter based, so
 * element i of a tensor is the same however the tensor is split over threads
 * or chunks, and any slice can be regenerated on its own.
 *
 *   at(key, i)   = the (i+1)-th output of SplitMix64 seeded with key
 *                  (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *                  generators", OOPSLA 2014; the finaliser is Stafford's
 *                  "Mix13" variant used by SplitMix64).
 *   normal(2j), normal(2j+1) = the Box-Muller pair (Box and Muller, 1958) of
 *                  u1 = ((at(key,2j) >> 11) + 0.5) * 2^-53   in (0, 1)
 *                  u2 =  (at(key,2j+1) >> 11)       * 2^-53   in [0, 1)
 *                  computed in IEEE double with the C library's log, sqrt,
 *                  cos and sin.
 *   bf16 tensors: value = bf16_rne((float)(mean + std * normal(i))).
 *   integers in [lo, hi): lo + (((at(key,i) >> 32) * (hi - lo)) >> 32).
 *   uniform doubles in [0, 1): (at(key,i) >> 11) * 2^-53.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t j = i >> 1;
  double u1 = ((double)(at(key, 2 * j) >> 11) + 0.5) * 0x1p-53;
  double u2 = (double)(at(key, 2 * j + 1) >> 11) * 0x1p-53;
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* float32 -> bf16 bits, round to nearest even; NaN kept quiet. */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t synth_at(uint64_t key, uint64_t i) { return at(key, i); }

double synth_normal_at(uint64_t key, uint64_t i) { return normal_at(key, i); }

/* out[k] = bf16(mean + std * normal(first + k)) for k in [0, n). */
void synth_normal_bf16(uint16_t* out, int64_t n, uint64_t key, uint64_t first, double mean,
                       double stdv, int nthreads) {
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t k = 0; k < n; ++k) {
    double z = normal_at(key, first + (uint64_t)k);
    out[k] = f32_to_bf16((float)(mean + stdv * z));
  }
}

/* out[k] = lo + floor(u32(at(key, first+k) >> 32) * (hi - lo) / 2^32). */
void synth_uniform_int(int32_t* out, int64_t n, uint64_t key, uint64_t first, int32_t lo,
                       int32_t hi) {
  uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo);
  for (int64_t k = 0; k < n; ++k) {
    uint64_t x = at(key, first + (uint64_t)k) >> 32;
    out[k] = (int32_t)((int64_t)lo + (int64_t)((x * span) >> 32));
  }
}

/* out[k] = (at(key, first+k) >> 11) * 2^-53, uniform in [0, 1). */
void synth_uniform_f64(double* out, int64_t n, uint64_t key, uint64_t first) {
  for (int64_t k = 0; k < n; ++k) out[k] = (double)(at(key, first + (uint64_t)k) >> 11) * 0x1p-53;
}
