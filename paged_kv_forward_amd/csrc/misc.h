// Small kernels of the path; see misc.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pie {

void launch_embed(const uint16_t* E, const int32_t* tok, int n_rows, int d, int vocab, float* y, float* ss,
                  hipStream_t st);
void launch_rope_table(const int32_t* pos, int n_rows, int hd, double theta, float* cs,
                       hipStream_t st);
void launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t st);
void launch_philox(uint64_t seed, uint32_t lane, uint32_t v0, int n, uint32_t* out, hipStream_t st);

}  // namespace pie
