// Kernel launchers (host side) used by the C ABI in ttq_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttq {

// Token-chunk split of the statistics reduction: returns the number of
// chunks (fp64 partial rows) and the rows per chunk.
int stats_chunks(int64_t T, int64_t K, int* rows_per_chunk);
// K-slice split of the low-rank Z = A X pass.
int lowrank_slices(int64_t T, int64_t K, int64_t* slice_len);

hipError_t launch_stats(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, double* ssq,
                        int accumulate, double* part, hipStream_t st);
hipError_t launch_awq_scales(const double* ssq, int64_t n_tokens, int64_t K, float alpha,
                             float lambda_rel, float* s, hipStream_t st);
hipError_t launch_quantize(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                           const float* s, int bits, int group, const float* B, const float* A,
                           int rank, uint32_t* codes, uint16_t* scale, uint16_t* zero,
                           hipStream_t st);
hipError_t launch_qgemm(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                        const float* s, const uint32_t* codes, const uint16_t* scale,
                        const uint16_t* zero, int64_t M, int bits, int group, void* Y, bool yf32,
                        int64_t ldy, hipStream_t st);
hipError_t launch_lowrank(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                          const float* A, const float* B, int64_t M, int rank, void* Y, bool yf32,
                          int64_t ldy, float* Zp, hipStream_t st);

}  // namespace ttq
