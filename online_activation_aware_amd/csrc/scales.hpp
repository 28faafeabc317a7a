// Shrunk AWQ scale arithmetic shared by the kernels that evaluate it, so that
// every path produces bitwise the same lambda and s.
//
// [TTQ §method b2-b4]: c[j] = ssq[j] / n (second moment of channel j over the
// prompt); lambda = lambda_rel * mean_j c[j] (shrinkage C + lambda I);
// s[j] = (c[j] + lambda)^(alpha / 2), in fp64, rounded once to fp32, and 1
// where c[j] + lambda == 0.
#pragma once

#include "common.hpp"

namespace ttq {

// Channel blocks of 64 for the shrinkage mean: at most 4096 (K <= 2^18).
constexpr int kMaxBlocks = 4096;

// Wave-wide sum in a fixed butterfly order: every lane receives the same,
// run-to-run reproducible value.
__device__ __forceinline__ double wave_sum_fixed(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Channel-block sum of the second moments: block b covers channels
// 64 b .. 64 b + 63 (lane l <-> channel 64 b + l; missing channels count 0).
__device__ __forceinline__ double cblock_sum(const double* __restrict__ ssq, int64_t b, int64_t K,
                                             double tn, int lane) {
    const int64_t j = 64 * b + lane;
    return wave_sum_fixed(j < K ? ssq[j] / tn : 0.0);
}

// Total of the nb block sums in a fixed order (one full wave calls this): lane
// l adds blocks l, l + 64, ... in order, then the 64 lane totals are combined
// by wave_sum_fixed.  mean(c) = blocks_total / K.
__device__ __forceinline__ double blocks_total(const double* bs, int64_t nb, int lane) {
    double t = 0.0;
    for (int64_t i = lane; i < nb; i += 64) t += bs[i];
    return wave_sum_fixed(t);
}

__device__ __forceinline__ float awq_scale(double ssq_j, double tn, double lam, double e) {
    const double cl = ssq_j / tn + lam;
    return cl == 0.0 ? 1.0f : (float)pow(cl, e);
}

}  // namespace ttq
