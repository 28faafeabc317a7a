// Shrunk AWQ scale arithmetic shared by the kernels that evaluate it, so that
// every path produces bitwise the same lambda and s.
//
// [TTQ §method b2-b4]: c[j] = ssq[j] / n (moment of order p of channel j over
// the prompt; p = 2: the second moment); lambda = lambda_rel * mean_j c[j]
// (shrinkage C + lambda I); s[j] = (c[j] + lambda)^(alpha / p), in fp64,
// rounded once to fp32, and 1 where c[j] + lambda == 0.
#pragma once

#include "common.hpp"

namespace ttq {

// Channel blocks of 16 for the shrinkage mean: at most 16384 (K <= 2^18).
constexpr int kBlockCh = 16;
constexpr int kMaxBlocks = (1 << 18) / kBlockCh;

// Wave-wide sum in a fixed butterfly order: every lane receives the same,
// run-to-run reproducible value.
__device__ __forceinline__ double wave_sum_fixed(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Sum over each aligned run of 16 lanes in a fixed butterfly (xor 8, 4, 2,
// 1): every lane of the run receives the same value.  All 64 lanes call it.
__device__ __forceinline__ double seg16_sum_fixed(double v) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Block sum of the second moments: block b covers channels 16 b .. 16 b + 15;
// lane l of a 16-lane run holds channel 16 b + l (missing channels count 0).
__device__ __forceinline__ double cblock_sum(const double* __restrict__ ssq, int64_t b, int64_t K,
                                             double tn, int l16) {
    const int64_t j = (int64_t)kBlockCh * b + l16;
    return seg16_sum_fixed(j < K ? ssq[j] / tn : 0.0);
}

// Total of the nb block sums in a fixed order (one full wave calls this): lane
// l adds blocks l, l + 64, ... in order, then the 64 lane totals are combined
// by wave_sum_fixed.  mean(c) = blocks_total / K.
__device__ __forceinline__ double blocks_total(const double* bs, int64_t nb, int lane) {
    double t = 0.0;
#pragma unroll 8
    for (int64_t i = lane; i < nb; i += 64) t += bs[i];
    return wave_sum_fixed(t);
}

// (c + lambda)^e in fp64, rounded once to fp32.  The exponents of the
// default settings, e = alpha / p = 1/4 (alpha 0.5, p 2) and 1/2, are
// evaluated by correctly rounded square roots (one-tenth of the cost of
// pow; the fp32 result equals the correctly rounded power except within
// ~1e-16 of an fp32 rounding boundary); other exponents by fp64 pow.
__device__ __forceinline__ float awq_scale(double ssq_j, double tn, double lam, double e) {
    const double cl = ssq_j / tn + lam;
    if (cl == 0.0) return 1.0f;
    if (e == 0.25) return (float)__builtin_sqrt(__builtin_sqrt(cl));
    if (e == 0.5) return (float)__builtin_sqrt(cl);
    return (float)pow(cl, e);
}

}  // namespace ttq
