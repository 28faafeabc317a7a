// Activation statistics and AWQ scales (gfx950).
//
// [TTQ §method b2, b3] (TTQ review page, "proposed method", bullets 2-3):
// the per-channel diagonal of the input covariance, estimated online from the
// prompt, and the shrunk closed-form AWQ scale built from it.
//
// k_stats: one launch, no partial sums.  A workgroup (8 waves) owns a block
// of 16 channels over all T tokens: lane l reads 8 channels (one 16-byte
// load of bf16, two of fp32) of rows l/2, l/2 + 256, ..., all of its loads
// issued before the first is used, and accumulates squares (or |x|^p for a
// moment order p != 2 [TTQ §method b4]) in fp64.  Lanes holding the same
// channels are combined by a fixed xor butterfly, the 8 waves in wave order,
// so every result is bitwise reproducible run to run.  The workgroup also
// leaves the block's sum of c = ssq / n (16-lane fixed butterfly), from which
// the consumers form the shrinkage mean.
//
// The blocks that share one 128-byte line of a row (four 16-channel blocks of
// bf16, two of fp32) run on one XCD: workgroups are dispatched to the eight
// XCDs round-robin by id, so ids w, w + 8, w + 16, ... are mapped to the
// blocks of one line, and that XCD's L2 serves the line to all of them.
#include "common.hpp"
#include "launch.hpp"
#include "scales.hpp"

namespace ttq {

constexpr int kStatsThreads = 512;
constexpr int kStatsWaves = kStatsThreads / kWave;
constexpr int kStatsRowStep = kStatsThreads / 2;   // rows covered by one pass of the workgroup
constexpr int kXcds = 8;

// |x|^p added to acc in fp64: PM = 2 squares (exact products), PM = 1 absolute
// values, PM = 0 any other p (fp64 pow of |x|; 0 for x = 0).
template <int PM>
__device__ __forceinline__ double add_moment(double x, double p, double acc) {
    if constexpr (PM == 2) return __builtin_fma(x, x, acc);
    else if constexpr (PM == 1) return acc + __builtin_fabs(x);
    else return acc + (x == 0.0 ? 0.0 : pow(__builtin_fabs(x), p));
}

template <bool XF32, int PM>
__global__ __launch_bounds__(kStatsThreads) void k_stats(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, double* __restrict__ ssq, int accumulate,
    double tn, double* __restrict__ bsum, double pexp, int64_t nblk, int sub) {
    // Block of this workgroup: XCD x = w % 8 takes lines x, x + 8, ... and
    // their `sub` blocks in consecutive slots.
    const int64_t w = blockIdx.x;
    const int64_t j = w / kXcds;
    const int64_t blk = (w % kXcds + (int64_t)kXcds * (j / sub)) * sub + j % sub;
    if (blk >= nblk) return;                      // whole workgroup: no barrier reached
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t c0 = blk * kBlockCh + 8 * (lane & 1);
    const int64_t r0 = (lane >> 1) + (int64_t)(kWave / 2) * wave;

    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    if (c0 < K) {
        if constexpr (XF32) {
            const float* base = (const float*)X + c0;
#pragma unroll 4
            for (int64_t t = r0; t < T; t += kStatsRowStep) {
                const f32x4* p = (const f32x4*)(base + t * ldx);
                f32x4 a = ld_nc(p), b = ld_nc(p + 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[i] = add_moment<PM>((double)a[i], pexp, acc[i]);
                    acc[4 + i] = add_moment<PM>((double)b[i], pexp, acc[4 + i]);
                }
            }
        } else {
            const uint16_t* base = (const uint16_t*)X + c0;
#pragma unroll 8
            for (int64_t t = r0; t < T; t += kStatsRowStep) {
                u32x4 v = ld_nc((const u32x4*)(base + t * ldx));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = add_moment<PM>((double)bf16lo_to_f32(v[i]), pexp, acc[2 * i]);
                    acc[2 * i + 1] = add_moment<PM>((double)bf16hi_to_f32(v[i]), pexp, acc[2 * i + 1]);
                }
            }
        }
    }
    // the wave's 32 rows: lanes l and l ^ 2, ^ 4, ... ^ 32 hold the same channels
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int m = 2; m <= 32; m <<= 1) acc[i] += __shfl_xor(acc[i], m);
    __shared__ double red[kStatsWaves][kBlockCh];
    if (lane < 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][8 * lane + i] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
        const int64_t jc = blk * kBlockCh + lane;
        const bool ok = lane < kBlockCh && jc < K;
        double tot = 0.0;
        if (ok) {
            tot = red[0][lane];
#pragma unroll
            for (int v = 1; v < kStatsWaves; ++v) tot += red[v][lane];
            if (accumulate) tot = ssq[jc] + tot;
            ssq[jc] = tot;
        }
        if (bsum != nullptr) {
            const double bs = seg16_sum_fixed(ok ? tot / tn : 0.0);
            if (lane == 0) bsum[blk] = bs;
        }
    }
}

// Standalone scales from ssq: one workgroup of 1024 threads.  The 16 waves
// form the 16-channel block sums (cblock_sum, four blocks per wave at a time)
// into LDS, wave 0 totals them (blocks_total), then every thread evaluates the
// scales of its channels.
constexpr int kScaleThreads = 1024;

__global__ __launch_bounds__(kScaleThreads) void k_awq_scales(const double* __restrict__ ssq,
                                                              int64_t n_tokens, int64_t K,
                                                              double e, double lambda_rel,
                                                              float* __restrict__ s) {
    __shared__ double bs[kMaxBlocks];
    __shared__ double lam_s;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const double tn = (double)n_tokens;
    const int64_t nb = (K + kBlockCh - 1) / kBlockCh;
    constexpr int kPer = kWave / kBlockCh;        // blocks per wave step
    for (int64_t b0 = (int64_t)wave * kPer; b0 < nb; b0 += (int64_t)(kScaleThreads / kWave) * kPer) {
        const int64_t b = b0 + lane / kBlockCh;
        const double v = cblock_sum(ssq, b, K, tn, lane % kBlockCh);
        if (lane % kBlockCh == 0 && b < nb) bs[b] = v;
    }
    __syncthreads();
    if (wave == 0) {
        const double sum = blocks_total(bs, nb, lane);
        if (lane == 0) lam_s = lambda_rel * (sum / (double)K);
    }
    __syncthreads();
    const double lam = lam_s;
    for (int64_t j = threadIdx.x; j < K; j += kScaleThreads) s[j] = awq_scale(ssq[j], tn, lam, e);
}

// ------------------------------------------------------------------ host

template <bool XF32>
static hipError_t launch_stats_t(const void* X, int64_t T, int64_t K, int64_t ldx, double* ssq, int accumulate,
                                 double tn, double* bsum, double p, hipStream_t st, StageTimer tm) {
    const int64_t nblk = (K + kBlockCh - 1) / kBlockCh;
    const int sub = XF32 ? 2 : 4;                 // 16-channel blocks per 128-byte line
    const int64_t lines = (nblk + sub - 1) / sub;
    const dim3 g((unsigned)(((lines + kXcds - 1) / kXcds) * kXcds * sub));
    if (p == 2.0)
        return launch_kernel(k_stats<XF32, 2>, g, dim3(kStatsThreads), 0, st, tm.start, tm.stop, X, T, K, ldx, ssq,
                             accumulate, tn, bsum, p, nblk, sub);
    if (p == 1.0)
        return launch_kernel(k_stats<XF32, 1>, g, dim3(kStatsThreads), 0, st, tm.start, tm.stop, X, T, K, ldx, ssq,
                             accumulate, tn, bsum, p, nblk, sub);
    return launch_kernel(k_stats<XF32, 0>, g, dim3(kStatsThreads), 0, st, tm.start, tm.stop, X, T, K, ldx, ssq,
                         accumulate, tn, bsum, p, nblk, sub);
}

hipError_t launch_stats(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, double* ssq,
                        int accumulate, hipStream_t st, double* bsum, StageTimer tm, double p) {
    const double tn = bsum != nullptr ? (double)T : 1.0;
    return xf32 ? launch_stats_t<true>(X, T, K, ldx, ssq, accumulate, tn, bsum, p, st, tm)
                : launch_stats_t<false>(X, T, K, ldx, ssq, accumulate, tn, bsum, p, st, tm);
}

hipError_t launch_awq_scales(const double* ssq, int64_t n_tokens, int64_t K, float alpha,
                             float lambda_rel, float p, float* s, hipStream_t st) {
    return launch_kernel(k_awq_scales, dim3(1), dim3(kScaleThreads), 0, st, nullptr, nullptr, ssq, n_tokens, K,
                         (double)alpha / (double)p, (double)lambda_rel, s);
}

}  // namespace ttq
