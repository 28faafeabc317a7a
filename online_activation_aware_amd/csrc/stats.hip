// Activation statistics and AWQ scales (gfx950).
//
// [TTQ §method b2, b3] (TTQ review page, "proposed method", bullets 2-3):
// the per-channel diagonal of the input covariance, estimated online from the
// prompt, and the shrunk closed-form AWQ scale built from it.
//
// k_stats: one launch, no partial sums.  A workgroup owns a block of CH
// channels (16 or 64) over all T tokens: lane l reads 8 channels (one
// 16-byte load of bf16, two of fp32) of every (64/CH*8)-th row, all U of a
// batch issued before the first is used, and accumulates squares (or |x|^p
// for a moment order p != 2 [TTQ §method b4]) in fp64.  Lanes holding the
// same channels are combined by a fixed xor butterfly, the waves in wave
// order, so every result is bitwise reproducible run to run.  The workgroup
// also leaves the sums of c = ssq / n over each 16 channels (fixed 16-lane
// butterfly), from which the consumers form the shrinkage mean.
//
// Block size by shape (measured on the 4096- and 14336-channel layers): a
// 64-channel block reads whole 128-byte lines of bf16 and is used when K
// gives at least 128 such blocks (14336 channels, 1024 tokens: 8.3 us
// against 16.5 us with 16-channel blocks); with fewer, 64-channel blocks
// leave most of the chip idle and 16-channel blocks are used (4096 x 2048:
// 9.0 us against 10.3 us).  The 16-channel blocks that share one line run
// on one XCD: workgroups are dispatched to the eight XCDs round-robin by id,
// so ids w, w + 8, w + 16, ... are mapped to the blocks of one line, and that
// XCD's L2 serves the line to all of them (ordinary cached loads).
#include "common.hpp"
#include "launch.hpp"
#include "scales.hpp"

namespace ttq {

constexpr int kXcds = 8;
constexpr int kStatsBatch = 8;                 // loads per lane issued together

// |x|^p added to acc in fp64: PM = 2 squares (exact products), PM = 1 absolute
// values, PM = 0 any other p (fp64 pow of |x|; 0 for x = 0).
template <int PM>
__device__ __forceinline__ double add_moment(double x, double p, double acc) {
    if constexpr (PM == 2) return __builtin_fma(x, x, acc);
    else if constexpr (PM == 1) return acc + __builtin_fabs(x);
    else return acc + (x == 0.0 ? 0.0 : pow(__builtin_fabs(x), p));
}

template <int CH>
struct StatsShape {
    static constexpr int kThreads = CH == 16 ? 512 : 1024;
    static constexpr int kWaves = kThreads / kWave;
    static constexpr int kLanesPerRow = CH / 8;
    static constexpr int kRowsPerWave = kWave / kLanesPerRow;
    static constexpr int kRowStep = kWaves * kRowsPerWave;   // rows covered by one pass of the workgroup
};

template <bool XF32, int PM, int CH>
__global__ __launch_bounds__(StatsShape<CH>::kThreads) void k_stats(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, double* __restrict__ ssq, int accumulate,
    double tn, double* __restrict__ bsum, double pexp, int64_t nblk, int sub) {
    using S = StatsShape<CH>;
    int64_t blk = blockIdx.x;
    if constexpr (CH == 16) {
        // XCD x = w % 8 takes lines x, x + 8, ... and their `sub` blocks in
        // consecutive slots.
        const int64_t w = blockIdx.x, j = w / kXcds;
        blk = (w % kXcds + (int64_t)kXcds * (j / sub)) * sub + j % sub;
    }
    if (blk >= nblk) return;                      // whole workgroup: no barrier reached
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t c0 = blk * CH + 8 * (lane % S::kLanesPerRow);
    const int64_t r0 = lane / S::kLanesPerRow + (int64_t)S::kRowsPerWave * wave;

    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    if (c0 < K) {
        for (int64_t tb = r0; tb < T; tb += (int64_t)kStatsBatch * S::kRowStep) {
            if constexpr (XF32) {
                f32x4 a[kStatsBatch], b[kStatsBatch];
#pragma unroll
                for (int u = 0; u < kStatsBatch; ++u) {
                    const int64_t t = tb + (int64_t)u * S::kRowStep;
                    if (t < T) {
                        const f32x4* p = (const f32x4*)((const float*)X + t * ldx + c0);
                        a[u] = p[0];
                        b[u] = p[1];
                    } else {
                        a[u] = b[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
#pragma unroll
                for (int u = 0; u < kStatsBatch; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[i] = add_moment<PM>((double)a[u][i], pexp, acc[i]);
                        acc[4 + i] = add_moment<PM>((double)b[u][i], pexp, acc[4 + i]);
                    }
            } else {
                u32x4 v[kStatsBatch];
#pragma unroll
                for (int u = 0; u < kStatsBatch; ++u) {
                    const int64_t t = tb + (int64_t)u * S::kRowStep;
                    v[u] = t < T ? *(const u32x4*)((const uint16_t*)X + t * ldx + c0) : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < kStatsBatch; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] = add_moment<PM>((double)bf16lo_to_f32(v[u][i]), pexp, acc[2 * i]);
                        acc[2 * i + 1] = add_moment<PM>((double)bf16hi_to_f32(v[u][i]), pexp, acc[2 * i + 1]);
                    }
            }
        }
    }
    // the wave's rows: lanes l and l ^ kLanesPerRow, ^ 2 kLanesPerRow, ...
    // hold the same channels
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int m = S::kLanesPerRow; m < kWave; m <<= 1) acc[i] += __shfl_xor(acc[i], m);
    __shared__ double red[S::kWaves][CH];
    if (lane < S::kLanesPerRow) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][8 * lane + i] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
        const int64_t jc = blk * CH + lane;
        const bool ok = lane < CH && jc < K;
        double tot = 0.0;
        if (ok) {
            tot = red[0][lane];
#pragma unroll
            for (int v = 1; v < S::kWaves; ++v) tot += red[v][lane];
            if (accumulate) tot = ssq[jc] + tot;
            ssq[jc] = tot;
        }
        if (bsum != nullptr) {
            const double bs = seg16_sum_fixed(ok ? tot / tn : 0.0);
            const int64_t b16 = blk * (CH / kBlockCh) + lane / kBlockCh;
            if (lane % kBlockCh == 0 && lane < CH && b16 * kBlockCh < K) bsum[b16] = bs;
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

// 64-channel blocks when K gives at least this many of them.
constexpr int64_t kStats64MinBlocks = 128;

template <bool XF32, int CH>
static hipError_t launch_stats_ch(const void* X, int64_t T, int64_t K, int64_t ldx, double* ssq, int accumulate,
                                  double tn, double* bsum, double p, hipStream_t st, StageTimer tm) {
    const int64_t nblk = (K + CH - 1) / CH;
    int sub = 1;
    int64_t grid = nblk;
    if constexpr (CH == 16) {
        sub = XF32 ? 2 : 4;                       // 16-channel blocks per 128-byte line
        const int64_t lines = (nblk + sub - 1) / sub;
        grid = ((lines + kXcds - 1) / kXcds) * kXcds * sub;
    }
    const dim3 g((unsigned)grid), b(StatsShape<CH>::kThreads);
    if (p == 2.0)
        return launch_kernel(k_stats<XF32, 2, CH>, g, b, 0, st, tm.start, tm.stop, X, T, K, ldx, ssq, accumulate, tn,
                             bsum, p, nblk, sub);
    if (p == 1.0)
        return launch_kernel(k_stats<XF32, 1, CH>, g, b, 0, st, tm.start, tm.stop, X, T, K, ldx, ssq, accumulate, tn,
                             bsum, p, nblk, sub);
    return launch_kernel(k_stats<XF32, 0, CH>, g, b, 0, st, tm.start, tm.stop, X, T, K, ldx, ssq, accumulate, tn,
                         bsum, p, nblk, sub);
}

template <bool XF32>
static hipError_t launch_stats_t(const void* X, int64_t T, int64_t K, int64_t ldx, double* ssq, int accumulate,
                                 double tn, double* bsum, double p, hipStream_t st, StageTimer tm) {
    if ((K + 63) / 64 >= kStats64MinBlocks)
        return launch_stats_ch<XF32, 64>(X, T, K, ldx, ssq, accumulate, tn, bsum, p, st, tm);
    return launch_stats_ch<XF32, 16>(X, T, K, ldx, ssq, accumulate, tn, bsum, p, st, tm);
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
