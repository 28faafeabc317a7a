// Activation statistics and AWQ scales (gfx950).
//
// [TTQ §method b2, b3] (TTQ review page, "proposed method", bullets 2-3):
// the per-channel diagonal of the input covariance, estimated online from the
// prompt, and the shrunk closed-form AWQ scale built from it.
//
// k_stats_partial: a coalesced column reduction.  Each lane owns 8
// consecutive channels (one 16-byte bf16 load per token row, or two for
// fp32); the 16 waves of a workgroup stride over the rows of one token chunk;
// squares (or, for a moment order p != 2 [TTQ §method b4], |x|^p) are
// accumulated in fp64; the wave partials are combined through LDS in a fixed
// order and each workgroup writes one fp64 partial row per chunk.
// k_stats_final sums the chunk partials in a fixed order.  Every sum has a
// fixed order and there are no atomics, so results are bitwise reproducible.
#include "common.hpp"
#include "launch.hpp"
#include "scales.hpp"

namespace ttq {

constexpr int kStatsThreads = 1024;         // 16 waves: all of a chunk's rows in flight at once
constexpr int kStatsWaves = kStatsThreads / kWave;
constexpr int kStatsChans = kWave * 8;      // channels per workgroup strip

// |x|^p added to acc in fp64: PM = 2 squares (exact products), PM = 1 absolute
// values, PM = 0 any other p (fp64 pow of |x|; 0 for x = 0).
template <int PM>
__device__ __forceinline__ double add_moment(double x, double p, double acc) {
    if constexpr (PM == 2) return __builtin_fma(x, x, acc);
    else if constexpr (PM == 1) return acc + __builtin_fabs(x);
    else return acc + (x == 0.0 ? 0.0 : pow(__builtin_fabs(x), p));
}

template <bool XF32, int PM>
__global__ __launch_bounds__(kStatsThreads) void k_stats_partial(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, int rows_per_chunk,
    double* __restrict__ part, double pexp) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t c0 = (int64_t)blockIdx.x * kStatsChans + lane * 8;
    const int64_t t0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t t1 = min(T, t0 + rows_per_chunk);

    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;

    if (c0 < K) {
        if constexpr (XF32) {
            const float* base = (const float*)X + c0;
#pragma unroll 4
            for (int64_t t = t0 + wave; t < t1; t += kStatsWaves) {
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
            for (int64_t t = t0 + wave; t < t1; t += kStatsWaves) {
                u32x4 w = ld_nc((const u32x4*)(base + t * ldx));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = add_moment<PM>((double)bf16lo_to_f32(w[i]), pexp, acc[2 * i]);
                    acc[2 * i + 1] = add_moment<PM>((double)bf16hi_to_f32(w[i]), pexp, acc[2 * i + 1]);
                }
            }
        }
    }

    __shared__ double red[kStatsWaves][kStatsChans];
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = acc[i];
    __syncthreads();
    // 512 channel sums; the 16 wave partials are added in wave order.
    if (threadIdx.x < kStatsChans) {
        const int c = threadIdx.x;
        const int64_t ch = (int64_t)blockIdx.x * kStatsChans + c;
        if (ch < K) {
            double s = red[0][c];
#pragma unroll
            for (int w = 1; w < kStatsWaves; ++w) s += red[w][c];
            part[(int64_t)blockIdx.y * K + ch] = s;
        }
    }
}

// Sum of the chunk partials: a workgroup covers one 64-channel block; its four
// waves each add a quarter of the chunks (in chunk order, all loads in flight
// at once) and wave 0 adds the four quarters in order.  With BSUM, wave 0 also
// stores the block's sum of c = ssq / n (cblock_sum order) in bsum[block];
// the consumer of lambda totals them after this kernel has finished.
// One pass for short prompts or many channels: a workgroup owns one block of
// 64 channels over all T tokens (lane: 8 channels of one row, 8 rows per
// wave, 16 waves), so ssq and the block's sum of c come out of one kernel.
// Rows are combined lane-wise in a fixed butterfly and waves in order, so
// the result is run-to-run reproducible.
template <bool XF32, int PM>
__global__ __launch_bounds__(kStatsThreads) void k_stats_block(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, double* __restrict__ ssq, int accumulate,
    double tn, double* __restrict__ bsum, double pexp) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane >> 3, c8 = lane & 7;
    const int64_t c0 = (int64_t)blockIdx.x * kWave + 8 * c8;
    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    if (c0 < K) {
        const int64_t tstart = 8 * wave + r;
        constexpr int64_t step = 8 * kStatsWaves;
        if constexpr (XF32) {
            const float* base = (const float*)X + c0;
#pragma unroll 4
            for (int64_t t = tstart; t < T; t += step) {
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
            for (int64_t t = tstart; t < T; t += step) {
                u32x4 w = ld_nc((const u32x4*)(base + t * ldx));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = add_moment<PM>((double)bf16lo_to_f32(w[i]), pexp, acc[2 * i]);
                    acc[2 * i + 1] = add_moment<PM>((double)bf16hi_to_f32(w[i]), pexp, acc[2 * i + 1]);
                }
            }
        }
    }
    // the 8 rows of the wave: lanes l, l ^ 8, l ^ 16, l ^ 32 hold the same channels
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc[i] += __shfl_xor(acc[i], 8);
        acc[i] += __shfl_xor(acc[i], 16);
        acc[i] += __shfl_xor(acc[i], 32);
    }
    __shared__ double red[kStatsWaves][kWave];
    if (r == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][8 * c8 + i] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
        double tot = red[0][lane];
#pragma unroll
        for (int w = 1; w < kStatsWaves; ++w) tot += red[w][lane];
        const int64_t j = (int64_t)blockIdx.x * kWave + lane;
        if (j < K) {
            if (accumulate) tot = ssq[j] + tot;
            ssq[j] = tot;
        }
        if (bsum != nullptr) {
            const double bs = wave_sum_fixed(j < K ? tot / tn : 0.0);
            if (lane == 0) bsum[blockIdx.x] = bs;
        }
    }
}

template <bool BSUM>
__global__ __launch_bounds__(256) void k_stats_final(const double* __restrict__ part, int nchunks, int64_t K,
                                                     double* __restrict__ ssq, int accumulate, double tn,
                                                     double* __restrict__ bsum) {
    __shared__ double red[4][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t j = (int64_t)blockIdx.x * kWave + lane;
    const int per = (nchunks + 3) / 4;
    const int ch0 = wave * per, ch1 = min(nchunks, ch0 + per);
    double acc = 0.0;
    if (j < K) {
#pragma unroll 8
        for (int ch = ch0; ch < ch1; ++ch) acc += part[(int64_t)ch * K + j];
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        double tot = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
        if (j < K) {
            if (accumulate) tot = ssq[j] + tot;
            ssq[j] = tot;
        }
        if constexpr (BSUM) {
            const double bs = wave_sum_fixed(j < K ? tot / tn : 0.0);
            if (lane == 0) bsum[blockIdx.x] = bs;
        }
    }
}

// Standalone scales from ssq: one workgroup of 1024 threads.  The 16 waves
// form the 64-channel block sums (cblock_sum) into LDS, wave 0 totals them
// (blocks_total), then every thread evaluates the scales of its channels.
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
    const int64_t nb = (K + 63) / 64;
    for (int64_t b = wave; b < nb; b += kScaleThreads / kWave) {
        const double v = cblock_sum(ssq, b, K, tn, lane);
        if (lane == 0) bs[b] = v;
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

int stats_chunks(int64_t T, int64_t K, int* rows_per_chunk) {
    // At most kMaxStatsChunks token chunks (the fp64 partials stay small next
    // to X), at least ~256 workgroups (one per compute unit) where T allows,
    // and whole multiples of the 16 waves' row stride.
    const int64_t strips = (K + kStatsChans - 1) / kStatsChans;
    int64_t want = (256 + strips - 1) / strips;
    if (want > kMaxStatsChunks) want = kMaxStatsChunks;
    if (want < 1) want = 1;
    int64_t rows = (T + want - 1) / want;
    rows = (rows + kStatsWaves - 1) / kStatsWaves * kStatsWaves;
    if (rows <= 0) rows = kStatsWaves;
    *rows_per_chunk = (int)rows;
    return T > 0 ? (int)((T + rows - 1) / rows) : 0;
}

template <bool XF32>
static hipError_t launch_partial(dim3 grid, const void* X, int64_t T, int64_t K, int64_t ldx, int rows,
                                 double* part, double p, hipStream_t st, hipEvent_t e0) {
    if (p == 2.0)
        return launch_kernel(k_stats_partial<XF32, 2>, grid, dim3(kStatsThreads), 0, st, e0, nullptr, X, T, K, ldx,
                             rows, part, p);
    if (p == 1.0)
        return launch_kernel(k_stats_partial<XF32, 1>, grid, dim3(kStatsThreads), 0, st, e0, nullptr, X, T, K, ldx,
                             rows, part, p);
    return launch_kernel(k_stats_partial<XF32, 0>, grid, dim3(kStatsThreads), 0, st, e0, nullptr, X, T, K, ldx,
                         rows, part, p);
}

// One-pass statistics when the 64-channel blocks alone fill most of the chip
// or the prompt is short (measured: 14336 channels x 1024 tokens 11.0 ->
// 9.7 us, 768 x 128 6.2 -> 5.0 us; 4096 x 2048 stays on two kernels, 9.3
// against 13.4 us with only 64 blocks).
static bool stats_one_pass(int64_t T, int64_t K) {
    return (K + kWave - 1) / kWave >= 160 || T <= 256;
}

template <bool XF32>
static hipError_t launch_block(const void* X, int64_t T, int64_t K, int64_t ldx, double* ssq, int accumulate,
                               double tn, double* bsum, double p, hipStream_t st, StageTimer tm) {
    const dim3 g((unsigned)((K + kWave - 1) / kWave));
    if (p == 2.0)
        return launch_kernel(k_stats_block<XF32, 2>, g, dim3(kStatsThreads), 0, st, tm.start, tm.stop, X, T, K, ldx,
                             ssq, accumulate, tn, bsum, p);
    if (p == 1.0)
        return launch_kernel(k_stats_block<XF32, 1>, g, dim3(kStatsThreads), 0, st, tm.start, tm.stop, X, T, K, ldx,
                             ssq, accumulate, tn, bsum, p);
    return launch_kernel(k_stats_block<XF32, 0>, g, dim3(kStatsThreads), 0, st, tm.start, tm.stop, X, T, K, ldx,
                         ssq, accumulate, tn, bsum, p);
}

hipError_t launch_stats(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, double* ssq,
                        int accumulate, double* part, hipStream_t st, double* bsum, StageTimer tm, double p) {
    if (stats_one_pass(T, K)) {
        const double tn = bsum != nullptr ? (double)T : 1.0;
        return xf32 ? launch_block<true>(X, T, K, ldx, ssq, accumulate, tn, bsum, p, st, tm)
                    : launch_block<false>(X, T, K, ldx, ssq, accumulate, tn, bsum, p, st, tm);
    }
    int rows = 0;
    const int nchunks = stats_chunks(T, K, &rows);
    if (nchunks > 0) {
        dim3 grid((unsigned)((K + kStatsChans - 1) / kStatsChans), (unsigned)nchunks);
        hipError_t e = xf32 ? launch_partial<true>(grid, X, T, K, ldx, rows, part, p, st, tm.start)
                            : launch_partial<false>(grid, X, T, K, ldx, rows, part, p, st, tm.start);
        if (e != hipSuccess) return e;
    }
    const dim3 g((unsigned)((K + kWave - 1) / kWave));
    hipEvent_t e0 = nchunks > 0 ? nullptr : tm.start;
    if (bsum != nullptr)
        return launch_kernel(k_stats_final<true>, g, dim3(256), 0, st, e0, tm.stop, (const double*)part, nchunks, K,
                             ssq, accumulate, (double)T, bsum);
    return launch_kernel(k_stats_final<false>, g, dim3(256), 0, st, e0, tm.stop, (const double*)part, nchunks, K,
                         ssq, accumulate, 1.0, (double*)nullptr);
}

hipError_t launch_awq_scales(const double* ssq, int64_t n_tokens, int64_t K, float alpha,
                             float lambda_rel, float p, float* s, hipStream_t st) {
    return launch_kernel(k_awq_scales, dim3(1), dim3(kScaleThreads), 0, st, nullptr, nullptr, ssq, n_tokens, K,
                         (double)alpha / (double)p, (double)lambda_rel, s);
}

}  // namespace ttq
