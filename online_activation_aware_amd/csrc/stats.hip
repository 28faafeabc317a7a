// Activation statistics and AWQ scales (gfx950).
//
// [TTQ §method b2, b3] (TTQ review page, "proposed method", bullets 2-3):
// the per-channel diagonal of the input covariance, estimated online from the
// prompt, and the shrunk closed-form AWQ scale built from it.
//
// k_stats_partial: a coalesced column reduction.  Each lane owns 8
// consecutive channels (one 16-byte bf16 load per token row, or two for
// fp32); the four waves of a workgroup stride over the rows of one token
// chunk; squares are accumulated in fp64; the four wave partials are combined
// through LDS in a fixed order and each workgroup writes one fp64 partial row
// per chunk.  k_stats_final sums the chunk partials in chunk order.  No
// atomics anywhere, so the result is bitwise reproducible.
#include "common.hpp"
#include "launch.hpp"

namespace ttq {

constexpr int kStatsThreads = 256;
constexpr int kStatsChans = kWave * 8;      // channels per workgroup strip

template <bool XF32>
__global__ __launch_bounds__(kStatsThreads) void k_stats_partial(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, int rows_per_chunk,
    double* __restrict__ part) {
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
#pragma unroll 8
            for (int64_t t = t0 + wave; t < t1; t += 4) {
                const f32x4* p = (const f32x4*)(base + t * ldx);
                f32x4 a = ld_nc(p), b = ld_nc(p + 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    double x = (double)a[i];
                    acc[i] = __builtin_fma(x, x, acc[i]);
                    double y = (double)b[i];
                    acc[4 + i] = __builtin_fma(y, y, acc[4 + i]);
                }
            }
        } else {
            const uint16_t* base = (const uint16_t*)X + c0;
#pragma unroll 8
            for (int64_t t = t0 + wave; t < t1; t += 4) {
                u32x4 w = ld_nc((const u32x4*)(base + t * ldx));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    double x = (double)bf16lo_to_f32(w[i]);
                    acc[2 * i] = __builtin_fma(x, x, acc[2 * i]);
                    double y = (double)bf16hi_to_f32(w[i]);
                    acc[2 * i + 1] = __builtin_fma(y, y, acc[2 * i + 1]);
                }
            }
        }
    }

    __shared__ double red[4][kStatsChans];
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = acc[i];
    __syncthreads();
    // 512 channel sums, two per thread; waves summed in order 0,1,2,3.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = threadIdx.x + h * kStatsThreads;
        const int64_t ch = (int64_t)blockIdx.x * kStatsChans + c;
        if (ch < K) {
            double s = red[0][c];
            s += red[1][c];
            s += red[2][c];
            s += red[3][c];
            part[(int64_t)blockIdx.y * K + ch] = s;
        }
    }
}

// Sum of the chunk partials: a workgroup covers 64 channels; its four waves
// take every fourth chunk and the four sums are added in wave order.
__global__ __launch_bounds__(256) void k_stats_final(const double* __restrict__ part, int nchunks,
                                                     int64_t K, double* __restrict__ ssq,
                                                     int accumulate) {
    __shared__ double red[4][64];
    const int c = threadIdx.x & 63, p = threadIdx.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + c;
    double s = 0.0;
    if (j < K) {
#pragma unroll 4
        for (int ch = p; ch < nchunks; ch += 4) s += part[(int64_t)ch * K + j];
    }
    red[p][c] = s;
    __syncthreads();
    if (p == 0 && j < K) {
        double tot = red[0][c];
        tot += red[1][c];
        tot += red[2][c];
        tot += red[3][c];
        ssq[j] = accumulate ? ssq[j] + tot : tot;
    }
}

// [TTQ §method b2-b4]: c = ssq / T; lambda = lambda_rel * mean(c);
// s = (c + lambda)^(alpha/2) in fp64, rounded once to fp32; 1 where c+lambda == 0.
// Every workgroup forms the same mean(c) (same fixed summation order), then
// the scales of its own 256 channels.
constexpr int kScaleThreads = 256;

__global__ __launch_bounds__(kScaleThreads) void k_awq_scales(const double* __restrict__ ssq,
                                                              int64_t n_tokens, int64_t K,
                                                              double alpha, double lambda_rel,
                                                              float* __restrict__ s) {
    __shared__ double red[kScaleThreads];
    const int tid = threadIdx.x;
    const double tn = (double)n_tokens;
    double part = 0.0;
    for (int64_t j = tid; j < K; j += kScaleThreads) part += ssq[j] / tn;
    red[tid] = part;
    __syncthreads();
    for (int w = kScaleThreads / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    const double lam = lambda_rel * (red[0] / (double)K);
    const double e = alpha / 2.0;
    const int64_t j = (int64_t)blockIdx.x * kScaleThreads + tid;
    if (j < K) {
        const double cl = ssq[j] / tn + lam;
        s[j] = cl == 0.0 ? 1.0f : (float)pow(cl, e);
    }
}

// ------------------------------------------------------------------ host

int stats_chunks(int64_t T, int64_t K, int* rows_per_chunk) {
    // At most 32 token chunks (the fp64 partials stay <= 32 K doubles, a small
    // fraction of the bytes read), at least ~1024 workgroups where T allows,
    // and whole multiples of the 4 waves' row stride.
    const int64_t strips = (K + kStatsChans - 1) / kStatsChans;
    int64_t want = (1024 + strips - 1) / strips;
    if (want > 32) want = 32;
    if (want < 1) want = 1;
    int64_t rows = (T + want - 1) / want;
    rows = (rows + 3) / 4 * 4;
    if (rows <= 0) rows = 4;
    *rows_per_chunk = (int)rows;
    return T > 0 ? (int)((T + rows - 1) / rows) : 0;
}

hipError_t launch_stats(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, double* ssq,
                        int accumulate, double* part, hipStream_t st) {
    int rows = 0;
    const int nchunks = stats_chunks(T, K, &rows);
    if (nchunks > 0) {
        dim3 grid((unsigned)((K + kStatsChans - 1) / kStatsChans), (unsigned)nchunks);
        if (xf32)
            k_stats_partial<true><<<grid, kStatsThreads, 0, st>>>(X, T, K, ldx, rows, part);
        else
            k_stats_partial<false><<<grid, kStatsThreads, 0, st>>>(X, T, K, ldx, rows, part);
    }
    k_stats_final<<<(unsigned)((K + 63) / 64), 256, 0, st>>>(part, nchunks, K, ssq, accumulate);
    return hipGetLastError();
}

hipError_t launch_awq_scales(const double* ssq, int64_t n_tokens, int64_t K, float alpha,
                             float lambda_rel, float* s, hipStream_t st) {
    k_awq_scales<<<(unsigned)((K + kScaleThreads - 1) / kScaleThreads), kScaleThreads, 0, st>>>(
        ssq, n_tokens, K, (double)alpha, (double)lambda_rel, s);
    return hipGetLastError();
}

}  // namespace ttq
