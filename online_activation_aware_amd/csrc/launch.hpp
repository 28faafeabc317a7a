// Kernel launchers (host side) used by the C ABI in ttq_api.cpp.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ttq.h"

namespace ttq {

// Stage timing: the first kernel of a stage records `start` as it starts and
// the last records `stop` as it ends (hipExtLaunchKernel stamps the dispatch
// itself, so nothing extra is enqueued).  Null events: a plain launch.
struct StageTimer {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Low-rank term added in the projection GEMM's epilogue: Y += Z B^T, fp32.
struct LowrankEpilogue {
    const float* Z;   // [nz][T][rank]: Z = the nz partials added in order
    const float* B;   // [M][rank]
    int rank;
    int nz = 1;
};

template <typename F, typename... Args>
inline hipError_t launch_kernel(F kern, dim3 grid, dim3 block, size_t lds, hipStream_t st, hipEvent_t e0,
                                hipEvent_t e1, Args... args) {
    hipExtLaunchKernelGGL(kern, grid, block, (std::uint32_t)lds, st, e0, e1, 0u, args...);
    return hipGetLastError();
}

// K-slice split of the low-rank Z = A X pass.
int lowrank_slices(int64_t T, int64_t K, int64_t* slice_len);

// Statistics in one launch (no workspace).  bsum (optional, ceil(K/16)
// doubles): per-16-channel block sums of c = ssq / T, from which the
// quantizer forms lambda = lambda_rel * mean(c).  p: moment order of the
// statistic, sum |x|^p (2: sums of squares).
hipError_t launch_stats(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, double* ssq,
                        int accumulate, hipStream_t st, double* bsum = nullptr, StageTimer tm = {},
                        double p = 2.0);
hipError_t launch_awq_scales(const double* ssq, int64_t n_tokens, int64_t K, float alpha,
                             float lambda_rel, float p, float* s, hipStream_t st);
// Scales evaluated inside the quantizer from the statistics (instead of a
// given s): lambda = lambda_rel * blocks_total(bsum) / K, then
// s[j] = awq_scale(ssq[j], tn, lambda, e), also stored to s_out.
struct QScaleSrc {
    const double* ssq;
    const double* bsum;
    double lambda_rel;
    double tn;
    double e;
    float* s_out;
};
hipError_t launch_quantize(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                           const float* s, int bits, int group, const float* B, const float* A,
                           int rank, uint32_t* codes, uint16_t* scale, uint16_t* zero,
                           uint16_t* wq, hipStream_t st, const QScaleSrc* qs = nullptr,
                           StageTimer tm = {});
hipError_t launch_qgemm(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                        const float* s, const uint32_t* codes, const uint16_t* scale,
                        const uint16_t* zero, int64_t M, int bits, int group, void* Y, bool yf32,
                        int64_t ldy, uint16_t* wq, hipStream_t st, StageTimer tm = {});
// Prompt-sized projections use the dequantized weight w~ ([M][K] bf16) and
// the matrix-core GEMM; smaller ones (and fp32 X) the fused kernel.
constexpr int64_t kDequantGemmMinT = 192;
bool gemm_bf16_supported(int64_t T, int64_t K, int64_t ldx, int64_t ldw);
// split_ws (optional, gemm_bf16_split_ws_bytes(T, K, M) bytes, 16-byte
// aligned): lets a projection with too few 128 x 256 tiles run as two K
// slices plus an ordered sum (only without the low-rank epilogue).
hipError_t launch_gemm_bf16(const uint16_t* X, int64_t T, int64_t K, int64_t ldx, const uint16_t* Wq,
                            int64_t ldw, int64_t M, void* Y, bool yf32, int64_t ldy, hipStream_t st,
                            StageTimer tm = {}, const LowrankEpilogue* lr = nullptr, float* split_ws = nullptr);
int gemm_bf16_splits(int64_t T, int64_t K, int64_t M);
size_t gemm_bf16_split_ws_bytes(int64_t T, int64_t K, int64_t M);
// Workspace of the prompt-sized projection: the dequantized weight (M x K
// bf16), then, 256-byte aligned, the K-slice partials.
inline size_t dequant_ws_bytes(int64_t M, int64_t K) {
    return ((size_t)M * (size_t)K * 2 + 255) / 256 * 256;
}
inline float* split_ws_after(uint16_t* wq, int64_t M, int64_t K) {
    return wq ? (float*)((char*)wq + dequant_ws_bytes(M, K)) : nullptr;
}
// Few-token projection (decode steps and short prompts): T <= kQgemvMaxT,
// K a multiple of 128 (at most 16384 for T > 4).  A batch of P prompts
// (T <= 4 only) reads prompt p's operands at the element strides of bt.
constexpr int64_t kQgemvMaxT = 128;
constexpr int64_t kQgemvBatchMaxT = 4;
struct QgemvBatch {
    int64_t x = 0, s = 0, codes = 0, sz = 0, y = 0;
};
bool qgemv_supported(int64_t T, int64_t K, int64_t ldx, bool xf32);
// kGsMinT <= T <= 16, bf16 X, 4-bit codes, groups of 32/64/128, K a
// multiple of 128: the group scale applied to sums on the matrix cores
// (qgemv_gs.hip); x/s and its 32-channel sums are formed in LDS by the same
// launch.  A workspace of qgemv_gs_ws_bytes(T, K, M) bytes (256-byte
// aligned; zero when K is not split) holds the fp32 partials of K slices.
constexpr int64_t kGsMinT = 5;
bool qgemv_gs_eligible(int64_t T, int64_t K, int64_t M, int bits, int group, bool xf32, int64_t ldx);
size_t qgemv_gs_ws_bytes(int64_t T, int64_t K, int64_t M);
hipError_t launch_qgemv_gs(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                           const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, int bits,
                           int group, void* Y, bool yf32, int64_t ldy, void* ws, hipStream_t st,
                           StageTimer tm = {});
// kSkMinT <= T <= 16, bf16 X, K a multiple of 128: split-K variant with an
// fp32 partial workspace P of qgemv_sk_ws_bytes(T, K, M) bytes.
constexpr int64_t kSkMinT = 12;
bool qgemv_sk_eligible(int64_t T, int64_t K, int64_t ldx, bool xf32);
size_t qgemv_sk_ws_bytes(int64_t T, int64_t K, int64_t M);
hipError_t launch_qgemv_sk(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                           const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, int bits,
                           int group, void* Y, bool yf32, int64_t ldy, float* P, hipStream_t st, StageTimer tm = {});
hipError_t launch_qgemv(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                        const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, int bits,
                        int group, void* Y, bool yf32, int64_t ldy, hipStream_t st, StageTimer tm = {},
                        int64_t P = 1, QgemvBatch bt = {});
// Z = X A^T (fp32, [T][rank]) on the matrix cores, for bf16 X, K % 32 == 0
// and a 16-byte-aligned A.
bool lowrank_z_mfma_ok(bool xf32, int64_t T, int64_t K, int64_t ldx, const float* A);
// parts > 1: K is cut into `parts` slices and Z holds their partials
// [parts][T][rank] (lowrank_zm_parts(T, K) fills the chip).
hipError_t launch_lowrank_z(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* A,
                            int rank, float* Z, hipStream_t st, StageTimer tm = {}, int parts = 1);
int lowrank_zm_parts(int64_t T, int64_t K);
hipError_t launch_lowrank(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                          const float* A, const float* B, int64_t M, int rank, void* Y, bool yf32,
                          int64_t ldy, float* Zp, hipStream_t st, StageTimer tm = {});


// Per-prompt low-rank factors (factors.hip): workspace regions and the call.
struct FactorsLayout {
    size_t wt, yp, ym, yk, gp, rinv, g, tb, ta, total;
};
FactorsLayout factors_layout(int64_t M, int64_t K, int l);
bool factors_supported(bool wf32, int64_t M, int64_t K, int64_t ldw, int l, int rank);
hipError_t launch_factors(const uint16_t* W, int64_t M, int64_t K, int64_t ldw, const float* s, const float* om,
                          int l, int q, int rank, float* B, float* A, char* ws, hipStream_t st);

// ttq_linear's argument checks (clearing the calling thread's error text
// first) and the workspace bytes the call needs (0 for an empty call).
ttq_status linear_check(const ttq_linear_args* a, size_t* need);
// Record `msg` as the calling thread's last error text; returns st.
ttq_status set_error(ttq_status st, const char* msg);

}  // namespace ttq
