// The libttq C ABI: argument validation, workspace layout, launches.
//
// Every check runs on the host before any HIP call; a failed check returns
// TTQ_ERR_INVALID / TTQ_ERR_UNSUPPORTED and launches nothing.  Global state:
// the per-thread error text, and a per-device memo of the quantizer's
// residency (a property of the code object, so it never changes a result).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include <hip/hip_runtime.h>

#include "ttq.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

ttq_status fail(ttq_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ttq_status fail(ttq_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

ttq_status device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return TTQ_OK;
    return fail(TTQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxK = (int64_t)1 << 18;    // input channels (block sums of the mean fit in LDS)
constexpr int kMaxRank = 64;
constexpr size_t kAlign = 256;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t round_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }
bool dtype_ok(int t) { return t == TTQ_F32 || t == TTQ_BF16; }
size_t esize(int t) { return t == TTQ_F32 ? 4 : 2; }
bool bits_ok(int b) { return b >= 2 && b <= 5; }
bool group_ok(int g) { return g == 16 || g == 32 || g == 64 || g == 128; }
bool dim_ok(int64_t n) { return n >= 0 && n <= kMaxDim; }

#define TTQ_REQUIRE(cond, ...)                                \
    do {                                                      \
        if (!(cond)) return fail(TTQ_ERR_INVALID, __VA_ARGS__); \
    } while (0)

// Checks for the output Y [T][M]: element-aligned, any row stride >= M.
ttq_status check_output(const void* p, int t, int64_t rows, int64_t M, int64_t ld) {
    TTQ_REQUIRE(dtype_ok(t), "Y: unknown dtype %d", t);
    TTQ_REQUIRE(ld >= M && ld <= kMaxDim, "Y: row stride %lld < row length %lld", (long long)ld, (long long)M);
    if (rows > 0 && M > 0) {
        TTQ_REQUIRE(p != nullptr, "Y: null pointer");
        TTQ_REQUIRE(aligned(p, esize(t)), "Y: pointer not aligned to its element size");
    }
    return TTQ_OK;
}

// Checks for a [rows][K] row-major matrix argument of dtype t.
ttq_status check_matrix(const char* name, const void* p, int t, int64_t rows, int64_t K, int64_t ld) {
    TTQ_REQUIRE(dtype_ok(t), "%s: unknown dtype %d", name, t);
    TTQ_REQUIRE(ld >= K && ld <= kMaxDim, "%s: row stride %lld < row length %lld", name, (long long)ld, (long long)K);
    if (rows > 0) {
        TTQ_REQUIRE(p != nullptr, "%s: null pointer", name);
        TTQ_REQUIRE(aligned(p, 16), "%s: pointer not 16-byte aligned", name);
        TTQ_REQUIRE((ld * (int64_t)esize(t)) % 16 == 0, "%s: row stride is not a multiple of 16 bytes", name);
    }
    return TTQ_OK;
}

ttq_status check_quant_shape(int64_t M, int64_t K, int bits, int group) {
    TTQ_REQUIRE(dim_ok(M), "M out of range");
    TTQ_REQUIRE(K > 0 && K <= kMaxK && K % 32 == 0, "K must be a positive multiple of 32, at most 2^18");
    if (!bits_ok(bits)) return fail(TTQ_ERR_INVALID, "bits must be 2, 3, 4 or 5 (got %d)", bits);
    if (!group_ok(group)) return fail(TTQ_ERR_INVALID, "group must be 16, 32, 64 or 128 (got %d)", group);
    TTQ_REQUIRE(K % group == 0, "K must be a multiple of the group size");
    return TTQ_OK;
}

ttq_status check_state(const float* s, const void* codes, const void* scale, const void* zero, bool need_s) {
    TTQ_REQUIRE(!need_s || s != nullptr, "s: null pointer");
    TTQ_REQUIRE(s == nullptr || aligned(s, 16), "s: pointer not 16-byte aligned");
    TTQ_REQUIRE(codes != nullptr && aligned(codes, 16), "codes: null or not 16-byte aligned");
    TTQ_REQUIRE(scale != nullptr && aligned(scale, 2), "scale_f16: null or misaligned");
    TTQ_REQUIRE(zero != nullptr && aligned(zero, 2), "zero_f16: null or misaligned");
    return TTQ_OK;
}

ttq_status check_lowrank(const float* B, const float* A, int rank, bool allow_zero) {
    TTQ_REQUIRE(rank >= (allow_zero ? 0 : 1) && rank <= kMaxRank, "rank must be in [%d, %d] (got %d)",
                allow_zero ? 0 : 1, kMaxRank, rank);
    TTQ_REQUIRE((B == nullptr) == (rank == 0) && (A == nullptr) == (rank == 0),
                "B and A must both be given iff rank > 0");
    TTQ_REQUIRE(B == nullptr || (aligned(B, 4) && aligned(A, 4)), "B/A: misaligned");
    return TTQ_OK;
}

ttq_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return TTQ_OK;
    TTQ_REQUIRE(ws != nullptr, "workspace: null pointer (%zu bytes needed)", need);
    TTQ_REQUIRE(aligned(ws, kAlign), "workspace: pointer not 256-byte aligned");
    TTQ_REQUIRE(ws_bytes >= need, "workspace: %zu bytes given, %zu needed", ws_bytes, need);
    return TTQ_OK;
}

// Prompt-sized projections stage the dequantized weight (M x K bf16) in the
// workspace; the size is requested whenever T allows that path.
size_t ws_qgemm(int64_t T, int64_t K, int64_t M) {
    // 5 <= T <= 16: the fp32 partials of the K slices of the sums kernel
    // (4-bit codes) or of the split-K few-token projection.
    if (T >= ttq::kGsMinT && T <= 16 && K % 128 == 0) {
        const size_t gs = round_up(ttq::qgemv_gs_ws_bytes(T, K, M));
        const size_t sk = T >= ttq::kSkMinT ? round_up(ttq::qgemv_sk_ws_bytes(T, K, M)) : 0;
        return gs > sk ? gs : sk;
    }
    if (T < ttq::kDequantGemmMinT) return 0;
    return ttq::dequant_ws_bytes(M, K) + round_up(ttq::gemm_bf16_split_ws_bytes(T, K, M));
}
bool use_dequant_gemm(int64_t T, bool xf32, int64_t K, int64_t ldx) {
    return !xf32 && T >= ttq::kDequantGemmMinT && ttq::gemm_bf16_supported(T, K, ldx, K);
}
size_t ws_lowrank(int64_t T, int64_t K, int rank) {
    if (rank <= 0 || T <= 0) return 0;
    int64_t len = 0;
    int ns = ttq::lowrank_slices(T, K, &len);
    if (ttq::lowrank_zm_parts(T, K) > ns) ns = ttq::lowrank_zm_parts(T, K);
    return round_up((size_t)ns * (size_t)T * (size_t)rank * sizeof(float));
}

struct StateLayout {
    size_t ssq, s, codes, scale, zero, bsum, scratch, total;
};
StateLayout state_layout(int64_t T, int64_t K, int64_t M, int bits, int group, int rank) {
    StateLayout L{};
    size_t off = 0;
    L.ssq = off;     off += round_up((size_t)K * sizeof(double));
    L.s = off;       off += round_up((size_t)K * sizeof(float));
    L.codes = off;   off += round_up((size_t)M * (size_t)(K * bits / 32) * sizeof(int32_t));
    L.scale = off;   off += round_up((size_t)M * (size_t)(K / group) * sizeof(uint16_t));
    L.zero = off;    off += round_up((size_t)M * (size_t)(K / group) * sizeof(uint16_t));
    L.bsum = off;    off += round_up((size_t)((K + 15) / 16) * sizeof(double));
    L.scratch = off;
    size_t scratch = 0;
    // prompt-sized projections: the dequantized weight, then Z = X A^T for
    // the low-rank epilogue
    const size_t proj = ws_qgemm(T, K, M) + (rank > 0 && T > 0 ? round_up((size_t)ttq::lowrank_zm_parts(T, K) *
                                                                          T * rank * sizeof(float)) : 0);
    if (proj > scratch) scratch = proj;
    if (ws_lowrank(T, K, rank) > scratch) scratch = ws_lowrank(T, K, rank);
    L.total = off + scratch;
    return L;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

}  // namespace

extern "C" {

const char* ttq_status_str(int status) {
    switch (status) {
        case TTQ_OK: return "TTQ_OK";
        case TTQ_ERR_INVALID: return "TTQ_ERR_INVALID";
        case TTQ_ERR_UNSUPPORTED: return "TTQ_ERR_UNSUPPORTED";
        case TTQ_ERR_DEVICE: return "TTQ_ERR_DEVICE";
    }
    return "TTQ_ERR_UNKNOWN";
}

const char* ttq_last_error(void) { return g_last_error.c_str(); }

size_t ttq_workspace_bytes(int64_t T, int64_t K, int64_t M, int bits, int group, int rank) {
    if (!dim_ok(T) || !dim_ok(M) || K <= 0 || K > kMaxK || K % 32 || !bits_ok(bits) ||
        !group_ok(group) || K % group || rank < 0 || rank > kMaxRank)
        return 0;
    return state_layout(T, K, M, bits, group, rank).total;
}

ttq_status ttq_stats(const void* X, int xt, int64_t T, int64_t K, int64_t ldx, double* ssq,
                     int accumulate, void* ws, size_t ws_bytes, void* stream) {
    return ttq_stats_p(X, xt, T, K, ldx, 2.0f, ssq, accumulate, ws, ws_bytes, stream);
}

ttq_status ttq_stats_p(const void* X, int xt, int64_t T, int64_t K, int64_t ldx, float p, double* msum,
                       int accumulate, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    double* ssq = msum;
    TTQ_REQUIRE(std::isfinite(p) && p > 0.f, "p must be finite and > 0");
    TTQ_REQUIRE(dim_ok(T), "T out of range");
    TTQ_REQUIRE(K > 0 && K <= kMaxK && K % 8 == 0, "K must be a positive multiple of 8, at most 2^18");
    if (ttq_status e = check_matrix("X", X, xt, T, K, ldx)) return e;
    TTQ_REQUIRE(ssq != nullptr && aligned(ssq, 8), "ssq: null or not 8-byte aligned");
    (void)ws;
    (void)ws_bytes;
    if (T == 0 && accumulate) return TTQ_OK;
    return device_status(ttq::launch_stats(X, xt == TTQ_F32, T, K, ldx, ssq, accumulate, as_stream(stream),
                                           nullptr, {}, (double)p),
                         "ttq_stats launch");
}

ttq_status ttq_awq_scales(const double* ssq, int64_t n_tokens, int64_t K, float alpha,
                          float lambda_rel, float p, float* s, void* stream) {
    g_last_error.clear();
    TTQ_REQUIRE(K > 0 && K <= kMaxK, "K must be in [1, 2^18]");
    TTQ_REQUIRE(n_tokens > 0, "n_tokens must be positive");
    TTQ_REQUIRE(ssq != nullptr && aligned(ssq, 8), "ssq: null or not 8-byte aligned");
    TTQ_REQUIRE(s != nullptr && aligned(s, 16), "s: null or not 16-byte aligned");
    TTQ_REQUIRE(std::isfinite(alpha) && alpha >= 0.f, "alpha must be finite and >= 0");
    TTQ_REQUIRE(std::isfinite(lambda_rel) && lambda_rel >= 0.f, "lambda_rel must be finite and >= 0");
    TTQ_REQUIRE(std::isfinite(p) && p > 0.f, "p must be finite and > 0");
    return device_status(ttq::launch_awq_scales(ssq, n_tokens, K, alpha, lambda_rel, p, s, as_stream(stream)),
                         "ttq_awq_scales launch");
}

ttq_status ttq_quantize_groups(const void* W, int wt, int64_t M, int64_t K, int64_t ldw,
                               const float* s, int bits, int group, const float* B, const float* A,
                               int rank, int32_t* codes, uint16_t* scale_f16, uint16_t* zero_f16,
                               void* stream) {
    g_last_error.clear();
    if (ttq_status e = check_quant_shape(M, K, bits, group)) return e;
    if (ttq_status e = check_matrix("W", W, wt, M, K, ldw)) return e;
    if (ttq_status e = check_lowrank(B, A, rank, true)) return e;
    if (M == 0) return TTQ_OK;
    if (ttq_status e = check_state(s, codes, scale_f16, zero_f16, false)) return e;
    return device_status(ttq::launch_quantize(W, wt == TTQ_F32, M, K, ldw, s, bits, group, B, A, rank,
                                              (uint32_t*)codes, scale_f16, zero_f16, nullptr,
                                              as_stream(stream)),
                         "ttq_quantize_groups launch");
}

ttq_status ttq_qgemm(const void* X, int xt, int64_t T, int64_t K, int64_t ldx, const float* s,
                     const int32_t* codes, const uint16_t* scale_f16, const uint16_t* zero_f16,
                     int64_t M, int bits, int group, void* Y, int yt, int64_t ldy, void* ws,
                     size_t ws_bytes, void* stream) {
    g_last_error.clear();
    TTQ_REQUIRE(dim_ok(T), "T out of range");
    if (ttq_status e = check_quant_shape(M, K, bits, group)) return e;
    if (ttq_status e = check_matrix("X", X, xt, T, K, ldx)) return e;
    if (ttq_status e = check_output(Y, yt, T, M, ldy)) return e;
    if (T == 0 || M == 0) return TTQ_OK;
    if (ttq_status e = check_state(s, codes, scale_f16, zero_f16, true)) return e;
    const bool xf32 = xt == TTQ_F32;
    const bool dq = use_dequant_gemm(T, xf32, K, ldx);
    const bool gs = ttq::qgemv_gs_eligible(T, K, M, bits, group, xf32, ldx);
    const bool sk = !gs && ttq::qgemv_sk_eligible(T, K, ldx, xf32);
    if (ttq_status e = check_ws(ws, ws_bytes, (dq || sk || gs) ? ws_qgemm(T, K, M) : 0)) return e;
    hipStream_t st = as_stream(stream);
    if (gs)
        return device_status(ttq::launch_qgemv_gs(X, xf32, T, K, ldx, s, (const uint32_t*)codes, scale_f16, zero_f16,
                                                  M, bits, group, Y, yt == TTQ_F32, ldy, ws, st),
                             "ttq_qgemm launch");
    if (sk)
        return device_status(ttq::launch_qgemv_sk(X, xf32, T, K, ldx, s, (const uint32_t*)codes, scale_f16, zero_f16,
                                                  M, bits, group, Y, yt == TTQ_F32, ldy, (float*)ws, st),
                             "ttq_qgemm launch");
    if (ttq::qgemv_supported(T, K, ldx, xf32))
        return device_status(ttq::launch_qgemv(X, xf32, T, K, ldx, s, (const uint32_t*)codes, scale_f16, zero_f16,
                                               M, bits, group, Y, yt == TTQ_F32, ldy, st),
                             "ttq_qgemm launch");
    return device_status(ttq::launch_qgemm(X, xf32, T, K, ldx, s, (const uint32_t*)codes,
                                           scale_f16, zero_f16, M, bits, group, Y, yt == TTQ_F32, ldy,
                                           dq ? (uint16_t*)ws : nullptr, st),
                         "ttq_qgemm launch");
}

size_t ttq_lowrank_factors_workspace_bytes(int64_t M, int64_t K, int l) {
    if (M <= 0 || K <= 0 || K > kMaxK || !dim_ok(M) || l < 1 || l > 32) return 0;
    return ttq::factors_layout(M, K, l).total;
}

ttq_status ttq_lowrank_factors(const void* W, int wt, int64_t M, int64_t K, int64_t ldw, const float* s,
                               const float* omega, int l, int q, int rank, float* B, float* A, void* ws,
                               size_t ws_bytes, void* stream) {
    g_last_error.clear();
    TTQ_REQUIRE(dim_ok(M) && M > 0, "M must be positive");
    TTQ_REQUIRE(K > 0 && K <= kMaxK && K % 32 == 0, "K must be a positive multiple of 32, at most 2^18");
    if (ttq_status e = check_matrix("W", W, wt, M, K, ldw)) return e;
    TTQ_REQUIRE(l >= 1 && l <= 32, "l (test vectors) must be in [1, 32]");
    TTQ_REQUIRE(rank >= 1 && rank <= l, "rank must be in [1, l]");
    TTQ_REQUIRE(l <= M && l <= K, "l must not exceed M or K");
    TTQ_REQUIRE(q >= 0 && q <= 64, "q (power iterations) must be in [0, 64]");
    TTQ_REQUIRE(s != nullptr && aligned(s, 4), "s: null or misaligned");
    TTQ_REQUIRE(omega != nullptr && aligned(omega, 4), "omega: null or misaligned");
    TTQ_REQUIRE(B != nullptr && aligned(B, 4) && A != nullptr && aligned(A, 4), "B/A: null or misaligned");
    if (wt == TTQ_F32) return fail(TTQ_ERR_UNSUPPORTED, "per-prompt factors need a bf16 weight");
    TTQ_REQUIRE(ttq::factors_supported(false, M, K, ldw, l, rank), "sizes exceed the factor kernels' addressing");
    if (ttq_status e = check_ws(ws, ws_bytes, ttq::factors_layout(M, K, l).total)) return e;
    return device_status(ttq::launch_factors((const uint16_t*)W, M, K, ldw, s, omega, l, q, rank, B, A, (char*)ws,
                                             as_stream(stream)),
                         "ttq_lowrank_factors launch");
}

ttq_status ttq_qgemm_batched(const void* X, int xt, int64_t P, int64_t T, int64_t K, int64_t ldx,
                             int64_t x_stride, const float* s, int64_t s_stride, const int32_t* codes,
                             int64_t codes_stride, const uint16_t* scale_f16, const uint16_t* zero_f16,
                             int64_t sz_stride, int64_t M, int bits, int group, void* Y, int yt, int64_t ldy,
                             int64_t y_stride, void* stream) {
    g_last_error.clear();
    TTQ_REQUIRE(P >= 1 && P <= 65535, "P (prompts) must be in [1, 65535]");
    TTQ_REQUIRE(T >= 1 && T <= ttq::kQgemvBatchMaxT, "T must be in [1, %d] for batched decode steps",
                (int)ttq::kQgemvBatchMaxT);
    if (ttq_status e = check_quant_shape(M, K, bits, group)) return e;
    TTQ_REQUIRE(K % 128 == 0, "K must be a multiple of 128");
    if (ttq_status e = check_matrix("X", X, xt, T, K, ldx)) return e;
    if (ttq_status e = check_output(Y, yt, T, M, ldy)) return e;
    if (M == 0) return TTQ_OK;
    if (ttq_status e = check_state(s, codes, scale_f16, zero_f16, true)) return e;
    const int64_t xe = esize(xt);
    TTQ_REQUIRE(x_stride >= 0 && (x_stride * xe) % 16 == 0 && (P == 1 || x_stride >= (T - 1) * ldx + K),
                "x_stride: negative, not a multiple of 16 bytes, or overlapping prompts");
    TTQ_REQUIRE(s_stride >= 0 && s_stride % 4 == 0, "s_stride: negative or not a multiple of 16 bytes");
    TTQ_REQUIRE(codes_stride >= 0 && codes_stride % 4 == 0, "codes_stride: negative or not a multiple of 16 bytes");
    TTQ_REQUIRE(sz_stride >= 0, "sz_stride: negative");
    TTQ_REQUIRE(y_stride >= 0 && (P == 1 || y_stride >= (T - 1) * ldy + M), "y_stride: negative or overlapping prompts");
    ttq::QgemvBatch bt;
    bt.x = x_stride; bt.s = s_stride; bt.codes = codes_stride; bt.sz = sz_stride; bt.y = y_stride;
    return device_status(ttq::launch_qgemv(X, xt == TTQ_F32, T, K, ldx, s, (const uint32_t*)codes, scale_f16, zero_f16,
                                           M, bits, group, Y, yt == TTQ_F32, ldy, as_stream(stream), {}, P, bt),
                         "ttq_qgemm_batched launch");
}

ttq_status ttq_lowrank_add(const void* X, int xt, int64_t T, int64_t K, int64_t ldx, const float* A,
                           const float* B, int64_t M, int rank, void* Y, int yt, int64_t ldy, void* ws,
                           size_t ws_bytes, void* stream) {
    g_last_error.clear();
    TTQ_REQUIRE(dim_ok(T) && dim_ok(M), "T or M out of range");
    TTQ_REQUIRE(K > 0 && K <= kMaxK && K % 8 == 0, "K must be a positive multiple of 8, at most 2^18");
    if (ttq_status e = check_lowrank(B, A, rank, false)) return e;
    if (ttq_status e = check_matrix("X", X, xt, T, K, ldx)) return e;
    if (ttq_status e = check_output(Y, yt, T, M, ldy)) return e;
    if (T == 0 || M == 0) return TTQ_OK;
    if (ttq_status e = check_ws(ws, ws_bytes, ws_lowrank(T, K, rank))) return e;
    return device_status(ttq::launch_lowrank(X, xt == TTQ_F32, T, K, ldx, A, B, M, rank, Y, yt == TTQ_F32,
                                             ldy, (float*)ws, as_stream(stream)),
                         "ttq_lowrank_add launch");
}

static ttq_status check_linear(const ttq_linear_args* a) {
    TTQ_REQUIRE(a != nullptr, "args: null pointer");
    TTQ_REQUIRE(dim_ok(a->T), "T out of range");
    if (ttq_status e = check_quant_shape(a->M, a->K, a->bits, a->group)) return e;
    if (ttq_status e = check_matrix("X", a->X, a->xt, a->T, a->K, a->ldx)) return e;
    if (ttq_status e = check_matrix("W", a->W, a->wt, a->M, a->K, a->ldw)) return e;
    if (ttq_status e = check_output(a->Y, a->yt, a->T, a->M, a->ldy)) return e;
    if (ttq_status e = check_lowrank(a->B, a->A, a->rank, true)) return e;
    TTQ_REQUIRE(std::isfinite(a->alpha) && a->alpha >= 0.f, "alpha must be finite and >= 0");
    TTQ_REQUIRE(std::isfinite(a->lambda_rel) && a->lambda_rel >= 0.f, "lambda_rel must be finite and >= 0");
    TTQ_REQUIRE(std::isfinite(a->p) && a->p > 0.f, "p must be finite and > 0");
    TTQ_REQUIRE(a->ssq == nullptr || aligned(a->ssq, 8), "ssq: not 8-byte aligned");
    TTQ_REQUIRE(a->s == nullptr || aligned(a->s, 16), "s: not 16-byte aligned");
    TTQ_REQUIRE(a->codes == nullptr || aligned(a->codes, 16), "codes: not 16-byte aligned");
    TTQ_REQUIRE(a->scale_f16 == nullptr || aligned(a->scale_f16, 2), "scale_f16: misaligned");
    TTQ_REQUIRE(a->zero_f16 == nullptr || aligned(a->zero_f16, 2), "zero_f16: misaligned");
    if (a->stage_events != nullptr)
        for (int i = 0; i < TTQ_LINEAR_STAGE_EVENTS; ++i)
            TTQ_REQUIRE(a->stage_events[i] != nullptr, "stage_events[%d]: null handle", i);
    return TTQ_OK;
}

// Stage i of ttq_linear is timed by events (2i, 2i+1), stamped by the
// stage's first and last kernel; a stage that launches nothing records both
// on the stream as markers.
struct StageMarks {
    void* const* ev;
    hipStream_t st;
    ttq::StageTimer timer(int i) const {
        if (ev == nullptr) return {};
        return {(hipEvent_t)ev[2 * i], (hipEvent_t)ev[2 * i + 1]};
    }
    ttq_status markers(int i) const {
        if (ev == nullptr) return TTQ_OK;
        for (int k = 0; k < 2; ++k)
            if (ttq_status e = device_status(hipEventRecord((hipEvent_t)ev[2 * i + k], st), "stage event"))
                return e;
        return TTQ_OK;
    }
};

// Everything after the statistics (ssq, and the block sums of c in bsum):
// scales, quantizer, projection and low-rank term, with the state and
// scratch regions of L in w.
static ttq_status linear_layer(const ttq_linear_args* a, const double* ssq, const double* bsum, char* w,
                               const StateLayout& L, hipStream_t st) {
    float* s = a->s ? a->s : (float*)(w + L.s);
    int32_t* codes = a->codes ? a->codes : (int32_t*)(w + L.codes);
    uint16_t* scale = a->scale_f16 ? a->scale_f16 : (uint16_t*)(w + L.scale);
    uint16_t* zero = a->zero_f16 ? a->zero_f16 : (uint16_t*)(w + L.zero);
    void* scratch = w + L.scratch;
    const bool xf32 = a->xt == TTQ_F32;
    const StageMarks sm{a->stage_events, st};
    auto timer = [&](int i) { return sm.timer(i); };
    auto markers = [&](int i) { return sm.markers(i); };
    if (a->M == 0) {
        // No rows to quantize: the scales still form part of the prompt state.
        if (ttq_status e = device_status(ttq::launch_awq_scales(ssq, a->T, a->K, a->alpha, a->lambda_rel, a->p, s, st),
                                         "scales"))
            return e;
        for (int i = 1; i < 4; ++i)
            if (ttq_status e = markers(i)) return e;
        return TTQ_OK;
    }
    // The quantizer evaluates the scales of its channels from (ssq, lambda)
    // with the same arithmetic as ttq_awq_scales, and stores s.
    const ttq::QScaleSrc qs{ssq, bsum, (double)a->lambda_rel, (double)a->T, (double)a->alpha / (double)a->p, s};
    // Prompt-sized projections: the quantizer also writes the dequantized
    // weight (into the scratch area, free again once the statistics are
    // reduced) and the projection is a plain matrix-core GEMM on it.
    const bool dq = use_dequant_gemm(a->T, xf32, a->K, a->ldx);
    uint16_t* wq = dq ? (uint16_t*)scratch : nullptr;
    if (ttq_status e = device_status(
            ttq::launch_quantize(a->W, a->wt == TTQ_F32, a->M, a->K, a->ldw, s, a->bits, a->group, a->B,
                                 a->A, a->rank, (uint32_t*)codes, scale, zero, wq, st, &qs, timer(1)),
            "quantize"))
        return e;
    if (ttq::qgemv_gs_eligible(a->T, a->K, a->M, a->bits, a->group, xf32, a->ldx)) {
        if (ttq_status e = device_status(
                ttq::launch_qgemv_gs(a->X, xf32, a->T, a->K, a->ldx, s, (const uint32_t*)codes, scale, zero, a->M,
                                     a->bits, a->group, a->Y, a->yt == TTQ_F32, a->ldy, scratch, st, timer(2)),
                "qgemv"))
            return e;
    } else if (ttq::qgemv_sk_eligible(a->T, a->K, a->ldx, xf32)) {
        if (ttq_status e = device_status(
                ttq::launch_qgemv_sk(a->X, xf32, a->T, a->K, a->ldx, s, (const uint32_t*)codes, scale, zero, a->M,
                                     a->bits, a->group, a->Y, a->yt == TTQ_F32, a->ldy, (float*)scratch, st,
                                     timer(2)),
                "qgemv"))
            return e;
    } else if (ttq::qgemv_supported(a->T, a->K, a->ldx, xf32)) {
        if (ttq_status e = device_status(
                ttq::launch_qgemv(a->X, xf32, a->T, a->K, a->ldx, s, (const uint32_t*)codes, scale, zero, a->M,
                                  a->bits, a->group, a->Y, a->yt == TTQ_F32, a->ldy, st, timer(2)),
                "qgemv"))
            return e;
    } else if (dq) {
        // With low-rank factors: Z = X A^T on the matrix cores first, then the
        // GEMM adds Z B^T in its epilogue (no second pass over Y).
        ttq::LowrankEpilogue lre{nullptr, a->B, a->rank};
        const bool fuse = a->rank > 0 && ttq::lowrank_z_mfma_ok(xf32, a->T, a->K, a->ldx, a->A);
        if (fuse) {
            float* Z = (float*)((char*)scratch + ws_qgemm(a->T, a->K, a->M));
            lre.nz = ttq::lowrank_zm_parts(a->T, a->K);
            if (ttq_status e = device_status(ttq::launch_lowrank_z(a->X, xf32, a->T, a->K, a->ldx, a->A, a->rank, Z,
                                                                   st, timer(3), lre.nz),
                                             "lowrank Z"))
                return e;
            lre.Z = Z;
        }
        if (ttq_status e = device_status(ttq::launch_gemm_bf16((const uint16_t*)a->X, a->T, a->K, a->ldx, wq,
                                                               a->K, a->M, a->Y, a->yt == TTQ_F32, a->ldy, st,
                                                               timer(2), fuse ? &lre : nullptr,
                                                               fuse ? nullptr : ttq::split_ws_after(wq, a->M, a->K)),
                                         "gemm"))
            return e;
        if (fuse) return TTQ_OK;
    } else if (ttq_status e = device_status(
                   ttq::launch_qgemm(a->X, xf32, a->T, a->K, a->ldx, s, (const uint32_t*)codes, scale, zero,
                                     a->M, a->bits, a->group, a->Y, a->yt == TTQ_F32, a->ldy, nullptr, st,
                                     timer(2)),
                   "qgemm")) {
        return e;
    }
    if (a->rank > 0)
        return device_status(ttq::launch_lowrank(a->X, xf32, a->T, a->K, a->ldx, a->A, a->B, a->M, a->rank, a->Y,
                                                 a->yt == TTQ_F32, a->ldy, (float*)scratch, st, timer(3)),
                             "lowrank");
    return markers(3);
}

}  // extern "C"

namespace ttq {

ttq_status linear_check(const ttq_linear_args* a, size_t* need) {
    g_last_error.clear();
    if (ttq_status e = check_linear(a)) return e;
    *need = a->T == 0 ? 0 : state_layout(a->T, a->K, a->M, a->bits, a->group, a->rank).total;
    return TTQ_OK;
}

ttq_status set_error(ttq_status st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace ttq

extern "C" {

ttq_status ttq_linear(const ttq_linear_args* a, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (ttq_status e = check_linear(a)) return e;
    if (a->T == 0) return TTQ_OK;   // no prompt tokens: nothing to estimate or project
    const StateLayout L = state_layout(a->T, a->K, a->M, a->bits, a->group, a->rank);
    if (ttq_status e = check_ws(ws, ws_bytes, L.total)) return e;
    char* w = (char*)ws;
    double* ssq = a->ssq ? a->ssq : (double*)(w + L.ssq);
    double* bsum = (double*)(w + L.bsum);
    hipStream_t st = as_stream(stream);
    // Statistics (sums of |x|^p); the reduction also leaves the 16-channel
    // block sums of c.
    const StageMarks sm{a->stage_events, st};
    if (ttq_status e = device_status(ttq::launch_stats(a->X, a->xt == TTQ_F32, a->T, a->K, a->ldx, ssq, 0, st,
                                                       bsum, sm.timer(0), (double)a->p),
                                     "stats"))
        return e;
    return linear_layer(a, ssq, bsum, w, L, st);
}

// Shared statistics: [ssq K fp64 | block sums] at the head of the workspace,
// then one layer's state and scratch at a time (layers run in order).
static size_t shared_head(int64_t K) { return round_up((size_t)K * 8) + round_up((size_t)((K + 15) / 16) * 8); }

size_t ttq_linear_shared_workspace_bytes(const ttq_linear_args* layers, int n) {
    if (layers == nullptr || n < 1) return 0;
    size_t mx = 0;
    for (int i = 0; i < n; ++i) {
        const ttq_linear_args* a = &layers[i];
        if (ttq_workspace_bytes(a->T, a->K, a->M, a->bits, a->group, a->rank) == 0) return 0;
        const size_t t = state_layout(a->T, a->K, a->M, a->bits, a->group, a->rank).total;
        if (t > mx) mx = t;
    }
    return shared_head(layers[0].K) + mx;
}

ttq_status ttq_linear_shared(const ttq_linear_args* layers, int n, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    TTQ_REQUIRE(layers != nullptr && n >= 1 && n <= 64, "layers: null, or n not in [1, 64]");
    const ttq_linear_args* a0 = &layers[0];
    for (int i = 0; i < n; ++i) {
        const ttq_linear_args* a = &layers[i];
        if (ttq_status e = check_linear(a)) return e;
        TTQ_REQUIRE(a->X == a0->X && a->xt == a0->xt && a->T == a0->T && a->K == a0->K && a->ldx == a0->ldx,
                    "layer %d: X, xt, T, K and ldx must equal layer 0's (one shared input)", i);
        TTQ_REQUIRE(a->alpha == a0->alpha && a->lambda_rel == a0->lambda_rel && a->p == a0->p,
                    "layer %d: alpha, lambda_rel and p must equal layer 0's", i);
        TTQ_REQUIRE(a->stage_events == nullptr, "layer %d: stage events are not recorded for shared layers", i);
        TTQ_REQUIRE(i == 0 || a->ssq == nullptr, "layer %d: only layer 0 receives the shared statistics", i);
    }
    if (a0->T == 0) return TTQ_OK;
    const size_t need = ttq_linear_shared_workspace_bytes(layers, n);
    TTQ_REQUIRE(need > 0, "sizes not accepted");
    if (ttq_status e = check_ws(ws, ws_bytes, need)) return e;
    char* w = (char*)ws;
    const size_t head = shared_head(a0->K);
    double* ssq = a0->ssq ? a0->ssq : (double*)w;
    double* bsum = (double*)(w + round_up((size_t)a0->K * 8));
    char* wl = w + head;
    hipStream_t st = as_stream(stream);
    if (ttq_status e = device_status(ttq::launch_stats(a0->X, a0->xt == TTQ_F32, a0->T, a0->K, a0->ldx, ssq, 0, st,
                                                       bsum, {}, (double)a0->p),
                                     "stats"))
        return e;
    for (int i = 0; i < n; ++i) {
        const ttq_linear_args* a = &layers[i];
        const StateLayout L = state_layout(a->T, a->K, a->M, a->bits, a->group, a->rank);
        if (ttq_status e = linear_layer(a, ssq, bsum, wl, L, st)) return e;
    }
    return TTQ_OK;
}

}  // extern "C"
