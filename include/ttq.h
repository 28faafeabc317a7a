/*
 * libttq — activation-aware test-time quantization (TTQ) of one linear layer,
 * per prompt, on AMD MI355X (gfx950).
 *
 * Source of the method: the nubint.ai review page "TTQ: Activation-Aware
 * Test-Time Quantization to Accelerate LLM Inference On The Fly", section
 * "proposed method" (bullets b1..b7).  "[TTQ §method b3]" below means its
 * third bullet.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Shapes: T tokens, K input channels, M output channels.
 *    X is [T][K] row-major with row stride ldx (elements),
 *    W is [M][K] row-major with row stride ldw (the Linear weight layout),
 *    Y is [T][M] row-major with row stride ldy.
 *  - Every pointer is DEVICE memory, allocated and owned by the caller; the
 *    library allocates nothing and never synchronises.  Every call only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream)
 *    and returns; results are ready when the stream reaches that point.
 *    Global state: the calling thread's last error text, and a per-device
 *    memo of kernel residency queried from the runtime once (a property of
 *    the code object: it never changes a result).  Calls are safe from any
 *    thread and on any stream.
 *  - Packed codes: for each output row, the K codes form a little-endian bit
 *    stream (code j occupies stream bits [bits*j, bits*j + bits), least
 *    significant bit first; stream bit i is bit i%32 of int32 word i/32).
 *    codes is dense: [M][K*bits/32] int32.
 *  - Per-group step and zero point: fp16 bit patterns, dense [M][K/group];
 *    the group of channel j is j / group (consecutive input channels of one
 *    output row).  The zero point is an integer stored as fp16.
 *  - Argument checks run on the host before any HIP call.  A failed check
 *    returns TTQ_ERR_INVALID (or TTQ_ERR_UNSUPPORTED for well-formed but
 *    unimplemented options) and launches nothing.  A failed launch returns
 *    TTQ_ERR_DEVICE.  Faults during execution surface at the caller's next
 *    synchronisation.  After a non-OK status the outputs are undefined.
 *    ttq_last_error() describes the last non-OK status of the calling thread.
 *  - Alignment: X, W and codes base pointers 16-byte aligned and the X/W row
 *    strides a multiple of 16 bytes; Y aligned to its element size, any row
 *    stride >= M; s 16-byte aligned; ssq 8-byte aligned; workspace 256-byte
 *    aligned.
 *  - Limits: K a positive multiple of 32 (of 8 for ttq_stats), at most 2^18;
 *    T, M and row strides at most 2^30; bits in
 *    {2,3,4,5}; group in {16,32,64,128} dividing K; 0 <= rank <= 64
 *    (ttq_lowrank_factors: rank <= l <= 32).
 *    T == 0 or M == 0 is a valid empty call (nothing is launched, except
 *    that ttq_stats with accumulate == 0 still zeroes ssq).
 *  - Inputs are expected to be finite.  The quantizer gives a NaN weight
 *    code 0 and leaves it out of its group's range; other non-finite inputs
 *    give unspecified (but memory-safe) outputs.
 */
#ifndef TTQ_H
#define TTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TTQ_OK = 0,
    TTQ_ERR_INVALID = 1,      /* malformed arguments: nothing launched      */
    TTQ_ERR_UNSUPPORTED = 2,  /* well-formed but not implemented            */
    TTQ_ERR_DEVICE = 3        /* the HIP runtime refused a launch           */
} ttq_status;

typedef enum {
    TTQ_F32 = 0,              /* IEEE binary32                              */
    TTQ_BF16 = 1              /* bfloat16 (upper half of a binary32)        */
} ttq_dtype;

/*
 * ttq_stats — per-channel sum of squares of the prompt's activations.
 * [TTQ §method b2, b3]: the diagonal of the input covariance, estimated
 * online from the prompt itself.
 *   ssq[j] (+)= sum_{t<T} X[t][j]^2, accumulated in fp64.
 *   X: [T][K] fp32 or bf16 (xt), stride ldx >= K.   ssq: [K] fp64, output.
 *   accumulate != 0 adds to the existing ssq (chunked prefill), else
 *   overwrites it.  ws, ws_bytes: unused (the reduction runs in one
 *   kernel without partial sums in memory); any value, NULL included.
 *   All sums are reduced in a fixed order, so results are bitwise
 *   reproducible run to run.  K must be a multiple of 8.
 */
ttq_status ttq_stats(const void* X, int xt, int64_t T, int64_t K, int64_t ldx,
                     double* ssq, int accumulate, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * ttq_stats_p — per-channel sum of |x|^p, for a moment order p fixed in
 * advance.  [TTQ §method b4]: alpha, lambda and p are fixed, not searched;
 * p = 2 is the diagonal covariance of ttq_stats, p = 1 the mean absolute
 * activation of the original AWQ statistic.
 *   msum[j] (+)= sum_{t<T} |X[t][j]|^p in fp64: exact squares for p = 2,
 *   exact |x| for p = 1, fp64 pow(|x|, p) otherwise (0 for x = 0).
 *   p finite and > 0 (else TTQ_ERR_INVALID).  Everything else (X, msum,
 *   accumulate, ws, ordering and reproducibility) is as for ttq_stats, which
 *   is this call with p = 2.  Feed msum to ttq_awq_scales with the same p.
 */
ttq_status ttq_stats_p(const void* X, int xt, int64_t T, int64_t K, int64_t ldx,
                       float p, double* msum, int accumulate, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * ttq_awq_scales — shrunk AWQ per-channel scales.
 * [TTQ §method b2-b4]: c = ssq / n_tokens; lambda = lambda_rel * mean(c)
 * (shrinkage C + lambda I); s[j] = (c[j] + lambda)^(alpha / p), evaluated in
 * fp64 and rounded once to fp32; s[j] = 1 where c[j] + lambda == 0.
 * alpha, lambda_rel, p are fixed in advance (no search).
 *   ssq: [K] fp64 input, the sums of |x|^p from ttq_stats_p with the same p
 *   (sums of squares for p = 2).  s: [K] fp32 output.  n_tokens > 0.
 *   alpha and lambda_rel finite and >= 0; p finite and > 0.
 */
ttq_status ttq_awq_scales(const double* ssq, int64_t n_tokens, int64_t K,
                          float alpha, float lambda_rel, float p, float* s,
                          void* stream);

/*
 * ttq_quantize_groups — group-wise RTN of the scaled (residual) weight.
 * [TTQ §method b1] group-wise RTN; [TTQ §method b2] the weight is scaled by
 * s per input channel; [TTQ §method b5] with low-rank factors the residual
 * W - B A is quantized.
 *   v[o][j] = fp32( (W[o][j] - sum_{k<rank} B[o][k] A[k][j]) * s[j] ), the
 *     residual accumulated in fp64 in rank order; without factors this is
 *     the correctly rounded fp32 product W*s.
 *   Per group: mn = min(0, min v), mx = max(0, max v);
 *     step = fp16 rounded up of fp32(mx - mn) / (2^bits - 1) (1 if zero);
 *     zero = clamp(rne(-mn / step), 0, 2^bits - 1);
 *     code = clamp(rne(v / step) + zero, 0, 2^bits - 1).
 *   W: [M][K] fp32/bf16 (wt), stride ldw.  s: [K] fp32, or NULL for s = 1.
 *   B: [M][rank] fp32 dense, A: [rank][K] fp32 dense; both NULL iff rank 0.
 *   Outputs: codes [M][K*bits/32], scale_f16 and zero_f16 [M][K/group].
 *   Codes whose v/step lies within ~1e-5 of a step of a rounding boundary
 *   may differ from an exact-division evaluation (v * (1/step) is used).
 */
ttq_status ttq_quantize_groups(const void* W, int wt, int64_t M, int64_t K, int64_t ldw,
                               const float* s, int bits, int group,
                               const float* B, const float* A, int rank,
                               int32_t* codes, uint16_t* scale_f16, uint16_t* zero_f16,
                               void* stream);

/*
 * ttq_qgemm — the quantized projection Y = W_hat (X / s).
 * [TTQ §method b7] quantized projection kernel; [TTQ §method b1] QDQ:
 * W_hat[o][j] = (code - zero) * step; [TTQ §method b2] inputs divided by s.
 *   Y[t][o] = sum_j W_hat[o][j] * X[t][j] / s[j].
 *   For T >= 5 the dequantized weight (code - zero) * step / s[j] is
 *   rounded once to bf16 and multiplied with X on the matrix cores with fp32
 *   accumulation (bf16 X is used as is; fp32 X is split into two bf16 halves
 *   and the weight too, three products, for near-fp32 accuracy).
 *   X: [T][K] (xt), s: [K], codes/scale/zero as produced by
 *   ttq_quantize_groups for (M, K, bits, group).  Y: [T][M] fp32 or bf16
 *   (yt), overwritten.  Y must not overlap any input.
 *   Execution paths: for T <= 4 with K a multiple of 128 (decode steps) the
 *   vector ALUs compute step * (sum code * x/s - zero * sum x/s) per group
 *   in fp32, with no bf16 rounding; for bf16 X with 5 <= T <= 16, 4-bit
 *   codes, groups of 32, 64 or 128 and K a multiple of 128 the matrix cores
 *   compute the same per-group sums with x * (1/s) rounded once to bf16
 *   (formed in LDS by the same launch, with its 32-channel sums) and each
 *   code taken exactly as the bf16 number 128 + code (K split over
 *   workgroups of 64 rows: fp32 partials in ws, added in slice order by a
 *   second kernel); otherwise, for 5 <= T <= 128 with K a multiple
 *   of 128 (at most 16384) the codes stream straight into registers and are
 *   expanded there to the bf16 weights above; for bf16 X with T >= 192 and
 *   K a multiple of 64 the weight is dequantized once into ws (M*K bf16) and
 *   multiplied by a matrix-core GEMM; otherwise codes are dequantized tile
 *   by tile inside the GEMM kernel.  The last three see bitwise the same
 *   bf16 weights.
 *   For bf16 X with 12 <= T <= 16 (where the sums path does not apply) the
 *   expansion runs split over K (each workgroup: 64 rows, one K slice; fp32
 *   partials in ws, added in slice order by a second kernel).  The T >= 192
 *   GEMM also runs as two K slices when its 128 x 256 output tiles number
 *   fewer than 192 and K >= 8192 (a multiple of 128): fp32 partial products
 *   in ws, then Y = P0 + P1.
 *   ws: at least ttq_workspace_bytes(T, K, M, bits, group, 0) bytes (for
 *   5 <= T <= 16 and K a multiple of 128: the larger of S*T*M*4 for the
 *   S K slices of the sums path (whole 512-channel sets, at most 8 a slice,
 *   S*ceil(M/64) about 256; none when S = 1) and, when T >= 12, the split
 *   partials S'*T*M*4 for S' <= K/128 slices; M*K*2 when T >= 192, plus 2*T*M'*4 with M' = M
 *   rounded up to 4 when the GEMM runs as two K slices; each part rounded up
 *   to 256; none otherwise); only read and written by the kernels this call
 *   enqueues.
 */
ttq_status ttq_qgemm(const void* X, int xt, int64_t T, int64_t K, int64_t ldx,
                     const float* s, const int32_t* codes, const uint16_t* scale_f16,
                     const uint16_t* zero_f16, int64_t M, int bits, int group,
                     void* Y, int yt, int64_t ldy, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * ttq_qgemm_batched — one decode step of P prompts in one launch.
 * [TTQ §method b7] the quantized projection, for several prompts at once:
 * every prompt has its own quantized state (its own s, codes, steps and
 * zeros: TTQ quantizes per prompt), so this is P independent projections
 * sharing one launch.  Prompt p uses
 *   X + p*x_stride ([T][K], stride ldx, elements of xt), s + p*s_stride,
 *   codes + p*codes_stride (int32 words), scale_f16/zero_f16 + p*sz_stride,
 *   Y + p*y_stride ([T][M], stride ldy, elements of yt),
 * and gets exactly what ttq_qgemm gives for it alone (the same kernel, bit
 * for bit).  1 <= T <= 4, K a multiple of 128, 1 <= P <= 65535; strides
 * >= 0, keeping every prompt's X, s and codes 16-byte aligned; prompts'
 * X and Y regions must not overlap.  No workspace.
 */
ttq_status ttq_qgemm_batched(const void* X, int xt, int64_t P, int64_t T, int64_t K, int64_t ldx,
                             int64_t x_stride, const float* s, int64_t s_stride,
                             const int32_t* codes, int64_t codes_stride,
                             const uint16_t* scale_f16, const uint16_t* zero_f16, int64_t sz_stride,
                             int64_t M, int bits, int group, void* Y, int yt, int64_t ldy,
                             int64_t y_stride, void* stream);

/*
 * ttq_lowrank_add — Y += B (A X), the dynamic low-rank term.
 * [TTQ §method b5]: W = W_q + B A, so the layer adds B (A X) to the
 * quantized projection.  Computed in fp32: Z[t][k] = sum_j A[k][j] X[t][j],
 * then Y[t][o] += sum_k B[o][k] Z[t][k].
 *   X: [T][K] (xt), A: [rank][K] fp32, B: [M][rank] fp32, Y: [T][M] (yt),
 *   updated in place.  ws: at least ttq_workspace_bytes(T, K, M, 2, 32, rank).
 */
ttq_status ttq_lowrank_add(const void* X, int xt, int64_t T, int64_t K, int64_t ldx,
                           const float* A, const float* B, int64_t M, int rank,
                           void* Y, int yt, int64_t ldy, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * ttq_lowrank_factors — the dynamic low-rank factors of one prompt.
 * [TTQ §method b5]: W = W_q + B A with factors formed per prompt.  The top
 * `rank` factors of W diag(s) (s from this prompt's ttq_awq_scales) are
 * estimated by randomized subspace iteration (Halko, Martinsson and Tropp,
 * "Finding structure with randomness", 2011): with A_s = W diag(s),
 *   Q = orth(A_s omega^T);  q times: Q = orth(A_s orth(A_s^T Q));
 *   Q^T A_s = U~ S V^T;  B = Q U~_r S_r,  A = V_r^T diag(1/s),
 * so that B A approximates W and B (A X) acts on the raw input; feed them
 * to ttq_quantize_groups / ttq_linear with the same s.  orth() is a
 * Cholesky QR with an fp64 Gram matrix; the inner orth of each power
 * iteration is omitted (orth(A_s orth(A_s^T Q)) = orth(A_s A_s^T Q) exactly,
 * the inner orth being a right product with an upper triangular matrix of
 * positive diagonal); the passes over W run on the matrix cores with fp32
 * accuracy; the small eigenproblem is a fp64 Jacobi iteration.
 *   W: [M][K] bf16 (wt; fp32 W returns TTQ_ERR_UNSUPPORTED), stride ldw,
 *   K a multiple of 32.  s: [K] fp32.  omega: [l][K] fp32, the caller's
 *   Gaussian test vectors (one per row), 1 <= rank <= l <= 32, l <= M, K.
 *   q: power iterations, 0..64.  Outputs B: [M][rank] fp32, A: [rank][K]
 *   fp32, dense.  Singular vectors are determined up to sign (and within
 *   repeated singular values); B A is the unique part.  A zero weight gives
 *   zero factors.  ws: ttq_lowrank_factors_workspace_bytes(M, K, l) bytes,
 *   256-byte aligned (it holds a bf16 transpose of W); results are bitwise
 *   reproducible run to run.
 */
ttq_status ttq_lowrank_factors(const void* W, int wt, int64_t M, int64_t K, int64_t ldw,
                               const float* s, const float* omega, int l, int q, int rank,
                               float* B, float* A, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for ttq_lowrank_factors (0 for sizes it does not accept). */
size_t ttq_lowrank_factors_workspace_bytes(int64_t M, int64_t K, int l);

/*
 * Workspace size (bytes) sufficient for every call above and for ttq_linear
 * with these sizes (including the intermediate ssq, s, codes, steps and
 * zeros that ttq_linear keeps there when the caller does not supply them).
 * Returns 0 for arguments that no call accepts.
 */
size_t ttq_workspace_bytes(int64_t T, int64_t K, int64_t M, int bits, int group, int rank);

/*
 * ttq_linear — the whole per-prompt path of one linear layer.
 * [TTQ §method b1-b5, b7]: statistics of this prompt's X (sums of |x|^p,
 * ttq_stats_p) -> shrunk AWQ scales with the same p -> group RTN of
 * (W - B A) diag(s) -> quantized projection, plus B (A X) when rank > 0.
 * Equivalent to the five calls above in order.
 * The optional outputs (ssq, s, codes, scale_f16, zero_f16) receive the
 * prompt's quantization state so that later decode steps can call ttq_qgemm
 * on it; when NULL they live in the workspace.
 * Execution: statistics (the reduction also forms lambda), then one
 * quantizer pass that evaluates s for its channels (same arithmetic as
 * ttq_awq_scales), writes codes, steps and zeros, and for bf16 X with
 * T >= 192 and K a multiple of 64 also the dequantized weight into ws, which
 * the matrix-core GEMM then multiplies (otherwise the fused kernel of
 * ttq_qgemm runs); then the low-rank term.
 * stage_events: NULL, or TTQ_LINEAR_STAGE_EVENTS hipEvent_t handles created
 * by the caller: a (start, stop) pair for each of the statistics, the
 * quantizer, the projection and the low-rank term, in that order.  The
 * stage's first kernel stamps `start` when it starts and its last kernel
 * stamps `stop` when it ends (kernel timestamps: nothing extra is enqueued);
 * a stage that launches nothing (the low-rank term when rank == 0) records
 * both on `stream` as markers.  For per-stage timing; never blocks.
 */
#define TTQ_LINEAR_STAGE_EVENTS 8
typedef struct ttq_linear_args {
    const void* X;  int xt;  int64_t T;  int64_t K;  int64_t ldx;
    const void* W;  int wt;  int64_t M;  int64_t ldw;
    float alpha;  float lambda_rel;  float p;
    int bits;  int group;
    const float* B;  const float* A;  int rank;
    void* Y;  int yt;  int64_t ldy;
    double* ssq;  float* s;  int32_t* codes;  uint16_t* scale_f16;  uint16_t* zero_f16;
    void* const* stage_events;
} ttq_linear_args;

ttq_status ttq_linear(const ttq_linear_args* args, void* ws, size_t ws_bytes, void* stream);

/*
 * ttq_linear_shared — several layers that read the same X (q, k and v; gate
 * and up), with one statistics pass for all of them.
 * [TTQ §method b3]: the statistics are those of the layer input X, so
 * projections of the same input share them (and hence lambda and s).
 *   layers[0..n-1], 1 <= n <= 64: ttq_linear arguments that agree in X, xt,
 *   T, K, ldx, alpha, lambda_rel and p; M, W, bits, group, the low-rank
 *   factors, Y and the state outputs are per layer.  The statistics are
 *   reduced once (into layers[0].ssq if given; every other ssq must be
 *   NULL), then each layer runs the quantizer and projection of ttq_linear
 *   in order, with results bitwise equal to separate ttq_linear calls.
 *   stage_events must be NULL.  ws: ttq_linear_shared_workspace_bytes(
 *   layers, n) bytes (the statistics plus the largest layer's state and
 *   scratch; layers run one after another on the stream and reuse it).
 */
ttq_status ttq_linear_shared(const ttq_linear_args* layers, int n, void* ws, size_t ws_bytes,
                             void* stream);

/* Workspace bytes for ttq_linear_shared (0 when some layer's sizes are not accepted). */
size_t ttq_linear_shared_workspace_bytes(const ttq_linear_args* layers, int n);

/*
 * ttq_linear_noalloc — ttq_linear without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The library allocates
 * nothing here either: the workspace is a device array inside the library,
 * TTQ_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it runs on, held until the
 * process ends.  Arguments, results and the other checks are those of
 * ttq_linear; a layer whose ttq_workspace_bytes(T, K, M, bits, group, rank)
 * exceeds TTQ_NOALLOC_SCRATCH_BYTES returns TTQ_ERR_INVALID (give the state
 * outputs ssq, s, codes, scale_f16, zero_f16 to keep them out of the array).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from threads without ordering) race and give
 * undefined results.  The array's address is resolved on the first call on
 * each device (TTQ_ERR_DEVICE if that fails).
 */
#define TTQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ttq_status ttq_linear_noalloc(const ttq_linear_args* args, void* stream);

/* Static text for a status code. */
const char* ttq_status_str(int status);

/* Text describing the calling thread's last non-OK status ("" if none). */
const char* ttq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TTQ_H */
