// Per-prompt low-rank factors of W diag(s) by randomized subspace iteration.
//
// [TTQ §method b5]: the low-rank factors are dynamic, i.e. formed for each
// prompt from the weight and this prompt's scales.  The top-r factors of
// A_s = W diag(s) are estimated with the randomized range finder plus q
// power iterations (Halko, Martinsson and Tropp, "Finding structure with
// randomness", SIAM Review 2011), then the SVD of the small projected
// matrix:
//   Q = orth(A_s Om^T);  q times: Q = orth(A_s orth(A_s^T Q));
//   P = W^T Q  (so C = Q^T A_s = P^T diag(s));  C C^T = U~ S^2 U~^T;
//   B = Q U~_r S_r,  A[k][j] = (P U~)[j][k] / S_k   (= V_r^T diag(1/s)).
// Om (l x K, l <= 32) is the caller's Gaussian test matrix.
//
// The passes over W are skinny products on the matrix cores (the Z = X A^T
// kernel of the low-rank term, with W or a bf16 transpose of W as X and the
// fp32 l-column operand split into three bf16 terms).  orth() is CholQR2:
// G = Y^T Y in fp64 (fixed-order reduction), G = R^T R, Y R^-1, twice.  The
// l x l eigenproblem is a cyclic Jacobi iteration in fp64 on one wave.
#include "common.hpp"
#include "launch.hpp"

namespace ttq {

constexpr int kFMaxL = 32;
constexpr int kGramRows = 64;                     // rows per Gram partial
constexpr int kGramStage = 64;                    // rows staged in LDS at a time

// Wt[j][o] = W[o][j] for o < M, 0 for M <= o < ldt (64 x 64 tiles via LDS).
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ W, int64_t M, int64_t K,
                                                        int64_t ldw, uint16_t* __restrict__ Wt, int64_t ldt) {
    __shared__ uint16_t tile[64][66];
    const int64_t o0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4
    for (int r = ty; r < 64; r += 4) {
        const int64_t o = o0 + r, j = j0 + tx;
        tile[r][tx] = (o < M && j < K) ? W[o * ldw + j] : (uint16_t)0;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t j = j0 + r, o = o0 + tx;
        if (j < K && o < ldt) Wt[j * ldt + o] = tile[tx][r];
    }
}

// out[i][j] = in[i][j] * s[j]   (l x K).
__global__ __launch_bounds__(256) void k_scale_cols(const float* __restrict__ in, int l, int64_t K,
                                                    const float* __restrict__ s, float* __restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)l * K) return;
    out[idx] = in[idx] * s[idx % K];
}

// Gram partials: chunk c (rows 64 c .. 64 c + 63 of Y [N][l], each row scaled
// by rs[n] if given) -> Gp[c][a][b] = sum_n y_na y_nb in fp64, rows in order
// (staged through LDS).
__global__ __launch_bounds__(1024) void k_gram_partial(const float* __restrict__ Y, int64_t N, int l,
                                                       const float* __restrict__ rs, double* __restrict__ Gp) {
    __shared__ double ys[kGramStage][kFMaxL];
    const int a = threadIdx.x / kFMaxL, b = threadIdx.x % kFMaxL;
    double acc = 0.0;
    for (int st = 0; st < kGramRows; st += kGramStage) {
        const int64_t n0 = (int64_t)blockIdx.x * kGramRows + st;
        __syncthreads();
        for (int idx = threadIdx.x; idx < kGramStage * l; idx += 1024) {
            const int r = idx / l, c = idx % l;
            const int64_t n = n0 + r;
            double v = 0.0;
            if (n < N) v = (double)Y[n * l + c] * (rs ? (double)rs[n] : 1.0);
            ys[r][c] = v;
        }
        __syncthreads();
        if (a < l && b < l)
            for (int r = 0; r < kGramStage; ++r) acc = __builtin_fma(ys[r][a], ys[r][b], acc);
    }
    if (a < l && b < l) Gp[((int64_t)blockIdx.x * l + a) * l + b] = acc;
}

// Sum of the chunk partials Gp[c] (l x l) by a 1024-thread block, into
// out[a][b] (LDS, row stride kFMaxL + 1): four groups of 256 threads add the
// chunks c = g, g + 4, ... (all loads independent), then the four group sums
// are added in group order.  Fixed order: bitwise reproducible.
__device__ void sum_partials(const double* __restrict__ Gp, int nchunks, int l, double (*part)[kFMaxL * kFMaxL],
                             double (*out)[kFMaxL + 1]) {
    const int grp = threadIdx.x >> 8, t = threadIdx.x & 255;
    const int ne = l * l;
    for (int e = t; e < ne; e += 256) {
        double acc = 0.0;
#pragma unroll 8
        for (int c = grp; c < nchunks; c += 4) acc += Gp[(int64_t)c * ne + e];
        part[grp][e] = acc;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < ne; e += 1024)
        out[e / l][e % l] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
    __syncthreads();
}

// G[a][b] = sum of the chunk partials.
__global__ __launch_bounds__(1024) void k_gram_reduce(const double* __restrict__ Gp, int nchunks, int l,
                                                      double* __restrict__ G) {
    __shared__ double part[4][kFMaxL * kFMaxL];
    __shared__ double g[kFMaxL][kFMaxL + 1];
    sum_partials(Gp, nchunks, l, part, g);
    for (int e = threadIdx.x; e < l * l; e += 1024) G[e] = g[e / l][e % l];
}

// One workgroup: G = sum of the partials (sum_partials); G = R^T R (R upper,
// right-looking Cholesky, one thread per entry), written to Rout.  A pivot
// <= 0 (exactly dependent columns, e.g. a zero weight) gives R_kk = 1 and
// R_kj = 0, so that column of Y R^-1 is the (zero) residual; `bad` counts
// such pivots (diagnostics only).
__global__ __launch_bounds__(1024) void k_chol(const double* __restrict__ Gp, int nchunks, int l,
                                               double* __restrict__ Rout, int* __restrict__ bad) {
    __shared__ double part[4][kFMaxL * kFMaxL];
    __shared__ double g[kFMaxL][kFMaxL + 1];
    __shared__ int nbad;
    const int a = threadIdx.x / kFMaxL, b = threadIdx.x % kFMaxL;
    if (threadIdx.x == 0) nbad = 0;
    const bool in = a < l && b < l;
    sum_partials(Gp, nchunks, l, part, g);
    for (int k = 0; k < l; ++k) {
        const double d = g[k][k];
        __syncthreads();
        if (a == k && in && b >= k)
            g[k][b] = d > 0.0 ? ((b == k) ? __builtin_sqrt(d) : g[k][b] / __builtin_sqrt(d)) : (b == k ? 1.0 : 0.0);
        if (threadIdx.x == 0 && !(d > 0.0)) nbad += 1;
        __syncthreads();
        if (in && a > k && b >= a) g[a][b] -= g[k][a] * g[k][b];
        __syncthreads();
    }
    if (in) Rout[a * l + b] = b >= a ? g[a][b] : 0.0;
    if (threadIdx.x == 0) *bad = nbad;
}

// out = (rs o Y) R^-1 per row n of Y [N][l]: q R = y by forward substitution
// (q_c = (y_c - sum_{k<c} q_k R_kc) / R_cc), in fp64, rounded to fp32.  A
// group of 32 lanes owns one row (lane c computes q_c; the q_k it needs come
// from lanes k < c by shuffles, in order).
// mode 0: out [N][l].  mode 1: out [l][ldo] transposed, times cs[n] if given
// (columns N <= n < ldo are zero).
__global__ __launch_bounds__(256) void k_apply_r(const float* __restrict__ Y, int64_t N, int l,
                                                 const float* __restrict__ rs, const double* __restrict__ R,
                                                 int mode, const float* __restrict__ cs, float* __restrict__ out,
                                                 int64_t ldo) {
    __shared__ double rr[kFMaxL * kFMaxL];
    for (int i = threadIdx.x; i < l * l; i += 256) rr[i] = R[i];
    __syncthreads();
    const int c = threadIdx.x & 31;
    const int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 32;
    const int64_t lim = mode == 0 ? N : ldo;
    if (n >= lim) return;                         // uniform over the 32 lanes of a row
    if (n >= N) {                                 // padding columns of the transposed operand
        if (c < l) out[c * ldo + n] = 0.f;
        return;
    }
    const double y = c < l ? (double)Y[n * l + c] * (rs ? (double)rs[n] : 1.0) : 0.0;
    double v = y, q = 0.0;
    for (int k = 0; k < l; ++k) {
        // q_k is final once lane k has subtracted the terms of lanes < k.
        const double qk = __shfl(c == k ? v / rr[k * l + k] : 0.0, k, 32);
        if (c == k) q = qk;
        if (c > k) v = __builtin_fma(-qk, rr[k * l + c], v);
    }
    if (c < l) {
        if (mode == 0) out[n * l + c] = (float)q;
        else out[c * ldo + n] = (float)(q * ((cs != nullptr) ? (double)cs[n] : 1.0));
    }
}

// Symmetric l x l eigenproblem G [l][l] by cyclic Jacobi.  A sweep is l-1
// rounds of l/2 disjoint rotations (round-robin pairing); in a round every
// index i has a partner p_i and a pair (c_i, s_i) with column i of the
// rotation J equal to c_i e_i + s_i e_{p_i}, so one thread per entry forms
// (J^T G J)[i][j] and (V J)[i][j] from the previous round's values.
// Output: eigenvalues descending as sigma = sqrt(max(ev, 0)) and the matching
// eigenvectors as columns of U [l][l].
__global__ __launch_bounds__(1024) void k_jacobi(const double* __restrict__ G, int l, double* __restrict__ sig,
                                                 double* __restrict__ U) {
    // Two copies of A and V: a round reads one and writes the other, so it
    // needs two barriers (rotations known, new values written) instead of a
    // third one before overwriting in place.
    __shared__ double a[2][kFMaxL][kFMaxL + 1];
    __shared__ double v[2][kFMaxL][kFMaxL + 1];
    __shared__ double rc[kFMaxL], rs_[kFMaxL];
    __shared__ int ptn[kFMaxL];
    __shared__ double wsum[16];
    __shared__ int order[kFMaxL];
    const int tid = threadIdx.x;
    const int i = tid / l, j = tid % l;           // blockDim = l*l rounded up to whole waves
    const bool in = tid < l * l;
    const int n = l + (l & 1);                    // even count for the pairing (a dummy index if odd)
    if (in) {
        a[0][i][j] = G[i * l + j];
        v[0][i][j] = (i == j) ? 1.0 : 0.0;
    }
    __syncthreads();
    int cur = 0;
    double scale = 0.0;
    for (int k = 0; k < l; ++k) scale += a[0][k][k];
    for (int sweep = 0; sweep < 30; ++sweep) {
        // Off-diagonal mass, reduced over the block in a fixed order.
        double o = (in && i != j) ? a[cur][i][j] * a[cur][i][j] : 0.0;
        for (int m = 32; m >= 1; m >>= 1) o += __shfl_xor(o, m);
        if ((tid & 63) == 0) wsum[tid >> 6] = o;
        __syncthreads();
        double tot = 0.0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += wsum[w];
        // Stop when the off-diagonal mass is at the rounding level of the
        // largest eigenvalues (cyclic Jacobi converges quadratically).
        if (!(tot > 1e-28 * scale * scale)) break;
        for (int round = 0; round < n - 1; ++round) {
            const double (*ac)[kFMaxL + 1] = a[cur];
            if (tid < n / 2) {
                int p, q;
                if (tid == 0) { p = n - 1; q = round % (n - 1); }
                else { p = (round + tid) % (n - 1); q = (round + n - 1 - tid) % (n - 1); }
                if (p > q) { const int t = p; p = q; q = t; }
                double c = 1.0, sn = 0.0;
                if (q < l && ac[p][q] != 0.0) {
                    const double th = (ac[q][q] - ac[p][p]) / (2.0 * ac[p][q]);
                    const double t = (th >= 0.0 ? 1.0 : -1.0) / (__builtin_fabs(th) + __builtin_sqrt(th * th + 1.0));
                    c = 1.0 / __builtin_sqrt(t * t + 1.0);
                    sn = t * c;
                }
                // J[p][p] = c, J[q][p] = -s, J[p][q] = s, J[q][q] = c.
                if (p < l) { ptn[p] = q < l ? q : p; rc[p] = c; rs_[p] = q < l ? -sn : 0.0; }
                if (q < l) { ptn[q] = p; rc[q] = c; rs_[q] = sn; }
            }
            __syncthreads();
            if (in) {
                const int pi = ptn[i], pj = ptn[j];
                const double ci = rc[i], si = rs_[i], cj = rc[j], sj = rs_[j];
                a[cur ^ 1][i][j] = ci * (cj * ac[i][j] + sj * ac[i][pj]) + si * (cj * ac[pi][j] + sj * ac[pi][pj]);
                v[cur ^ 1][i][j] = cj * v[cur][i][j] + sj * v[cur][i][pj];
            }
            __syncthreads();
            cur ^= 1;
        }
    }
    // Sort by eigenvalue, descending (ties keep index order).
    const double (*af)[kFMaxL + 1] = a[cur];
    if (tid == 0) {
        for (int k = 0; k < l; ++k) order[k] = k;
        for (int k = 0; k < l; ++k) {
            int best = k;
            for (int m = k + 1; m < l; ++m)
                if (af[order[m]][order[m]] > af[order[best]][order[best]]) best = m;
            const int t = order[k]; order[k] = order[best]; order[best] = t;
        }
    }
    __syncthreads();
    if (tid < l) {
        const double ev = af[order[tid]][order[tid]];
        sig[tid] = __builtin_sqrt(ev > 0.0 ? ev : 0.0);
    }
    if (in) U[i * l + j] = v[cur][i][order[j]];
}

static unsigned jacobi_threads(int l) { return (unsigned)((l * l + 63) / 64 * 64); }

// B[o][k] = sig_k * sum_i Q[o][i] U[i][k]   (k < rank), one thread per entry.
__global__ __launch_bounds__(256) void k_form_b(const float* __restrict__ Q, int64_t M, int l, int rank,
                                                const double* __restrict__ U, const double* __restrict__ sig,
                                                float* __restrict__ B) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * rank) return;
    const int64_t o = idx / rank;
    const int k = (int)(idx % rank);
    double acc = 0.0;
    for (int i = 0; i < l; ++i) acc = __builtin_fma((double)Q[o * l + i], U[i * l + k], acc);
    B[idx] = (float)(acc * sig[k]);
}

// A[k][j] = (sum_i P[j][i] U[i][k]) / sig_k   (k < rank; P = W^T Q), one
// thread per entry (consecutive threads: consecutive j).
__global__ __launch_bounds__(256) void k_form_a(const float* __restrict__ P, int64_t K, int l, int rank,
                                                const double* __restrict__ U, const double* __restrict__ sig,
                                                float* __restrict__ A) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= K * rank) return;
    const int k = (int)(idx / K);
    const int64_t j = idx % K;
    double acc = 0.0;
    for (int i = 0; i < l; ++i) acc = __builtin_fma((double)P[j * l + i], U[i * l + k], acc);
    A[idx] = sig[k] > 0.0 ? (float)(acc / sig[k]) : 0.0f;
}

// ------------------------------------------------------------------ host

static int64_t round32(int64_t x) { return (x + 31) / 32 * 32; }

FactorsLayout factors_layout(int64_t M, int64_t K, int l) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    FactorsLayout F{};
    const int64_t M32 = round32(M);
    const int64_t N = M > K ? M : K;
    const int64_t NP = M32 > K ? M32 : K;
    size_t off = 0;
    F.wt = off;    off += up((size_t)K * M32 * 2);
    F.y = off;     off += up((size_t)N * l * 4);          // pass output [N][l]
    F.q1 = off;    off += up((size_t)N * l * 4);          // first CholQR basis [N][l]
    F.qrow = off;  off += up((size_t)M * l * 4);          // final Q [M][l]
    F.op = off;    off += up((size_t)l * NP * 4);         // next pass operand [l][K or M32]
    F.gp = off;    off += up((size_t)((N + kGramRows - 1) / kGramRows) * l * l * 8);
    F.rinv = off;  off += up((size_t)l * l * 8);
    F.g = off;     off += up((size_t)l * l * 8);
    F.sig = off;   off += up((size_t)l * 8);
    F.u = off;     off += up((size_t)l * l * 8);
    F.bad = off;   off += up(sizeof(int) * 2);
    F.total = off;
    return F;
}

bool factors_supported(bool wf32, int64_t M, int64_t K, int l, int rank) {
    return !wf32 && M > 0 && K > 0 && K % 32 == 0 && l >= 1 && l <= kFMaxL && rank >= 1 && rank <= l &&
           l <= M && l <= K && (int64_t)16 * (round32(M) > K ? round32(M) : K) * 2 < ((int64_t)1 << 31);
}

hipError_t launch_factors(const uint16_t* W, int64_t M, int64_t K, int64_t ldw, const float* s, const float* om,
                          int l, int q, int rank, float* B, float* A, char* ws, hipStream_t st) {
    const FactorsLayout F = factors_layout(M, K, l);
    const int64_t M32 = round32(M);
    uint16_t* Wt = (uint16_t*)(ws + F.wt);
    float* Y = (float*)(ws + F.y);
    float* Q1 = (float*)(ws + F.q1);
    float* Qrow = (float*)(ws + F.qrow);
    float* op = (float*)(ws + F.op);
    double* Gp = (double*)(ws + F.gp);
    double* Rm = (double*)(ws + F.rinv);
    double* Gm = (double*)(ws + F.g);
    double* sig = (double*)(ws + F.sig);
    double* U = (double*)(ws + F.u);
    int* bad = (int*)(ws + F.bad);
    hipError_t e;
#define TTQ_F(call) if ((e = (call)) != hipSuccess) return e
    TTQ_F(launch_kernel(k_transpose_bf16, dim3((unsigned)((K + 63) / 64), (unsigned)((M32 + 63) / 64)), dim3(256), 0,
                        st, nullptr, nullptr, W, M, K, ldw, Wt, M32));
    // orth(rs o Y) for Y [N][l]; result in op (mode 1, [l][ldo], times cs) and,
    // when qrow is given, also row-major there.
    auto cholqr2 = [&](const float* Yin, int64_t N, const float* rs, const float* cs, int64_t ldo,
                       float* qrow) -> hipError_t {
        const unsigned nch = (unsigned)((N + kGramRows - 1) / kGramRows);
        auto rows_grid = [](int64_t n) { return dim3((unsigned)((n * 32 + 255) / 256)); };
        hipError_t r;
        if ((r = launch_kernel(k_gram_partial, dim3(nch), dim3(1024), 0, st, nullptr, nullptr, Yin, N, l, rs, Gp)))
            return r;
        if ((r = launch_kernel(k_chol, dim3(1), dim3(1024), 0, st, nullptr, nullptr, (const double*)Gp, (int)nch, l,
                               Rm, bad)))
            return r;
        if ((r = launch_kernel(k_apply_r, rows_grid(N), dim3(256), 0, st, nullptr, nullptr, Yin, N, l, rs,
                               (const double*)Rm, 0, (const float*)nullptr, Q1, (int64_t)0)))
            return r;
        if ((r = launch_kernel(k_gram_partial, dim3(nch), dim3(1024), 0, st, nullptr, nullptr, (const float*)Q1, N,
                               l, (const float*)nullptr, Gp)))
            return r;
        if ((r = launch_kernel(k_chol, dim3(1), dim3(1024), 0, st, nullptr, nullptr, (const double*)Gp, (int)nch, l,
                               Rm, bad + 1)))
            return r;
        if (qrow != nullptr &&
            (r = launch_kernel(k_apply_r, rows_grid(N), dim3(256), 0, st, nullptr, nullptr, (const float*)Q1, N, l,
                               (const float*)nullptr, (const double*)Rm, 0, (const float*)nullptr, qrow,
                               (int64_t)0)))
            return r;
        return launch_kernel(k_apply_r, rows_grid(ldo), dim3(256), 0, st, nullptr, nullptr, (const float*)Q1, N, l,
                             (const float*)nullptr, (const double*)Rm, 1, cs, op, ldo);
    };
    // Y = W (Om diag(s))^T;  Q = orth(Y) as the [l][M32] operand of W^T Q.
    TTQ_F(launch_kernel(k_scale_cols, dim3((unsigned)(((int64_t)l * K + 255) / 256)), dim3(256), 0, st, nullptr,
                        nullptr, om, l, K, s, op));
    TTQ_F(launch_lowrank_z(W, false, M, K, ldw, op, l, Y, st, {}));
    TTQ_F(cholqr2(Y, M, nullptr, nullptr, M32, q == 0 ? Qrow : nullptr));
    for (int it = 0; it < q; ++it) {
        // P = W^T Q; Z = orth(diag(s) P) as the operand (diag(s) Z)^T [l][K].
        TTQ_F(launch_lowrank_z(Wt, false, K, M32, M32, op, l, Y, st, {}));
        TTQ_F(cholqr2(Y, K, s, s, K, nullptr));
        // Y = W (diag(s) Z);  Q = orth(Y).
        TTQ_F(launch_lowrank_z(W, false, M, K, ldw, op, l, Y, st, {}));
        TTQ_F(cholqr2(Y, M, nullptr, nullptr, M32, it == q - 1 ? Qrow : nullptr));
    }
    // P = W^T Q (in Y [K][l]); C C^T = Gram of diag(s) P; factors.
    TTQ_F(launch_lowrank_z(Wt, false, K, M32, M32, op, l, Y, st, {}));
    const unsigned nch = (unsigned)((K + kGramRows - 1) / kGramRows);
    TTQ_F(launch_kernel(k_gram_partial, dim3(nch), dim3(1024), 0, st, nullptr, nullptr, (const float*)Y, K, l, s, Gp));
    TTQ_F(launch_kernel(k_gram_reduce, dim3(1), dim3(1024), 0, st, nullptr, nullptr, (const double*)Gp, (int)nch, l,
                        Gm));
    TTQ_F(launch_kernel(k_jacobi, dim3(1), dim3(jacobi_threads(l)), 0, st, nullptr, nullptr, (const double*)Gm, l,
                        sig, U));
    TTQ_F(launch_kernel(k_form_b, dim3((unsigned)((M * rank + 255) / 256)), dim3(256), 0, st, nullptr, nullptr,
                        (const float*)Qrow, M, l, rank, (const double*)U, (const double*)sig, B));
    TTQ_F(launch_kernel(k_form_a, dim3((unsigned)((K * rank + 255) / 256)), dim3(256), 0, st, nullptr, nullptr,
                        (const float*)Y, K, l, rank, (const double*)U, (const double*)sig, A));
#undef TTQ_F
    return hipSuccess;
}

}  // namespace ttq
