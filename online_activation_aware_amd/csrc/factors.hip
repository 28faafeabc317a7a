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
// by rs[n] if given) -> Gp[c][a][b] = sum_n y_na y_nb in fp64, rows in order.
__global__ __launch_bounds__(1024) void k_gram_partial(const float* __restrict__ Y, int64_t N, int l,
                                                       const float* __restrict__ rs, double* __restrict__ Gp) {
    __shared__ double ys[kGramRows][kFMaxL];
    const int64_t n0 = (int64_t)blockIdx.x * kGramRows;
    for (int idx = threadIdx.x; idx < kGramRows * l; idx += 1024) {
        const int r = idx / l, c = idx % l;
        const int64_t n = n0 + r;
        double v = 0.0;
        if (n < N) v = (double)Y[n * l + c] * (rs ? (double)rs[n] : 1.0);
        ys[r][c] = v;
    }
    __syncthreads();
    const int a = threadIdx.x / kFMaxL, b = threadIdx.x % kFMaxL;
    if (a < l && b < l) {
        double acc = 0.0;
        for (int r = 0; r < kGramRows; ++r) acc = __builtin_fma(ys[r][a], ys[r][b], acc);
        Gp[((int64_t)blockIdx.x * l + a) * l + b] = acc;
    }
}

// One workgroup: G = sum of the partials in chunk order; G = R^T R (R upper,
// right-looking Cholesky); Rinv = R^-1 (upper).  `bad` records whether a
// pivot was <= 0 (diagnostics only).
__global__ __launch_bounds__(1024) void k_chol_inv(const double* __restrict__ Gp, int nchunks, int l,
                                                   double* __restrict__ Rinv, int* __restrict__ bad) {
    __shared__ double g[kFMaxL][kFMaxL + 1];
    __shared__ double rinv[kFMaxL][kFMaxL + 1];
    __shared__ int nbad;
    const int a = threadIdx.x / kFMaxL, b = threadIdx.x % kFMaxL;
    if (threadIdx.x == 0) nbad = 0;
    const bool in = a < l && b < l;
    if (in) {
        double acc = 0.0;
        for (int c = 0; c < nchunks; ++c) acc += Gp[((int64_t)c * l + a) * l + b];
        g[a][b] = acc;
    }
    __syncthreads();
    for (int k = 0; k < l; ++k) {
        // Row k of R: R_kk = sqrt(g_kk), R_kj = g_kj / R_kk (kept in g's row k).
        const double d = g[k][k];
        __syncthreads();
        // A pivot <= 0 (exactly dependent columns, e.g. a zero weight): R_kk = 1
        // and R_kj = 0, so that column of Y R^-1 is the (zero) residual.
        if (a == k && in && b >= k)
            g[k][b] = d > 0.0 ? ((b == k) ? __builtin_sqrt(d) : g[k][b] / __builtin_sqrt(d)) : (b == k ? 1.0 : 0.0);
        if (threadIdx.x == 0 && !(d > 0.0)) nbad += 1;
        __syncthreads();
        if (in && a > k && b >= a) g[a][b] -= g[k][a] * g[k][b];
        __syncthreads();
    }
    // Rinv column b by back substitution (one thread per column).
    if (threadIdx.x < l) {
        const int c = threadIdx.x;
        for (int i = l - 1; i >= 0; --i) {
            double v = (i == c) ? 1.0 : 0.0;
            for (int k = i + 1; k <= c; ++k) v -= g[i][k] * rinv[k][c];
            rinv[i][c] = (i <= c) ? v / g[i][i] : 0.0;
        }
    }
    __syncthreads();
    if (in) Rinv[a * l + b] = rinv[a][b];
    if (threadIdx.x == 0) *bad = nbad;
}

// out = (rs o Y) Rinv, per row n of Y [N][l], in fp64, rounded to fp32.
// mode 0: out [N][l].  mode 1: out [l][ldo] transposed, times cs[n] if given
// (columns N <= n < ldo are zero).
__global__ __launch_bounds__(256) void k_apply_rinv(const float* __restrict__ Y, int64_t N, int l,
                                                    const float* __restrict__ rs, const double* __restrict__ Rinv,
                                                    int mode, const float* __restrict__ cs, float* __restrict__ out,
                                                    int64_t ldo) {
    __shared__ double ri[kFMaxL * kFMaxL];
    for (int i = threadIdx.x; i < l * l; i += 256) ri[i] = Rinv[i];
    __syncthreads();
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t lim = mode == 0 ? N : ldo;
    if (n >= lim) return;
    if (n >= N) {                                 // padding columns of the transposed operand
        for (int c = 0; c < l; ++c) out[c * ldo + n] = 0.f;
        return;
    }
    // Static indices throughout (y stays in registers); l <= 32 is uniform.
    double y[kFMaxL];
    const double sc = rs ? (double)rs[n] : 1.0;
#pragma unroll
    for (int k = 0; k < kFMaxL; ++k) y[k] = k < l ? (double)Y[n * l + k] * sc : 0.0;
    const double cm = (mode == 1 && cs) ? (double)cs[n] : 1.0;
#pragma unroll
    for (int c = 0; c < kFMaxL; ++c) {
        if (c < l) {
            double v = 0.0;
#pragma unroll
            for (int k = 0; k <= c; ++k) v = __builtin_fma(y[k], ri[k * l + c], v);
            if (mode == 0) out[n * l + c] = (float)v;
            else out[c * ldo + n] = (float)(v * cm);
        }
    }
}

// Symmetric l x l eigenproblem (G = sum of Gram partials) by cyclic Jacobi
// on one wave: a sweep is l-1 rounds of l/2 disjoint rotations (round-robin
// pairing), each applied to the columns, then to the rows, and accumulated
// into V.  Output: eigenvalues descending as sigma = sqrt(max(ev, 0)) and
// the matching eigenvectors as columns of U [l][l].
__global__ __launch_bounds__(64) void k_jacobi(const double* __restrict__ Gp, int nchunks, int l,
                                               double* __restrict__ sig, double* __restrict__ U) {
    __shared__ double a[kFMaxL][kFMaxL + 1];
    __shared__ double v[kFMaxL][kFMaxL + 1];
    __shared__ double cs_[kFMaxL / 2], sn_[kFMaxL / 2];
    __shared__ int pp[kFMaxL / 2], qq[kFMaxL / 2];
    __shared__ int order[kFMaxL];
    __shared__ double offs;
    const int lane = threadIdx.x;
    const int n = l + (l & 1);                    // even count for the pairing (a dummy index if odd)
    for (int idx = lane; idx < kFMaxL * kFMaxL; idx += 64) {
        const int i = idx / kFMaxL, j = idx % kFMaxL;
        double acc = 0.0;
        if (i < l && j < l)
            for (int c = 0; c < nchunks; ++c) acc += Gp[((int64_t)c * l + i) * l + j];
        a[i][j] = acc;
        v[i][j] = (i == j) ? 1.0 : 0.0;
    }
    __syncthreads();
    double scale = 0.0;
    for (int i = 0; i < l; ++i) scale += a[i][i];
    for (int sweep = 0; sweep < 30; ++sweep) {
        if (lane == 0) {
            double o = 0.0;
            for (int i = 0; i < l; ++i)
                for (int j = 0; j < l; ++j)
                    if (i != j) o += a[i][j] * a[i][j];
            offs = o;
        }
        __syncthreads();
        if (!(offs > 1e-30 * scale * scale)) break;
        for (int round = 0; round < n - 1; ++round) {
            // Round-robin pairs: index n-1 fixed, the others rotate.
            if (lane < n / 2) {
                int p, q;
                if (lane == 0) { p = n - 1; q = round % (n - 1); }
                else { p = (round + lane) % (n - 1); q = (round + n - 1 - lane) % (n - 1); }
                if (p > q) { const int t = p; p = q; q = t; }
                double c = 1.0, s = 0.0;
                if (q < l && p < l && a[p][q] != 0.0) {
                    const double th = (a[q][q] - a[p][p]) / (2.0 * a[p][q]);
                    const double t = (th >= 0.0 ? 1.0 : -1.0) / (__builtin_fabs(th) + __builtin_sqrt(th * th + 1.0));
                    c = 1.0 / __builtin_sqrt(t * t + 1.0);
                    s = t * c;
                }
                pp[lane] = p; qq[lane] = q; cs_[lane] = c; sn_[lane] = s;
            }
            __syncthreads();
            // Columns: a[:, p], a[:, q] and v[:, p], v[:, q].
            for (int idx = lane; idx < (n / 2) * l; idx += 64) {
                const int r = idx / l, k = idx % l;
                const int p = pp[r], q = qq[r];
                if (q >= l) continue;
                const double c = cs_[r], s = sn_[r];
                const double akp = a[k][p], akq = a[k][q];
                a[k][p] = c * akp - s * akq;
                a[k][q] = s * akp + c * akq;
                const double vkp = v[k][p], vkq = v[k][q];
                v[k][p] = c * vkp - s * vkq;
                v[k][q] = s * vkp + c * vkq;
            }
            __syncthreads();
            // Rows: a[p, :], a[q, :].
            for (int idx = lane; idx < (n / 2) * l; idx += 64) {
                const int r = idx / l, k = idx % l;
                const int p = pp[r], q = qq[r];
                if (q >= l) continue;
                const double c = cs_[r], s = sn_[r];
                const double apk = a[p][k], aqk = a[q][k];
                a[p][k] = c * apk - s * aqk;
                a[q][k] = s * apk + c * aqk;
            }
            __syncthreads();
        }
    }
    // Sort by eigenvalue, descending (ties keep index order).
    if (lane == 0) {
        for (int i = 0; i < l; ++i) order[i] = i;
        for (int i = 0; i < l; ++i) {
            int best = i;
            for (int j = i + 1; j < l; ++j)
                if (a[order[j]][order[j]] > a[order[best]][order[best]]) best = j;
            const int t = order[i]; order[i] = order[best]; order[best] = t;
        }
    }
    __syncthreads();
    if (lane < l) {
        const double ev = a[order[lane]][order[lane]];
        sig[lane] = __builtin_sqrt(ev > 0.0 ? ev : 0.0);
    }
    for (int idx = lane; idx < l * l; idx += 64) {
        const int i = idx / l, k = idx % l;
        U[i * l + k] = v[i][order[k]];
    }
}

// B[o][k] = sig_k * sum_i Q[o][i] U[i][k]   (k < rank).
__global__ __launch_bounds__(256) void k_form_b(const float* __restrict__ Q, int64_t M, int l, int rank,
                                                const double* __restrict__ U, const double* __restrict__ sig,
                                                float* __restrict__ B) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= M) return;
    for (int k = 0; k < rank; ++k) {
        double acc = 0.0;
        for (int i = 0; i < l; ++i) acc = __builtin_fma((double)Q[o * l + i], U[i * l + k], acc);
        B[o * rank + k] = (float)(acc * sig[k]);
    }
}

// A[k][j] = (sum_i P[j][i] U[i][k]) / sig_k   (k < rank; P = W^T Q).
__global__ __launch_bounds__(256) void k_form_a(const float* __restrict__ P, int64_t K, int l, int rank,
                                                const double* __restrict__ U, const double* __restrict__ sig,
                                                float* __restrict__ A) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    for (int k = 0; k < rank; ++k) {
        double acc = 0.0;
        for (int i = 0; i < l; ++i) acc = __builtin_fma((double)P[j * l + i], U[i * l + k], acc);
        A[k * K + j] = sig[k] > 0.0 ? (float)(acc / sig[k]) : 0.0f;
    }
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
    double* Rinv = (double*)(ws + F.rinv);
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
        hipError_t r;
        if ((r = launch_kernel(k_gram_partial, dim3(nch), dim3(1024), 0, st, nullptr, nullptr, Yin, N, l, rs, Gp)))
            return r;
        if ((r = launch_kernel(k_chol_inv, dim3(1), dim3(1024), 0, st, nullptr, nullptr, (const double*)Gp,
                               (int)nch, l, Rinv, bad)))
            return r;
        if ((r = launch_kernel(k_apply_rinv, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, nullptr, nullptr,
                               Yin, N, l, rs, (const double*)Rinv, 0, (const float*)nullptr, Q1, (int64_t)0)))
            return r;
        if ((r = launch_kernel(k_gram_partial, dim3(nch), dim3(1024), 0, st, nullptr, nullptr, (const float*)Q1, N,
                               l, (const float*)nullptr, Gp)))
            return r;
        if ((r = launch_kernel(k_chol_inv, dim3(1), dim3(1024), 0, st, nullptr, nullptr, (const double*)Gp,
                               (int)nch, l, Rinv, bad + 1)))
            return r;
        if (qrow != nullptr &&
            (r = launch_kernel(k_apply_rinv, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, nullptr, nullptr,
                               (const float*)Q1, N, l, (const float*)nullptr, (const double*)Rinv, 0,
                               (const float*)nullptr, qrow, (int64_t)0)))
            return r;
        return launch_kernel(k_apply_rinv, dim3((unsigned)((ldo + 255) / 256)), dim3(256), 0, st, nullptr, nullptr,
                             (const float*)Q1, N, l, (const float*)nullptr, (const double*)Rinv, 1, cs, op, ldo);
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
    TTQ_F(launch_kernel(k_jacobi, dim3(1), dim3(64), 0, st, nullptr, nullptr, (const double*)Gp, (int)nch, l, sig, U));
    TTQ_F(launch_kernel(k_form_b, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, st, nullptr, nullptr,
                        (const float*)Qrow, M, l, rank, (const double*)U, (const double*)sig, B));
    TTQ_F(launch_kernel(k_form_a, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, nullptr, nullptr,
                        (const float*)Y, K, l, rank, (const double*)U, (const double*)sig, A));
#undef TTQ_F
    return hipSuccess;
}

}  // namespace ttq
