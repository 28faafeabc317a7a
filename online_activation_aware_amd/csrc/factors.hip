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
// orth(Y) = Y R^-1 with Y^T Y = R^T R: a Cholesky QR with the Gram matrix
// accumulated in fp64 from the stored fp32 rows, which leaves Q orthonormal
// to fp32 rounding.  The inner orth of each power iteration is left out:
// orth(A_s^T Q) = A_s^T Q R^-1 with R upper triangular with a positive
// diagonal, and orth(X R^-1) = orth(X) for such R, so
// orth(A_s orth(A_s^T Q)) = orth(A_s A_s^T Q) exactly.
//
// Two launches per pass over W (one stream, no host synchronisation):
//  * k_fpass: Yp = X OP^T on the matrix cores for X = W or Wt (a bf16
//    transpose of W made once by k_transpose_bf16).  A workgroup owns 128
//    rows and one K slice and writes the slice's partial product.  It loads
//    its operand inputs first and its slice of X after them, then forms the
//    operand in LDS while X is in flight: the test vectors times s for the
//    first pass, s^2 o P for the passes over W after a pass over W^T, and
//    Q = Y R^-1 (fp64) for the passes over W^T.  OP is rounded to fp32 and
//    split into three bf16 terms hi + mid + lo (fp32 accuracy against the
//    exact bf16 X).
//  * k_fgram: adds the slice partials of 128 rows in slice order and, where
//    a Gram matrix is needed, forms the fp64 Gram partial of those rows
//    (of rs o Y); then k_fgram_sum (one workgroup) adds the partials in
//    block order and factors the sum (one wave: Cholesky and R^-1 in
//    registers, each step's pivot row and column of R exchanged through
//    LDS).
// Then k_fjacobi solves the l x l eigenproblem C C^T by parallel cyclic
// Jacobi in fp64 (2 x 2 blocks per thread, one barrier per round; a
// separate wave computes each round's rotations during the previous round)
// and forms the small transforms of B and A, which k_fform applies.
// Every reduction has a fixed order: results are bitwise reproducible.
#include "common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace ttq {

constexpr int kFMaxL = 32;
constexpr int kPassWaves = 8;
constexpr int kPassRows = 16 * kPassWaves;        // rows of X per pass workgroup
constexpr int kPassMaxKS = 512;                   // K slice per pass workgroup
constexpr int kGramRows = 128;                    // rows per Gram partial
constexpr int kGramThreads = 256;

static int64_t round32(int64_t x) { return (x + 31) / 32 * 32; }
static int round4(int x) { return (x + 3) / 4 * 4; }

// Wt[j][o] = W[o][j] for o < M, 0 for M <= o < ldt; 64 x 64 tiles, 16-byte
// loads and stores, the transposition in LDS.
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ W, int64_t M, int64_t K,
                                                        int64_t ldw, uint16_t* __restrict__ Wt, int64_t ldt) {
    __shared__ uint32_t tile[64][33];             // [o][j pair], 2 bf16 per word
    const int64_t o0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
    const int t = threadIdx.x;
    const int64_t rows = min((int64_t)64, M - o0);
    const rsrc_t rw = make_rsrc(W + o0 * ldw, ((rows - 1) * ldw + K) * 2);   // rows >= M read as 0
    {
        const int r = t >> 3, c8 = (t & 7) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rr = r + 32 * h;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (j0 + c8 < K)
                v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rw, (int)((rr * ldw + j0 + c8) * 2), 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) tile[rr][c8 / 2 + e] = v[e];
        }
    }
    __syncthreads();
    const int o8 = (t & 7) * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int jr = (t >> 3) + 32 * h;
        const int64_t j = j0 + jr;
        if (j >= K || o0 + o8 >= ldt) continue;
        u32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a = tile[o8 + 2 * e][jr >> 1], b = tile[o8 + 2 * e + 1][jr >> 1];
            const uint32_t lo = (jr & 1) ? (a >> 16) : (a & 0xFFFFu);
            const uint32_t hi = (jr & 1) ? (b >> 16) : (b & 0xFFFFu);
            out[e] = lo | (hi << 16);
        }
        *(u32x4*)(Wt + j * ldt + o0 + o8) = out;
    }
}

// hi + mid + lo bf16 split of two fp32 values (the remainder is below 2^-24
// of each), as packed pairs.
__device__ __forceinline__ void split3(float x0, float x1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    hi = pack_bf16x2(x0, x1);
    const float r0 = x0 - bf16lo_to_f32(hi), r1 = x1 - bf16hi_to_f32(hi);
    mid = pack_bf16x2(r0, r1);
    lo = pack_bf16x2(r0 - bf16lo_to_f32(mid), r1 - bf16hi_to_f32(mid));
}

// 1/sqrt(x) in fp64: the hardware estimate refined by two Newton steps (to
// fp64 rounding level).
__device__ __forceinline__ double rsq_f64(double x) {
    double y = __builtin_amdgcn_rsq(x);
    const double h = 0.5 * x;
    double e = __builtin_fma(-h * y, y, 0.5);
    y = __builtin_fma(y, e, y);
    e = __builtin_fma(-h * y, y, 0.5);
    return __builtin_fma(y, e, y);
}

// One wave: G = R^T R (R upper, right-looking Cholesky) and Rinv = R^-1,
// fp64.  Lane a holds row a of the working matrix in registers (G on
// entry, zero outside [l][l]).  Step k: lane k publishes its row, and every
// lane a its column-k entry R[a][k] (final for a < k), in LDS; each lane
// reads them back (the same addresses in every lane), forms
//   Rinv[a][k] = (delta_ak - sum_{m < k} Rinv[a][m] R[m][k]) / R_kk
// (the sum split over four accumulators, m mod 4, added (0 + 1) + (2 + 3))
// and, for a > k, subtracts G[a][k] G[k][b] / G[k][k] from its row.  Row k
// is final after step k: R[k][b] = row_k[b] / R_kk.  A pivot <= 0 (exactly
// dependent columns, e.g. a zero weight) gives R_kk = 1 and R_kj = 0, so
// that column of Y R^-1 is the (zero) residual.  pub: LDS scratch of
// 2 * kFMaxL doubles.  Writes Rinv [l][l] (zero below the diagonal).
__device__ __forceinline__ void chol_inverse_wave(const double (*g)[kFMaxL + 1], int l, double* __restrict__ pub,
                                                  double* __restrict__ Rinv) {
    const int a = threadIdx.x & (kWave - 1);
    double row[kFMaxL], z[kFMaxL];                // z[m] = Rinv[a][m]
    double dvself = 0.0;                          // 1 / R_aa (0 for a rejected pivot)
#pragma unroll
    for (int b = 0; b < kFMaxL; ++b) {
        row[b] = a < kFMaxL ? g[a][b] : 0.0;
        z[b] = 0.0;
    }
    double* rowk = pub;                           // [kFMaxL]
    double* colk = pub + kFMaxL;                  // [kFMaxL]: R[m][k]
#pragma unroll
    for (int k = 0; k < kFMaxL; ++k) {
        if (k >= l) continue;                     // uniform
        if (a == k) {
#pragma unroll
            for (int b = 0; b < kFMaxL; b += 2) *(double2*)(rowk + b) = double2{row[b], row[b + 1]};
        }
        if (a < k) colk[a] = row[k] * dvself;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the writes above have landed
        __builtin_amdgcn_wave_barrier();
        double rk[kFMaxL];
#pragma unroll
        for (int b = 0; b < kFMaxL; b += 2) {
            const double2 v = *(const double2*)(rowk + b);
            rk[b] = v.x;
            rk[b + 1] = v.y;
        }
        const double d = rk[k];
        const bool ok = d > 0.0;
        const double ir = ok ? rsq_f64(d) : 1.0;  // 1 / R_kk
        const double dv = ok ? ir : 0.0;          // R[k][b] = row_k[b] dv for b > k
        if (a == k) dvself = dv;
        double a4[4] = {a == k ? 1.0 : 0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int m = 0; m < k; ++m) a4[m & 3] = __builtin_fma(-z[m], colk[m], a4[m & 3]);
        const double yk = ((a4[0] + a4[1]) + (a4[2] + a4[3])) * ir;
        z[k] = yk;
        if (a < l) Rinv[a * l + k] = yk;
        // Trailing update of rows a > k.
        const double w = a > k ? row[k] * (dv * dv) : 0.0;
#pragma unroll
        for (int b = k + 1; b < kFMaxL; ++b)
            if (b < l) row[b] = __builtin_fma(-w, rk[b], row[b]);
        // Every lane has read rowk / colk before the next step rewrites them.
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
    }
}

// Operand of a pass: OP[i][k] for the K slice [kb, kb + kn).
//   Yprev == nullptr: OP[i][k] = om[i][k] * (cs ? cs[k] : 1)   (om [l][ldo]).
//   otherwise:        OP[i][k] = (sum_{c <= i} rs_k Yprev[k][c] Rinv[c][i]) * cs_k
//                     in fp64 (Rinv [l][l] upper triangular; Rinv == nullptr:
//                     the identity), rows k >= Nprev zero (Yprev [Nprev][LS]).
struct PassOp {
    const float* om;
    int64_t ldo;
    const float* Yprev;
    int64_t Nprev;
    const double* Rinv;
    const float* rs;
    const float* cs;
};

// Skinny product on the matrix cores: Yp[y][n][i] = sum over the K slice y
// of X[n][k] * OP[i][k], i < 16 RT (rows i >= l of OP are zero), stored with
// row stride LS.  X bf16 [N][ldx].  Wave w owns rows n0 + 16 w .. + 15;
// thread t forms operand column kb + t.
template <int RT>
__global__ __launch_bounds__(kPassWaves * kWave) void k_fpass(const uint16_t* __restrict__ X, int64_t N,
                                                              int64_t ldx, int64_t K, PassOp po, int l, int LS,
                                                              int64_t ks, float* __restrict__ Yp) {
    constexpr int kSteps = kPassMaxKS / 32;
    constexpr int kRow = kPassMaxKS / 2 + 4;      // words per plane row (16-byte pad)
    static_assert(kPassMaxKS == kPassWaves * kWave && kFMaxL * kFMaxL <= 2 * kPassMaxKS, "one operand row per thread");
    __shared__ uint32_t sop[3][16 * RT][kRow];
    __shared__ double rt[kFMaxL][kFMaxL];         // Rinv transposed: rt[i][c] = Rinv[c][i]
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int r16 = lane & 15, q = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * kPassRows;
    const int64_t kb = (int64_t)blockIdx.y * ks;
    const int kn = (int)min(ks, K - kb);          // a multiple of 32
    const int nsteps = kn / 32;
    const int64_t rows = min((int64_t)kPassRows, N - n0);
    const rsrc_t rx = make_rsrc(X + n0 * ldx, ((rows - 1) * ldx + K) * 2);   // rows >= N read as 0

    // Operand inputs first: the X loads issued after them stay in flight
    // while the operand is formed (loads complete in issue order).
    const int g8 = kn / 8;
    constexpr int kOmIt = (16 * RT * (kPassMaxKS / 8) + kPassWaves * kWave - 1) / (kPassWaves * kWave);
    float om8[kOmIt][8];
    const int64_t k = kb + tid;
    const bool kin = po.Yprev != nullptr && tid < kn && k < po.Nprev;
    f32x4 yv[kFMaxL / 4];
    double gv[2] = {0.0, 0.0};                    // Rinv entries tid, tid + 512
    double rsk = 1.0, sck = 1.0;
    if (po.Yprev == nullptr) {
#pragma unroll
        for (int it = 0; it < kOmIt; ++it) {
            const int idx = tid + it * kPassWaves * kWave;
            const int i = idx / g8, c8 = (idx % g8) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) om8[it][e] = 0.f;
            if (idx < 16 * RT * g8 && i < l) {
                const float* src = po.om + (int64_t)i * po.ldo + kb + c8;
#pragma unroll
                for (int e = 0; e < 8; ++e) om8[it][e] = src[e];
                if (po.cs != nullptr)
#pragma unroll
                    for (int e = 0; e < 8; ++e) om8[it][e] *= po.cs[kb + c8 + e];
            }
        }
    } else {
        if (po.Rinv != nullptr)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (tid + u * kPassWaves * kWave < l * l) gv[u] = po.Rinv[tid + u * kPassWaves * kWave];
        if (kin) {
            if (po.rs != nullptr) rsk = (double)po.rs[k];
            if (po.cs != nullptr) sck = (double)po.cs[k];
        }
#pragma unroll
        for (int c4 = 0; c4 < kFMaxL; c4 += 4)
            yv[c4 / 4] = (kin && c4 < LS) ? *(const f32x4*)(po.Yprev + k * LS + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    u32x4 xb[kSteps];
    const int64_t xrow = (int64_t)(16 * wave + r16) * ldx + kb + 8 * q;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
        xb[s] = s < nsteps ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rx, (int)((xrow + 32 * s) * 2), 0, 0))
                           : u32x4{0u, 0u, 0u, 0u};

    if (po.Yprev == nullptr) {
#pragma unroll
        for (int it = 0; it < kOmIt; ++it) {
            const int idx = tid + it * kPassWaves * kWave;
            if (idx >= 16 * RT * g8) continue;
            const int i = idx / g8, c8 = (idx % g8) * 8;
            u32x4 hi, mid, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t h0, m0, l0;
                split3(om8[it][2 * e], om8[it][2 * e + 1], h0, m0, l0);
                hi[e] = h0;
                mid[e] = m0;
                lo[e] = l0;
            }
            *(u32x4*)&sop[0][i][c8 / 2] = hi;
            *(u32x4*)&sop[1][i][c8 / 2] = mid;
            *(u32x4*)&sop[2][i][c8 / 2] = lo;
        }
    } else {
        // Row k = kb + tid of this slice, all outputs; pairs of rows are
        // packed into bf16 words by the even lane.
        float o[16 * RT];
        if (po.Rinv != nullptr) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int e = tid + u * kPassWaves * kWave;
                if (e < l * l) rt[e % l][e / l] = gv[u];
            }
            __syncthreads();                      // rt ready
            double y[kFMaxL];
#pragma unroll
            for (int c = 0; c < kFMaxL; ++c) y[c] = (double)yv[c / 4][c % 4] * rsk;
#pragma unroll
            for (int i = 0; i < 16 * RT; ++i) {
                o[i] = 0.f;
                if (i < l) {
                    double acc = 0.0;
#pragma unroll
                    for (int c = 0; c <= i; ++c)
                        if (c < l) acc = __builtin_fma(y[c], rt[i][c], acc);
                    o[i] = (float)(acc * sck);
                }
            }
        } else {
            const double sc2 = rsk * sck;
#pragma unroll
            for (int i = 0; i < 16 * RT; ++i) o[i] = i < l ? (float)((double)yv[i / 4][i % 4] * sc2) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16 * RT; ++i) {
            const float on = __shfl_xor(o[i], 1);
            if ((tid & 1) == 0 && tid < kn) {
                uint32_t hi, mid, lo;
                split3(o[i], on, hi, mid, lo);
                sop[0][i][tid >> 1] = hi;
                sop[1][i][tid >> 1] = mid;
                sop[2][i][tid >> 1] = lo;
            }
        }
    }
    __syncthreads();

    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        if (s >= nsteps) continue;                // wave-uniform
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int w = 16 * s + 4 * q;
            const u32x4 hi = *(const u32x4*)&sop[0][16 * rt + r16][w];
            const u32x4 mid = *(const u32x4*)&sop[1][16 * rt + r16][w];
            const u32x4 lo = *(const u32x4*)&sop[2][16 * rt + r16][w];
            acc[rt] = mfma_16x16x32(hi, xb[s], acc[rt]);
            acc[rt] = mfma_16x16x32(mid, xb[s], acc[rt]);
            acc[rt] = mfma_16x16x32(lo, xb[s], acc[rt]);
        }
    }
    // Lane holds OUT^T[16 rt + 4 q + i][n0 + 16 wave + r16], i = 0..3.
    const int64_t n = n0 + 16 * wave + r16;
    if (n < N) {
        float* yo = Yp + ((int64_t)blockIdx.y * N + n) * LS;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            if (16 * rt + 4 * q < LS) *(f32x4*)(yo + 16 * rt + 4 * q) = acc[rt];
    }
}

// Ysum[n] = sum of the S slice partials of row n (slice order) and the fp64
// Gram partial of rows kGramRows c .. + kGramRows - 1 scaled by rs[n] if
// given: Gp[c][a][b] = sum_n (rs_n y_na)(rs_n y_nb), rows in order
// (k_fgram_sum adds them).  Gp == nullptr: the slice sum only.
__global__ __launch_bounds__(kGramThreads) void k_fgram(const float* __restrict__ Yp, int S, int64_t N, int LS, int l,
                                                        const float* __restrict__ rs, float* __restrict__ Ysum,
                                                        double* __restrict__ Gp) {
    __shared__ double ys[kGramRows][kFMaxL + 2];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * kGramRows;
    const int g4 = LS / 4;
    for (int idx = tid; idx < kGramRows * g4; idx += kGramThreads) {
        const int r = idx / g4, c4 = (idx % g4) * 4;
        const int64_t n = n0 + r;
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        double sc = 0.0;
        if (n < N) {
            // Slices in order, eight loads in flight at a time.
            v = *(const f32x4*)(Yp + n * LS + c4);
            for (int y0 = 1; y0 < S; y0 += 8) {
                f32x4 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    w[u] = y0 + u < S ? *(const f32x4*)(Yp + ((int64_t)(y0 + u) * N + n) * LS + c4)
                                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (y0 + u < S)
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] += w[u][e];
            }
            *(f32x4*)(Ysum + n * LS + c4) = v;
            sc = rs != nullptr ? (double)rs[n] : 1.0;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) ys[r][c4 + e] = (double)v[e] * sc;
    }
    if (Gp == nullptr) return;
    __syncthreads();
    // Thread: the 4 x 4 block (ba, bb) of G over rows part, part + 4, ...
    // (part = tid % 4); the four parts are added by shuffles, (0 + 1) + (2 + 3).
    const int64_t ne = (int64_t)l * l;
    {
        const int blk = tid >> 2, part = tid & 3;
        const int ba = blk >> 3, bb = blk & 7;
        const bool act = 4 * ba < l && 4 * bb < l;
        double acc[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[u][w] = 0.0;
        if (act) {
#pragma unroll 4
            for (int r = part; r < kGramRows; r += 4) {
                double x[4], y[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    x[u] = ys[r][4 * ba + u];
                    y[u] = ys[r][4 * bb + u];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int w = 0; w < 4; ++w) acc[u][w] = __builtin_fma(x[u], y[w], acc[u][w]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc[u][w] += __shfl_xor(acc[u][w], 1);
                acc[u][w] += __shfl_xor(acc[u][w], 2);
            }
        if (act && part == 0) {
            double* gp = Gp + (int64_t)blockIdx.x * ne;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    if (4 * ba + u < l && 4 * bb + w < l) gp[(4 * ba + u) * l + 4 * bb + w] = acc[u][w];
        }
    }
}

// G = sum of the nch Gram partials in block order (one workgroup; a second
// launch after k_fgram instead of a completion count, since a device-scope
// fence in every k_fgram workgroup writes back and invalidates its XCD's L2)
// and, if Rinv is given, its Cholesky factor's inverse (chol_inverse_wave).
__global__ __launch_bounds__(kGramThreads) void k_fgram_sum(const double* __restrict__ Gp, int nch, int l,
                                                            double* __restrict__ G, double* __restrict__ Rinv) {
    __shared__ double gs[kFMaxL][kFMaxL + 1];
    __shared__ double pub[2 * kFMaxL];
    const int tid = threadIdx.x;
    const int64_t ne = (int64_t)l * l;
    for (int e = tid; e < ne; e += kGramThreads) {
        double acc = 0.0;
        for (int c0 = 0; c0 < nch; c0 += 32) {
            double v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = c0 + u < nch ? Gp[(int64_t)(c0 + u) * ne + e] : 0.0;
#pragma unroll
            for (int u = 0; u < 32; ++u) acc += v[u];
        }
        G[e] = acc;
        gs[e / l][e % l] = acc;
    }
    if (Rinv == nullptr) return;
    for (int e = tid; e < kFMaxL * kFMaxL; e += kGramThreads)
        if (e / kFMaxL >= l || e % kFMaxL >= l) gs[e / kFMaxL][e % kFMaxL] = 0.0;
    __syncthreads();
    if (tid < kWave) chol_inverse_wave(gs, l, pub, Rinv);
}

// Rotation that zeroes a_pq (p < q): J[p][p] = J[q][q] = c, J[p][q] = s,
// J[q][p] = -s with t = sgn(d) e / (|d| + r), d = a_qq - a_pp, e = 2 a_pq,
// r = sqrt(d^2 + e^2), c = 1/sqrt(1 + t^2), s = t c (Golub and Van Loan,
// Matrix Computations, the symmetric Schur decomposition), evaluated as
// c = sqrt(w), w = (|d| + r) / (2 r), and s = sgn(d) e / (2 r sqrt(w)),
// which follow from 1 + t^2 = 2 r / (|d| + r): two reciprocal square roots.
__device__ __forceinline__ void jacobi_cs(double app, double aqq, double apq, double& c, double& s) {
    c = 1.0;
    s = 0.0;
    if (apq == 0.0) return;
    const double d = aqq - app, e = 2.0 * apq;
    const double h = __builtin_fma(d, d, e * e);
    const double y = rsq_f64(h);                  // 1 / r
    const double w = 0.5 * (__builtin_fabs(d) + h * y) * y;
    const double z = rsq_f64(w);
    c = w * z;
    s = (d >= 0.0 ? 0.5 : -0.5) * e * y * z;
}

// Partner of index x in round r of the round-robin ordering of n = m + 1
// indices (x paired with m when x == r, m with r, otherwise with
// (2 r - x) mod m), or x itself when the partner is the padding index (>= l).
__device__ __forceinline__ int jacobi_partner(int x, int r, int m, int l) {
    int p;
    if (x == m) p = r;
    else if (x == r) p = m;
    else {
        p = 2 * r - x;
        p = p < 0 ? p + m : (p >= m ? p - m : p);
    }
    return p < l ? p : x;
}

// (J^T A J)[x][y] for the rotation of this round: column x of J is
// c_x e_x + s_x e_{p_x}.
__device__ __forceinline__ double jacobi_entry(const double (*a)[kFMaxL + 1], int x, int y, double cx, double sx,
                                               int px, double cy, double sy, int py) {
    const double t1 = __builtin_fma(sy, a[x][py], cy * a[x][y]);
    const double t2 = __builtin_fma(sy, a[px][py], cy * a[px][y]);
    return __builtin_fma(sx, t2, cx * t1);
}

// Symmetric l x l eigenproblem of G = C C^T by cyclic Jacobi: a sweep is
// n - 1 rounds of n/2 disjoint rotations in round-robin order (n = l rounded
// up to even; in round r pair t is (r, n - 1) for t = 0, else
// ((r + t) mod (n - 1), (r - t) mod (n - 1)); an index paired with n - 1 >= l
// is not rotated), tabulated once.  Each round forms A' = J^T A J and
// V' = V J: thread (tr, tc) of the first group owns the 2 x 2 block of A at
// the rows of pair tr and the columns of pair tc (the rotation mixes exactly
// those), thread (tr, tc) of the second group the same block of V, both
// reading the previous round's copy; meanwhile lanes t < n/2 of the last
// wave form the three entries of the next round's pair t from the same copy
// and its rotation, so a round needs one barrier.  Stops when the
// off-diagonal mass is at the rounding level of the trace (at most 30
// sweeps).  Then, with sigma_k = sqrt(max(ev, 0)) descending, U~ the
// matching eigenvectors and Rinv = R^-1 of the last basis (Q = YM R^-1):
//   TB = R^-1 U~_r diag(sigma_r),  TA = U~_r diag(1/sigma_r) (0 where
//   sigma = 0), both [l][rank] fp64.
// blockDim: 2 (n/2)^2 threads rounded up to whole waves, plus one wave.
__global__ __launch_bounds__(640) void k_fjacobi(const double* __restrict__ G, const double* __restrict__ Rinv, int l,
                                                 int rank, double* __restrict__ TB, double* __restrict__ TA) {
    __shared__ double a[2][kFMaxL][kFMaxL + 1];
    __shared__ double v[2][kFMaxL][kFMaxL + 1];
    __shared__ double rc[2][kFMaxL], rsn[2][kFMaxL];
    __shared__ int ptab[kFMaxL][kFMaxL / 2];      // pair t of round r: p | q << 8, p < q
    __shared__ int xtab[kFMaxL][kFMaxL];          // partner of x in round r (x itself if padding)
    __shared__ double wsum[16];
    __shared__ int order[kFMaxL];
    __shared__ double sg[kFMaxL];
    const int tid = threadIdx.x;
    const int nt = (int)blockDim.x, nw = nt >> 6;
    const bool pw = (tid >> 6) == nw - 1;         // the pair wave: the last one
    const int pt = tid & (kWave - 1);
    const int n = l + (l & 1), m = n - 1, np = n / 2, nb = np * np;
    const bool ta = tid < nb, tv = tid >= nb && tid < 2 * nb;
    const int bi = ta ? tid : tid - nb;
    const int tr = bi / np, tc = bi % np;
    for (int e = tid; e < l * l; e += nt) {
        a[0][e / l][e % l] = G[e];
        v[0][e / l][e % l] = (e / l == e % l) ? 1.0 : 0.0;
    }
    for (int e = tid; e < m * np; e += nt) {
        const int r = e / np, t = e % np;
        int p, q;
        if (t == 0) { p = r; q = m; }
        else { p = (r + t) % m; q = (r + m - t) % m; }
        if (p > q) { const int x = p; p = q; q = x; }
        ptab[r][t] = p | (q << 8);
        xtab[r][p] = q < l ? q : p;
        if (q < l) xtab[r][q] = p;
    }
    __syncthreads();
    auto publish = [&](int buf, int p, int q, double c, double s) {
        if (q < l) {
            rc[buf][p] = c; rsn[buf][p] = -s;
            rc[buf][q] = c; rsn[buf][q] = s;
        } else {
            rc[buf][p] = 1.0; rsn[buf][p] = 0.0;
        }
    };
    if (pw && pt < np) {                          // round 0 rotations from G
        const int pq = ptab[0][pt], p = pq & 255, q = pq >> 8;
        double c = 1.0, s = 0.0;
        if (q < l) jacobi_cs(a[0][p][p], a[0][q][q], a[0][p][q], c, s);
        publish(0, p, q, c, s);
    }
    __syncthreads();
    int cur = 0;
    double scale = 0.0;
    for (int k = 0; k < l; ++k) scale += a[0][k][k];
    for (int sweep = 0; sweep < 30; ++sweep) {
        double o = 0.0;
        for (int e = tid; e < l * l; e += nt)
            if (e / l != e % l) o = __builtin_fma(a[cur][e / l][e % l], a[cur][e / l][e % l], o);
        for (int msk = 32; msk >= 1; msk >>= 1) o += __shfl_xor(o, msk);
        if ((tid & 63) == 0) wsum[tid >> 6] = o;
        __syncthreads();
        double tot = 0.0;
        for (int w = 0; w < nw; ++w) tot += wsum[w];
        // Every thread holds the same tot; readfirstlane makes the exit
        // visibly uniform, so the round loop runs on scalar control flow.
        if (!__builtin_amdgcn_readfirstlane(tot > 1e-28 * scale * scale ? 1 : 0)) break;
        for (int r = 0; r < m; ++r) {
            const double (*ac)[kFMaxL + 1] = a[cur];
            if (ta || tv) {
                const int px = ptab[r][tr], py = ptab[r][tc];
                const int x0 = px & 255, x1 = px >> 8, y0 = py & 255, y1 = py >> 8;
                const bool xv = x1 < l, yv = y1 < l;
                const int x1c = xv ? x1 : x0, y1c = yv ? y1 : y0;
                const double cy0 = rc[cur][y0], sy0 = rsn[cur][y0];
                const double cy1 = rc[cur][y1c], sy1 = yv ? rsn[cur][y1c] : 0.0;
                if (ta) {
                    const double cx0 = rc[cur][x0], sx0 = rsn[cur][x0];
                    const double cx1 = rc[cur][x1c], sx1 = xv ? rsn[cur][x1c] : 0.0;
                    const double a00 = ac[x0][y0], a01 = yv ? ac[x0][y1c] : 0.0;
                    const double a10 = xv ? ac[x1c][y0] : 0.0, a11 = (xv && yv) ? ac[x1c][y1c] : 0.0;
                    // Columns (A J), then rows (J^T (A J)).
                    const double b00 = __builtin_fma(sy0, a01, cy0 * a00), b01 = __builtin_fma(sy1, a00, cy1 * a01);
                    const double b10 = __builtin_fma(sy0, a11, cy0 * a10), b11 = __builtin_fma(sy1, a10, cy1 * a11);
                    double (*an)[kFMaxL + 1] = a[cur ^ 1];
                    an[x0][y0] = __builtin_fma(sx0, b10, cx0 * b00);
                    if (yv) an[x0][y1] = __builtin_fma(sx0, b11, cx0 * b01);
                    if (xv) an[x1][y0] = __builtin_fma(sx1, b00, cx1 * b10);
                    if (xv && yv) an[x1][y1] = __builtin_fma(sx1, b01, cx1 * b11);
                } else {
                    // V J on rows x0, x1.
                    const double (*vc)[kFMaxL + 1] = v[cur];
                    double (*vn)[kFMaxL + 1] = v[cur ^ 1];
                    const double v00 = vc[x0][y0], v01 = vc[x0][y1c];
                    const double v10 = vc[x1c][y0], v11 = vc[x1c][y1c];
                    vn[x0][y0] = __builtin_fma(sy0, v01, cy0 * v00);
                    if (yv) vn[x0][y1] = __builtin_fma(sy1, v00, cy1 * v01);
                    if (xv) {
                        vn[x1][y0] = __builtin_fma(sy0, v11, cy0 * v10);
                        if (yv) vn[x1][y1] = __builtin_fma(sy1, v10, cy1 * v11);
                    }
                }
            }
            if (pw && pt < np) {                  // next round's rotation of pair pt
                const int pq2 = ptab[r + 1 == m ? 0 : r + 1][pt], p = pq2 & 255, q = pq2 >> 8;
                double c = 1.0, s = 0.0;
                if (q < l) {
                    const int pp = xtab[r][p], pq = xtab[r][q];
                    const double cp = rc[cur][p], sp = rsn[cur][p], cq = rc[cur][q], sq = rsn[cur][q];
                    jacobi_cs(jacobi_entry(ac, p, p, cp, sp, pp, cp, sp, pp),
                              jacobi_entry(ac, q, q, cq, sq, pq, cq, sq, pq),
                              jacobi_entry(ac, p, q, cp, sp, pp, cq, sq, pq), c, s);
                }
                publish(cur ^ 1, p, q, c, s);
            }
            __syncthreads();
            cur ^= 1;
        }
    }
    // Descending eigenvalue order (ties keep index order): rank of each index.
    const double (*af)[kFMaxL + 1] = a[cur];
    if (tid < l) {
        const double ev = af[tid][tid];
        int rk = 0;
        for (int k = 0; k < l; ++k) {
            const double ek = af[k][k];
            rk += (ek > ev || (ek == ev && k < tid)) ? 1 : 0;
        }
        order[rk] = tid;
    }
    __syncthreads();
    if (tid < l) {
        const double ev = af[order[tid]][order[tid]];
        sg[tid] = __builtin_sqrt(ev > 0.0 ? ev : 0.0);
    }
    __syncthreads();
    // U~[x][k] = v[x][order[k]].
    for (int e = tid; e < l * rank; e += nt) {
        const int x = e / rank, k = e % rank;
        const double sk = sg[k];
        double t = 0.0;
        for (int y = x; y < l; ++y) t = __builtin_fma(Rinv[x * l + y], v[cur][y][order[k]], t);
        TB[e] = t * sk;
        TA[e] = sk > 0.0 ? v[cur][x][order[k]] / sk : 0.0;
    }
}

// Blocks [0, nbb): B[o][k] = sum_c YM[o][c] TB[c][k] (o < M); the blocks
// after them: A[k][j] = sum_c P[j][c] TA[c][k] (j < K); k < rank, fp64 sums
// rounded to fp32.  YM and P have row stride LS; a block stages its 64 rows
// and the transform in LDS, and thread (r, g) forms outputs k = g, g + 4, ...
// of row r.
__global__ __launch_bounds__(256) void k_fform(const float* __restrict__ YM, int64_t M, const float* __restrict__ P,
                                               int64_t K, int LS, int l, int rank, const double* __restrict__ TB,
                                               const double* __restrict__ TA, float* __restrict__ B,
                                               float* __restrict__ A, unsigned nbb) {
    __shared__ float rows[64][kFMaxL + 1];
    __shared__ double tr[kFMaxL][kFMaxL];
    const int tid = threadIdx.x;
    const bool isb = blockIdx.x < nbb;
    const int64_t r0 = (int64_t)(isb ? blockIdx.x : blockIdx.x - nbb) * 64;
    const int64_t nrow = isb ? M : K;
    const float* src = isb ? YM : P;
    const double* T = isb ? TB : TA;
    for (int e = tid; e < l * rank; e += 256) tr[e / rank][e % rank] = T[e];
    const int g4 = LS / 4;
    for (int e = tid; e < 64 * g4; e += 256) {
        const int r = e / g4, c4 = (e % g4) * 4;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (r0 + r < nrow) x = *(const f32x4*)(src + (r0 + r) * LS + c4);
#pragma unroll
        for (int u = 0; u < 4; ++u) rows[r][c4 + u] = x[u];
    }
    __syncthreads();
    const int r = tid >> 2, g = tid & 3;
    const int64_t row = r0 + r;
    if (row >= nrow) return;
    double x[kFMaxL];
#pragma unroll
    for (int c = 0; c < kFMaxL; ++c) x[c] = c < l ? (double)rows[r][c] : 0.0;
    for (int k = g; k < rank; k += 4) {
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < kFMaxL; ++c)
            if (c < l) acc = __builtin_fma(x[c], tr[c][k], acc);
        if (isb) B[row * rank + k] = (float)acc;
        else A[(int64_t)k * K + row] = (float)acc;
    }
}

// ------------------------------------------------------------------ host

// K slices of a pass over N rows with reduction length K: slices of at most
// kPassMaxKS channels, more (down to 64 channels) while the row blocks alone
// leave most of the 256 compute units idle.
static int64_t pass_slice(int64_t N, int64_t K) {
    const int64_t rb = (N + kPassRows - 1) / kPassRows;
    int64_t ks = kPassMaxKS;
    while (ks > 64 && rb * ((K + ks - 1) / ks) < 256) ks /= 2;
    return ks;
}
static int64_t pass_slices(int64_t N, int64_t K) {
    const int64_t ks = pass_slice(N, K);
    return (K + ks - 1) / ks;
}

FactorsLayout factors_layout(int64_t M, int64_t K, int l) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    FactorsLayout F{};
    const int64_t M32 = round32(M);
    const int LS = round4(l);
    const int64_t N = M > K ? M : K;
    const int64_t ypn = pass_slices(M, K) * M > pass_slices(K, M32) * K ? pass_slices(M, K) * M
                                                                        : pass_slices(K, M32) * K;
    size_t off = 0;
    F.wt = off;    off += up((size_t)K * M32 * 2);
    F.yp = off;    off += up((size_t)ypn * LS * 4);        // pass partials [S][N][LS]
    F.ym = off;    off += up((size_t)M * LS * 4);          // summed W pass [M][LS]
    F.yk = off;    off += up((size_t)K * LS * 4);          // summed W^T pass [K][LS]
    F.gp = off;    off += up((size_t)((N + kGramRows - 1) / kGramRows) * l * l * 8);
    F.rinv = off;  off += up((size_t)l * l * 8);           // R^-1 of the latest basis
    F.g = off;     off += up((size_t)l * l * 8);           // the latest Gram matrix
    F.tb = off;    off += up((size_t)l * l * 8);
    F.ta = off;    off += up((size_t)l * l * 8);
    F.total = off;
    return F;
}

bool factors_supported(bool wf32, int64_t M, int64_t K, int64_t ldw, int l, int rank) {
    const int64_t M32 = round32(M);
    return !wf32 && M > 0 && K > 0 && K % 32 == 0 && l >= 1 && l <= kFMaxL && rank >= 1 && rank <= l &&
           l <= M && l <= K && ldw >= K && (int64_t)kPassRows * (ldw > M32 ? ldw : M32) * 2 < ((int64_t)1 << 31);
}

hipError_t launch_factors(const uint16_t* W, int64_t M, int64_t K, int64_t ldw, const float* s, const float* om,
                          int l, int q, int rank, float* B, float* A, char* ws, hipStream_t st) {
    const FactorsLayout F = factors_layout(M, K, l);
    const int64_t M32 = round32(M);
    const int LS = round4(l);
    uint16_t* Wt = (uint16_t*)(ws + F.wt);
    float* Yp = (float*)(ws + F.yp);
    float* YM = (float*)(ws + F.ym);
    float* YK = (float*)(ws + F.yk);
    double* Gp = (double*)(ws + F.gp);
    double* G = (double*)(ws + F.g);
    double* Rinv = (double*)(ws + F.rinv);
    double* TB = (double*)(ws + F.tb);
    double* TA = (double*)(ws + F.ta);
    hipError_t e;
#define TTQ_F(call) if ((e = (call)) != hipSuccess) return e
    TTQ_F(launch_kernel(k_transpose_bf16, dim3((unsigned)((K + 63) / 64), (unsigned)((M32 + 63) / 64)), dim3(256), 0,
                        st, nullptr, nullptr, W, M, K, ldw, Wt, M32));
    // Yp = slices of X OP^T (X: N rows, reduction length Kr); then the slice
    // sum into Ysum and (gram) the Gram matrix of rs o Ysum into G, factored
    // into Rinv when chol is set.
    auto pass = [&](const uint16_t* X, int64_t N, int64_t ldx, int64_t Kr, const PassOp& po, float* Ysum,
                    const float* rs, bool gram, bool chol) -> hipError_t {
        const int64_t ks = pass_slice(N, Kr);
        const int S = (int)((Kr + ks - 1) / ks);
        const dim3 g((unsigned)((N + kPassRows - 1) / kPassRows), (unsigned)S);
        hipError_t r = l <= 16 ? launch_kernel(k_fpass<1>, g, dim3(kPassWaves * kWave), 0, st, nullptr, nullptr, X,
                                               N, ldx, Kr, po, l, LS, ks, Yp)
                               : launch_kernel(k_fpass<2>, g, dim3(kPassWaves * kWave), 0, st, nullptr, nullptr, X,
                                               N, ldx, Kr, po, l, LS, ks, Yp);
        if (r != hipSuccess) return r;
        const unsigned nch = (unsigned)((N + kGramRows - 1) / kGramRows);
        r = launch_kernel(k_fgram, dim3(nch), dim3(kGramThreads), 0, st, nullptr, nullptr, (const float*)Yp, S, N,
                          LS, l, rs, Ysum, gram ? Gp : nullptr);
        if (r != hipSuccess || !gram) return r;
        return launch_kernel(k_fgram_sum, dim3(1), dim3(kGramThreads), 0, st, nullptr, nullptr, (const double*)Gp,
                             (int)nch, l, G, chol ? Rinv : nullptr);
    };
    // Y = W (Om diag(s))^T;  Y^T Y = R^T R;  Q = Y R^-1.
    TTQ_F(pass(W, M, ldw, K, PassOp{om, K, nullptr, 0, nullptr, nullptr, s}, YM, nullptr, true, true));
    for (int it = 0; it < q; ++it) {
        // P = W^T Q.  The inner orth is left out: orth(A_s^T Q) = A_s^T Q R^-1
        // with R upper triangular with a positive diagonal, and
        // orth(A_s A_s^T Q R^-1) = orth(A_s A_s^T Q).
        TTQ_F(pass(Wt, K, M32, M32, PassOp{nullptr, 0, YM, M, Rinv, nullptr, nullptr}, YK, nullptr, false, false));
        // Y = A_s (A_s^T Q) = W (s^2 o P);  Y^T Y = R^T R.
        TTQ_F(pass(W, M, ldw, K, PassOp{nullptr, 0, YK, K, nullptr, s, s}, YM, nullptr, true, true));
    }
    // P = W^T Q;  G = C C^T = Gram of diag(s) P;  eigenproblem;  factors.
    TTQ_F(pass(Wt, K, M32, M32, PassOp{nullptr, 0, YM, M, Rinv, nullptr, nullptr}, YK, s, true, false));
    const int np = (l + 1) / 2;
    const unsigned jt = (unsigned)((2 * np * np + 63) / 64 * 64 + kWave);
    TTQ_F(launch_kernel(k_fjacobi, dim3(1), dim3(jt), 0, st, nullptr, nullptr, (const double*)G,
                        (const double*)Rinv, l, rank, TB, TA));
    const unsigned nbb = (unsigned)((M + 63) / 64);
    TTQ_F(launch_kernel(k_fform, dim3(nbb + (unsigned)((K + 63) / 64)), dim3(256), 0, st, nullptr, nullptr,
                        (const float*)YM, M, (const float*)YK, K, LS, l, rank, (const double*)TB, (const double*)TA,
                        B, A, nbb));
#undef TTQ_F
    return hipSuccess;
}

}  // namespace ttq
