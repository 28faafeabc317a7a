// Dynamic low-rank term Y += B (A X), fp32.
//
// [TTQ §method b5]: W = W_q + B A, so the quantized layer adds B (A X).
// The term is kept in fp32 end to end: it can carry much of Y's energy.
//
// k_lowrank_zm (bf16 X, K % 32 == 0): Z on the matrix cores.  A (fp32) is
// split into three bf16 terms hi + mid + lo (the remainder is below 2^-24 of
// A), X is bf16 already and the MFMA accumulates in fp32, so Z keeps fp32
// accuracy.  A workgroup owns 16 tokens and one K slice (grid.y; one slice
// unless the token tiles alone leave most compute units idle); its 16 waves
// take the slice's 32-wide K steps w, w + 16, ... and their tiles are added in
// wave order.  Slice y writes its partial Z to Z + y T rank.
// k_lowrank_z (fp32 X or other K): one wave per 64 tokens and K slice (lane =
// token); A's values are the same for every lane, so they come through scalar
// loads, and each lane accumulates rank partial sums of its token over the
// slice.
// k_lowrank_y: a 64 x 64 (tokens x rows) tile per workgroup; the slice
// partials are summed in slice order into LDS together with the B rows, and
// each thread adds a 4 x 4 block of B Z^T into Y.  No atomics.
#include "common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace ttq {

constexpr int kMaxRank = 64;

constexpr int kZWaves = 16;

template <int RT>
__global__ __launch_bounds__(kZWaves * kWave) void k_lowrank_zm(const uint16_t* __restrict__ X, int64_t T,
                                                                int64_t K, int64_t ldx,
                                                                const float* __restrict__ A, int rank,
                                                                float* __restrict__ Z) {
    __shared__ f32x4 red[kZWaves][RT][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15, q = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    const int64_t rows = min((int64_t)16, T - t0);
    const rsrc_t rx = make_rsrc(X + t0 * ldx, ((rows - 1) * ldx + K) * 2);   // tokens >= T read as 0

    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t nsall = K / 32;
    const int64_t spp = (nsall + gridDim.y - 1) / gridDim.y;       // steps per slice
    const int64_t sbeg = (int64_t)blockIdx.y * spp;
    const int64_t nsteps = min(nsall, sbeg + spp);                  // end of this slice
    Z += (int64_t)blockIdx.y * T * rank;
    constexpr int U = 4;                          // steps whose loads are in flight together
    for (int64_t sb = sbeg + wave; sb < nsteps; sb += (int64_t)U * kZWaves) {
        u32x4 xb[U];
        f32x4 a0[U][RT], a1[U][RT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t step = sb + (int64_t)u * kZWaves;
            const int64_t k0 = step * 32 + 8 * q;
            const bool in = step < nsteps;
            xb[u] = in ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rx, (int)((r16 * ldx + k0) * 2), 0, 0))
                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int kr = 16 * rt + r16;         // rank row of this lane's operand
                a0[u][rt] = a1[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (in && kr < rank) {
                    a0[u][rt] = *(const f32x4*)(A + (int64_t)kr * K + k0);
                    a1[u][rt] = *(const f32x4*)(A + (int64_t)kr * K + k0 + 4);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (sb + (int64_t)u * kZWaves >= nsteps) break;   // wave-uniform
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float a[8] = {a0[u][rt][0], a0[u][rt][1], a0[u][rt][2], a0[u][rt][3],
                                    a1[u][rt][0], a1[u][rt][1], a1[u][rt][2], a1[u][rt][3]};
                u32x4 hi, mid, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = pack_bf16x2(a[2 * e], a[2 * e + 1]);
                    const float r0 = a[2 * e] - bf16lo_to_f32(hi[e]), r1 = a[2 * e + 1] - bf16hi_to_f32(hi[e]);
                    mid[e] = pack_bf16x2(r0, r1);
                    lo[e] = pack_bf16x2(r0 - bf16lo_to_f32(mid[e]), r1 - bf16hi_to_f32(mid[e]));
                }
                acc[rt] = mfma_16x16x32(hi, xb[u], acc[rt]);
                acc[rt] = mfma_16x16x32(mid, xb[u], acc[rt]);
                acc[rt] = mfma_16x16x32(lo, xb[u], acc[rt]);
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) red[wave][rt][lane] = acc[rt];
    __syncthreads();
    // Lane of wave rt holds Z^T[16 rt + 4 q + i][t0 + r16], i = 0..3.
    if (wave < RT) {
        const int rt = wave;
        f32x4 sum = red[0][rt][lane];
        for (int w = 1; w < kZWaves; ++w) {
            const f32x4 v = red[w][rt][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[i] += v[i];
        }
        const int64_t t = t0 + r16;
        if (t < T) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = 16 * rt + 4 * q + i;
                if (k < rank) Z[t * rank + k] = sum[i];
            }
        }
    }
}

bool lowrank_z_mfma_ok(bool xf32, int64_t T, int64_t K, int64_t ldx, const float* A) {
    return !xf32 && K % 32 == 0 && (int64_t)16 * ldx * 2 < ((int64_t)1 << 31) && T > 0 &&
           (uintptr_t)A % 16 == 0;
}

// K slices for Z when its 16-token tiles leave most of the 256 compute units
// idle (2048 tokens: 128 tiles, 2 slices), each slice at least one step per
// wave; at most 8.
int lowrank_zm_parts(int64_t T, int64_t K) {
    const int64_t tiles = (T + 15) / 16;
    int64_t s = (256 + tiles - 1) / tiles;
    const int64_t smax = (K / 32) / kZWaves;
    if (s > 8) s = 8;
    if (s > smax) s = smax;
    return s < 1 ? 1 : (int)s;
}

hipError_t launch_lowrank_z(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* A,
                            int rank, float* Z, hipStream_t st, StageTimer tm, int parts) {
    if (!lowrank_z_mfma_ok(xf32, T, K, ldx, A) || parts < 1) return hipErrorInvalidValue;
    const dim3 g((unsigned)((T + 15) / 16), (unsigned)parts);
    if (rank <= 16)
        return launch_kernel(k_lowrank_zm<1>, g, dim3(kZWaves * kWave), 0, st, tm.start, tm.stop,
                             (const uint16_t*)X, T, K, ldx, A, rank, Z);
    if (rank <= 32)
        return launch_kernel(k_lowrank_zm<2>, g, dim3(kZWaves * kWave), 0, st, tm.start, tm.stop,
                             (const uint16_t*)X, T, K, ldx, A, rank, Z);
    if (rank > kMaxRank) return hipErrorInvalidValue;
    return launch_kernel(k_lowrank_zm<4>, g, dim3(kZWaves * kWave), 0, st, tm.start, tm.stop, (const uint16_t*)X,
                         T, K, ldx, A, rank, Z);
}

template <bool XF32, int RMAX>
__global__ __launch_bounds__(64) void k_lowrank_z(const void* __restrict__ X, int64_t T, int64_t K,
                                                  int64_t ldx, const float* __restrict__ A, int rank,
                                                  int64_t slice, float* __restrict__ Zp) {
    const int lane = threadIdx.x;
    const int64_t t = (int64_t)blockIdx.x * 64 + lane;
    const int64_t j0 = (int64_t)blockIdx.y * slice;
    const int64_t j1 = min(K, j0 + slice);
    float z[RMAX];
#pragma unroll
    for (int k = 0; k < RMAX; ++k) z[k] = 0.f;
    if (t < T) {
        for (int64_t j = j0; j < j1; j += 8) {
            float x[8];
            if constexpr (XF32) {
                const f32x4* p = (const f32x4*)((const float*)X + t * ldx + j);
                f32x4 a = ld_nc(p), b = ld_nc(p + 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
            } else {
                u32x4 w = ld_nc((const u32x4*)((const uint16_t*)X + t * ldx + j));
#pragma unroll
                for (int i = 0; i < 4; ++i) { x[2 * i] = bf16lo_to_f32(w[i]); x[2 * i + 1] = bf16hi_to_f32(w[i]); }
            }
#pragma unroll
            for (int k = 0; k < RMAX; ++k) {
                if (k >= rank) break;
                const float* ak = A + (int64_t)k * K + j;
#pragma unroll
                for (int i = 0; i < 8; ++i) z[k] = __builtin_fmaf(ak[i], x[i], z[k]);
            }
        }
        float* zo = Zp + ((int64_t)blockIdx.y * T + t) * rank;
#pragma unroll
        for (int k = 0; k < RMAX; ++k)
            if (k < rank) zo[k] = z[k];
    }
}

template <bool YF32, int RMAX>
__global__ __launch_bounds__(256) void k_lowrank_y(const float* __restrict__ Zp, int nslices,
                                                   const float* __restrict__ B, int rank, int64_t T,
                                                   int64_t M, void* __restrict__ Y, int64_t ldy) {
    __shared__ float sZ[64][RMAX + 1];
    __shared__ float sB[64][RMAX + 1];
    const int tid = threadIdx.x;
    const int64_t tb = (int64_t)blockIdx.y * 64, ob = (int64_t)blockIdx.x * 64;
    for (int idx = tid; idx < 64 * RMAX; idx += 256) {
        const int r = idx / RMAX, k = idx % RMAX;
        float zs = 0.f, bv = 0.f;
        if (k < rank) {
            if (tb + r < T)
                for (int sl = 0; sl < nslices; ++sl) zs += Zp[((int64_t)sl * T + tb + r) * rank + k];
            if (ob + r < M) bv = B[(ob + r) * rank + k];
        }
        sZ[r][k] = zs;
        sB[r][k] = bv;
    }
    __syncthreads();
    const int tt = (tid >> 4) * 4, oo = (tid & 15) * 4;
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < RMAX; ++k)
                if (k < rank) s = __builtin_fmaf(sB[oo + b][k], sZ[tt + a][k], s);
            acc[a][b] = s;
        }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int64_t t = tb + tt + a;
        if (t >= T) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t o = ob + oo + b;
            if (o >= M) continue;
            if constexpr (YF32) {
                float* yp = (float*)Y + t * ldy + o;
                *yp = *yp + acc[a][b];
            } else {
                uint16_t* yp = (uint16_t*)Y + t * ldy + o;
                *yp = (uint16_t)f32_to_bf16(bf16_to_f32(*yp) + acc[a][b]);
            }
        }
    }
}

int lowrank_slices(int64_t T, int64_t K, int64_t* slice_len) {
    const int64_t tblocks = (T + 63) / 64;
    int64_t ns = tblocks >= 512 ? 1 : (512 + tblocks - 1) / tblocks;
    int64_t len = (K + ns - 1) / ns;
    len = (len + 7) / 8 * 8;
    if (len < 64) len = 64;
    *slice_len = len;
    return (int)((K + len - 1) / len);
}

template <int RMAX>
static hipError_t launch_lr(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                            const float* A, const float* B, int64_t M, int rank, void* Y, bool yf32,
                            int64_t ldy, float* Zp, hipStream_t st, StageTimer tm) {
    int ns = 1;
    if (lowrank_z_mfma_ok(xf32, T, K, ldx, A)) {
        ns = lowrank_zm_parts(T, K);
        if (hipError_t e = launch_lowrank_z(X, xf32, T, K, ldx, A, rank, Zp, st, {tm.start, nullptr}, ns)) return e;
    } else {
        int64_t len = 0;
        ns = lowrank_slices(T, K, &len);
        dim3 gz((unsigned)((T + 63) / 64), (unsigned)ns);
        hipError_t e = xf32 ? launch_kernel(k_lowrank_z<true, RMAX>, gz, dim3(64), 0, st, tm.start, nullptr, X,
                                            T, K, ldx, A, rank, len, Zp)
                            : launch_kernel(k_lowrank_z<false, RMAX>, gz, dim3(64), 0, st, tm.start, nullptr, X,
                                            T, K, ldx, A, rank, len, Zp);
        if (e != hipSuccess) return e;
    }
    dim3 gy((unsigned)((M + 63) / 64), (unsigned)((T + 63) / 64));
    return yf32 ? launch_kernel(k_lowrank_y<true, RMAX>, gy, dim3(256), 0, st, nullptr, tm.stop, (const float*)Zp,
                                ns, B, rank, T, M, Y, ldy)
                : launch_kernel(k_lowrank_y<false, RMAX>, gy, dim3(256), 0, st, nullptr, tm.stop, (const float*)Zp,
                                ns, B, rank, T, M, Y, ldy);
}

hipError_t launch_lowrank(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                          const float* A, const float* B, int64_t M, int rank, void* Y, bool yf32,
                          int64_t ldy, float* Zp, hipStream_t st, StageTimer tm) {
    // The accumulators are sized by the smallest of 8/16/32/64 that holds rank.
    if (rank <= 8) return launch_lr<8>(X, xf32, T, K, ldx, A, B, M, rank, Y, yf32, ldy, Zp, st, tm);
    if (rank <= 16) return launch_lr<16>(X, xf32, T, K, ldx, A, B, M, rank, Y, yf32, ldy, Zp, st, tm);
    if (rank <= 32) return launch_lr<32>(X, xf32, T, K, ldx, A, B, M, rank, Y, yf32, ldy, Zp, st, tm);
    if (rank <= kMaxRank) return launch_lr<64>(X, xf32, T, K, ldx, A, B, M, rank, Y, yf32, ldy, Zp, st, tm);
    return hipErrorInvalidValue;
}

}  // namespace ttq
