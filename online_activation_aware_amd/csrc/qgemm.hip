// Quantized projection Y = W_hat (X / s) on the gfx950 matrix cores.
//
// [TTQ §method b7] a quantized-projection GEMM kernel; [TTQ §method b1] QDQ,
// W_hat = (code - zero) * step; [TTQ §method b2] the input is divided by the
// AWQ scale s.  The 1/s factor is folded into the dequantized weight, so the
// only rounding on the operand path is the single bf16 rounding of
//   w~[o][j] = (code - zero) * step * (1/s[j]),
// and X (already bf16) enters the MFMA untouched.  fp32 X is split into
// hi + lo bf16 halves, and w~ too, giving three MFMAs per tile product.
//
// Tiling: a 256-thread workgroup computes a BM x BN = 128 x 128 tile of Y^T
// (128 output rows o x 128 tokens t); four waves in a 2 x 2 arrangement own
// 64 x 64 each, i.e. 4 x 4 v_mfma_f32_16x16x32_bf16 per 32-deep K slice.  Per
// 64-deep K step every thread dequantizes 4 units of 8 codes into LDS and
// stages 4 x 16 bytes of X; the next step's global loads are issued before
// the current step's MFMAs so their latency hides behind the math.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace ttq {

constexpr int kGBM = 128, kGBN = 128, kGBK = 64, kGLdsK = kGBK + 8;  // 144-byte LDS rows
constexpr int kGThreads = 256;

// Extract the 8*BITS-bit field of the 8 codes starting at column kcol of a row.
template <int BITS>
__device__ __forceinline__ uint64_t load_unit_field(const uint32_t* __restrict__ row, int64_t kcol) {
    const int64_t bit = (int64_t)BITS * kcol;
    const int64_t wi = bit >> 5;
    const int off = (int)(bit & 31);
    uint64_t w = row[wi];
    if (off + 8 * BITS > 32) w |= (uint64_t)row[wi + 1] << 32;
    return w >> off;
}

template <int BITS, bool XF32>
struct WUnit {
    u32x4 hi;
    u32x4 lo;
};

template <int BITS, bool XF32>
__device__ __forceinline__ void dequant_unit(uint64_t field, float zf, float df, const float* inv,
                                             WUnit<BITS, XF32>& out) {
    constexpr uint64_t MASK = (1u << BITS) - 1;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = (float)(uint32_t)((field >> (BITS * i)) & MASK);
        w[i] = ((q - zf) * df) * inv[i];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t h0 = f32_to_bf16(w[2 * p]), h1 = f32_to_bf16(w[2 * p + 1]);
        out.hi[p] = h0 | (h1 << 16);
        if constexpr (XF32) {
            const float r0 = w[2 * p] - bf16_to_f32(h0), r1 = w[2 * p + 1] - bf16_to_f32(h1);
            out.lo[p] = pack_bf16x2(r0, r1);
        }
    }
}

template <int BITS, int GROUP, bool XF32, bool YF32>
__global__ __launch_bounds__(kGThreads) void k_qgemm(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, const float* __restrict__ s,
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ zero, int64_t M, void* __restrict__ Y, int64_t ldy, int yvec) {
    constexpr int NB = XF32 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t sW[NB][kGBM * kGLdsK];
    __shared__ __attribute__((aligned(16))) uint16_t sX[NB][kGBN * kGLdsK];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t o0 = (int64_t)blockIdx.x * kGBM;
    const int64_t t0 = (int64_t)blockIdx.y * kGBN;

    const int64_t words_per_row = K * BITS / 32;
    const int64_t groups_per_row = K / GROUP;
    const int cu = tid & 7;          // 8-column unit inside the K step (dequant role)
    const int rsub = tid >> 3;       // row 0..31 (+32 i)

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Register stage for the next K step.
    u32x4 xh[4], xl[4];
    uint64_t fld[4];
    float zf[4], df[4];
    float inv[8];

    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + kGThreads * i;
            const int64_t t = t0 + (c >> 3);
            const int64_t k = k0 + 8 * (c & 7);
            if (t < T && k < K) {
                if constexpr (XF32) {
                    const f32x4* p = (const f32x4*)((const float*)X + t * ldx + k);
                    f32x4 a = ld_nc(p), b = ld_nc(p + 1);
                    float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t h0 = f32_to_bf16(v[2 * q]), h1 = f32_to_bf16(v[2 * q + 1]);
                        xh[i][q] = h0 | (h1 << 16);
                        xl[i][q] = pack_bf16x2(v[2 * q] - bf16_to_f32(h0), v[2 * q + 1] - bf16_to_f32(h1));
                    }
                } else {
                    xh[i] = ld_nc((const u32x4*)((const uint16_t*)X + t * ldx + k));
                }
            } else {
                xh[i] = u32x4{0u, 0u, 0u, 0u};
                xl[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        const int64_t kcol = k0 + 8 * cu;
        const bool kin = kcol < K;
        if (kin) {
            // 1/s by v_rcp_f32 (<= 1 ulp): far below the bf16 rounding of w~.
            f32x4 a = *(const f32x4*)(s + kcol), b = *(const f32x4*)(s + kcol + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                inv[q] = __builtin_amdgcn_rcpf(a[q]);
                inv[4 + q] = __builtin_amdgcn_rcpf(b[q]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) inv[q] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t o = o0 + rsub + 32 * i;
            if (kin && o < M) {
                fld[i] = load_unit_field<BITS>(codes + o * words_per_row, kcol);
                const int64_t gi = o * groups_per_row + kcol / GROUP;
                zf[i] = f16_to_f32(zero[gi]);
                df[i] = f16_to_f32(scale[gi]);
            } else {
                fld[i] = 0;
                zf[i] = 0.f;
                df[i] = 0.f;
            }
        }
    };

    load_stage(0);
    for (int64_t k0 = 0; k0 < K; k0 += kGBK) {
        // Dequantize the staged codes, then publish the step to LDS.
        WUnit<BITS, XF32> wu[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dequant_unit<BITS, XF32>(fld[i], zf[i], df[i], inv, wu[i]);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + kGThreads * i;
            const int xo = (c >> 3) * kGLdsK + 8 * (c & 7);
            *(u32x4*)&sX[0][xo] = xh[i];
            if constexpr (XF32) *(u32x4*)&sX[NB - 1][xo] = xl[i];
            const int wo = (rsub + 32 * i) * kGLdsK + 8 * cu;
            *(u32x4*)&sW[0][wo] = wu[i].hi;
            if constexpr (XF32) *(u32x4*)&sW[NB - 1][wo] = wu[i].lo;
        }
        __syncthreads();
        if (k0 + kGBK < K) load_stage(k0 + kGBK);

#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int koff = 32 * kk + 8 * (lane >> 4);
            u32x4 a[NB][4], b[NB][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ro = (wm * 64 + 16 * i + (lane & 15)) * kGLdsK + koff;
                const int rt = (wn * 64 + 16 * i + (lane & 15)) * kGLdsK + koff;
#pragma unroll
                for (int h = 0; h < NB; ++h) {
                    a[h][i] = *(const u32x4*)&sW[h][ro];
                    b[h][i] = *(const u32x4*)&sX[h][rt];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = mfma_16x16x32(a[0][i], b[0][j], acc[i][j]);
                    if constexpr (XF32) {
                        acc[i][j] = mfma_16x16x32(a[0][i], b[1][j], acc[i][j]);
                        acc[i][j] = mfma_16x16x32(a[1][i], b[0][j], acc[i][j]);
                    }
                }
        }
    }

    // Epilogue: lane holds Y^T[o + r][t] for r = 0..3, i.e. 4 consecutive o of token t.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t o = o0 + wm * 64 + 16 * i + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t t = t0 + wn * 64 + 16 * j + (lane & 15);
            if (t >= T) continue;
            store_y4<YF32>(Y, t * ldy + o, M - o, yvec, acc[i][j]);
        }
    }
}

// ---------------------------------------------------------------------------
// Dequantize once: w~[o][j] = bf16(((code - zero) * step) * (1/s[j])), with
// exactly the arithmetic of the fused kernel above ((code - zero) * step is
// exact in fp32; 1/s by v_rcp_f32; one RNE rounding), written densely as
// [M][K] bf16 for the matrix-core GEMM.  One thread per 8 codes: the codes
// are read as whole dwords, the 8 weights stored as one 16-byte vector.
// Grid: x over the K/8 units of a row, y over rows (grid-strided).  A w~
// larger than 64 MiB is written by streaming stores (stream_stage).
template <int BITS, int GROUP, bool NT>
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ codes,
                                                 const uint16_t* __restrict__ scale,
                                                 const uint16_t* __restrict__ zero,
                                                 const float* __restrict__ s, int64_t M, int64_t K,
                                                 uint16_t* __restrict__ wq) {
    const int64_t col = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (col >= K) return;
    const f32x4 a = *(const f32x4*)(s + col), b = *(const f32x4*)(s + col + 4);
    float inv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        inv[q] = __builtin_amdgcn_rcpf(a[q]);
        inv[4 + q] = __builtin_amdgcn_rcpf(b[q]);
    }
    const int64_t wpr = K * BITS / 32, gpr = K / GROUP;
    for (int64_t o = blockIdx.y; o < M; o += gridDim.y) {
        const uint64_t f = load_unit_field<BITS>(codes + o * wpr, col);
        const int64_t gi = o * gpr + col / GROUP;
        WUnit<BITS, false> w;
        dequant_unit<BITS, false>(f, f16_to_f32(zero[gi]), f16_to_f32(scale[gi]), inv, w);
        st_nt<NT>((u32x4*)(wq + o * K + col), w.hi);
    }
}

template <int BITS, int GROUP>
static hipError_t launch_g3(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                            const float* s, const uint32_t* codes, const uint16_t* scale,
                            const uint16_t* zero, int64_t M, void* Y, bool yf32, int64_t ldy,
                            uint16_t* wq, hipStream_t st, StageTimer tm) {
    if (wq != nullptr) {
        dim3 gd((unsigned)((K / 8 + 255) / 256), (unsigned)(M < 8192 ? M : 8192));
        hipError_t e = stream_stage(M, K)
                           ? launch_kernel(k_dequant<BITS, GROUP, true>, gd, dim3(256), 0, st, tm.start, nullptr,
                                           codes, scale, zero, s, M, K, wq)
                           : launch_kernel(k_dequant<BITS, GROUP, false>, gd, dim3(256), 0, st, tm.start, nullptr,
                                           codes, scale, zero, s, M, K, wq);
        if (e != hipSuccess) return e;
        return launch_gemm_bf16((const uint16_t*)X, T, K, ldx, wq, K, M, Y, yf32, ldy, st, {nullptr, tm.stop},
                                nullptr, split_ws_after(wq, M, K));
    }
    // 4 consecutive outputs are stored as one vector when Y's rows allow it.
    const int yvec = ((uintptr_t)Y % 16 == 0) && ((ldy * (yf32 ? 4 : 2)) % 16 == 0);
    dim3 grid((unsigned)((M + kGBM - 1) / kGBM), (unsigned)((T + kGBN - 1) / kGBN));
#define TTQ_G_LAUNCH(XF, YF)                                                                           \
    return launch_kernel(k_qgemm<BITS, GROUP, XF, YF>, grid, dim3(kGThreads), 0, st, tm.start, tm.stop, X, T, \
                         K, ldx, s, codes, scale, zero, M, Y, ldy, yvec)
    if (xf32) {
        if (yf32) TTQ_G_LAUNCH(true, true); else TTQ_G_LAUNCH(true, false);
    } else {
        if (yf32) TTQ_G_LAUNCH(false, true); else TTQ_G_LAUNCH(false, false);
    }
#undef TTQ_G_LAUNCH
}

template <int BITS>
static hipError_t launch_g2(int group, const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                            const float* s, const uint32_t* codes, const uint16_t* scale,
                            const uint16_t* zero, int64_t M, void* Y, bool yf32, int64_t ldy,
                            uint16_t* wq, hipStream_t st, StageTimer tm) {
    switch (group) {
        case 16: return launch_g3<BITS, 16>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, wq, st, tm);
        case 32: return launch_g3<BITS, 32>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, wq, st, tm);
        case 64: return launch_g3<BITS, 64>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, wq, st, tm);
        case 128: return launch_g3<BITS, 128>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, wq, st, tm);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_qgemm(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                        const float* s, const uint32_t* codes, const uint16_t* scale,
                        const uint16_t* zero, int64_t M, int bits, int group, void* Y, bool yf32,
                        int64_t ldy, uint16_t* wq, hipStream_t st, StageTimer tm) {
    switch (bits) {
        case 2: return launch_g2<2>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, wq, st, tm);
        case 3: return launch_g2<3>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, wq, st, tm);
        case 4: return launch_g2<4>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, wq, st, tm);
        case 5: return launch_g2<5>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, wq, st, tm);
    }
    return hipErrorInvalidValue;
}

}  // namespace ttq
