// Quantized projection for few tokens (decode steps, short prompts):
// Y = W_hat (X / s) with T <= 128, bound by the stream of packed codes.
//
// [TTQ §method b7] quantized projection kernel; [TTQ §method b1] QDQ,
// w~[o][j] = bf16(((code - zero) * step) * (1/s[j])) exactly as in the other
// projection kernels; [TTQ §method b2] the input divided by s.  The point of
// the method at decode time is that only b/8 + 4/g bytes per weight cross
// HBM, so the codes go straight from HBM into registers (no LDS staging) and
// are expanded there.
//
// Mapping: a workgroup of 16 (or 8) waves owns 16 output rows; wave w takes
// the 128-wide K chunks w, w + 16, ...  Inside a chunk, lane l (row l % 16,
// quarter q = l / 16) owns the 32 consecutive channels 128 c + 32 q ..+31:
// BITS dwords of codes and one or two groups.  MFMA 16x16x32 j (j = 0..3)
// takes its 8 K-slots per lane from channels 128 c + 32 q + 8 j ..+7, and the
// token operand uses the same channel map, so each channel meets its own
// weight.  Tokens are the 16 columns of the MFMA (T > 16: several token
// tiles reuse the expanded weights).  The per-wave K-slice tiles are added
// through LDS in wave order (deterministic), and the 1/s of all K channels
// is staged in LDS once per workgroup.
#include "common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace ttq {

// Waves per workgroup: 16 for one or two token tiles (more code loads in
// flight), 8 for four or eight (room for the extra accumulators).
constexpr int vwaves(int nt) { return nt <= 2 ? 16 : 8; }
constexpr int kVChunk = 128;                      // channels per wave per step
constexpr int kVMaxK = 16384;                     // 1/s of every channel fits in LDS (64 KiB)
constexpr int kVPrefetch = 4;                     // chunks whose codes are in flight together

template <int BITS>
struct CodeWords {
    uint32_t w[BITS];
};

template <int BITS>
__device__ __forceinline__ void load_codes(CodeWords<BITS>& c, const uint32_t* __restrict__ p) {
    if constexpr (BITS == 4) {
        const u32x4 v = ld_nc((const u32x4*)p);
#pragma unroll
        for (int i = 0; i < 4; ++i) c.w[i] = v[i];
    } else if constexpr (BITS == 2) {
        const u32x2 v = ld_nc((const u32x2*)p);
        c.w[0] = v[0];
        c.w[1] = v[1];
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i) c.w[i] = ld_nc(p + i);
    }
}

// Code i (0..31) of a lane's 32-code field.
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const CodeWords<BITS>& c, int i) {
    const int bit = BITS * i;
    const int wi = bit >> 5, off = bit & 31;
    uint32_t v = c.w[wi] >> off;
    if (off + BITS > 32) v |= c.w[wi + 1] << (32 - off);
    return v & ((1u << BITS) - 1);
}

template <int BITS, int GROUP, bool XF32, bool YF32, int NT>
__global__ __launch_bounds__(vwaves(NT) * kWave) void k_qgemv(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, const float* __restrict__ s,
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ zero, int64_t M, void* __restrict__ Y, int64_t ldy) {
    constexpr int kVWaves = vwaves(NT);
    constexpr int kVThreads = kVWaves * kWave;
    __shared__ __attribute__((aligned(16))) float sinv[kVMaxK];
    __shared__ f32x4 red[kVWaves][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15, q = lane >> 4;
    const int64_t o0 = (int64_t)blockIdx.x * 16;
    const int64_t o = o0 + r;
    const bool orow = o < M;

    // 1/s by v_rcp_f32, as in the other projection kernels.
    for (int64_t j = threadIdx.x; j < K; j += kVThreads) sinv[j] = __builtin_amdgcn_rcpf(s[j]);

    const int64_t wpr = K * BITS / 32, gpr = K / GROUP;
    const uint32_t* crow = codes + (orow ? o : o0) * wpr;
    const uint16_t* srow = scale + (orow ? o : o0) * gpr;
    const uint16_t* zrow = zero + (orow ? o : o0) * gpr;
    // Token operand: rows >= T read as zero through the buffer bounds.
    const int64_t esz = XF32 ? 4 : 2;
    const rsrc_t rx = make_rsrc(X, ((T - 1) * ldx + K) * esz);

    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    const int64_t nchunks = K / kVChunk;
    for (int64_t c0 = wave; c0 < nchunks; c0 += (int64_t)kVWaves * kVPrefetch) {
        CodeWords<BITS> cw[kVPrefetch];
        uint16_t dh[kVPrefetch][GROUP < 32 ? 2 : 1], zh[kVPrefetch][GROUP < 32 ? 2 : 1];
#pragma unroll
        for (int p = 0; p < kVPrefetch; ++p) {
            const int64_t c = c0 + (int64_t)kVWaves * p;
            if (c < nchunks) {
                const int64_t k0 = c * kVChunk + 32 * q;
                load_codes<BITS>(cw[p], crow + k0 * BITS / 32);
                dh[p][0] = srow[k0 / GROUP];
                zh[p][0] = zrow[k0 / GROUP];
                if constexpr (GROUP < 32) {
                    dh[p][1] = srow[k0 / GROUP + 1];
                    zh[p][1] = zrow[k0 / GROUP + 1];
                }
            }
        }
#pragma unroll
        for (int p = 0; p < kVPrefetch; ++p) {
            const int64_t c = c0 + (int64_t)kVWaves * p;
            if (c >= nchunks) break;                  // wave-uniform
            const int64_t k0 = c * kVChunk + 32 * q;
            // Expand the lane's 32 weights into 4 MFMA operands (hi/lo for fp32 X).
            u32x4 ah[4], al[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int gsel = GROUP < 32 ? (8 * j) / GROUP : 0;
                const float df = f16_to_f32(dh[p][gsel]), zf = f16_to_f32(zh[p][gsel]);
                const f32x4 i0 = *(const f32x4*)(sinv + k0 + 8 * j);
                const f32x4 i1 = *(const f32x4*)(sinv + k0 + 8 * j + 4);
                const float inv[8] = {i0[0], i0[1], i0[2], i0[3], i1[0], i1[1], i1[2], i1[3]};
                float w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float qv = (float)code_at<BITS>(cw[p], 8 * j + e);
                    w[e] = ((qv - zf) * df) * inv[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ah[j][e] = pack_bf16x2(w[2 * e], w[2 * e + 1]);
                    if constexpr (XF32) {
                        const float r0 = w[2 * e] - bf16lo_to_f32(ah[j][e]);
                        const float r1 = w[2 * e + 1] - bf16hi_to_f32(ah[j][e]);
                        al[j][e] = pack_bf16x2(r0, r1);
                    }
                }
            }
            if (!orow) {
#pragma unroll
                for (int j = 0; j < 4; ++j) ah[j] = al[j] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                // One token tile's operands at a time (bounded registers; the
                // other waves cover the latency).
                if (n > 0) __builtin_amdgcn_sched_barrier(0);
                const int t = 16 * n + r;             // token of this lane's operand column
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int voff = (int)((t * ldx + k0 + 8 * j) * esz);
                    if constexpr (XF32) {
                        const f32x4 xa = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff, 0, 0));
                        const f32x4 xb = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + 16, 0, 0));
                        const float xv[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
                        u32x4 bh, bl;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            bh[e] = pack_bf16x2(xv[2 * e], xv[2 * e + 1]);
                            bl[e] = pack_bf16x2(xv[2 * e] - bf16lo_to_f32(bh[e]),
                                                xv[2 * e + 1] - bf16hi_to_f32(bh[e]));
                        }
                        acc[n] = mfma_16x16x32(ah[j], bh, acc[n]);
                        acc[n] = mfma_16x16x32(ah[j], bl, acc[n]);
                        acc[n] = mfma_16x16x32(al[j], bh, acc[n]);
                    } else {
                        const u32x4 xb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff, 0, 0));
                        acc[n] = mfma_16x16x32(ah[j], xb, acc[n]);
                    }
                }
            }
        }
    }

    // Lane holds Y^T[o0 + 4 q + i][16 n + r] for i = 0..3; the 16 K-slice
    // tiles of each token tile are added in wave order by one wave.
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        if (n > 0) __syncthreads();               // the previous tile's sums have been read
        red[wave][lane] = acc[n];
        __syncthreads();
        if (wave == n % kVWaves) {
            f32x4 sum = red[0][lane];
#pragma unroll
            for (int w = 1; w < kVWaves; ++w) {
                const f32x4 v = red[w][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) sum[i] += v[i];
            }
            const int64_t t = 16 * n + r;
            const int64_t ob = o0 + 4 * q;
            if (t < T) store_y4<YF32>(Y, t * ldy + ob, M - ob, 0, sum);
        }
    }
}

// Token rows up to 127 are addressed (padded tiles read as zero) with 32-bit
// buffer offsets.
bool qgemv_supported(int64_t T, int64_t K, int64_t ldx, bool xf32) {
    return T >= 1 && T <= kQgemvMaxT && K % kVChunk == 0 && K <= kVMaxK &&
           (int64_t)kQgemvMaxT * ldx * (xf32 ? 4 : 2) < ((int64_t)1 << 31);
}

template <int BITS, int GROUP, bool XF32, bool YF32>
static hipError_t launch_v4(const void* X, int64_t T, int64_t K, int64_t ldx, const float* s,
                            const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M,
                            void* Y, int64_t ldy, hipStream_t st, StageTimer tm) {
    const dim3 grid((unsigned)((M + 15) / 16));
#define TTQ_V_LAUNCH(NT)                                                                                  \
    return launch_kernel(k_qgemv<BITS, GROUP, XF32, YF32, NT>, grid, dim3(vwaves(NT) * kWave), 0, st,     \
                         tm.start, tm.stop, X, T, K, ldx, s, codes, scale, zero, M, Y, ldy)
    if (T <= 16) TTQ_V_LAUNCH(1);
    if (T <= 32) TTQ_V_LAUNCH(2);
    if (T <= 64) TTQ_V_LAUNCH(4);
    TTQ_V_LAUNCH(8);
#undef TTQ_V_LAUNCH
}

template <int BITS, int GROUP>
static hipError_t launch_v3(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                            const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M,
                            void* Y, bool yf32, int64_t ldy, hipStream_t st, StageTimer tm) {
    if (xf32) {
        if (yf32) return launch_v4<BITS, GROUP, true, true>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm);
        return launch_v4<BITS, GROUP, true, false>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm);
    }
    if (yf32) return launch_v4<BITS, GROUP, false, true>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm);
    return launch_v4<BITS, GROUP, false, false>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm);
}

template <int BITS>
static hipError_t launch_v2(int group, const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                            const float* s, const uint32_t* codes, const uint16_t* scale, const uint16_t* zero,
                            int64_t M, void* Y, bool yf32, int64_t ldy, hipStream_t st, StageTimer tm) {
    switch (group) {
        case 16: return launch_v3<BITS, 16>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm);
        case 32: return launch_v3<BITS, 32>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm);
        case 64: return launch_v3<BITS, 64>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm);
        case 128: return launch_v3<BITS, 128>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_qgemv(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                        const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, int bits,
                        int group, void* Y, bool yf32, int64_t ldy, hipStream_t st, StageTimer tm) {
    switch (bits) {
        case 2: return launch_v2<2>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm);
        case 3: return launch_v2<3>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm);
        case 4: return launch_v2<4>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm);
        case 5: return launch_v2<5>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm);
    }
    return hipErrorInvalidValue;
}

}  // namespace ttq
