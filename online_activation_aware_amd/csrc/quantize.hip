// Group-wise RTN of the scaled (residual) weight, packed into int32 words.
//
// [TTQ §method b1] group-wise RTN; [TTQ §method b2] the weight is scaled by the
// AWQ scale of its input channel; [TTQ §method b5] with dynamic low-rank factors
// the residual W - B A is what gets quantized.
//
// Mapping: a workgroup (4 waves) owns a strip of 512 input channels and a
// block of output rows; lane l owns 8 consecutive channels (one 16-byte bf16
// load, two for fp32), so a group of g channels spans g/8 adjacent lanes and
// its min/max needs log2(g/8) xor-shuffles.  Four adjacent lanes hold 32
// codes = `bits` int32 words, assembled with quad shuffles and written by the
// first `bits` lanes of the quad.  With low-rank factors, the strip of A
// (rank x 512 fp32) is staged once in LDS and reused for every row.
#include "common.hpp"
#include "launch.hpp"

namespace ttq {

constexpr int kQThreads = 256;
constexpr int kQChans = kWave * 8;

// Group RTN of one lane's 8 values and packing of the quad's 32 codes.
// All 64 lanes of the wave must call this together (it shuffles).
template <int BITS, int GROUP>
__device__ __forceinline__ void quantize_and_store(const float (&v)[8], bool active, int lane, int64_t cu,
                                                   int64_t col, int64_t o, int64_t words_per_row,
                                                   int64_t groups_per_row, uint32_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scale, uint16_t* __restrict__ zero) {
    constexpr float QMAX = (float)((1 << BITS) - 1);
    constexpr int GL = GROUP / 8;                 // lanes per group
    // Group range (NaN ignored: v_min/v_max return the non-NaN operand).
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
#pragma unroll
    for (int m = 1; m < GL; m <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, m));
        mx = fmaxf(mx, __shfl_xor(mx, m));
    }
    mn = fminf(0.0f, mn);
    mx = fmaxf(0.0f, mx);
    const float d32 = (mx - mn) / QMAX;
    const uint16_t dh = d32 == 0.0f ? (uint16_t)0x3C00 : f32_to_f16_up(d32);
    const float df = f16_to_f32(dh);
    const float z = fminf(fmaxf(rintf((-mn) / df), 0.0f), QMAX);
    const float inv = 1.0f / df;

    uint64_t field = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float q = fminf(fmaxf(rintf(v[i] * inv) + z, 0.0f), QMAX);
        q = (v[i] != v[i]) ? 0.0f : q;
        field |= (uint64_t)(uint32_t)q << (BITS * i);
    }

    // Quad assembly: lanes 4m..4m+3 hold 32 codes = BITS words.
    const int qbase = lane & ~3;
    uint64_t fq[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint64_t lo = (uint32_t)__shfl((int)(uint32_t)field, qbase + k);
        uint64_t hi = 0;
        if constexpr (BITS * 8 > 32) hi = (uint32_t)__shfl((int)(uint32_t)(field >> 32), qbase + k);
        fq[k] = lo | (hi << 32);
    }
    auto word = [&](int j) -> uint32_t {
        uint32_t wv = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int off = 8 * BITS * k - 32 * j;
            if (off >= 32 || off + 8 * BITS <= 0) continue;
            wv |= off >= 0 ? (uint32_t)(fq[k] << off) : (uint32_t)(fq[k] >> (-off));
        }
        return wv;
    };
    if (active) {
        const int j = lane & 3;
        uint32_t* wrow = codes + o * words_per_row + (cu >> 2) * BITS;
        if (j < BITS) wrow[j] = word(j);
        if (BITS > 4 && j == 0) wrow[4] = word(4);
        if ((cu % GL) == 0) {
            const int64_t gi = o * groups_per_row + col / GROUP;
            scale[gi] = dh;
            zero[gi] = f32_to_f16_rne(z);
        }
    }
}

template <int BITS, int GROUP, bool WF32, bool LOWRANK>
__global__ __launch_bounds__(kQThreads) void k_quantize(
    const void* __restrict__ W, int64_t M, int64_t K, int64_t ldw, const float* __restrict__ s,
    const float* __restrict__ B, const float* __restrict__ A, int rank, int rows_per_block,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale, uint16_t* __restrict__ zero) {
    extern __shared__ float sA[];                 // [rank][kQChans] when LOWRANK

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t cu = (int64_t)blockIdx.x * kWave + lane;   // 8-channel unit in the row
    const int64_t col = cu * 8;
    const bool active = col < K;
    const int64_t row0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t row1 = min(M, row0 + rows_per_block);

    float sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[i] = 1.0f;
    if (s != nullptr && active) {
        f32x4 a = *(const f32x4*)(s + col), b = *(const f32x4*)(s + col + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { sc[i] = a[i]; sc[4 + i] = b[i]; }
    }

    if constexpr (LOWRANK) {
        const int64_t cbase = (int64_t)blockIdx.x * kQChans;
        for (int idx = threadIdx.x; idx < rank * kQChans; idx += kQThreads) {
            const int k = idx / kQChans, c = idx % kQChans;
            sA[idx] = (cbase + c < K) ? A[(int64_t)k * K + cbase + c] : 0.0f;
        }
        __syncthreads();
    }

    const int64_t words_per_row = K * BITS / 32;
    const int64_t groups_per_row = K / GROUP;

    constexpr int RB = 4;                         // rows per wave whose loads are in flight together
    constexpr int WSTRIDE = kQThreads / kWave;    // waves per workgroup
    for (int64_t ob = row0 + wave; ob < row1; ob += WSTRIDE * RB) {
        float wbuf[RB][8];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t o = ob + (int64_t)WSTRIDE * r;
            if (active && o < row1) {
                if constexpr (WF32) {
                    const f32x4* p = (const f32x4*)((const float*)W + o * ldw + col);
                    f32x4 a = ld_nc(p), b = ld_nc(p + 1);
#pragma unroll
                    for (int i = 0; i < 4; ++i) { wbuf[r][i] = a[i]; wbuf[r][4 + i] = b[i]; }
                } else {
                    u32x4 p = ld_nc((const u32x4*)((const uint16_t*)W + o * ldw + col));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        wbuf[r][2 * i] = bf16lo_to_f32(p[i]);
                        wbuf[r][2 * i + 1] = bf16hi_to_f32(p[i]);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) wbuf[r][i] = 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t o = ob + (int64_t)WSTRIDE * r;
            if (o >= row1) break;                 // wave-uniform
            float v[8];
            if constexpr (LOWRANK) {
                double acc[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = (double)wbuf[r][i];
                const float* Brow = B + o * rank;
                for (int k = 0; k < rank; ++k) {
                    const double nb = -(double)Brow[k];
                    const f32x4* ak = (const f32x4*)(sA + k * kQChans + lane * 8);
                    f32x4 a0 = ak[0], a1 = ak[1];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[i] = __builtin_fma(nb, (double)a0[i], acc[i]);
                        acc[4 + i] = __builtin_fma(nb, (double)a1[i], acc[4 + i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = (float)(acc[i] * (double)sc[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = wbuf[r][i] * sc[i];
            }
            quantize_and_store<BITS, GROUP>(v, active, lane, cu, col, o, words_per_row, groups_per_row,
                                            codes, scale, zero);
        }
    }
}

template <int BITS, int GROUP>
static hipError_t launch_q3(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                            const float* s, const float* B, const float* A, int rank,
                            uint32_t* codes, uint16_t* scale, uint16_t* zero, hipStream_t st) {
    const bool lr = rank > 0;
    const int rows = lr ? 64 : 16;
    dim3 grid((unsigned)((K + kQChans - 1) / kQChans), (unsigned)((M + rows - 1) / rows));
    const size_t lds = lr ? (size_t)rank * kQChans * sizeof(float) : 0;
#define TTQ_Q_LAUNCH(WF, LR)                                                                       \
    k_quantize<BITS, GROUP, WF, LR><<<grid, kQThreads, lds, st>>>(W, M, K, ldw, s, B, A, rank,     \
                                                                  rows, codes, scale, zero)
    if (wf32) {
        if (lr) TTQ_Q_LAUNCH(true, true); else TTQ_Q_LAUNCH(true, false);
    } else {
        if (lr) TTQ_Q_LAUNCH(false, true); else TTQ_Q_LAUNCH(false, false);
    }
#undef TTQ_Q_LAUNCH
    return hipGetLastError();
}

template <int BITS>
static hipError_t launch_q2(int group, const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                            const float* s, const float* B, const float* A, int rank,
                            uint32_t* codes, uint16_t* scale, uint16_t* zero, hipStream_t st) {
    switch (group) {
        case 16: return launch_q3<BITS, 16>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, st);
        case 32: return launch_q3<BITS, 32>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, st);
        case 64: return launch_q3<BITS, 64>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, st);
        case 128: return launch_q3<BITS, 128>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_quantize(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                           const float* s, int bits, int group, const float* B, const float* A,
                           int rank, uint32_t* codes, uint16_t* scale, uint16_t* zero,
                           hipStream_t st) {
    switch (bits) {
        case 2: return launch_q2<2>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, st);
        case 3: return launch_q2<3>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, st);
        case 4: return launch_q2<4>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, st);
        case 5: return launch_q2<5>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ttq
