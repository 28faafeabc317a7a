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
//
// Optionally the kernel also writes the dequantized weight of [TTQ §method b1]
// (QDQ) with the input scale folded back, w~ = bf16(((code - zero) * step) *
// (1/s)), dense [M][K] bf16: the operand of the prompt-sized projection, so
// that the codes need not be read and expanded a second time.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "scales.hpp"

namespace ttq {

constexpr int kQThreads = 256;
constexpr int kQChans = kWave * 8;

// Group RTN of one lane's 8 values and packing of the quad's 32 codes.
// All 64 lanes of the wave must call this together (it shuffles).
template <int BITS, int GROUP>
__device__ __forceinline__ void quantize_and_store(const float (&v)[8], bool active, int lane, int64_t cu,
                                                   int64_t col, int64_t o, int64_t words_per_row,
                                                   int64_t groups_per_row, uint32_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scale, uint16_t* __restrict__ zero,
                                                   const float (&sinv)[8], uint16_t* __restrict__ wq, int64_t K) {
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
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float q = fminf(fmaxf(rintf(v[i] * inv) + z, 0.0f), QMAX);
        q = (v[i] != v[i]) ? 0.0f : q;
        qv[i] = q;
        field |= (uint64_t)(uint32_t)q << (BITS * i);
    }
    if (wq != nullptr && active) {
        // (q - z) * step is exact in fp32 (a small integer times an fp16 value).
        u32x4 pk;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            pk[p] = pack_bf16x2(((qv[2 * p] - z) * df) * sinv[2 * p], ((qv[2 * p + 1] - z) * df) * sinv[2 * p + 1]);
        *(u32x4*)(wq + o * K + col) = pk;
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

// Row batch held in registers: raw bf16 (one 16-byte vector) or fp32 (two).
template <bool WF32>
struct RawRow {
    u32x4 a;
    u32x4 b;
};

template <bool WF32>
__device__ __forceinline__ void load_row(RawRow<WF32>& r, const void* W, int64_t o, int64_t ldw, int64_t col) {
    if constexpr (WF32) {
        const u32x4* p = (const u32x4*)((const float*)W + o * ldw + col);
        r.a = ld_nc(p);
        r.b = ld_nc(p + 1);
    } else {
        r.a = ld_nc((const u32x4*)((const uint16_t*)W + o * ldw + col));
    }
}

template <bool WF32>
__device__ __forceinline__ void unpack_row(const RawRow<WF32>& r, float (&w)[8]) {
    if constexpr (WF32) {
        // Whole-vector casts: this compiler mis-lowers a bit cast whose operand
        // is a single vector element (it reads element 0).
        const f32x4 fa = __builtin_bit_cast(f32x4, r.a), fb = __builtin_bit_cast(f32x4, r.b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = fa[i];
            w[4 + i] = fb[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = bf16lo_to_f32(r.a[i]);
            w[2 * i + 1] = bf16hi_to_f32(r.a[i]);
        }
    }
}

template <int BITS, int GROUP, bool WF32, bool LOWRANK, bool SFUSE>
__global__ __launch_bounds__(kQThreads) void k_quantize(
    const void* __restrict__ W, int64_t M, int64_t K, int64_t ldw, const float* __restrict__ s,
    const float* __restrict__ B, const float* __restrict__ A, int rank, int rows_per_block,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale, uint16_t* __restrict__ zero,
    uint16_t* __restrict__ wq, QScaleSrc qs) {
    extern __shared__ float sA[];                 // [rank][kQChans] when LOWRANK

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t cu = (int64_t)blockIdx.x * kWave + lane;   // 8-channel unit in the row
    const int64_t col = cu * 8;
    const bool active = col < K;
    const int64_t cbase = (int64_t)blockIdx.x * kQChans;

    if constexpr (LOWRANK) {
        for (int idx = threadIdx.x; idx < rank * kQChans; idx += kQThreads) {
            const int k = idx / kQChans, c = idx % kQChans;
            sA[idx] = (cbase + c < K) ? A[(int64_t)k * K + cbase + c] : 0.0f;
        }
    }

    // Per-channel scales of this lane's 8 channels, and 1/s by v_rcp_f32
    // (exactly 1 for s = 1) for the dequantized weight.
    float sc[8], sinv[8];
    if constexpr (SFUSE) {
        // Each of the strip's 512 scales is evaluated once per workgroup.
        __shared__ float ssc[kQChans];
        const double lam = *qs.lam;
#pragma unroll
        for (int h = 0; h < kQChans / kQThreads; ++h) {
            const int c = threadIdx.x + h * kQThreads;
            const int64_t j = cbase + c;
            const float v = j < K ? awq_scale(qs.ssq[j], qs.tn, lam, qs.e) : 1.0f;
            ssc[c] = v;
            if (j < K && blockIdx.y == 0) qs.s_out[j] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = ssc[lane * 8 + i];
    } else {
        if constexpr (LOWRANK) __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = 1.0f;
        if (s != nullptr && active) {
            f32x4 a = *(const f32x4*)(s + col), b = *(const f32x4*)(s + col + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) { sc[i] = a[i]; sc[4 + i] = b[i]; }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sinv[i] = __builtin_amdgcn_rcpf(sc[i]);

    const int64_t words_per_row = K * BITS / 32;
    const int64_t groups_per_row = K / GROUP;

    // Rows per wave whose loads are in flight together.
    constexpr int RB = (LOWRANK || WF32) ? 4 : 8;
    constexpr int WSTRIDE = kQThreads / kWave;    // waves per workgroup
    // Row blocks rb = blockIdx.y, + gridDim.y, ... (the grid is sized to the
    // number of workgroups the device holds at once).
    const int64_t nrb = (M + rows_per_block - 1) / rows_per_block;
    for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
        const int64_t row0 = rb * rows_per_block;
        const int64_t row1 = min(M, row0 + rows_per_block);
        for (int64_t ob = row0 + wave; ob < row1; ob += WSTRIDE * RB) {
            RawRow<WF32> raw[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t o = ob + (int64_t)WSTRIDE * r;
                if (active && o < row1) {
                    load_row<WF32>(raw[r], W, o, ldw, col);
                } else {
                    raw[r].a = u32x4{0u, 0u, 0u, 0u};
                    raw[r].b = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t o = ob + (int64_t)WSTRIDE * r;
                if (o >= row1) break;                 // wave-uniform
                float wv[8];
                unpack_row<WF32>(raw[r], wv);
                float v[8];
                if constexpr (LOWRANK) {
                    double acc[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = (double)wv[i];
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
                    for (int i = 0; i < 8; ++i) v[i] = wv[i] * sc[i];
                }
                quantize_and_store<BITS, GROUP>(v, active, lane, cu, col, o, words_per_row, groups_per_row,
                                                codes, scale, zero, sinv, wq, K);
            }
        }
    }
}

template <int BITS, int GROUP>
static hipError_t launch_q3(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                            const float* s, const float* B, const float* A, int rank,
                            uint32_t* codes, uint16_t* scale, uint16_t* zero, uint16_t* wq,
                            const QScaleSrc* qs, hipStream_t st, StageTimer tm) {
    const bool lr = rank > 0;
    // Rows per block: one batch of loads per wave (4 waves x 8 rows for
    // bf16, x 4 for fp32); with low-rank factors more rows amortise staging A.
    const int rows = lr ? 64 : (wf32 ? 16 : 32);
    const int64_t strips = (K + kQChans - 1) / kQChans;
    const int64_t nrb = (M + rows - 1) / rows;
    const size_t lds = lr ? (size_t)rank * kQChans * sizeof(float) : 0;
    const QScaleSrc q = qs ? *qs : QScaleSrc{};
    // Persistent row loop: as many workgroups as the device holds at once
    // (workgroups per compute unit cached per kernel and LDS size).
    auto grid_for = [&](const void* kern, std::atomic<int>& cache) -> dim3 {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        int per_cu = lr ? 0 : cache.load(std::memory_order_relaxed);
        if (per_cu < 1) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kQThreads, lds) != hipSuccess ||
                per_cu < 1)
                per_cu = 1;
            if (!lr) cache.store(per_cu, std::memory_order_relaxed);
        }
        int64_t gy = ((int64_t)cus * per_cu + strips - 1) / strips;
        if (gy > nrb) gy = nrb;
        if (gy > 65535) gy = 65535;
        return dim3((unsigned)strips, (unsigned)gy);
    };
#define TTQ_Q_LAUNCH(WF, LR, SF)                                                                         \
    do {                                                                                                 \
        static std::atomic<int> occ{0};                                                                  \
        auto kern = k_quantize<BITS, GROUP, WF, LR, SF>;                                                 \
        return launch_kernel(kern, grid_for((const void*)kern, occ), dim3(kQThreads), lds, st, tm.start,  \
                             tm.stop, W, M, K, ldw, s, B, A, rank, rows, codes, scale, zero, wq, q);     \
    } while (0)
#define TTQ_Q_LAUNCH2(WF, LR) \
    if (qs) TTQ_Q_LAUNCH(WF, LR, true); else TTQ_Q_LAUNCH(WF, LR, false)
    if (wf32) {
        if (lr) { TTQ_Q_LAUNCH2(true, true); } else { TTQ_Q_LAUNCH2(true, false); }
    } else {
        if (lr) { TTQ_Q_LAUNCH2(false, true); } else { TTQ_Q_LAUNCH2(false, false); }
    }
#undef TTQ_Q_LAUNCH2
#undef TTQ_Q_LAUNCH
    return hipGetLastError();
}

template <int BITS>
static hipError_t launch_q2(int group, const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                            const float* s, const float* B, const float* A, int rank,
                            uint32_t* codes, uint16_t* scale, uint16_t* zero, uint16_t* wq,
                            const QScaleSrc* qs, hipStream_t st, StageTimer tm) {
    switch (group) {
        case 16: return launch_q3<BITS, 16>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 32: return launch_q3<BITS, 32>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 64: return launch_q3<BITS, 64>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 128: return launch_q3<BITS, 128>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_quantize(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                           const float* s, int bits, int group, const float* B, const float* A,
                           int rank, uint32_t* codes, uint16_t* scale, uint16_t* zero,
                           uint16_t* wq, hipStream_t st, const QScaleSrc* qs, StageTimer tm) {
    switch (bits) {
        case 2: return launch_q2<2>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 3: return launch_q2<3>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 4: return launch_q2<4>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 5: return launch_q2<5>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
    }
    return hipErrorInvalidValue;
}

}  // namespace ttq
