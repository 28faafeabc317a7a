// Group-wise RTN of the scaled (residual) weight, packed into int32 words.
//
// [TTQ §method b1] group-wise RTN; [TTQ §method b2] the weight is scaled by the
// AWQ scale of its input channel; [TTQ §method b5] with dynamic low-rank factors
// the residual W - B A is what gets quantized.
//
// Mapping: a workgroup (4 waves) owns a strip of 512 input channels and a
// block of output rows; lane l owns 8 consecutive channels (one 16-byte bf16
// load, two for fp32), so a group of g channels spans g/8 adjacent lanes and
// its min/max needs log2(g/8) DPP lane exchanges.  Four adjacent lanes hold
// 32 codes = `bits` int32 words, assembled with quad broadcasts and written
// by the first `bits` lanes of the quad.  With low-rank factors, the strip of A
// (up to 32 ranks x 512 fp32) is staged once in LDS and reused for every row;
// ranks 32..63 are read from global memory.
//
// Optionally the kernel also writes the dequantized weight of [TTQ §method b1]
// (QDQ) with the input scale folded back, w~ = bf16(((code - zero) * step) *
// (1/s)), dense [M][K] bf16: the operand of the prompt-sized projection, so
// that the codes need not be read and expanded a second time.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "scales.hpp"

namespace ttq {

constexpr int kQThreads = 256;
constexpr int kQChans = kWave * 8;
constexpr int kQLdsRanks = 32;       // ranks of A staged in LDS (64 KB)

// Workgroups of one quantizer kernel resident at once, per device and per
// number of A ranks staged in LDS (0 = not yet queried).
constexpr int kMaxDevices = 64;
struct OccMemo {
    std::atomic<int> resident[kMaxDevices][kQLdsRanks + 1];
};

// Cross-lane moves through DPP (they run in the VALU pipeline, no LDS round
// trip).  Quad permutations: lane i of each quad reads lane perm[i]
// (control perm0 | perm1 << 2 | perm2 << 4 | perm3 << 6); row mirrors
// reverse 8 or 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;     // [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane l of 8 <- lane 7 - l
constexpr int kDppMirror = 0x140;      // lane l of 16 <- lane 15 - l

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, dpp_u<CTRL>(__builtin_bit_cast(uint32_t, x)));
}

// min/max over the GL = GROUP/8 lanes of a group (aligned runs of GL lanes).
template <int GL>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
    static_assert(GL == 2 || GL == 4 || GL == 8 || GL == 16, "lanes per group");
    mn = fminf(mn, dpp_f<kDppQuadXor1>(mn));
    mx = fmaxf(mx, dpp_f<kDppQuadXor1>(mx));
    if constexpr (GL >= 4) {
        mn = fminf(mn, dpp_f<kDppQuadXor2>(mn));
        mx = fmaxf(mx, dpp_f<kDppQuadXor2>(mx));
    }
    if constexpr (GL >= 8) {             // each quad holds its own range: pair it with the mirrored quad
        mn = fminf(mn, dpp_f<kDppHalfMirror>(mn));
        mx = fmaxf(mx, dpp_f<kDppHalfMirror>(mx));
    }
    if constexpr (GL >= 16) {
        mn = fminf(mn, dpp_f<kDppMirror>(mn));
        mx = fmaxf(mx, dpp_f<kDppMirror>(mx));
    }
}

// Group RTN of one lane's 8 values and packing of the quad's 32 codes.
// All 64 lanes of the wave must call this together (cross-lane moves).
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
    group_minmax<GL>(mn, mx);
    mn = fminf(0.0f, mn);
    mx = fmaxf(0.0f, mx);
    const float d32 = (mx - mn) / QMAX;           // correctly rounded
    const uint16_t dh = d32 == 0.0f ? (uint16_t)0x3C00 : f32_to_f16_up(d32);
    const float df = f16_to_f32(dh);
    const float z = fminf(fmaxf(rintf((-mn) / df), 0.0f), QMAX);
    // Codes decided on v * (1/step) (v_rcp_f32, <= 1 ulp): only values within
    // ~1e-7 of a step from a rounding boundary can differ from a division.
    const float inv = __builtin_amdgcn_rcpf(df);

    // 8 codes of 8*BITS bits; a NaN value gives NaN + z, which the clamp's
    // v_max_f32 turns into 0.
    typedef typename std::conditional<(8 * BITS <= 32), uint32_t, uint64_t>::type field_t;
    field_t field = 0;
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = fminf(fmaxf(rintf(v[i] * inv) + z, 0.0f), QMAX);
        qv[i] = q;
        field |= (field_t)(uint32_t)q << (BITS * i);
    }
    if (wq != nullptr && active) {
        // (q - z) * step is exact in fp32 (a small integer times an fp16 value).
        u32x4 pk;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            pk[p] = pack_bf16x2(((qv[2 * p] - z) * df) * sinv[2 * p], ((qv[2 * p + 1] - z) * df) * sinv[2 * p + 1]);
        *(u32x4*)(wq + o * K + col) = pk;
    }

    // Quad assembly: lanes 4m..4m+3 hold 32 codes = BITS words; every lane
    // of the quad receives the quad's four fields by quad broadcasts.
    uint64_t fq[4];
    {
        const uint32_t lo = (uint32_t)field;
        fq[0] = dpp_u<0x00>(lo);
        fq[1] = dpp_u<0x55>(lo);
        fq[2] = dpp_u<0xAA>(lo);
        fq[3] = dpp_u<0xFF>(lo);
        if constexpr (8 * BITS > 32) {
            const uint32_t hi = (uint32_t)((uint64_t)field >> 32);
            fq[0] |= (uint64_t)dpp_u<0x00>(hi) << 32;
            fq[1] |= (uint64_t)dpp_u<0x55>(hi) << 32;
            fq[2] |= (uint64_t)dpp_u<0xAA>(hi) << 32;
            fq[3] |= (uint64_t)dpp_u<0xFF>(hi) << 32;
        }
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

template <int BITS, int GROUP, bool WF32, bool LOWRANK, bool SFUSE, bool RB4>
__global__ __launch_bounds__(kQThreads) void k_quantize(
    const void* __restrict__ W, int64_t M, int64_t K, int64_t ldw, const float* __restrict__ s,
    const float* __restrict__ B, const float* __restrict__ A, int rank, int rows_per_block,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale, uint16_t* __restrict__ zero,
    uint16_t* __restrict__ wq, QScaleSrc qs) {
    // [min(rank, kQLdsRanks)][kQChans] when LOWRANK (16-byte reads); ranks
    // beyond kQLdsRanks are read from A in global memory (L2-resident).
    extern __shared__ __attribute__((aligned(16))) float sA[];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // row addressing stays scalar
    const int64_t cu = (int64_t)blockIdx.x * kWave + lane;   // 8-channel unit in the row
    const int64_t col = cu * 8;
    const bool active = col < K;
    const int64_t cbase = (int64_t)blockIdx.x * kQChans;

    // A row block is WSTRIDE x RB rows: each wave takes RB of them (a batch).
    // The workgroup walks row blocks rb = blockIdx.y, + gridDim.y, ... (the
    // grid is sized to the number of workgroups the device holds at once),
    // and each wave issues the loads of its next batch before it processes
    // the current one, so loads stay in flight while the VALU works.
    constexpr int RB = (LOWRANK || WF32 || RB4) ? 4 : 8;
    constexpr int WSTRIDE = kQThreads / kWave;    // waves per workgroup
    const int64_t nrb = (M + rows_per_block - 1) / rows_per_block;
    auto load_batch = [&](RawRow<WF32> (&dst)[RB], int64_t rb) __attribute__((always_inline)) {
        const int64_t ob = rb * rows_per_block + wave;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t o = ob + (int64_t)WSTRIDE * r;
            if (rb < nrb && active && o < M) {
                load_row<WF32>(dst[r], W, o, ldw, col);
            } else {
                dst[r].a = u32x4{0u, 0u, 0u, 0u};
                dst[r].b = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    const int lds_ranks = rank < kQLdsRanks ? rank : kQLdsRanks;
    if constexpr (LOWRANK) {
        for (int idx = threadIdx.x; idx < lds_ranks * kQChans; idx += kQThreads) {
            const int k = idx / kQChans, c = idx % kQChans;
            sA[idx] = (cbase + c < K) ? A[(int64_t)k * K + cbase + c] : 0.0f;
        }
    }

    // Per-channel scales of this lane's 8 channels, and 1/s by v_rcp_f32
    // (exactly 1 for s = 1) for the dequantized weight.
    float sc[8], sinv[8];
    if constexpr (SFUSE) {
        // lambda from the statistics' block sums (same order as
        // ttq_awq_scales), then each of the strip's 512 scales once per
        // workgroup.
        __shared__ float ssc[kQChans];
        __shared__ double lam_s;
        if (wave == 0) {
            const double tot = blocks_total(qs.bsum, (K + kBlockCh - 1) / kBlockCh, lane);
            if (lane == 0) lam_s = qs.lambda_rel * (tot / (double)K);
        }
        __syncthreads();
        const double lam = lam_s;
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

    RawRow<WF32> cur[RB];
    load_batch(cur, blockIdx.y);
    for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
        RawRow<WF32> nxt[RB];
        load_batch(nxt, rb + gridDim.y);
        const int64_t ob = rb * rows_per_block + wave;
        if constexpr (LOWRANK) {
            // Residual of the batch's RB rows, rank-ordered fp64 sums per
            // element: each A value is read from LDS and widened once per
            // batch and used for all RB rows.
            double acc[RB][8];
            const float* Brow[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                float wv[8];
                unpack_row<WF32>(cur[r], wv);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[r][i] = (double)wv[i];
                const int64_t o = ob + (int64_t)WSTRIDE * r;
                Brow[r] = B + (o < M ? o : M - 1) * rank;
            }
            for (int k = 0; k < rank; ++k) {
                double ad[8];
                if (k < lds_ranks) {
                    const f32x4* ak = (const f32x4*)(sA + k * kQChans + lane * 8);
                    const f32x4 a0 = ak[0], a1 = ak[1];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ad[i] = (double)a0[i];
                        ad[4 + i] = (double)a1[i];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) ad[i] = active ? (double)A[(int64_t)k * K + col + i] : 0.0;
                }
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const double nb = -(double)Brow[r][k];
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[r][i] = __builtin_fma(nb, ad[i], acc[r][i]);
                }
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t o = ob + (int64_t)WSTRIDE * r;
                if (o >= M) break;                // wave-uniform
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = (float)(acc[r][i] * (double)sc[i]);
                quantize_and_store<BITS, GROUP>(v, active, lane, cu, col, o, words_per_row, groups_per_row,
                                                codes, scale, zero, sinv, wq, K);
            }
        } else {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t o = ob + (int64_t)WSTRIDE * r;
                if (o >= M) break;                // wave-uniform
                float wv[8];
                unpack_row<WF32>(cur[r], wv);
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = wv[i] * sc[i];
                quantize_and_store<BITS, GROUP>(v, active, lane, cu, col, o, words_per_row, groups_per_row,
                                                codes, scale, zero, sinv, wq, K);
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) cur[r] = nxt[r];
    }
}

template <int BITS, int GROUP>
static hipError_t launch_q3(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                            const float* s, const float* B, const float* A, int rank,
                            uint32_t* codes, uint16_t* scale, uint16_t* zero, uint16_t* wq,
                            const QScaleSrc* qs, hipStream_t st, StageTimer tm) {
    const bool lr = rank > 0;
    // Rows per block: one batch per wave (4 waves x 8 rows for bf16, x 4 for
    // fp32 or with low-rank factors).  Large bf16 weights (more than 2^25
    // values) also take batches of 4 rows: measured faster there (the
    // 14336 x 4096 layer 64.8 -> 54.4 us, 4096 x 14336 51.7 -> 50.4 us),
    // slower on 4096 x 4096 (19.9 -> 22.4 us).
    const bool rb4 = !lr && !wf32 && M * K > ((int64_t)1 << 25);
    const int rows = (lr || wf32 || rb4) ? 16 : 32;
    const int64_t strips = (K + kQChans - 1) / kQChans;
    const int64_t nrb = (M + rows - 1) / rows;
    const size_t lds = lr ? (size_t)(rank < kQLdsRanks ? rank : kQLdsRanks) * kQChans * sizeof(float) : 0;
    const QScaleSrc q = qs ? *qs : QScaleSrc{};
    // Persistent row loop: as many workgroups as the device holds at once.
    // The residency of each kernel instantiation is memoized per device and
    // per LDS size (0..32 staged ranks of A): a value the runtime derives
    // from the code object, the same on every call, so the memo never
    // changes a result.
    const int lds_ranks = lr ? (rank < kQLdsRanks ? rank : kQLdsRanks) : 0;
    auto grid_for = [&](const void* kern, OccMemo& memo) -> dim3 {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = -1;
        std::atomic<int>* slot = (dev >= 0 && dev < kMaxDevices) ? &memo.resident[dev][lds_ranks] : nullptr;
        int resident = slot ? slot->load(std::memory_order_relaxed) : 0;
        if (resident < 1) {
            int cus = 256, per_cu = 1;
            if (dev >= 0) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kQThreads, lds) != hipSuccess ||
                per_cu < 1)
                per_cu = 1;
            resident = cus * per_cu;
            if (slot) slot->store(resident, std::memory_order_relaxed);
        }
        int64_t gy = ((int64_t)resident + strips - 1) / strips;
        if (gy > nrb) gy = nrb;
        if (gy > 65535) gy = 65535;
        return dim3((unsigned)strips, (unsigned)gy);
    };
#define TTQ_Q_LAUNCH(WF, LR, SF, R4)                                                                     \
    do {                                                                                                 \
        static OccMemo memo;                                                                             \
        auto kern = k_quantize<BITS, GROUP, WF, LR, SF, R4>;                                             \
        return launch_kernel(kern, grid_for((const void*)kern, memo), dim3(kQThreads), lds, st, tm.start, \
                             tm.stop, W, M, K, ldw, s, B, A, rank, rows, codes, scale, zero, wq, q);     \
    } while (0)
#define TTQ_Q_LAUNCH2(WF, LR, R4) \
    if (qs) TTQ_Q_LAUNCH(WF, LR, true, R4); else TTQ_Q_LAUNCH(WF, LR, false, R4)
    if (wf32) {
        if (lr) { TTQ_Q_LAUNCH2(true, true, false); } else { TTQ_Q_LAUNCH2(true, false, false); }
    } else {
        if (lr) { TTQ_Q_LAUNCH2(false, true, false); }
        else if (rb4) { TTQ_Q_LAUNCH2(false, false, true); }
        else { TTQ_Q_LAUNCH2(false, false, false); }
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
