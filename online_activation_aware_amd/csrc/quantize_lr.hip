// Group-wise RTN of the residual W - B A of the dynamic low-rank factors.
//
// [TTQ §method b5]: W = W_q + B A with the residual W_q quantized at once;
// [TTQ §method b1, b2] group-wise RTN of the residual scaled by the AWQ scale
// of its input channel.  The value quantized is
//   v = fp32((W - sum_k B[o][k] A[k][j]) * s[j]),
// the residual accumulated in fp64 in rank order (every product of two fp32
// values is exact in fp64), then one fp64 multiply by s and one rounding.
//
// The residual costs `rank` fp64 fmas per weight, so this kernel is laid out
// for them: a workgroup (4 waves) owns a strip of 512 input channels, lane l
// owns 8 consecutive channels, and each wave takes batches of 4 rows, so that
// every A value read serves 4 fmas.  The strip of A (up to 16 ranks, 32 KB)
// and each wave's B values for its batch are staged in LDS, and the rank
// loop runs in chunks of 4 ranks whose LDS reads are all issued before their
// fmas; ranks beyond 16 read A from global memory.  Group RTN and the code
// arithmetic are those of the kernel without factors (rtn.hpp); a quad of
// lanes holds 32 codes = `bits` words, joined by quad broadcasts.  Optionally
// the dequantized weight w~ is written, as there.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "quant_launch.hpp"
#include "rtn.hpp"
#include "scales.hpp"

namespace ttq {

constexpr int kLrThreads = 256;
constexpr int kLrLaneCh = 8;
constexpr int kLrChans = kWave * kLrLaneCh;   // channels per strip
constexpr int kLrLdsRanks = 16;               // ranks of A staged in LDS (32 KB)
constexpr int kLrMaxRank = 64;
constexpr int kLrRB = 4;                      // rows per wave batch
constexpr int kLrChunk = 4;                   // ranks whose LDS reads are issued together

// 8 raw weights: bf16 (one 16-byte vector) or fp32 (two).
template <bool WF32>
struct RawRow8 {
    u32x4 a[WF32 ? 2 : 1];
};

template <bool WF32>
__device__ __forceinline__ void load_row8(RawRow8<WF32>& r, const void* W, int64_t o, int64_t ldw, int64_t col) {
    if constexpr (WF32) {
        const u32x4* p = (const u32x4*)((const float*)W + o * ldw + col);
        r.a[0] = ld_nc(p);
        r.a[1] = ld_nc(p + 1);
    } else {
        r.a[0] = ld_nc((const u32x4*)((const uint16_t*)W + o * ldw + col));
    }
}

template <bool WF32>
__device__ __forceinline__ void unpack_row8(const RawRow8<WF32>& r, double (&w)[kLrLaneCh]) {
    if constexpr (WF32) {
        // Whole-vector casts: this compiler mis-lowers a bit cast whose operand
        // is a single vector element (it reads element 0).
        const f32x4 fa = __builtin_bit_cast(f32x4, r.a[0]), fb = __builtin_bit_cast(f32x4, r.a[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = (double)fa[i];
            w[4 + i] = (double)fb[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = (double)bf16lo_to_f32(r.a[0][i]);
            w[2 * i + 1] = (double)bf16hi_to_f32(r.a[0][i]);
        }
    }
}

// Group RTN of one lane's 8 values and the stores of the quad's 32 codes,
// the step and zero, and (optionally) the dequantized weights.  All 64 lanes
// of the wave must call this together (cross-lane moves).
template <int BITS, int GROUP, bool NT>
__device__ __forceinline__ void quantize8_and_store(const float (&v)[kLrLaneCh], bool active, int lane, int64_t cu,
                                                    int64_t col, int64_t o, int64_t words_per_row,
                                                    int64_t groups_per_row, uint32_t* __restrict__ codes,
                                                    uint16_t* __restrict__ scale, uint16_t* __restrict__ zero,
                                                    const float (&sinv)[kLrLaneCh], uint16_t* __restrict__ wq,
                                                    int64_t K) {
    constexpr int GL = GROUP / kLrLaneCh;         // lanes per group
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < kLrLaneCh; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
    group_minmax<GL>(mn, mx);
    const GroupStep g = group_step<BITS>(mn, mx);
    const float mz = kMagic + g.z;

    typedef typename std::conditional<(kLrLaneCh * BITS <= 32), uint32_t, uint64_t>::type field_t;
    field_t field = 0;
    float qm[kLrLaneCh];
#pragma unroll
    for (int i = 0; i < kLrLaneCh; ++i) {
        qm[i] = code_magic<BITS>(v[i], g, mz);
        field |= (field_t)(__builtin_bit_cast(uint32_t, qm[i]) - kMagicBits) << (BITS * i);
    }
    if (wq != nullptr && active) {
        // (code - zero) * step is exact in fp32 (a small integer times an fp16 value).
        u32x4 pk;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            pk[p] = pack_bf16x2(((qm[2 * p] - mz) * g.df) * sinv[2 * p], ((qm[2 * p + 1] - mz) * g.df) * sinv[2 * p + 1]);
        st_nt<NT>((u32x4*)(wq + o * K + col), pk);
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
        if constexpr (kLrLaneCh * BITS > 32) {
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
            const int off = kLrLaneCh * BITS * k - 32 * j;
            if (off >= 32 || off + kLrLaneCh * BITS <= 0) continue;
            wv |= off >= 0 ? (uint32_t)(fq[k] << off) : (uint32_t)(fq[k] >> (-off));
        }
        return wv;
    };
    if (active) {
        const int j = lane & 3;
        uint32_t* wrow = codes + o * words_per_row + (cu >> 2) * BITS;
        if (j < BITS) wrow[j] = word(j);                   // single words: plain stores
        if (BITS > 4 && j == 0) wrow[4] = word(4);
        if ((cu % GL) == 0) {
            const int64_t gi = o * groups_per_row + col / GROUP;
            scale[gi] = g.dh;
            zero[gi] = f32_to_f16_rne(g.z);
        }
    }
}

template <int BITS, int GROUP, bool WF32, bool SFUSE, bool NT>
__global__ __launch_bounds__(kLrThreads) void k_quantize_lr(
    const void* __restrict__ W, int64_t M, int64_t K, int64_t ldw, const float* __restrict__ s,
    const float* __restrict__ B, const float* __restrict__ A, int rank, uint32_t* __restrict__ codes,
    uint16_t* __restrict__ scale, uint16_t* __restrict__ zero, uint16_t* __restrict__ wq, QScaleSrc qs) {
    // A strip: [ranks staged, a multiple of kLrChunk, zero past rank][kLrChans] fp32
    extern __shared__ __attribute__((aligned(16))) float sA[];
    constexpr int WSTRIDE = kLrThreads / kWave;
    // each wave's B values for its batch of rows: [rank][kLrRB] fp32
    __shared__ __attribute__((aligned(16))) float sB[WSTRIDE][kLrMaxRank][kLrRB];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // row addressing stays scalar
    const int64_t cu = (int64_t)blockIdx.x * kWave + lane;   // 8-channel unit in the row
    const int64_t col = cu * kLrLaneCh;
    const bool active = col < K;
    const int64_t cbase = (int64_t)blockIdx.x * kLrChans;

    constexpr int RPB = WSTRIDE * kLrRB;
    const int64_t nrb = (M + RPB - 1) / RPB;
    auto load_batch = [&](RawRow8<WF32> (&dst)[kLrRB], int64_t rb) __attribute__((always_inline)) {
        const int64_t ob = rb * RPB + wave;
#pragma unroll
        for (int r = 0; r < kLrRB; ++r) {
            const int64_t o = ob + (int64_t)WSTRIDE * r;
            if (rb < nrb && active && o < M) {
                load_row8<WF32>(dst[r], W, o, ldw, col);
            } else {
#pragma unroll
                for (int k = 0; k < (WF32 ? 2 : 1); ++k) dst[r].a[k] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // the first batch of rows is in flight during the set-up below
    RawRow8<WF32> cur[kLrRB];
    load_batch(cur, blockIdx.y);

    const int lds_ranks = rank < kLrLdsRanks ? rank : kLrLdsRanks;
    const int lds_pad = (lds_ranks + kLrChunk - 1) / kLrChunk * kLrChunk;
    for (int idx = threadIdx.x; idx < lds_pad * kLrChans; idx += kLrThreads) {
        const int k = idx / kLrChans, c = idx % kLrChans;
        sA[idx] = (k < lds_ranks && cbase + c < K) ? A[(int64_t)k * K + cbase + c] : 0.0f;
    }

    float sc[kLrLaneCh], sinv[kLrLaneCh];
    if constexpr (SFUSE) {
        // lambda from the statistics' block sums (same order as
        // ttq_awq_scales), then each of the strip's 512 scales once per
        // workgroup; the loads of both are issued before either is used.
        __shared__ float ssc[kLrChans];
        __shared__ double lam_s;
        double ssqv[kLrChans / kLrThreads];
#pragma unroll
        for (int h = 0; h < kLrChans / kLrThreads; ++h) {
            const int64_t j = cbase + threadIdx.x + h * kLrThreads;
            ssqv[h] = j < K ? qs.ssq[j] : 0.0;
        }
        if (wave == 0) {
            const double tot = blocks_total(qs.bsum, (K + kBlockCh - 1) / kBlockCh, lane);
            if (lane == 0) lam_s = qs.lambda_rel * (tot / (double)K);
        }
        __syncthreads();
        const double lam = lam_s;
#pragma unroll
        for (int h = 0; h < kLrChans / kLrThreads; ++h) {
            const int c = threadIdx.x + h * kLrThreads;
            const int64_t j = cbase + c;
            const float v = j < K ? awq_scale(ssqv[h], qs.tn, lam, qs.e) : 1.0f;
            ssc[c] = v;
            if (j < K && blockIdx.y == 0) qs.s_out[j] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kLrLaneCh; ++i) sc[i] = ssc[lane * kLrLaneCh + i];
    } else {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kLrLaneCh; ++i) sc[i] = 1.0f;
        if (s != nullptr && active) {
            const f32x4 a = *(const f32x4*)(s + col), b = *(const f32x4*)(s + col + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) { sc[i] = a[i]; sc[4 + i] = b[i]; }
        }
    }
#pragma unroll
    for (int i = 0; i < kLrLaneCh; ++i) sinv[i] = __builtin_amdgcn_rcpf(sc[i]);

    const int64_t words_per_row = K * BITS / 32;
    const int64_t groups_per_row = K / GROUP;
    const int rank_pad = (rank + kLrChunk - 1) / kLrChunk * kLrChunk;

    for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
        RawRow8<WF32> nxt[kLrRB];
        load_batch(nxt, rb + gridDim.y);
        const int64_t ob = rb * RPB + wave;
        // this wave's B rows for the batch, rank-major (zero past rank and
        // past M: the fma then leaves the residual unchanged)
        for (int idx = lane; idx < rank_pad * kLrRB; idx += kWave) {
            const int k = idx / kLrRB, r = idx % kLrRB;
            const int64_t o = ob + (int64_t)WSTRIDE * r;
            sB[wave][k][r] = (k < rank && o < M) ? B[o * rank + k] : 0.0f;
        }
        double acc[kLrRB][kLrLaneCh];
#pragma unroll
        for (int r = 0; r < kLrRB; ++r) unpack_row8<WF32>(cur[r], acc[r]);
        // the wave's own LDS writes are complete (ds ordering within a wave)
        __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0)
        // Ranks in chunks: all LDS reads of a chunk are issued, then its fmas
        // run rank by rank in order.
        for (int k0 = 0; k0 < rank_pad; k0 += kLrChunk) {
            f32x4 av[kLrChunk][2], bv[kLrChunk];
#pragma unroll
            for (int c = 0; c < kLrChunk; ++c) {
                const int k = k0 + c;
                bv[c] = *(const f32x4*)&sB[wave][k][0];
                if (k < lds_pad) {
                    const f32x4* ak = (const f32x4*)(sA + k * kLrChans + lane * kLrLaneCh);
                    av[c][0] = ak[0];
                    av[c][1] = ak[1];
                } else {
                    // ranks beyond the LDS strip: A from global memory
                    const bool in = active && k < rank;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        av[c][0][i] = in ? A[(int64_t)k * K + col + i] : 0.0f;
                        av[c][1][i] = in ? A[(int64_t)k * K + col + 4 + i] : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < kLrChunk; ++c) {
                double ad[kLrLaneCh];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ad[i] = (double)av[c][0][i];
                    ad[4 + i] = (double)av[c][1][i];
                }
#pragma unroll
                for (int r = 0; r < kLrRB; ++r) {
                    const double nb = -(double)bv[c][r];
#pragma unroll
                    for (int i = 0; i < kLrLaneCh; ++i) acc[r][i] = __builtin_fma(nb, ad[i], acc[r][i]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kLrRB; ++r) {
            const int64_t o = ob + (int64_t)WSTRIDE * r;
            if (o >= M) break;                    // wave-uniform
            float v[kLrLaneCh];
#pragma unroll
            for (int i = 0; i < kLrLaneCh; ++i) v[i] = (float)(acc[r][i] * (double)sc[i]);
            quantize8_and_store<BITS, GROUP, NT>(v, active, lane, cu, col, o, words_per_row, groups_per_row, codes,
                                                 scale, zero, sinv, wq, K);
        }
#pragma unroll
        for (int r = 0; r < kLrRB; ++r) cur[r] = nxt[r];
    }
}

template <int BITS, int GROUP>
static hipError_t launch_lr3(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw, const float* s,
                             const float* B, const float* A, int rank, uint32_t* codes, uint16_t* scale,
                             uint16_t* zero, uint16_t* wq, const QScaleSrc* qs, hipStream_t st, StageTimer tm) {
    const int64_t strips = (K + kLrChans - 1) / kLrChans;
    const int64_t nrb = (M + kLrThreads / kWave * kLrRB - 1) / (kLrThreads / kWave * kLrRB);
    const int lds_ranks = rank < kLrLdsRanks ? rank : kLrLdsRanks;
    const size_t lds = (size_t)((lds_ranks + kLrChunk - 1) / kLrChunk * kLrChunk) * kLrChans * sizeof(float);
    const QScaleSrc q = qs ? *qs : QScaleSrc{};
    const int wnt = wq != nullptr && stream_stage(M, K);   // streaming stores for a large staged w~
#define TTQ_LR_LAUNCH(WF, SF, NT)                                                                              \
    do {                                                                                                       \
        static OccMemo memo;                                                                                   \
        auto kern = k_quantize_lr<BITS, GROUP, WF, SF, NT>;                                                    \
        const int64_t gy = persistent_rows_grid(resident_workgroups((const void*)kern, kLrThreads, lds, memo,     \
                                                                    lds_ranks),                                \
                                                strips, nrb);                                                  \
        return launch_kernel(kern, dim3((unsigned)strips, (unsigned)gy), dim3(kLrThreads), lds, st, tm.start,   \
                             tm.stop, W, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, q);                 \
    } while (0)
    // Streaming stores are instantiated for bf16 weights only.
    if (wf32) {
        if (qs) TTQ_LR_LAUNCH(true, true, false); else TTQ_LR_LAUNCH(true, false, false);
    } else if (wnt) {
        if (qs) TTQ_LR_LAUNCH(false, true, true); else TTQ_LR_LAUNCH(false, false, true);
    } else {
        if (qs) TTQ_LR_LAUNCH(false, true, false); else TTQ_LR_LAUNCH(false, false, false);
    }
#undef TTQ_LR_LAUNCH
}

template <int BITS>
static hipError_t launch_lr2(int group, const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw, const float* s,
                             const float* B, const float* A, int rank, uint32_t* codes, uint16_t* scale,
                             uint16_t* zero, uint16_t* wq, const QScaleSrc* qs, hipStream_t st, StageTimer tm) {
    switch (group) {
        case 16: return launch_lr3<BITS, 16>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 32: return launch_lr3<BITS, 32>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 64: return launch_lr3<BITS, 64>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 128: return launch_lr3<BITS, 128>(W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_quantize_lr(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw, const float* s, int bits,
                              int group, const float* B, const float* A, int rank, uint32_t* codes, uint16_t* scale,
                              uint16_t* zero, uint16_t* wq, hipStream_t st, const QScaleSrc* qs, StageTimer tm) {
    if (rank < 1 || rank > 64) return hipErrorInvalidValue;
    switch (bits) {
        case 2: return launch_lr2<2>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 3: return launch_lr2<3>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 4: return launch_lr2<4>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
        case 5: return launch_lr2<5>(group, W, wf32, M, K, ldw, s, B, A, rank, codes, scale, zero, wq, qs, st, tm);
    }
    return hipErrorInvalidValue;
}

}  // namespace ttq
