// Group-wise RTN of the scaled weight, packed into int32 words.
//
// [TTQ §method b1] group-wise RTN; [TTQ §method b2] the weight is scaled by the
// AWQ scale of its input channel.  (With dynamic low-rank factors, [TTQ
// §method b5], the residual W - B A is quantized by quantize_lr.hip.)
//
// Mapping: a workgroup (4 waves) owns a strip of 1024 input channels and walks
// blocks of output rows; lane l owns 16 consecutive channels (two 16-byte
// loads of bf16, four of fp32), so a group of g channels spans g/16 adjacent
// lanes and its min/max needs log2(g/16) DPP lane exchanges.  The group's
// step, zero point and 1/step are formed once per lane and row and serve its
// 16 weights.
//
// Arithmetic (rtn.hpp):
//  - v = fp32(w * s);
//  - step: fp32(mx - mn) / (2^b - 1) by a multiply with the rounded
//    reciprocal of the constant and one fma correction, which equals the
//    correctly rounded division for every finite operand (checked
//    exhaustively over all non-negative fp32 values for 3, 7, 15 and 31);
//    then fp16 rounded toward +inf; zero = rne(-mn / step) by an IEEE
//    division;
//  - code: rne(v * (1/step)) + zero, clamped to [0, 2^b - 1].  One fma
//    forms v * (1/step) + (1.5 * 2^23 + zero); the fp32 spacing there is 1,
//    so the result holds the rounded code in its low significand bits; the
//    clamp is one v_med3 (a NaN value gives the lower bound, code 0), and the
//    code is the low bits of the result's bit pattern.  v * (1/step)
//    differs from v / step by a few ulps, and an exact tie (v / step =
//    k + 1/2) goes to whichever side that error puts it, with zero already
//    added: only values within ~1e-6 of a step of a rounding boundary can be
//    decided differently from the oracle.
//  - packing: a lane's 16 codes form 16 * b bits of its row's stream; each
//    code's bit pattern (1.5 * 2^23 + code) is shifted into place with one
//    shift-and-add, and the shifted copies of 1.5 * 2^23 are subtracted as a
//    compile-time constant per word.  For odd b, lane pairs join their
//    fields (96 or 160 bits = 3 or 5 words) after one DPP exchange.
//
// Optionally the kernel also writes the dequantized weight of [TTQ §method b1]
// (QDQ) with the input scale folded back, w~ = bf16(((code - zero) * step) *
// (1/s)), dense [M][K] bf16: the operand of the prompt-sized projection, so
// that the codes need not be read and expanded a second time.  (code - zero)
// comes out exactly as sum - (1.5 * 2^23 + zero).  A w~ larger than 64 MiB
// is written, with the codes of even bit widths (whole 4- or 8-byte fields
// per lane), by streaming stores (stream_stage); the single-word code stores
// of odd widths measured slower streamed.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "quant_launch.hpp"
#include "rtn.hpp"
#include "scales.hpp"

namespace ttq {

constexpr int kQThreads = 256;
constexpr int kLaneCh = 16;                // channels per lane
constexpr int kQChans = kWave * kLaneCh;   // channels per strip (workgroup)

// Sum of the shifted copies of kMagicBits in word wd of a lane's field
// (codes whose first bit lies in that word), modulo 2^32.
template <int BITS>
__device__ __forceinline__ constexpr uint32_t magic_sum(int wd) {
    uint32_t c = 0;
    for (int i = 0; i < kLaneCh; ++i) {
        const int sh = BITS * i - 32 * wd;
        if (sh >= 0 && sh < 32) c += kMagicBits << sh;
    }
    return c;
}

// The 16 * BITS bits of one lane's codes (code i at bits [BITS i, BITS i +
// BITS)) as NW words, the last one partial for odd BITS.  qb holds the bit
// patterns kMagicBits + code.  A code that straddles two words puts its high
// bits at the bottom of the next word.
template <int BITS>
struct LaneField {
    static constexpr int NW = (kLaneCh * BITS + 31) / 32;
    uint32_t w[NW];
};

template <int BITS>
__device__ __forceinline__ LaneField<BITS> pack_lane(const uint32_t (&qb)[kLaneCh]) {
    LaneField<BITS> f;
#pragma unroll
    for (int wd = 0; wd < LaneField<BITS>::NW; ++wd) {
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < kLaneCh; ++i) {
            const int sh = BITS * i - 32 * wd;
            if (sh >= 32 || sh + BITS <= 0) continue;
            if (sh >= 0) acc += qb[i] << sh;                          // shift-and-add
            else acc += (qb[i] - kMagicBits) >> (-sh);                // high bits of a straddling code
        }
        f.w[wd] = acc - magic_sum<BITS>(wd);
    }
    return f;
}

// Group RTN of one lane's 16 values and the stores of its codes, step, zero
// and (optionally) dequantized weights.  All 64 lanes of the wave must call
// this together (cross-lane moves).
template <int BITS, int GROUP, bool NT>
__device__ __forceinline__ void quantize_and_store(const float (&v)[kLaneCh], bool active, int lane, int64_t cu,
                                                   int64_t col, int64_t o, int64_t words_per_row,
                                                   int64_t groups_per_row, uint32_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scale, uint16_t* __restrict__ zero,
                                                   const float (&sinv)[kLaneCh], uint16_t* __restrict__ wq,
                                                   int64_t K) {
    constexpr int GL = GROUP / kLaneCh;           // lanes per group
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < kLaneCh; ++i) { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
    group_minmax<GL>(mn, mx);
    const GroupStep g = group_step<BITS>(mn, mx);
    const float mz = kMagic + g.z;                // exact

    // Codes as kMagic + code (exact integers in fp32).
    float qm[kLaneCh];
    uint32_t qb[kLaneCh];
#pragma unroll
    for (int i = 0; i < kLaneCh; ++i) {
        qm[i] = code_magic<BITS>(v[i], g, mz);
        qb[i] = __builtin_bit_cast(uint32_t, qm[i]);
    }
    if (wq != nullptr && active) {
        // (code - zero) * step is exact in fp32 (a small integer times an fp16 value).
        u32x4 pk0, pk1;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            pk0[p] = pack_bf16x2(((qm[2 * p] - mz) * g.df) * sinv[2 * p],
                                 ((qm[2 * p + 1] - mz) * g.df) * sinv[2 * p + 1]);
            pk1[p] = pack_bf16x2(((qm[8 + 2 * p] - mz) * g.df) * sinv[8 + 2 * p],
                                 ((qm[9 + 2 * p] - mz) * g.df) * sinv[9 + 2 * p]);
        }
        u32x4* dst = (u32x4*)(wq + o * K + col);
        st_nt<NT>(dst, pk0);
        st_nt<NT>(dst + 1, pk1);
    }

    const LaneField<BITS> f = pack_lane<BITS>(qb);
    if constexpr ((BITS & 1) == 0) {
        // 16 b bits = b/2 whole words per lane.
        if (active) {
            uint32_t* wrow = codes + o * words_per_row + cu * (BITS / 2);
            if constexpr (BITS == 2) {
                st_nt<NT>(wrow, f.w[0]);
            } else {
                u32x2 pr = {f.w[0], f.w[1]};
                st_nt<NT>((u32x2*)wrow, pr);
            }
        }
    } else {
        // Odd b: lanes 2m and 2m + 1 hold 16 b bits each (the last word
        // half full); their joint 32 b bits are b whole words.  Each lane
        // receives its partner's field.
        constexpr int NW = LaneField<BITS>::NW;   // 2 (b = 3) or 3 (b = 5)
        static_assert((kLaneCh * BITS) % 32 == 16, "odd bit widths leave half a word per lane");
        uint32_t pw[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) pw[k] = dpp_u<kDppQuadXor1>(f.w[k]);
        const bool even = (lane & 1) == 0;
        uint32_t Lw[NW], Rw[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            Lw[k] = even ? f.w[k] : pw[k];
            Rw[k] = even ? pw[k] : f.w[k];
        }
        // the pair's words: L0 .. L(NW-2), L(NW-1) | R0 << 16, R0 >> 16 | R1 << 16, ...
        uint32_t pair[BITS];
#pragma unroll
        for (int k = 0; k < NW - 1; ++k) pair[k] = Lw[k];
        pair[NW - 1] = (Lw[NW - 1] & 0xFFFFu) | (Rw[0] << 16);
#pragma unroll
        for (int k = 1; k < NW; ++k) pair[NW - 1 + k] = (Rw[k - 1] >> 16) | (Rw[k] << 16);
        if (active) {
            uint32_t* wrow = codes + o * words_per_row + (cu >> 1) * BITS;
            // even lane: the first NW words, odd lane: the remaining BITS - NW
#pragma unroll
            for (int k = 0; k < BITS; ++k)
                if ((k < NW) == even) wrow[k] = pair[k];   // single words: plain stores
        }
    }
    if (active && (cu % GL) == 0) {
        const int64_t gi = o * groups_per_row + col / GROUP;
        scale[gi] = g.dh;
        zero[gi] = f32_to_f16_rne(g.z);
    }
}

// Row batch held in registers: 16 raw bf16 (two 16-byte vectors) or fp32
// (four).
template <bool WF32>
struct RawRow {
    u32x4 a[WF32 ? 4 : 2];
};

// Ordinary (cached) loads: each load instruction of a wave uses half of
// every line it touches (lanes 32 or 64 bytes apart), and the next
// instruction takes the other half from the cache.
template <bool WF32>
__device__ __forceinline__ void load_row(RawRow<WF32>& r, const void* W, int64_t o, int64_t ldw, int64_t col) {
    if constexpr (WF32) {
        const u32x4* p = (const u32x4*)((const float*)W + o * ldw + col);
#pragma unroll
        for (int k = 0; k < 4; ++k) r.a[k] = p[k];
    } else {
        const u32x4* p = (const u32x4*)((const uint16_t*)W + o * ldw + col);
        r.a[0] = p[0];
        r.a[1] = p[1];
    }
}

template <bool WF32>
__device__ __forceinline__ void zero_row(RawRow<WF32>& r) {
#pragma unroll
    for (int k = 0; k < (WF32 ? 4 : 2); ++k) r.a[k] = u32x4{0u, 0u, 0u, 0u};
}

template <bool WF32>
__device__ __forceinline__ void unpack_row(const RawRow<WF32>& r, float (&w)[kLaneCh]) {
    if constexpr (WF32) {
        // Whole-vector casts: this compiler mis-lowers a bit cast whose operand
        // is a single vector element (it reads element 0).
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f32x4 fa = __builtin_bit_cast(f32x4, r.a[k]);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[4 * k + i] = fa[i];
        }
    } else {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[8 * k + 2 * i] = bf16lo_to_f32(r.a[k][i]);
                w[8 * k + 2 * i + 1] = bf16hi_to_f32(r.a[k][i]);
            }
    }
}

template <int BITS, int GROUP, bool WF32, bool SFUSE, bool NT>
__global__ __launch_bounds__(kQThreads) void k_quantize(
    const void* __restrict__ W, int64_t M, int64_t K, int64_t ldw, const float* __restrict__ s,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale, uint16_t* __restrict__ zero,
    uint16_t* __restrict__ wq, QScaleSrc qs) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // row addressing stays scalar
    const int64_t cu = (int64_t)blockIdx.x * kWave + lane;   // 16-channel unit in the row
    const int64_t col = cu * kLaneCh;
    const bool active = col < K;
    const int64_t cbase = (int64_t)blockIdx.x * kQChans;

    // A row block is WSTRIDE x RB rows: each wave takes RB of them (a batch).
    // The workgroup walks row blocks rb = blockIdx.y, + gridDim.y, ... (the
    // grid is sized to the number of workgroups the device holds at once),
    // and each wave issues the loads of its next batch before it processes
    // the current one, so loads stay in flight while the VALU works.
    constexpr int RB = WF32 ? 2 : 4;
    constexpr int WSTRIDE = kQThreads / kWave;    // waves per workgroup
    constexpr int RPB = WSTRIDE * RB;             // rows per block
    const int64_t nrb = (M + RPB - 1) / RPB;
    auto load_batch = [&](RawRow<WF32> (&dst)[RB], int64_t rb) __attribute__((always_inline)) {
        const int64_t ob = rb * RPB + wave;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t o = ob + (int64_t)WSTRIDE * r;
            if (rb < nrb && active && o < M) load_row<WF32>(dst[r], W, o, ldw, col);
            else zero_row<WF32>(dst[r]);
        }
    };

    // the first batch of rows is in flight during the set-up below
    RawRow<WF32> cur[RB];
    load_batch(cur, blockIdx.y);

    // Per-channel scales of this lane's 16 channels, and 1/s by v_rcp_f32
    // (exactly 1 for s = 1) for the dequantized weight.
    float sc[kLaneCh], sinv[kLaneCh];
    if constexpr (SFUSE) {
        // lambda from the statistics' block sums (same order as
        // ttq_awq_scales), then each of the strip's 1024 scales once per
        // workgroup; the loads of both are issued before either is used.
        __shared__ float ssc[kQChans];
        __shared__ double lam_s;
        double ssqv[kQChans / kQThreads];
#pragma unroll
        for (int h = 0; h < kQChans / kQThreads; ++h) {
            const int64_t j = cbase + threadIdx.x + h * kQThreads;
            ssqv[h] = j < K ? qs.ssq[j] : 0.0;
        }
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
            const float v = j < K ? awq_scale(ssqv[h], qs.tn, lam, qs.e) : 1.0f;
            ssc[c] = v;
            if (j < K && blockIdx.y == 0) qs.s_out[j] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kLaneCh; ++i) sc[i] = ssc[lane * kLaneCh + i];
    } else {
#pragma unroll
        for (int i = 0; i < kLaneCh; ++i) sc[i] = 1.0f;
        if (s != nullptr && active) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const f32x4 a = *(const f32x4*)(s + col + 4 * k);
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[4 * k + i] = a[i];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kLaneCh; ++i) sinv[i] = __builtin_amdgcn_rcpf(sc[i]);

    const int64_t words_per_row = K * BITS / 32;
    const int64_t groups_per_row = K / GROUP;

    for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
        RawRow<WF32> nxt[RB];
        load_batch(nxt, rb + gridDim.y);
        const int64_t ob = rb * RPB + wave;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t o = ob + (int64_t)WSTRIDE * r;
            if (o >= M) break;                    // wave-uniform
            float wv[kLaneCh];
            unpack_row<WF32>(cur[r], wv);
            float v[kLaneCh];
#pragma unroll
            for (int i = 0; i < kLaneCh; ++i) v[i] = wv[i] * sc[i];
            quantize_and_store<BITS, GROUP, NT>(v, active, lane, cu, col, o, words_per_row, groups_per_row, codes,
                                                scale, zero, sinv, wq, K);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) cur[r] = nxt[r];
    }
}

// Workgroups per row strip so that the row blocks split evenly over the
// workgroups the device holds at once (each walks the same number of them).
int64_t persistent_rows_grid(int64_t resident, int64_t strips, int64_t nrb) {
    int64_t gy = (resident + strips - 1) / strips;
    if (gy > nrb) gy = nrb;
    if (gy > 65535) gy = 65535;
    if (gy < 1) gy = 1;
    const int64_t rounds = (nrb + gy - 1) / gy;
    return (nrb + rounds - 1) / rounds;
}

int resident_workgroups(const void* kern, int threads, size_t lds, OccMemo& memo, int slot_index) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    std::atomic<int>* slot = (dev >= 0 && dev < kMaxDevices) ? &memo.resident[dev][slot_index] : nullptr;
    int resident = slot ? slot->load(std::memory_order_relaxed) : 0;
    if (resident < 1) {
        int cus = 256, per_cu = 1;
        if (dev >= 0) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds) != hipSuccess || per_cu < 1)
            per_cu = 1;
        resident = cus * per_cu;
        if (slot) slot->store(resident, std::memory_order_relaxed);
    }
    return resident;
}

template <int BITS, int GROUP>
static hipError_t launch_q3(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw, const float* s,
                            uint32_t* codes, uint16_t* scale, uint16_t* zero, uint16_t* wq,
                            const QScaleSrc* qs, hipStream_t st, StageTimer tm) {
    const int64_t strips = (K + kQChans - 1) / kQChans;
    const int rpb = wf32 ? 8 : 16;                // rows per block: 4 waves x RB
    const int64_t nrb = (M + rpb - 1) / rpb;
    const QScaleSrc q = qs ? *qs : QScaleSrc{};
    const int wnt = wq != nullptr && stream_stage(M, K);   // streaming stores for a large staged w~
    // Persistent row loop over as many workgroups as the device holds at
    // once.  The residency of each kernel instantiation is memoized per
    // device: a value the runtime derives from the code object, the same on
    // every call, so the memo never changes a result.
#define TTQ_Q_LAUNCH(WF, SF, NT)                                                                           \
    do {                                                                                                   \
        static OccMemo memo;                                                                               \
        auto kern = k_quantize<BITS, GROUP, WF, SF, NT>;                                                   \
        const int64_t gy = persistent_rows_grid(resident_workgroups((const void*)kern, kQThreads, 0, memo, 0), \
                                                strips, nrb);                                              \
        return launch_kernel(kern, dim3((unsigned)strips, (unsigned)gy), dim3(kQThreads), 0, st, tm.start, \
                             tm.stop, W, M, K, ldw, s, codes, scale, zero, wq, q);                         \
    } while (0)
    // Streaming stores are instantiated for bf16 weights only.
    if (wf32) {
        if (qs) TTQ_Q_LAUNCH(true, true, false); else TTQ_Q_LAUNCH(true, false, false);
    } else if (wnt) {
        if (qs) TTQ_Q_LAUNCH(false, true, true); else TTQ_Q_LAUNCH(false, false, true);
    } else {
        if (qs) TTQ_Q_LAUNCH(false, true, false); else TTQ_Q_LAUNCH(false, false, false);
    }
#undef TTQ_Q_LAUNCH
}

template <int BITS>
static hipError_t launch_q2(int group, const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw, const float* s,
                            uint32_t* codes, uint16_t* scale, uint16_t* zero, uint16_t* wq,
                            const QScaleSrc* qs, hipStream_t st, StageTimer tm) {
    switch (group) {
        case 16: return launch_q3<BITS, 16>(W, wf32, M, K, ldw, s, codes, scale, zero, wq, qs, st, tm);
        case 32: return launch_q3<BITS, 32>(W, wf32, M, K, ldw, s, codes, scale, zero, wq, qs, st, tm);
        case 64: return launch_q3<BITS, 64>(W, wf32, M, K, ldw, s, codes, scale, zero, wq, qs, st, tm);
        case 128: return launch_q3<BITS, 128>(W, wf32, M, K, ldw, s, codes, scale, zero, wq, qs, st, tm);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_quantize(const void* W, bool wf32, int64_t M, int64_t K, int64_t ldw,
                           const float* s, int bits, int group, const float* B, const float* A,
                           int rank, uint32_t* codes, uint16_t* scale, uint16_t* zero,
                           uint16_t* wq, hipStream_t st, const QScaleSrc* qs, StageTimer tm) {
    if (rank > 0)
        return launch_quantize_lr(W, wf32, M, K, ldw, s, bits, group, B, A, rank, codes, scale, zero, wq, st, qs, tm);
    switch (bits) {
        case 2: return launch_q2<2>(group, W, wf32, M, K, ldw, s, codes, scale, zero, wq, qs, st, tm);
        case 3: return launch_q2<3>(group, W, wf32, M, K, ldw, s, codes, scale, zero, wq, qs, st, tm);
        case 4: return launch_q2<4>(group, W, wf32, M, K, ldw, s, codes, scale, zero, wq, qs, st, tm);
        case 5: return launch_q2<5>(group, W, wf32, M, K, ldw, s, codes, scale, zero, wq, qs, st, tm);
    }
    return hipErrorInvalidValue;
}

}  // namespace ttq
