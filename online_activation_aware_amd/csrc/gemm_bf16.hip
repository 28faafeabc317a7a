// Projection with an already dequantized (QDQ) weight: Y = X W~^T on the
// gfx950 matrix cores, bf16 operands, fp32 accumulation.
//
// [TTQ §method b1] quantization with QDQ operations: for prompt-sized token
// counts the weight is dequantized once, w~[o][j] = bf16((code - zero) * step
// * (1/s[j])) (written by the quantizer, or by k_dequant from packed codes),
// and every token tile then reuses it.  The per-element arithmetic is exactly
// that of the fused dequantize-in-LDS kernel, so both paths see identical
// bf16 weights.
//
// Tiling: 128 output rows x 256 tokens per workgroup; when such tiles would
// leave most compute units idle, two K slices (fp32 partials, then their
// ordered sum) or 128 x 128 tiles.  8 waves (2 per SIMD), each 64 x 64 (or
// 64 x 32): 4 x 4 (4 x 2) MFMA 16x16x32 per 32-deep slice.  Both operands arrive
// by buffer->LDS DMA into 3-slot rings issued two steps ahead (no staging
// registers); 128-byte LDS rows with an XOR chunk swizzle (conflict-free);
// one barrier per 64-deep K step, each wave waiting only for its own DMA.
// Fragments are double-buffered in registers: the LDS reads of one 32-deep
// half overlap the MFMAs of the other.  (Raising the wave priority around the
// MFMA phases measured ~0.3 us slower on the 4096 x 4096, T = 2048 layer.)
// Optionally the epilogue adds the low-rank term Z B^T (fp32, rank <= 64)
// before the store.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace ttq {

constexpr int kBM = 128, kBK = 64;            // token tile BN: 256, or 128 for small grids
constexpr int kBThreads = 512;
constexpr int kBRowB = kBK * 2;                  // 128-byte LDS rows
constexpr unsigned kXcds = 8, kXcdRows = 8;     // XCDs; row tiles per XCD block

template <int BN, bool YF32, bool LR>
__global__ __launch_bounds__(kBThreads, 1) void k_gemm_bf16(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, int64_t ldx, const uint16_t* __restrict__ Wq,
    int64_t ldw, int64_t M, void* __restrict__ Y, int64_t ldy, int yvec, const float* __restrict__ Z,
    const float* __restrict__ Bm, int rank, int nz, int64_t zstride) {
    constexpr int NW = kBThreads / kWave;                       // 8 waves
    constexpr int WT = BN / 4;                                  // tokens per wave (64 or 32)
    constexpr int FB = WT / 16;                                 // token fragments per wave
    constexpr int XOPS = BN * kBRowB / 1024 / NW;               // 1 KB DMA ops per wave for X (4 or 2)
    constexpr int WOPS = kBM * kBRowB / 1024 / NW;              // ... for W~ (2)
    constexpr int OPS = XOPS + WOPS;
    __shared__ __attribute__((aligned(1024))) uint8_t sX0[BN * kBRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sX1[BN * kBRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sX2[BN * kBRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sW0[kBM * kBRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sW1[kBM * kBRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sW2[kBM * kBRowB];

    // Split over K (grid.z > 1): slice z multiplies input channels
    // [z K, (z + 1) K) and stores its partial product at Y + z zstride.
    if (gridDim.z > 1) {
        X += (int64_t)blockIdx.z * K;
        Wq += (int64_t)blockIdx.z * K;
        Y = (char*)Y + (int64_t)blockIdx.z * zstride * (YF32 ? 4 : 2);
    }
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 2, wn = wave & 3;      // 2 x 4 waves of 64 x WT
    // Tile order for the eight XCDs, each with its own L2: workgroups are
    // dispatched to XCDs round-robin by linear id, so the n/8 ids an XCD
    // receives are given consecutive places in an order that walks groups of
    // 8 row tiles across the token tiles; each XCD then covers a compact
    // block of the output (4096 x 2048 output: 8 row x 4 token tiles per XCD,
    // 16.8 MB of operands read instead of 21).  Grids that do not divide
    // keep the plain order.
    int64_t ob = blockIdx.x, tb = blockIdx.y;
    {
        const unsigned mt = gridDim.x, nt = gridDim.y, n = mt * nt;
        if (n % kXcds == 0 && mt % kXcdRows == 0) {
            const unsigned b = blockIdx.x + mt * blockIdx.y;
            const unsigned v = (b % kXcds) * (n / kXcds) + b / kXcds;
            const unsigned r = v % (kXcdRows * nt);
            ob = (int64_t)(v / (kXcdRows * nt)) * kXcdRows + r % kXcdRows;
            tb = r / kXcdRows;
        }
    }
    const int64_t o0 = ob * kBM;
    const int64_t t0 = tb * BN;
    const int rows_x = (int)min((int64_t)BN, T - t0);
    const int rows_w = (int)min((int64_t)kBM, M - o0);
    const rsrc_t rx = make_rsrc(X + t0 * ldx, ((int64_t)(rows_x - 1) * ldx + K) * 2);
    const rsrc_t rw = make_rsrc(Wq + o0 * ldw, ((int64_t)(rows_w - 1) * ldw + K) * 2);

    // DMA op i of this wave fills LDS rows 8 (ops*wave + i) .. +7; lane l lands
    // in row (.. + l/8) at chunk position l%8, holding chunk (l%8) ^ (row & 7).
    const int rl = lane >> 3;
    const int ch = (lane & 7) ^ rl;
    const int xoff0 = ((wave * 8 * XOPS + rl) * (int)ldx + 8 * ch) * 2;
    const int woff0 = ((wave * 8 * WOPS + rl) * (int)ldw + 8 * ch) * 2;
    const int xrow8 = 8 * (int)ldx * 2, wrow8 = 8 * (int)ldw * 2;

    f32x4 acc[4][FB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](uint8_t* xd, uint8_t* wd, int64_t k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XOPS; ++i)
            dma_to_lds<16>(rx, xd + (wave * XOPS + i) * 1024, xoff0 + i * xrow8, (int)k0 * 2);
#pragma unroll
        for (int i = 0; i < WOPS; ++i)
            dma_to_lds<16>(rw, wd + (wave * WOPS + i) * 1024, woff0 + i * wrow8, (int)k0 * 2);
    };
    // Fragments of one 32-deep half of a K step: a = 4 row fragments of W~,
    // b = FB token fragments of X.  Set 0 holds the first half, set 1 the
    // second, so the matrix cores work on one set while the other is read.
    u32x4 a0[4], b0[FB], a1[4], b1[FB];
    auto rd = [&](u32x4* a, u32x4* b, const uint8_t* xs, const uint8_t* ws, int kk) __attribute__((always_inline)) {
        const int c = 4 * kk + (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *(const u32x4*)(ws + lds_swz(wm * 64 + 16 * i + (lane & 15), c));
#pragma unroll
        for (int j = 0; j < FB; ++j) b[j] = *(const u32x4*)(xs + lds_swz(wn * WT + 16 * j + (lane & 15), c));
    };
    auto mm = [&](const u32x4* a, const u32x4* b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < FB; ++j) acc[i][j] = mfma_16x16x32(a[i], b[j], acc[i][j]);
    };
    // Step kt (ring slot xc/wc): its first-half fragments are read while the
    // previous step's second half runs on the matrix cores; then the DMA two
    // steps ahead is issued and the second-half fragments are read while the
    // first half runs.  Every LDS read of the slot has completed before the
    // closing barrier, so the slot can be refilled one step later, and the
    // loop iterations begin with no LDS read in flight.
    auto step = [&](bool first, bool more, const uint8_t* xc, const uint8_t* wc, uint8_t* xn, uint8_t* wn_,
                    int64_t kt) __attribute__((always_inline)) {
        rd(a0, b0, xc, wc, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (!first) mm(a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        if (more) issue(xn, wn_, (kt + 2) * kBK);
        rd(a1, b1, xc, wc, 1);
        __builtin_amdgcn_sched_barrier(0);
        mm(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        if (more) wait_vmcnt<OPS>();              // step kt+1's operands have landed
        else wait_vmcnt<0>();
        sync_lds();
    };

    const int64_t nk = K / kBK;
    issue(sX0, sW0, 0);
    if (nk > 1) {
        issue(sX1, sW1, kBK);
        wait_vmcnt<OPS>();
    } else {
        wait_vmcnt<0>();
    }
    sync_lds();
    step(true, 2 < nk, sX0, sW0, sX2, sW2, 0);
    int64_t kt = 1;
    for (; kt + 5 <= nk; kt += 3) {
        step(false, true, sX1, sW1, sX0, sW0, kt + 0);
        step(false, true, sX2, sW2, sX1, sW1, kt + 1);
        step(false, true, sX0, sW0, sX2, sW2, kt + 2);
    }
    for (; kt < nk; kt += 3) {
        step(false, kt + 2 < nk, sX1, sW1, sX0, sW0, kt + 0);
        if (kt + 1 < nk) step(false, kt + 3 < nk, sX2, sW2, sX1, sW1, kt + 1);
        if (kt + 2 < nk) step(false, kt + 4 < nk, sX0, sW0, sX2, sW2, kt + 2);
    }
    mm(a1, b1);

    if constexpr (LR) {
        // [TTQ §method b5] low-rank term Y += B (A X) = Z B^T, in fp32, added
        // before the store.  Every DMA has landed and every wave has passed
        // the last barrier, so the ring slots are free: the tile's Z (BN
        // tokens) and B (128 rows) are staged there transposed (rank-major,
        // so lanes read consecutive tokens / rows), 32 ranks at a time (what
        // one slot holds); the ranks are added in order.
        float* zs = (float*)sX0;                  // [32][BN]
        float* bs = (float*)sW0;                  // [32][128]
        for (int kc = 0; kc < rank; kc += 32) {
            const int nk = min(32, rank - kc);
            if (kc > 0) __syncthreads();          // the previous chunk's reads are done
            for (int idx = tid; idx < nk * BN; idx += kBThreads) {
                const int k = kc + idx / BN, tt = idx % BN;
                float zv = 0.0f;
                if (t0 + tt < T) {                // Z's K-slice partials, added in slice order
                    zv = Z[(t0 + tt) * rank + k];
                    for (int p = 1; p < nz; ++p) zv += Z[((int64_t)p * T + t0 + tt) * rank + k];
                }
                zs[idx] = zv;
            }
            for (int idx = tid; idx < nk * kBM; idx += kBThreads) {
                const int k = kc + idx / kBM, oo = idx % kBM;
                bs[idx] = (o0 + oo < M) ? Bm[(o0 + oo) * rank + k] : 0.0f;
            }
            __syncthreads();
            for (int k = 0; k < nk; ++k) {
                float zt[FB];
#pragma unroll
                for (int j = 0; j < FB; ++j) zt[j] = zs[k * BN + wn * WT + 16 * j + (lane & 15)];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 bo = *(const f32x4*)(bs + k * kBM + wm * 64 + 16 * i + 4 * (lane >> 4));
#pragma unroll
                    for (int j = 0; j < FB; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(bo[r], zt[j], acc[i][j][r]);
                }
            }
        }
    }

    // Lane holds Y^T[o + r][t] for r = 0..3 (4 consecutive o of token t).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t o = o0 + wm * 64 + 16 * i + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            const int64_t t = t0 + wn * WT + 16 * j + (lane & 15);
            if (t >= T) continue;
            store_y4<YF32>(Y, t * ldy + o, M - o, yvec, acc[i][j]);
        }
    }
}

bool gemm_bf16_supported(int64_t T, int64_t K, int64_t ldx, int64_t ldw) {
    return T > 0 && K % kBK == 0 && (int64_t)256 * ldx * 2 < ((int64_t)1 << 31) &&
           (int64_t)kBM * ldw * 2 < ((int64_t)1 << 31);
}

// Y = P[0] + P[1] + ... (fp32 partial products of the K slices, added in
// slice order, rows of ldp floats), stored as fp32 or bf16 (RNE).  The
// partials are read with the nontemporal hint: they are dead afterwards
// (14336 -> 4096, T = 1024: layer 184.8 -> 181.9 us).
template <bool YF32>
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ P, int S, int64_t T, int64_t M,
                                                   int64_t ldp, int64_t zstride, void* __restrict__ Y, int64_t ldy,
                                                   int yvec) {
    const int64_t nq = (M + 3) / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < T * nq; i += (int64_t)gridDim.x * 256) {
        const int64_t t = i / nq, o = 4 * (i % nq);
        f32x4 acc = ld_nc((const f32x4*)(P + t * ldp + o));
        for (int s = 1; s < S; ++s) {
            const f32x4 v = ld_nc((const f32x4*)(P + s * zstride + t * ldp + o));
            acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
        }
        store_y4<YF32>(Y, t * ldy + o, M - o, yvec, acc);
    }
}

// K slices for a projection whose 128 x 256 tiles alone would leave most
// compute units idle: two slices of at least 4096 channels each keep the
// 256-token tiles (and their lower LDS traffic per flop) and double the
// workgroups; otherwise none (the 128 x 128 tiles are used instead).
int gemm_bf16_splits(int64_t T, int64_t K, int64_t M) {
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((T + 255) / 256);
    if (tiles >= 192 || tiles * 2 > 512) return 1;
    if (K % (2 * kBK) != 0 || K / 2 < 4096) return 1;
    return 2;
}

static int64_t split_ld(int64_t M) { return (M + 3) / 4 * 4; }

size_t gemm_bf16_split_ws_bytes(int64_t T, int64_t K, int64_t M) {
    const int S = gemm_bf16_splits(T, K, M);
    return S > 1 ? (size_t)S * (size_t)T * (size_t)split_ld(M) * sizeof(float) : 0;
}

hipError_t launch_gemm_bf16(const uint16_t* X, int64_t T, int64_t K, int64_t ldx, const uint16_t* Wq,
                            int64_t ldw, int64_t M, void* Y, bool yf32, int64_t ldy, hipStream_t st,
                            StageTimer tm, const LowrankEpilogue* lr, float* split_ws) {
    const int yvec = ((uintptr_t)Y % 16 == 0) && ((ldy * (yf32 ? 4 : 2)) % 16 == 0);
    const int64_t mt = (M + kBM - 1) / kBM;
    const float* Z = lr ? lr->Z : nullptr;
    const float* B = lr ? lr->B : nullptr;
    const int rank = lr ? lr->rank : 0;
    const int nz = lr ? lr->nz : 1;
    const int S = (lr == nullptr && split_ws != nullptr) ? gemm_bf16_splits(T, K, M) : 1;
    if (S > 1) {
        // fp32 partials of the K slices into the workspace (rows of ldp
        // floats, 16-byte aligned), then their ordered sum into Y.
        const int64_t ldp = split_ld(M), zs = T * ldp;
        const dim3 grid((unsigned)mt, (unsigned)((T + 255) / 256), (unsigned)S);
        hipError_t e = launch_kernel(k_gemm_bf16<256, true, false>, grid, dim3(kBThreads), 0, st, tm.start,
                                     nullptr, X, T, K / S, ldx, Wq, ldw, M, (void*)split_ws, ldp, 1,
                                     (const float*)nullptr, (const float*)nullptr, 0, 1, zs);
        if (e != hipSuccess) return e;
        const int64_t work = T * ((M + 3) / 4);
        const unsigned blocks = (unsigned)std::min<int64_t>((work + 255) / 256, 4096);
        if (yf32)
            return launch_kernel(k_split_sum<true>, dim3(blocks), dim3(256), 0, st, nullptr, tm.stop,
                                 (const float*)split_ws, S, T, M, ldp, zs, Y, ldy, yvec);
        return launch_kernel(k_split_sum<false>, dim3(blocks), dim3(256), 0, st, nullptr, tm.stop,
                             (const float*)split_ws, S, T, M, ldp, zs, Y, ldy, yvec);
    }
    // 128 x 256 tiles, unless they would leave most compute units idle; then
    // 128 x 128 (twice the workgroups).
    const bool narrow = mt * ((T + 255) / 256) < 192;
    const dim3 grid((unsigned)mt, (unsigned)((T + (narrow ? 127 : 255)) / (narrow ? 128 : 256)));
#define TTQ_B_LAUNCH(BN, YF, LRF)                                                                          \
    return launch_kernel(k_gemm_bf16<BN, YF, LRF>, grid, dim3(kBThreads), 0, st, tm.start, tm.stop, X, T, K, \
                         ldx, Wq, ldw, M, Y, ldy, yvec, Z, B, rank, nz, (int64_t)0)
#define TTQ_B_LAUNCH2(BN)                                 \
    if (rank > 0) {                                       \
        if (yf32) TTQ_B_LAUNCH(BN, true, true);           \
        TTQ_B_LAUNCH(BN, false, true);                    \
    }                                                     \
    if (yf32) TTQ_B_LAUNCH(BN, true, false);              \
    TTQ_B_LAUNCH(BN, false, false)
    if (narrow) { TTQ_B_LAUNCH2(128); }
    TTQ_B_LAUNCH2(256);
#undef TTQ_B_LAUNCH2
#undef TTQ_B_LAUNCH
}

}  // namespace ttq
