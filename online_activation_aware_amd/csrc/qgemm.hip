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
            if constexpr (YF32) {
                float* yp = (float*)Y + t * ldy + o;
                if (yvec && o + 4 <= M) {
                    *(f32x4*)yp = acc[i][j];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (o + r < M) yp[r] = acc[i][j][r];
                }
            } else {
                uint16_t* yp = (uint16_t*)Y + t * ldy + o;
                if (yvec && o + 4 <= M) {
                    u32x2 v = {pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
                    *(u32x2*)yp = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (o + r < M) yp[r] = (uint16_t)f32_to_bf16(acc[i][j][r]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Wide-tile variant for bf16 X and prompt-sized T: 128 rows x 256 tokens per
// workgroup, so each dequantized weight feeds 256 tokens.  Two LDS stages
// (108 KiB): while the MFMAs read stage k, the codes and X of step k+1 are
// already in flight from global memory, and are dequantized into the other
// stage right after; one barrier per 64-deep K step.  Waves are 2 x 2, each
// owning 64 rows x 128 tokens (4 x 8 MFMA tiles, 128 accumulators).

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit buffer, gfx9-family descriptor

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// 8 codes (a 8*BITS-bit field, already shifted down) -> 8 bf16 weights
// (code - zero) * step * (1/s), packed in pairs.
template <int BITS>
__device__ __forceinline__ u32x4 dequant8(uint64_t field, float zf, float df, const float (&inv)[8]) {
    float q[8];
    if constexpr (BITS == 4) {
        const uint32_t w = (uint32_t)field;
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            q[2 * b] = (float)((lo >> (8 * b)) & 0xFFu);      // v_cvt_f32_ubyteN
            q[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = (float)(uint32_t)((field >> (BITS * i)) & ((1u << BITS) - 1));
    }
    const float nzd = -zf * df;                   // exact: small integer times an fp16 value
    u32x4 out;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float w0 = __builtin_fmaf(q[2 * p], df, nzd) * inv[2 * p];
        const float w1 = __builtin_fmaf(q[2 * p + 1], df, nzd) * inv[2 * p + 1];
        out[p] = pack_bf16x2(w0, w1);
    }
    return out;
}

constexpr int kWBM = 128, kWBN = 256, kWBK = 64;
constexpr int kWRowB = kWBK * 2;                 // 128-byte LDS rows (8 chunks of 16 B)

// s_waitcnt vmcnt(n) (expcnt / lgkmcnt left unconstrained), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

typedef __attribute__((address_space(3))) void lds_void;

// Buffer -> LDS DMA of LS bytes per lane (64 lanes land contiguously at
// `lds`).  The size operand must be a literal for the host compilation pass,
// hence the explicit dispatch.
template <int LS>
__device__ __forceinline__ void dma_to_lds(rsrc_t r, void* lds, int voff, int soff) {
    static_assert(LS == 2 || LS == 4 || LS == 12 || LS == 16, "DMA lane size");
    if constexpr (LS == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
    else if constexpr (LS == 12) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 12, voff, soff, 0, 0);
    else if constexpr (LS == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, soff, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 2, voff, soff, 0, 0);
}

// Workgroup barrier for LDS hand-off only.  __syncthreads() carries a release
// fence, which would also wait for every LDS DMA still in flight (including
// the prefetch of two steps ahead); here the caller waits for exactly the
// DMA it needs (wait_vmcnt) and this waits for this wave's own LDS stores.
// The empty asm statements keep the compiler from moving memory operations
// across the barrier.
__device__ __forceinline__ void sync_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0); vmcnt, expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS tiles use 128-byte rows of eight 16-byte chunks; chunk j of row r is
// stored at position j ^ (r & 7), so that 8 consecutive rows read at the same
// chunk hit 8 different bank groups (conflict-free 16-byte reads/writes).
__device__ __forceinline__ int swz(int row, int chunk) { return row * kWRowB + ((chunk ^ (row & 7)) << 4); }

// Per-step side data of the wide kernel (codes, steps, zeros, s), staged in
// LDS by bulk DMA.  Sizes per 128-row x 64-column step:
template <int BITS, int GROUP>
struct SideLayout {
    static constexpr int CB = 8 * BITS;                                   // code bytes per row
    static constexpr int CLS = (CB % 16 == 0) ? 16 : 4;                   // DMA lane size (bytes)
    static constexpr int CL = CB / CLS;                                   // code lanes per row
    static constexpr int C = kWBM * CL / kWave;                           // code DMA ops
    static constexpr int DB = 2 * (GROUP <= 64 ? 64 / GROUP : 1);         // step/zero bytes per row
    // DMA lanes are at least 4 bytes (narrower lanes still land 4 bytes
    // apart), so with 2 bytes per row (groups of 64, 128) each row fetches
    // the aligned dword that contains its value.
    static constexpr bool DWORD_PAD = DB < 4;
    static constexpr int DBL = DWORD_PAD ? 4 : DB;                         // LDS bytes per row
    static constexpr int DLS = 4;
    static constexpr int DL = DBL / DLS;
    static constexpr int D = kWBM * DL / kWave;                           // DMA ops for steps (and zeros)
    static constexpr int NS = C + 2 * D + 1;                              // + one for s
    static constexpr int OFF_C = 0;
    static constexpr int OFF_D = OFF_C + kWBM * CB;
    static constexpr int OFF_Z = OFF_D + kWBM * DBL;
    static constexpr int OFF_S = OFF_Z + kWBM * DBL;
    static constexpr int BYTES = (OFF_S + kWBK * 4 + 255) / 256 * 256;
    static_assert(kWBM * CL % kWave == 0 && kWBM * DL % kWave == 0, "whole DMA ops");
};

// vmcnt(n) for a wave-uniform runtime n (0..15).
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
    switch (n) {
        case 0: wait_vmcnt<0>(); break;   case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;   case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;   case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;   case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;   case 9: wait_vmcnt<9>(); break;
        case 10: wait_vmcnt<10>(); break; case 11: wait_vmcnt<11>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

constexpr int kWThreads = 512;                   // 8 waves: two per SIMD
constexpr int kWMath = 4;                        // waves 0..3: MFMA; 4..7: producers

// Requires K % 64 == 0 and 256 rows of X addressable with 32-bit offsets.
//
// 128 rows x 256 tokens per workgroup, 8 waves with split roles so that on
// every SIMD the matrix unit and the vector ALU work at the same time:
//   math waves 0..3 (one per SIMD): 2 x 2 tiles of 64 rows x 128 tokens,
//     4 x 8 MFMA 16x16x32 per 32-deep slice; they only read LDS;
//   producer waves 4..7: issue every DMA and dequantize the weights.
// All global data arrives by buffer->LDS DMA (few memory instructions):
//   X     : 3-slot ring, step kt+2 issued during step kt;
//   side  : codes, steps, zeros and s of a step, 3-slot ring, step kt+3
//           issued during step kt (it is consumed one step early);
//   W~    : step kt+1 dequantized while step kt's MFMAs run, written to the
//           other slot of a 2-slot ring.
// One barrier per 64-deep K step; each producer wave waits only for its own
// DMA of the data the next step needs.
template <int BITS, int GROUP, bool YF32>
__global__ __launch_bounds__(kWThreads, 1) void k_qgemm_wide(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, int64_t ldx, const float* __restrict__ s,
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ zero, int64_t M, void* __restrict__ Y, int64_t ldy, int yvec) {
    using SL = SideLayout<BITS, GROUP>;
    constexpr bool STRADDLE = (8 * BITS) % 32 != 0 && BITS != 2;
    constexpr int NPROD = kWThreads / kWave - kWMath;                 // producer waves (4)
    constexpr int XDMA = kWBN * kWRowB / 1024 / NPROD;                // 1 KB X DMA ops per producer (8)
    constexpr int PTHREADS = NPROD * kWave;                            // 256
    constexpr int UNITS = kWBM * kWBK / 8 / PTHREADS;                  // 8-code units per producer thread (4)
    constexpr int RSTRIDE = PTHREADS / 8;                              // 32
    __shared__ __attribute__((aligned(1024))) uint8_t sX0[kWBN * kWRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sX1[kWBN * kWRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sX2[kWBN * kWRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sW0[kWBM * kWRowB];
    __shared__ __attribute__((aligned(1024))) uint8_t sW1[kWBM * kWRowB];
    __shared__ __attribute__((aligned(256))) uint8_t sS0[SL::BYTES];
    __shared__ __attribute__((aligned(256))) uint8_t sS1[SL::BYTES];
    __shared__ __attribute__((aligned(256))) uint8_t sS2[SL::BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const bool math = wave < kWMath;
    const int wm = wave >> 1, wn = wave & 1;      // math tile (valid for math waves)
    const int pw = wave - kWMath;                 // producer index (valid for producers)
    const int ptid = tid - kWMath * kWave;
    const int64_t o0 = (int64_t)blockIdx.x * kWBM;
    const int64_t t0 = (int64_t)blockIdx.y * kWBN;
    const int rows_x = (int)min((int64_t)kWBN, T - t0);
    const int rows_w = (int)min((int64_t)kWBM, M - o0);
    const int wprb = (int)(K * BITS / 32) * 4;    // code bytes per row
    const int gprb = (int)(K / GROUP) * 2;        // step/zero bytes per row

    // Buffer descriptors: out-of-range rows read as zero.
    const rsrc_t rx = make_rsrc(X + t0 * ldx, ((int64_t)(rows_x - 1) * ldx + K) * 2);
    const rsrc_t rc = make_rsrc((const uint8_t*)codes + o0 * wprb, (int64_t)rows_w * wprb);
    // Step/zero extents rounded up to whole dwords: with 2-byte rows the last
    // dword of a tile may end in the next tile's first row (the dispatch keeps
    // M * K / group even for that case, so the array itself ends on a dword).
    const int64_t szb = ((int64_t)rows_w * gprb + 3) & ~(int64_t)3;
    const rsrc_t rsz = make_rsrc((const uint8_t*)scale + o0 * gprb, szb);
    const rsrc_t rzz = make_rsrc((const uint8_t*)zero + o0 * gprb, szb);
    const rsrc_t rs = make_rsrc(s, K * 4);

    // X DMA (producer pw, op i): fills LDS rows 8(XDMA pw + i) .. +7; lane l
    // lands in row 8(XDMA pw + i) + l/8 at chunk position l%8, which holds
    // chunk (l%8)^(row&7).
    const int xrow_l = lane >> 3;
    const int xchunk = (lane & 7) ^ xrow_l;
    const int xoff0 = ((pw * 8 * XDMA + xrow_l) * (int)ldx + 8 * xchunk) * 2;
    const int xrow8 = 8 * (int)ldx * 2;           // byte distance of 8 token rows

    // Side DMA: ops q = pw, pw + NPROD, ... of SL::NS.
    const int my_side = (!math && pw < SL::NS) ? (SL::NS - pw + NPROD - 1) / NPROD : 0;

    // Dequant role: unit cu = ptid % 8 (8 columns) of rows rsub + 32 i.
    const int cu = ptid & 7;
    const int rsub = ptid >> 3;
    const int ubit = 8 * cu * BITS;               // bit offset of the unit in its row's step segment
    const int ushift = ubit & 31;
    const int gi = GROUP <= 64 ? (8 * cu) / GROUP : 0;
    const int wdst = swz(rsub, cu);               // + RSTRIDE i rows (same swizzle: 32 i % 8 == 0)

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue_x = [&](uint8_t* dst, int64_t k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XDMA; ++i)
            dma_to_lds<16>(rx, dst + (pw * XDMA + i) * 1024, xoff0 + i * xrow8, (int)k0 * 2);
    };
    auto issue_side = [&](uint8_t* dst, int64_t k0) __attribute__((always_inline)) {
        const int kc = (int)(k0 * BITS / 8);      // byte offset of the step in a code row
        const int kg = (int)(k0 / GROUP) * 2;
        for (int q = pw; q < SL::NS; q += NPROD) {
            if (q < SL::C) {
                const int li = q * kWave + lane, r = li / SL::CL, sg = li % SL::CL;
                dma_to_lds<SL::CLS>(rc, dst + SL::OFF_C + q * kWave * SL::CLS, r * wprb + sg * SL::CLS, kc);
            } else if (q < SL::C + 2 * SL::D) {
                const bool isz = q >= SL::C + SL::D;
                const int p = q - SL::C - (isz ? SL::D : 0);
                const int li = p * kWave + lane, r = li / SL::DL, sg = li % SL::DL;
                int voff, soff;
                if constexpr (SL::DWORD_PAD) {
                    voff = (r * gprb + kg) & ~3;
                    soff = 0;
                } else {
                    voff = r * gprb + sg * SL::DLS;
                    soff = kg;
                }
                if (isz) dma_to_lds<SL::DLS>(rzz, dst + SL::OFF_Z + p * kWave * SL::DLS, voff, soff);
                else dma_to_lds<SL::DLS>(rsz, dst + SL::OFF_D + p * kWave * SL::DLS, voff, soff);
            } else {
                dma_to_lds<4>(rs, dst + SL::OFF_S, lane * 4, (int)k0 * 4);
            }
        }
    };
    auto dequant_store = [&](const uint8_t* side, uint8_t* dst, int64_t k0) __attribute__((always_inline)) {
        const int kg_cur = (int)(k0 / GROUP) * 2;
        (void)kg_cur;
        const f32x4 sa = *(const f32x4*)(side + SL::OFF_S + 32 * cu);
        const f32x4 sb = *(const f32x4*)(side + SL::OFF_S + 32 * cu + 16);
        float inv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            inv[q] = __builtin_amdgcn_rcpf(sa[q]);
            inv[4 + q] = __builtin_amdgcn_rcpf(sb[q]);
        }
#pragma unroll
        for (int i = 0; i < UNITS; ++i) {
            const int r = rsub + RSTRIDE * i;
            const uint32_t* cw = (const uint32_t*)(side + SL::OFF_C + r * SL::CB) + (ubit >> 5);
            uint64_t f;
            if constexpr (STRADDLE) f = (((uint64_t)cw[1] << 32) | cw[0]) >> ushift;
            else f = (uint64_t)(cw[0] >> ushift);
            uint16_t dh, zh;
            if constexpr (SL::DWORD_PAD) {
                const int half = ((r * gprb + kg_cur) >> 1) & 1;
                dh = (uint16_t)(*(const uint32_t*)(side + SL::OFF_D + r * 4) >> (16 * half));
                zh = (uint16_t)(*(const uint32_t*)(side + SL::OFF_Z + r * 4) >> (16 * half));
            } else {
                dh = *(const uint16_t*)(side + SL::OFF_D + r * SL::DB + 2 * gi);
                zh = *(const uint16_t*)(side + SL::OFF_Z + r * SL::DB + 2 * gi);
            }
            const u32x4 wv = dequant8<BITS>(f, f16_to_f32(zh), f16_to_f32(dh), inv);
            *(u32x4*)(dst + wdst + i * RSTRIDE * kWRowB) = wv;
        }
    };
    auto compute = [&](const uint8_t* xs, const uint8_t* ws) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c = 4 * kk + (lane >> 4);
            u32x4 a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = *(const u32x4*)(ws + swz(wm * 64 + 16 * i + (lane & 15), c));
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) {
                u32x4 b[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    b[j] = *(const u32x4*)(xs + swz(wn * 128 + 64 * jh + 16 * j + (lane & 15), c));
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][4 * jh + j] = mfma_16x16x32(a[i], b[j], acc[i][4 * jh + j]);
            }
        }
    };

    // Step kt with static slots: xc/xn = X slots of kt / kt+2, wc/wn_ = W~
    // slots of kt / kt+1, s1 = side slot of kt+1 (dequantized now), s3 = side
    // slot for kt+3 (issued now); side/xnext/next: steps kt+3 / kt+2 / kt+1 exist.
    auto step = [&](bool side, bool xnext, bool next, uint8_t* xc, uint8_t* xn, uint8_t* wc, uint8_t* wn_,
                    const uint8_t* s1, uint8_t* s3, int64_t kt) __attribute__((always_inline)) {
        if (math) {
            compute(xc, wc);
        } else {
            if (side) issue_side(s3, (kt + 3) * kWBK);
            if (xnext) issue_x(xn, (kt + 2) * kWBK);
            if (next) dequant_store(s1, wn_, (kt + 1) * kWBK);
            // The DMA issued during this step may stay in flight; all older
            // DMA (step kt+1's X, step kt+2's side data) must have landed.
            wait_vmcnt_rt((side ? my_side : 0) + (xnext ? XDMA : 0));
        }
        sync_lds();
    };

    const int64_t nk = K / kWBK;
    // Prologue (producers): side 0, X 0, side 1, X 1, side 2; dequantize step 0.
    if (!math) {
        issue_side(sS0, 0);
        issue_x(sX0, 0);
        int pending = 0;                          // DMA ops allowed to remain in flight
        if (nk > 1) {
            issue_side(sS1, kWBK);
            issue_x(sX1, kWBK);
            pending = XDMA;
        }
        if (nk > 2) {
            issue_side(sS2, 2 * kWBK);
            pending += my_side;
        }
        wait_vmcnt_rt(nk > 1 ? pending : 0);      // side 0, X 0 and side 1 have landed
    }
    sync_lds();
    if (!math) dequant_store(sS0, sW0, 0);
    sync_lds();

    // Slot sequence (period 6): X slot kt%3, W~ slot kt%2, side slot kt%3.
    int64_t kt = 0;
    for (; kt + 9 <= nk; kt += 6) {
        step(true, true, true, sX0, sX2, sW0, sW1, sS1, sS0, kt + 0);
        step(true, true, true, sX1, sX0, sW1, sW0, sS2, sS1, kt + 1);
        step(true, true, true, sX2, sX1, sW0, sW1, sS0, sS2, kt + 2);
        step(true, true, true, sX0, sX2, sW1, sW0, sS1, sS0, kt + 3);
        step(true, true, true, sX1, sX0, sW0, sW1, sS2, sS1, kt + 4);
        step(true, true, true, sX2, sX1, sW1, sW0, sS0, sS2, kt + 5);
    }
    for (; kt < nk; kt += 6) {
#define TTQ_TAIL(J, XC, XN, WC, WN, S1, S3)                                                             \
        if (kt + J < nk)                                                                                \
            step(kt + J + 3 < nk, kt + J + 2 < nk, kt + J + 1 < nk, XC, XN, WC, WN, S1, S3, kt + J)
        TTQ_TAIL(0, sX0, sX2, sW0, sW1, sS1, sS0);
        TTQ_TAIL(1, sX1, sX0, sW1, sW0, sS2, sS1);
        TTQ_TAIL(2, sX2, sX1, sW0, sW1, sS0, sS2);
        TTQ_TAIL(3, sX0, sX2, sW1, sW0, sS1, sS0);
        TTQ_TAIL(4, sX1, sX0, sW0, sW1, sS2, sS1);
        TTQ_TAIL(5, sX2, sX1, sW1, sW0, sS0, sS2);
#undef TTQ_TAIL
    }

    if (!math) return;
    // Epilogue: lane holds Y^T[o + r][t] for r = 0..3 (4 consecutive o of token t).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t o = o0 + wm * 64 + 16 * i + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t t = t0 + wn * 128 + 16 * j + (lane & 15);
            if (t >= T) continue;
            if constexpr (YF32) {
                float* yp = (float*)Y + t * ldy + o;
                if (yvec && o + 4 <= M) {
                    *(f32x4*)yp = acc[i][j];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (o + r < M) yp[r] = acc[i][j][r];
                }
            } else {
                uint16_t* yp = (uint16_t*)Y + t * ldy + o;
                if (yvec && o + 4 <= M) {
                    u32x2 v = {pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
                    *(u32x2*)yp = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (o + r < M) yp[r] = (uint16_t)f32_to_bf16(acc[i][j][r]);
                }
            }
        }
    }
}

template <int BITS, int GROUP>
static hipError_t launch_g3(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                            const float* s, const uint32_t* codes, const uint16_t* scale,
                            const uint16_t* zero, int64_t M, void* Y, bool yf32, int64_t ldy,
                            hipStream_t st) {
    // 4 consecutive outputs are stored as one vector when Y's rows allow it.
    const int yvec = ((uintptr_t)Y % 16 == 0) && ((ldy * (yf32 ? 4 : 2)) % 16 == 0);
    // 32-bit buffer offsets must reach 256 rows of X and 128 rows of codes.
    const bool wide_ok = K % kWBK == 0 && (int64_t)kWBN * ldx * 2 < ((int64_t)1 << 31) &&
                         (GROUP < 64 || (M * (K / GROUP)) % 2 == 0);
    if (!xf32 && T >= 192 && wide_ok) {
        dim3 gw((unsigned)((M + kWBM - 1) / kWBM), (unsigned)((T + kWBN - 1) / kWBN));
        if (yf32)
            k_qgemm_wide<BITS, GROUP, true><<<gw, kWThreads, 0, st>>>((const uint16_t*)X, T, K, ldx, s, codes,
                                                                     scale, zero, M, Y, ldy, yvec);
        else
            k_qgemm_wide<BITS, GROUP, false><<<gw, kWThreads, 0, st>>>((const uint16_t*)X, T, K, ldx, s, codes,
                                                                      scale, zero, M, Y, ldy, yvec);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((M + kGBM - 1) / kGBM), (unsigned)((T + kGBN - 1) / kGBN));
#define TTQ_G_LAUNCH(XF, YF)                                                                   \
    k_qgemm<BITS, GROUP, XF, YF><<<grid, kGThreads, 0, st>>>(X, T, K, ldx, s, codes, scale, \
                                                             zero, M, Y, ldy, yvec)
    if (xf32) {
        if (yf32) TTQ_G_LAUNCH(true, true); else TTQ_G_LAUNCH(true, false);
    } else {
        if (yf32) TTQ_G_LAUNCH(false, true); else TTQ_G_LAUNCH(false, false);
    }
#undef TTQ_G_LAUNCH
    return hipGetLastError();
}

template <int BITS>
static hipError_t launch_g2(int group, const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                            const float* s, const uint32_t* codes, const uint16_t* scale,
                            const uint16_t* zero, int64_t M, void* Y, bool yf32, int64_t ldy,
                            hipStream_t st) {
    switch (group) {
        case 16: return launch_g3<BITS, 16>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st);
        case 32: return launch_g3<BITS, 32>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st);
        case 64: return launch_g3<BITS, 64>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st);
        case 128: return launch_g3<BITS, 128>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_qgemm(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                        const float* s, const uint32_t* codes, const uint16_t* scale,
                        const uint16_t* zero, int64_t M, int bits, int group, void* Y, bool yf32,
                        int64_t ldy, hipStream_t st) {
    switch (bits) {
        case 2: return launch_g2<2>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st);
        case 3: return launch_g2<3>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st);
        case 4: return launch_g2<4>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st);
        case 5: return launch_g2<5>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace ttq
