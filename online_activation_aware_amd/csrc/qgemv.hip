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

constexpr int kTChan = 32;                        // channels per lane field

template <int N>
__device__ __forceinline__ float cvt_ubyte(uint32_t v) {
    float f;
    if constexpr (N == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(v));
    else if constexpr (N == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(v));
    else if constexpr (N == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(v));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(v));
    return f;
}

// The 32 codes of a lane's field as fp32 values, code i at bits BITS*i of the
// little-endian bit stream.
template <int BITS>
__device__ __forceinline__ void field_codes(const CodeWords<BITS>& c, float (&q)[kTChan]) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = c.w[i] & 0x0F0F0F0Fu, hi = (c.w[i] >> 4) & 0x0F0F0F0Fu;
            q[8 * i + 0] = cvt_ubyte<0>(lo);
            q[8 * i + 1] = cvt_ubyte<0>(hi);
            q[8 * i + 2] = cvt_ubyte<1>(lo);
            q[8 * i + 3] = cvt_ubyte<1>(hi);
            q[8 * i + 4] = cvt_ubyte<2>(lo);
            q[8 * i + 5] = cvt_ubyte<2>(hi);
            q[8 * i + 6] = cvt_ubyte<3>(lo);
            q[8 * i + 7] = cvt_ubyte<3>(hi);
        }
    } else if constexpr (BITS == 2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t m = (c.w[i] >> (2 * j)) & 0x03030303u;   // codes 4 b + j of this word
                q[16 * i + j] = cvt_ubyte<0>(m);
                q[16 * i + 4 + j] = cvt_ubyte<1>(m);
                q[16 * i + 8 + j] = cvt_ubyte<2>(m);
                q[16 * i + 12 + j] = cvt_ubyte<3>(m);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kTChan; ++i) q[i] = (float)code_at<BITS>(c, i);
    }
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
    {
        // Token block blockIdx.y: tokens 16 NT y .. 16 NT y + 16 NT - 1.
        const int64_t tb = (int64_t)blockIdx.y * NT * 16;
        X = XF32 ? (const void*)((const float*)X + tb * ldx) : (const void*)((const uint16_t*)X + tb * ldx);
        Y = YF32 ? (void*)((float*)Y + tb * ldy) : (void*)((uint16_t*)Y + tb * ldy);
        T = T - tb < (int64_t)NT * 16 ? T - tb : (int64_t)NT * 16;
    }

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
            // (q - z) * step = fma(q, step, -z * step) exactly (small integers
            // times an fp16 step), then times 1/s.  Rows >= M read row o0 and
            // their outputs are never stored.
            // The first token tile's operands (bf16 X) are requested before the
            // weights are expanded, so that the expansion covers their latency.
            u32x4 xb0[4];
            if constexpr (!XF32) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xb0[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rx, (int)((r * ldx + k0 + 8 * j) * esz), 0, 0));
            }
            u32x4 ah[4], al[4];
            float qall[kTChan];
            field_codes<BITS>(cw[p], qall);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int gsel = GROUP < 32 ? (8 * j) / GROUP : 0;
                const float df = f16_to_f32(dh[p][gsel]);
                const float nzd = -f16_to_f32(zh[p][gsel]) * df;
                const f32x4 i0 = *(const f32x4*)(sinv + k0 + 8 * j);
                const f32x4 i1 = *(const f32x4*)(sinv + k0 + 8 * j + 4);
                const float inv[8] = {i0[0], i0[1], i0[2], i0[3], i1[0], i1[1], i1[2], i1[3]};
                float w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = __builtin_fmaf(qall[8 * j + e], df, nzd) * inv[e];
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
                        const u32x4 xb = n == 0 ? xb0[j]
                                                : __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                                rx, voff, 0, 0));
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

// ---------------------------------------------------------------------------
// One to four tokens: the vector ALUs, with the group affine map applied to
// sums instead of to weights.
//
// For a group h of row o, sum_k (q_k - z_h) * step_h * xs_k
//   = step_h * (sum_k q_k * xs_k - z_h * sum_k xs_k),     xs = x / s,
// and sum_k xs_k does not depend on o.  A lane therefore converts each code
// to fp32 once (v_cvt_f32_ubyteN on masked nibbles for b = 4) and does one
// FMA per code and token; the step and zero cost two FMAs per group.  xs is
// formed once per wave in fp32 (x * v_rcp(s)), so the only rounding is fp32
// accumulation: no bf16 rounding of weights or tokens on this path.
//
// Mapping: a piece is 64 lanes x 32 consecutive channels (2048 channels;
// b x 256 bytes of codes per row).  A workgroup owns RW rows; its NS waves
// take the pieces w, w + NS, ...; per piece a wave issues the codes of all
// RW rows (one contiguous 16-byte load per lane and row at b = 4) before it
// computes, so each load instruction reads a contiguous b x 256-byte run of
// one row.  Per-lane sums are added over the wave by a fixed butterfly and
// over the waves in wave order (deterministic).
constexpr int kTPiece = kTChan * kWave;           // channels per piece
constexpr int kTMaxWaves = 8;
// 16 rows per workgroup: the grid's waves fit the chip in one round.  Rows
// in flight per wave: 3 for one token, 2 for two, 1 for four (registers).
constexpr int trows(int tt) { return 16; }
constexpr int tdepth(int tt) { return tt == 1 ? 3 : tt == 2 ? 2 : 1; }

template <int BITS, int SG>
struct RowField {
    CodeWords<BITS> cw;
    uint16_t dh[SG], zh[SG];
};

// Prompt p = blockIdx.y of a batched call reads X + p * x, s + p * s, ...
// (element strides; all zero for one prompt).
template <int BITS, int GROUP, bool XF32, bool YF32, int TT>
__global__ __launch_bounds__(kTMaxWaves * kWave) void k_qgemv_t(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, const float* __restrict__ s,
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ zero, int64_t M, void* __restrict__ Y, int64_t ldy, QgemvBatch bt) {
    constexpr int RW = trows(TT);
    constexpr int D = tdepth(TT);
    constexpr int SG = GROUP < kTChan ? kTChan / GROUP : 1;   // groups per lane field
    constexpr int SGC = kTChan / SG;                          // channels per group part
    constexpr int NV = RW * TT;
    __shared__ float red[kTMaxWaves][NV];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int NS = blockDim.x / kWave;
    const int64_t o0 = (int64_t)blockIdx.x * RW;
    const int64_t wpr = K * BITS / 32, gpr = K / GROUP;
    const int64_t npieces = (K + kTPiece - 1) / kTPiece;
    {
        const int64_t pb = blockIdx.y;
        X = XF32 ? (const void*)((const float*)X + pb * bt.x) : (const void*)((const uint16_t*)X + pb * bt.x);
        s += pb * bt.s;
        codes += pb * bt.codes;
        scale += pb * bt.sz;
        zero += pb * bt.sz;
        Y = YF32 ? (void*)((float*)Y + pb * bt.y) : (void*)((uint16_t*)Y + pb * bt.y);
    }

    float acc[RW][TT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[r][t] = 0.f;

    for (int64_t p = wave; p < npieces; p += NS) {
        const int64_t k0 = p * kTPiece + (int64_t)lane * kTChan;
        if (k0 < K) {                             // K % 32 == 0: a field is all in or all out
            auto load_row = [&](RowField<BITS, SG>& f, int r) __attribute__((always_inline)) {
                const int64_t o = o0 + r < M ? o0 + r : M - 1;
                load_codes<BITS>(f.cw, codes + o * wpr + k0 * BITS / 32);
#pragma unroll
                for (int h = 0; h < SG; ++h) {
                    f.dh[h] = scale[o * gpr + k0 / GROUP + h];
                    f.zh[h] = zero[o * gpr + k0 / GROUP + h];
                }
            };
            // Requests in the order they are waited for (the vector memory
            // counter drains in order): scales and tokens of this field, then
            // the first D rows.  fp32 tokens with four token slots are fetched
            // after the rows, one token at a time, to bound registers.
            constexpr bool kEarlyX = !(XF32 && TT == 4);
            constexpr int XW = XF32 ? kTChan : kTChan / 2;     // 32-bit words per token field
            float sv[kTChan];
#pragma unroll
            for (int v = 0; v < kTChan / 4; ++v) {
                const f32x4 a = *(const f32x4*)(s + k0 + 4 * v);
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[4 * v + e] = a[e];
            }
            auto load_x = [&](uint32_t (&xr)[XW], int t) __attribute__((always_inline)) {
                const u32x4* xp = XF32 ? (const u32x4*)((const float*)X + t * ldx + k0)
                                       : (const u32x4*)((const uint16_t*)X + t * ldx + k0);
#pragma unroll
                for (int v = 0; v < XW / 4; ++v) {
                    const u32x4 a = t < T ? xp[v] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 4; ++e) xr[4 * v + e] = a[e];
                }
            };
            uint32_t xr[kEarlyX ? TT : 1][XW];
            if constexpr (kEarlyX) {
#pragma unroll
                for (int t = 0; t < TT; ++t) load_x(xr[t], t);
            }
            RowField<BITS, SG> ring[D];
#pragma unroll
            for (int r = 0; r < D; ++r) load_row(ring[r], r);
            __builtin_amdgcn_sched_barrier(0);              // all D rows requested before any wait

            // xs = x * (1/s) and its sums over each group part.
#pragma unroll
            for (int i = 0; i < kTChan; ++i) sv[i] = __builtin_amdgcn_rcpf(sv[i]);
            float xs[TT][kTChan], S[TT][SG];
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if constexpr (!kEarlyX) load_x(xr[0], t);
                const uint32_t(&xt)[XW] = xr[kEarlyX ? t : 0];
#pragma unroll
                for (int i = 0; i < kTChan; ++i) {
                    float x;
                    if constexpr (XF32) x = __builtin_bit_cast(float, xt[i]);
                    else x = (i & 1) ? bf16hi_to_f32(xt[i / 2]) : bf16lo_to_f32(xt[i / 2]);
                    xs[t][i] = x * sv[i];
                }
#pragma unroll
                for (int h = 0; h < SG; ++h) {
                    float a = xs[t][h * SGC];
#pragma unroll
                    for (int i = 1; i < SGC; ++i) a += xs[t][h * SGC + i];
                    S[t][h] = a;
                }
            }

            // Rows stream through a ring of D fields: row r + D is requested
            // before row r is computed.
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const RowField<BITS, SG> f = ring[r % D];
                if (r + D < RW) load_row(ring[r % D], r + D);
                float q[kTChan];
                field_codes<BITS>(f.cw, q);
#pragma unroll
                for (int h = 0; h < SG; ++h) {
                    const float df = f16_to_f32(f.dh[h]), zf = f16_to_f32(f.zh[h]);
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        float d = q[h * SGC] * xs[t][h * SGC];
#pragma unroll
                        for (int i = 1; i < SGC; ++i) d = __builtin_fmaf(q[h * SGC + i], xs[t][h * SGC + i], d);
                        acc[r][t] = __builtin_fmaf(df, __builtin_fmaf(-zf, S[t][h], d), acc[r][t]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);          // rows are not interleaved (registers)
            }
        }
    }

    // Sum over the wave: at each butterfly step a lane keeps half of its
    // values and adds its partner's copy of them; afterwards lane l holds the
    // wave total of value idx(l), whose bits are lane bits 5, 4, ... .
    float v[NV];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < TT; ++t) v[r * TT + t] = acc[r][t];
    int n = NV, idx = 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        if (n > 1) {
            const int half = n / 2;
            const bool up = (lane & m) != 0;
#pragma unroll
            for (int i = 0; i < half; ++i) {
                // Selects written on the bit patterns: a per-lane choice between
                // two array elements must not become a dynamic array index.
                const uint32_t a = __builtin_bit_cast(uint32_t, v[i]);
                const uint32_t b = __builtin_bit_cast(uint32_t, v[i + half]);
                const uint32_t um = up ? 0xFFFFFFFFu : 0u;
                const float send = __builtin_bit_cast(float, (a & um) | (b & ~um));
                const float keep = __builtin_bit_cast(float, (b & um) | (a & ~um));
                v[i] = keep + __shfl_xor(send, m);
            }
            idx = 2 * idx + (up ? 1 : 0);
            n = half;
        } else {
            v[0] += __shfl_xor(v[0], m);
        }
    }
    constexpr int kLowBits = 6 - __builtin_ctz(NV);            // lane bits below the index bits
    if ((lane & ((1 << kLowBits) - 1)) == 0) red[wave][idx] = v[0];
    __syncthreads();
    if (threadIdx.x < NV) {
        const int vi = threadIdx.x;
        float a = red[0][vi];
        for (int w = 1; w < NS; ++w) a += red[w][vi];
        const int r = vi / TT, t = vi % TT;
        const int64_t o = o0 + r;
        if (o < M && t < T) {
            if constexpr (YF32) ((float*)Y)[t * ldy + o] = a;
            else ((uint16_t*)Y)[t * ldy + o] = (uint16_t)f32_to_bf16(a);
        }
    }
}

template <int BITS, int GROUP, bool XF32, bool YF32, int TT>
static hipError_t launch_t(const void* X, int64_t T, int64_t K, int64_t ldx, const float* s,
                           const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, void* Y,
                           int64_t ldy, hipStream_t st, StageTimer tm, int64_t P, const QgemvBatch& bt) {
    const int64_t np = (K + kTPiece - 1) / kTPiece;
    const int64_t rounds = (np + kTMaxWaves - 1) / kTMaxWaves;
    const int ns = (int)((np + rounds - 1) / rounds);           // waves, each taking `rounds` pieces
    const dim3 grid((unsigned)((M + trows(TT) - 1) / trows(TT)), (unsigned)P);
    return launch_kernel(k_qgemv_t<BITS, GROUP, XF32, YF32, TT>, grid, dim3(ns * kWave), 0, st, tm.start, tm.stop,
                         X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, bt);
}

// ---------------------------------------------------------------------------
// 12 <= T <= 16 with a workspace: split K.  A workgroup owns 64 output rows
// (four MFMA row tiles) and one of KS slices of K.  Its 16 waves take the
// slice's 128-channel chunks in turn; per chunk a wave requests the codes of
// all four row tiles and the token fragments, then expands the tiles one by
// one (as k_qgemv: the same bf16 w/s per weight) into four accumulators, so
// each token fragment read from L2 serves 64 rows instead of 16.  The wave
// tiles are added in wave order and the workgroup's fp32 partial goes to
// P[ks][T][M]; k_sk_reduce adds the KS partials in slice order.
constexpr int kSkTiles = 4;                       // 16-row MFMA tiles per workgroup
constexpr int kSkWaves = 16;
constexpr int64_t kSkMaxSlice = 8192;             // channels per slice (1/s staged in LDS)

template <int BITS, int GROUP, bool XF32>
__global__ __launch_bounds__(kSkWaves * kWave) void k_qgemv_sk(
    const void* __restrict__ X, int64_t T, int64_t K, int64_t ldx, const float* __restrict__ s,
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ zero, int64_t M, int64_t kslice, float* __restrict__ P) {
    constexpr int G2 = GROUP < 32 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) float sinv[kSkMaxSlice];
    __shared__ f32x4 red[kSkWaves][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15, q = lane >> 4;
    const int64_t o0 = (int64_t)blockIdx.x * 16 * kSkTiles;
    const int64_t ks = blockIdx.y;
    const int64_t kbeg = ks * kslice;
    const int64_t kend = kbeg + kslice < K ? kbeg + kslice : K;

    for (int64_t j = threadIdx.x; j < kend - kbeg; j += kSkWaves * kWave)
        sinv[j] = __builtin_amdgcn_rcpf(s[kbeg + j]);

    const int64_t wpr = K * BITS / 32, gpr = K / GROUP;
    const uint32_t* crow[kSkTiles];
    const uint16_t* srow[kSkTiles];
    const uint16_t* zrow[kSkTiles];
#pragma unroll
    for (int rt = 0; rt < kSkTiles; ++rt) {
        int64_t o = o0 + 16 * rt + r;
        if (o >= M) o = M - 1;                    // rows past M: loads stay in bounds, outputs unused
        crow[rt] = codes + o * wpr;
        srow[rt] = scale + o * gpr;
        zrow[rt] = zero + o * gpr;
    }
    const int64_t esz = XF32 ? 4 : 2;
    const rsrc_t rx = make_rsrc(X, ((T - 1) * ldx + K) * esz);   // tokens >= T read as zero

    f32x4 acc[kSkTiles];
#pragma unroll
    for (int rt = 0; rt < kSkTiles; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    const int64_t nch = (kend - kbeg) / kVChunk;
    for (int64_t c = wave; c < nch; c += kSkWaves) {
        const int64_t kl = c * kVChunk + 32 * q;  // channel within the slice
        const int64_t k0 = kbeg + kl;
        CodeWords<BITS> cw[kSkTiles];
        uint16_t dh[kSkTiles][G2], zh[kSkTiles][G2];
#pragma unroll
        for (int rt = 0; rt < kSkTiles; ++rt) {
            load_codes<BITS>(cw[rt], crow[rt] + k0 * BITS / 32);
#pragma unroll
            for (int h = 0; h < G2; ++h) {
                dh[rt][h] = srow[rt][k0 / GROUP + h];
                zh[rt][h] = zrow[rt][k0 / GROUP + h];
            }
        }
        // Token fragments of this chunk (bf16 hi [+ lo for fp32 X]).
        u32x4 bh[4], bl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int voff = (int)((r * ldx + k0 + 8 * j) * esz);
            if constexpr (XF32) {
                const f32x4 xa = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff, 0, 0));
                const f32x4 xc = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + 16, 0, 0));
                const float xv[8] = {xa[0], xa[1], xa[2], xa[3], xc[0], xc[1], xc[2], xc[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bh[j][e] = pack_bf16x2(xv[2 * e], xv[2 * e + 1]);
                    bl[j][e] = pack_bf16x2(xv[2 * e] - bf16lo_to_f32(bh[j][e]), xv[2 * e + 1] - bf16hi_to_f32(bh[j][e]));
                }
            } else {
                bh[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff, 0, 0));
            }
        }
#pragma unroll
        for (int rt = 0; rt < kSkTiles; ++rt) {
            float qall[kTChan];
            field_codes<BITS>(cw[rt], qall);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int gsel = GROUP < 32 ? (8 * j) / GROUP : 0;
                const float df = f16_to_f32(dh[rt][gsel]);
                const float nzd = -f16_to_f32(zh[rt][gsel]) * df;
                const f32x4 i0 = *(const f32x4*)(sinv + kl + 8 * j);
                const f32x4 i1 = *(const f32x4*)(sinv + kl + 8 * j + 4);
                const float inv[8] = {i0[0], i0[1], i0[2], i0[3], i1[0], i1[1], i1[2], i1[3]};
                u32x4 ah, al;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float w0 = __builtin_fmaf(qall[8 * j + 2 * e], df, nzd) * inv[2 * e];
                    const float w1 = __builtin_fmaf(qall[8 * j + 2 * e + 1], df, nzd) * inv[2 * e + 1];
                    ah[e] = pack_bf16x2(w0, w1);
                    if constexpr (XF32) al[e] = pack_bf16x2(w0 - bf16lo_to_f32(ah[e]), w1 - bf16hi_to_f32(ah[e]));
                }
                acc[rt] = mfma_16x16x32(ah, bh[j], acc[rt]);
                if constexpr (XF32) {
                    acc[rt] = mfma_16x16x32(ah, bl[j], acc[rt]);
                    acc[rt] = mfma_16x16x32(al, bh[j], acc[rt]);
                }
            }
        }
    }

    // Lane holds Y^T[o0 + 16 rt + 4 q + i][r] for tile rt; the 16 wave tiles
    // are added in wave order by one wave per row tile.
    float* Pk = P + ks * T * M;
#pragma unroll
    for (int rt = 0; rt < kSkTiles; ++rt) {
        if (rt > 0) __syncthreads();
        red[wave][lane] = acc[rt];
        __syncthreads();
        if (wave == rt) {
            f32x4 sum = red[0][lane];
            for (int w = 1; w < kSkWaves; ++w) {
                const f32x4 v = red[w][lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) sum[i] += v[i];
            }
            const int64_t ob = o0 + 16 * rt + 4 * q;
            if (r < T)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (ob + i < M) Pk[(int64_t)r * M + ob + i] = sum[i];
        }
    }
}

// Y[t][o] = sum over slices ks = 0.. of P[ks][t][o], in slice order.
template <bool YF32>
__global__ __launch_bounds__(256) void k_sk_reduce(const float* __restrict__ P, int ksn, int64_t T, int64_t M,
                                                   void* __restrict__ Y, int64_t ldy) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * M) return;
    const int64_t t = idx / M, o = idx % M;
    float a = P[idx];
    for (int k = 1; k < ksn; ++k) a += P[(int64_t)k * T * M + idx];
    if constexpr (YF32) ((float*)Y)[t * ldy + o] = a;
    else ((uint16_t*)Y)[t * ldy + o] = (uint16_t)f32_to_bf16(a);
}

// Slices for the split-K path: enough workgroups to fill the chip, each
// slice a whole number of chunks and at most kSkMaxSlice channels.
int64_t qgemv_sk_slices(int64_t K, int64_t M) {
    const int64_t gx = (M + 16 * kSkTiles - 1) / (16 * kSkTiles);
    const int64_t nch = K / kVChunk;
    int64_t ks = (256 + gx - 1) / gx;
    if (ks > nch) ks = nch;
    while ((nch + ks - 1) / ks * kVChunk > kSkMaxSlice) ++ks;
    return ks < 1 ? 1 : ks;
}

// bf16 X only (with fp32 X the three-product expansion does not fit the
// registers of 16 waves), and T >= 12: below that the second launch costs
// about what the shared token fragments save (measured: T = 5 and 8 equal or
// slower, T = 16 29.1 -> 26.0 us on the 14336 -> 4096 layer).
bool qgemv_sk_eligible(int64_t T, int64_t K, int64_t ldx, bool xf32) {
    return !xf32 && T >= kSkMinT && T <= 16 && K % kVChunk == 0 && (int64_t)16 * ldx * 2 < ((int64_t)1 << 31);
}

size_t qgemv_sk_ws_bytes(int64_t T, int64_t K, int64_t M) {
    return (size_t)qgemv_sk_slices(K, M) * (size_t)T * (size_t)M * sizeof(float);
}

template <int BITS, int GROUP, bool XF32>
static hipError_t launch_sk3(const void* X, int64_t T, int64_t K, int64_t ldx, const float* s, const uint32_t* codes,
                             const uint16_t* scale, const uint16_t* zero, int64_t M, void* Y, bool yf32, int64_t ldy,
                             float* P, hipStream_t st, StageTimer tm) {
    const int64_t ksn = qgemv_sk_slices(K, M);
    const int64_t nch = K / kVChunk;
    const int64_t kslice = (nch + ksn - 1) / ksn * kVChunk;
    const int64_t ksr = (K + kslice - 1) / kslice;             // slices actually used
    const dim3 grid((unsigned)((M + 16 * kSkTiles - 1) / (16 * kSkTiles)), (unsigned)ksr);
    if (hipError_t e = launch_kernel(k_qgemv_sk<BITS, GROUP, XF32>, grid, dim3(kSkWaves * kWave), 0, st, tm.start,
                                     nullptr, X, T, K, ldx, s, codes, scale, zero, M, kslice, P))
        return e;
    const dim3 g2((unsigned)((T * M + 255) / 256));
    return yf32 ? launch_kernel(k_sk_reduce<true>, g2, dim3(256), 0, st, nullptr, tm.stop, (const float*)P, (int)ksr,
                                T, M, Y, ldy)
                : launch_kernel(k_sk_reduce<false>, g2, dim3(256), 0, st, nullptr, tm.stop, (const float*)P,
                                (int)ksr, T, M, Y, ldy);
}

template <int BITS>
static hipError_t launch_sk2(int group, bool xf32, const void* X, int64_t T, int64_t K, int64_t ldx, const float* s,
                             const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, void* Y,
                             bool yf32, int64_t ldy, float* P, hipStream_t st, StageTimer tm) {
#define TTQ_SK(G) return launch_sk3<BITS, G, false>(X, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, P, st, tm)
    switch (group) {
        case 16: TTQ_SK(16);
        case 32: TTQ_SK(32);
        case 64: TTQ_SK(64);
        case 128: TTQ_SK(128);
    }
#undef TTQ_SK
    return hipErrorInvalidValue;
}

hipError_t launch_qgemv_sk(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                           const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, int bits,
                           int group, void* Y, bool yf32, int64_t ldy, float* P, hipStream_t st, StageTimer tm) {
    if (!qgemv_sk_eligible(T, K, ldx, xf32)) return hipErrorInvalidValue;
    switch (bits) {
        case 2: return launch_sk2<2>(group, xf32, X, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, P, st, tm);
        case 3: return launch_sk2<3>(group, xf32, X, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, P, st, tm);
        case 4: return launch_sk2<4>(group, xf32, X, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, P, st, tm);
        case 5: return launch_sk2<5>(group, xf32, X, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, P, st, tm);
    }
    return hipErrorInvalidValue;
}

// T <= 4 runs k_qgemv_t (64-bit addressing, any K).  Above that, token rows
// up to 127 are addressed (padded tiles read as zero) with 32-bit buffer
// offsets, and 1/s of every channel is staged in LDS.
bool qgemv_supported(int64_t T, int64_t K, int64_t ldx, bool xf32) {
    if (T < 1 || T > kQgemvMaxT || K % kVChunk != 0) return false;
    if (T <= 4) return true;
    return K <= kVMaxK && (int64_t)kQgemvMaxT * ldx * (xf32 ? 4 : 2) < ((int64_t)1 << 31);
}

template <int BITS, int GROUP, bool XF32, bool YF32>
static hipError_t launch_v4(const void* X, int64_t T, int64_t K, int64_t ldx, const float* s,
                            const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M,
                            void* Y, int64_t ldy, hipStream_t st, StageTimer tm, int64_t P, const QgemvBatch& bt) {
    if (T == 1)
        return launch_t<BITS, GROUP, XF32, YF32, 1>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm, P, bt);
    if (T == 2)
        return launch_t<BITS, GROUP, XF32, YF32, 2>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm, P, bt);
    if (T <= 4)
        return launch_t<BITS, GROUP, XF32, YF32, 4>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm, P, bt);
    if (P != 1) return hipErrorInvalidValue;      // batched calls are for T <= 4
    // Token tiles per workgroup: all of them, unless the row blocks alone
    // would leave most compute units idle; then the tiles are split over a
    // second grid dimension (each such workgroup expands its rows' weights).
    const int64_t gx = (M + 15) / 16;
    int nt = T <= 16 ? 1 : T <= 32 ? 2 : T <= 64 ? 4 : 8;
    while (nt > 1 && gx * ((T + 16 * nt - 1) / (16 * nt)) < 256) nt /= 2;
    const dim3 grid((unsigned)gx, (unsigned)((T + 16 * nt - 1) / (16 * nt)));
#define TTQ_V_LAUNCH(NT)                                                                                  \
    return launch_kernel(k_qgemv<BITS, GROUP, XF32, YF32, NT>, grid, dim3(vwaves(NT) * kWave), 0, st,     \
                         tm.start, tm.stop, X, T, K, ldx, s, codes, scale, zero, M, Y, ldy)
    if (nt == 1) TTQ_V_LAUNCH(1);
    if (nt == 2) TTQ_V_LAUNCH(2);
    if (nt == 4) TTQ_V_LAUNCH(4);
    TTQ_V_LAUNCH(8);
#undef TTQ_V_LAUNCH
}

template <int BITS, int GROUP>
static hipError_t launch_v3(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                            const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M,
                            void* Y, bool yf32, int64_t ldy, hipStream_t st, StageTimer tm, int64_t P,
                            const QgemvBatch& bt) {
    if (xf32) {
        if (yf32) return launch_v4<BITS, GROUP, true, true>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm, P, bt);
        return launch_v4<BITS, GROUP, true, false>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm, P, bt);
    }
    if (yf32) return launch_v4<BITS, GROUP, false, true>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm, P, bt);
    return launch_v4<BITS, GROUP, false, false>(X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, st, tm, P, bt);
}

template <int BITS>
static hipError_t launch_v2(int group, const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx,
                            const float* s, const uint32_t* codes, const uint16_t* scale, const uint16_t* zero,
                            int64_t M, void* Y, bool yf32, int64_t ldy, hipStream_t st, StageTimer tm,
                            int64_t P, const QgemvBatch& bt) {
    switch (group) {
        case 16: return launch_v3<BITS, 16>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm, P, bt);
        case 32: return launch_v3<BITS, 32>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm, P, bt);
        case 64: return launch_v3<BITS, 64>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm, P, bt);
        case 128: return launch_v3<BITS, 128>(X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm, P, bt);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_qgemv(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                        const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, int bits,
                        int group, void* Y, bool yf32, int64_t ldy, hipStream_t st, StageTimer tm, int64_t P,
                        QgemvBatch bt) {
    switch (bits) {
        case 2: return launch_v2<2>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm, P, bt);
        case 3: return launch_v2<3>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm, P, bt);
        case 4: return launch_v2<4>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm, P, bt);
        case 5: return launch_v2<5>(group, X, xf32, T, K, ldx, s, codes, scale, zero, M, Y, yf32, ldy, st, tm, P, bt);
    }
    return hipErrorInvalidValue;
}

}  // namespace ttq
