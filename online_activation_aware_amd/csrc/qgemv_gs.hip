// Quantized projection for T <= 16 tokens with the group scale applied to
// sums: Y[t][o] = sum_g step_og (sum_{j in g} (q_oj - z_og) x~_tj),
// x~ = X / s.
//
// [TTQ §method b7] quantized projection kernel; [TTQ §method b1] QDQ with
// group-wise RTN (W_hat = (code - zero) * step); [TTQ §method b2] the input
// divided by s.  The codes are never expanded to weights: a 4-bit code q
// becomes the exact bf16 number 128 + q by one byte permute with the
// exponent byte 0x43, and the matrix cores form, per 32-channel subgroup,
//   P[t][o] = sum_j (128 + q_oj) x~_tj          (bf16 x~, fp32 accumulation)
// with tokens as the 16 rows and weight rows as the 16 columns of a
// 16x16x32 MFMA.  Per group:  step * P - step * (z + 128) * S_t, where
// S_t = sum_j x~_tj over the group; step * (z + 128) is exact in fp32 (an
// 11-bit step times an 8-bit integer), and the S term of a 128-channel
// chunk is one fp32 16x16x4 MFMA (S as the token operand, the per-group
// constants as the row operand) accumulated with the opposite sign.
//
// One launch.  A workgroup owns 64 output rows (four 16-row tiles) and a
// slice of K of up to eight 512-channel sets; wave w takes set w.  Each
// wave first requests its share of the slice's tokens and 1/s, then the
// steps, zeros and codes of its set (16 bytes per lane and row tile and
// chunk: words 4q..4q+3 of row r, one row's 64-byte run per four lanes),
// and while the codes stream in it writes x~ = bf16(x * (1/s)) (each
// 8-channel slot in the order 0 2 4 6 1 3 5 7, the order the code permute
// produces) and the 32-channel sums of x~ into LDS.  A 4x4 exchange across
// the lane quarters (v_permlane32_swap, v_permlane16_swap) turns the code
// words into word 4j + q for MFMA j, so each MFMA covers one 32-channel
// subgroup.  The wave tiles are added in wave order through LDS; with
// several K slices each workgroup stores its fp32 partial and k_gs_reduce
// adds the slices in slice order (a second launch: ordering the slices
// inside one launch would need a counter in known state or a device-scope
// fence per workgroup, which writes back and invalidates the L2 of its
// XCD).  Both orders are fixed, so results do not depend on timing.
#include "common.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace ttq {

constexpr int kGsMaxWaves = 8;
constexpr int kGsMaxT = 16;
constexpr int64_t kGsRows = 64;                   // output rows per workgroup (four MFMA row tiles)
constexpr int kGsChunk = 128;                     // channels per chunk
constexpr int kGsSet = 4;                         // chunks per wave
constexpr int kGsSetCh = kGsSet * kGsChunk;       // channels per set
constexpr int kGsLds = 140 * 1024;                // tokens and sums of a slice (and the wave tiles)

// LDS of a slice of gps sets for T tokens: x~ rows of gps * 1024 + 16
// bytes (the 16 spread the token rows over the banks) and sums rows of
// gps * 16 + 4 floats.
__host__ __device__ inline int64_t gs_row_bytes(int64_t gps) { return gps * kGsSetCh * 2 + 16; }
__host__ __device__ inline int64_t gs_srow(int64_t gps) { return gps * 16 + 4; }
static int64_t gs_lds_need(int64_t T, int64_t gps) { return T * gs_row_bytes(gps) + T * gs_srow(gps) * 4; }

// Work split over the chip: row blocks x K slices, enough workgroups to
// cover 256 compute units, at most eight sets (one per wave) a slice.
struct GsPlan {
    int64_t rb, ng4, gps, slices;
};
static GsPlan gs_plan(int64_t T, int64_t K, int64_t M) {
    GsPlan p;
    p.rb = (M + kGsRows - 1) / kGsRows;
    p.ng4 = (K / kGsChunk + kGsSet - 1) / kGsSet;
    int64_t s = (256 + p.rb - 1) / p.rb;
    if (s > p.ng4) s = p.ng4;
    if (s < 1) s = 1;
    p.gps = (p.ng4 + s - 1) / s;
    if (p.gps > kGsMaxWaves) p.gps = kGsMaxWaves;
    while (p.gps > 1 && gs_lds_need(T, p.gps) > kGsLds) --p.gps;
    p.slices = (p.ng4 + p.gps - 1) / p.gps;
    return p;
}

// Workspace (several slices): the fp32 partials [slices][T][M].
static size_t gs_ws_bytes(int64_t T, int64_t K, int64_t M) {
    const GsPlan p = gs_plan(T, K, M);
    return p.slices > 1 ? ((size_t)p.slices * T * M * 4 + 255) / 256 * 256 : 0;
}

// Four bf16 pairs (128 + q) from one word of eight 4-bit codes (code i at
// bits 4 i), in slot order 0 2 4 6 1 3 5 7.
__device__ __forceinline__ u32x4 codes_as_bf16(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    constexpr uint32_t k43 = 0x43434343u;
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(k43, lo, 0x04010400u);   // codes 0, 2
    r[1] = __builtin_amdgcn_perm(k43, lo, 0x04030402u);   // codes 4, 6
    r[2] = __builtin_amdgcn_perm(k43, hi, 0x04010400u);   // codes 1, 3
    r[3] = __builtin_amdgcn_perm(k43, hi, 0x04030402u);   // codes 5, 7
    return r;
}

// 4x4 exchange between the lane quarters (16-lane rows) and the four words
// of a lane: word j of quarter q becomes word q of quarter j.
__device__ __forceinline__ void swap_quarters(u32x4& w) {
    const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    w[0] = c[0];
    w[1] = c[1];
    w[2] = d[0];
    w[3] = d[1];
}

__device__ __forceinline__ float h2f_lo(uint32_t d) { return f16_to_f32((uint16_t)(d & 0xFFFFu)); }
__device__ __forceinline__ float h2f_hi(uint32_t d) { return f16_to_f32((uint16_t)(d >> 16)); }

// NH fp16 values at byte offset off of a buffer (aligned to W bytes) as
// NH / 2 packed words; bytes past the end of the buffer read as zero.
template <int NH, int W>
__device__ __forceinline__ void load_halves(uint32_t (&d)[NH / 2], rsrc_t r, uint32_t off) {
    if constexpr (W == 16) {
#pragma unroll
        for (int v = 0; v < NH / 8; ++v) {
            const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16 * v), 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) d[4 * v + e] = a[e];
        }
    } else if constexpr (W == 8) {
#pragma unroll
        for (int v = 0; v < NH / 4; ++v) {
            const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off + 8 * v), 0, 0));
            d[2 * v] = a[0];
            d[2 * v + 1] = a[1];
        }
    } else if constexpr (W == 4) {
#pragma unroll
        for (int v = 0; v < NH / 2; ++v) d[v] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + 4 * v), 0, 0);
    } else {
#pragma unroll
        for (int v = 0; v < NH / 2; ++v)
            d[v] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)(off + 4 * v), 0, 0) |
                   ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)(off + 4 * v + 2), 0, 0) << 16);
    }
}

// Lane l: token l % 16 of the token operand, weight row l % 16 of the code
// operand, quarter l / 16; it holds the outputs of tokens 4 (l / 16) + i
// and row l % 16 of each row tile.  SZW: bytes per step / zero load (the
// alignment the row length of the step array allows).
template <int GROUP, bool YF32, int SZW>
__global__ __launch_bounds__(kGsMaxWaves * kWave) void k_qgemv_gs(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, int64_t ldx, const float* __restrict__ s,
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero,
    int64_t M, void* __restrict__ Y, int64_t ldy, float* __restrict__ P, int64_t gps) {
    constexpr int NG = kGsChunk / GROUP;          // groups per chunk
    constexpr int SPG = GROUP / 32;               // subgroups per group
    constexpr int NH = kGsSet * NG;               // groups per set
    __shared__ __attribute__((aligned(16))) unsigned char smem[kGsLds];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nw = blockDim.x / kWave;
    const int r16 = lane & 15, q = lane >> 4;
    const int64_t rb = blockIdx.x, sl = blockIdx.y, nsl = gridDim.y;
    const int64_t o0 = rb * kGsRows;
    const int64_t nch = K / kGsChunk;
    const int64_t kb = sl * gps * kGsSetCh;       // first channel of the slice
    const int64_t ks = K - kb < gps * kGsSetCh ? K - kb : gps * kGsSetCh;
    const int64_t wpr = K / 8, gpr = K / GROUP;
    const int64_t rowb = gs_row_bytes(gps), srow = gs_srow(gps);
    unsigned char* xs = smem;                     // [T][rowb]
    float* ss = (float*)(smem + T * rowb);        // [T][srow]

    // Requests in the order of use.  1) This thread's 8 channels of the
    // slice (channel kb + 8 tid) for every token, and their s; past the
    // slice or past T they read zeros through the buffer bounds.
    const rsrc_t rxr = make_rsrc(X, ((T - 1) * ldx + K) * 2);
    const rsrc_t rsr = make_rsrc(s, K * 4);
    const bool pu = 8 * tid < ks;
    const uint32_t pc = pu ? (uint32_t)(kb + 8 * tid) : 0x40000000u;
    const f32x4 sa = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsr, (int)(pc * 4), 0, 0));
    const f32x4 sb = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsr, (int)(pc * 4 + 16), 0, 0));
    u32x4 xr[kGsMaxT];
#pragma unroll
    for (int t = 0; t < kGsMaxT; ++t)
        xr[t] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rxr, (int)(t < T && pu ? (uint32_t)((t * ldx) * 2) + pc * 2 : 0x80000000u), 0, 0));
    __builtin_amdgcn_sched_barrier(0);

    // 2) Steps, zeros and codes of this wave's set (global set g; a wave
    // past the end of K loads the last set and does not use it, so that no
    // branch surrounds the loads).
    const bool active = wave * kGsSetCh < ks;     // wave-uniform
    const int64_t ng4 = (nch + kGsSet - 1) / kGsSet;
    const int64_t g = active ? sl * gps + wave : ng4 - 1;
    const uint32_t* crow[4];
    uint32_t szo[4];                              // byte offset of the row's steps / zeros
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        int64_t o = o0 + 16 * rt + r16;
        if (o >= M) o = M - 1;                    // rows past M: loads stay in bounds, outputs unused
        crow[rt] = codes + o * wpr + 4 * q;
        szo[rt] = (uint32_t)(o * gpr * 2);
    }
    const rsrc_t rsc = make_rsrc(scale, M * gpr * 2);
    const rsrc_t rze = make_rsrc(zero, M * gpr * 2);
    uint32_t sw[4][NH / 2], zw[4][NH / 2];
    u32x4 cw[kGsSet][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        load_halves<NH, SZW>(sw[rt], rsc, szo[rt] + (uint32_t)(g * NH * 2));
        load_halves<NH, SZW>(zw[rt], rze, szo[rt] + (uint32_t)(g * NH * 2));
    }
#pragma unroll
    for (int i = 0; i < kGsSet; ++i) {
        int64_t c = kGsSet * g + i;
        if (c >= nch) c = nch - 1;                // past the last chunk: codes stay in bounds, unused
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) cw[i][rt] = ld_nc((const u32x4*)(crow[rt] + 16 * c));
    }
    __builtin_amdgcn_sched_barrier(0);

    // 3) x~ = bf16(x * (1/s)) of this thread's channels into LDS, slot order
    // 0 2 4 6 1 3 5 7, and the 32-channel sums of x~ (fp32, slots in order
    // within a thread, then ((a + b) + (c + d)) over the four threads of a
    // subgroup).  Channels past the slice are written as zeros.
    {
        float rs[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            rs[e] = pu ? __builtin_amdgcn_rcpf(sa[e]) : 0.f;
            rs[4 + e] = pu ? __builtin_amdgcn_rcpf(sb[e]) : 0.f;
        }
        constexpr int kOrd[8] = {0, 2, 4, 6, 1, 3, 5, 7};
        const bool own = 8 * tid < gps * kGsSetCh;   // this thread's slot lies in the LDS row
#pragma unroll
        for (int t = 0; t < kGsMaxT; ++t) {
            if (t >= T) continue;                 // uniform
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16lo_to_f32(xr[t][e]) * rs[2 * e];
                x[2 * e + 1] = bf16hi_to_f32(xr[t][e]) * rs[2 * e + 1];
            }
            u32x4 o;
            float sum = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                o[d] = pack_bf16x2(x[kOrd[2 * d]], x[kOrd[2 * d + 1]]);
                sum += bf16lo_to_f32(o[d]);
                sum += bf16hi_to_f32(o[d]);
            }
            const float p1 = sum + __shfl_xor(sum, 1);
            const float p2 = p1 + __shfl_xor(p1, 2);
            if (own) {
                *(u32x4*)(xs + t * rowb + 16 * tid) = o;
                if ((tid & 3) == 0) ss[t * srow + tid / 4] = p2;
            }
        }
    }
    // LDS writes visible to the workgroup; the code loads stay in flight.
    __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) {
        // Token operand of MFMA j in quarter q: channels 32 j + 8 q .. +7 of
        // the chunk (the codes after the quarter exchange); with 128-channel
        // groups the exchange is skipped (one group per chunk: any channel
        // order that matches the codes will do) and it is 32 q + 8 j .. +7.
        // Lanes of tokens >= T read token 0: their output rows are not stored.
        constexpr int kXq = GROUP < 128 ? 16 : 64, kXj = GROUP < 128 ? 64 : 16;
        const int tl = r16 < T ? r16 : 0;
        const unsigned char* xl = xs + tl * rowb + kXq * q + (int64_t)wave * kGsSetCh * 2;
        const float* sl4 = ss + tl * srow + wave * 16 + q;
        const bool q1 = (q & 1) != 0, q2 = (q & 2) != 0;
#pragma unroll
        for (int i = 0; i < kGsSet; ++i) {
            // A chunk past K adds nothing: its steps and sums are taken as
            // zero (its token operand is zero in LDS).
            const bool cv = kGsSet * g + i < nch;
            const float si = cv ? sl4[4 * i] : 0.f;
            u32x4 xa[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xa[j] = *(const u32x4*)(xl + i * kGsChunk * 2 + kXj * j);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                u32x4 w = cw[i][rt];
                if constexpr (GROUP < 128) swap_quarters(w);
                f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p = mfma_16x16x32(xa[j], codes_as_bf16(w[j]), p);
                    if ((j + 1) % SPG == 0) {
                        const int gl = i * NG + j / SPG;
                        float st = (gl & 1) ? h2f_hi(sw[rt][gl / 2]) : h2f_lo(sw[rt][gl / 2]);
                        st = cv ? st : 0.f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[rt][e] = __builtin_fmaf(st, p[e], acc[rt][e]);
                        p = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
                // step (z + 128) of the group of subgroup q of this chunk.
                uint32_t sd, zd;
                bool hi;
                if constexpr (NG == 4) {          // group 4 i + q
                    sd = q2 ? sw[rt][2 * i + 1] : sw[rt][2 * i];
                    zd = q2 ? zw[rt][2 * i + 1] : zw[rt][2 * i];
                    hi = q1;
                } else if constexpr (NG == 2) {   // group 2 i + q / 2
                    sd = sw[rt][i];
                    zd = zw[rt][i];
                    hi = q2;
                } else {                          // group i
                    sd = sw[rt][i / 2];
                    zd = zw[rt][i / 2];
                    hi = (i & 1) != 0;
                }
                const float st = hi ? h2f_hi(sd) : h2f_lo(sd);
                const float zf = hi ? h2f_hi(zd) : h2f_lo(zd);
                const float nb = cv ? -(st * (zf + 128.f)) : 0.f;
                acc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(si, nb, acc[rt], 0, 0, 0);
            }
        }
    }

    // Wave tiles added in wave order (the LDS of the tokens reused once all
    // waves have read it); one wave per row tile.
    __syncthreads();
    f32x4* red = (f32x4*)smem;                    // [nw][4][kWave]
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) red[(wave * 4 + rt) * kWave + lane] = acc[rt];
    __syncthreads();
    for (int rt = wave; rt < 4; rt += nw) {
        f32x4 sum = red[rt * kWave + lane];
        for (int w = 1; w < nw; ++w) {
            const f32x4 v = red[(w * 4 + rt) * kWave + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[e] += v[e];
        }
        const int64_t o = o0 + 16 * rt + r16;
        if (o < M) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = 4 * q + e;
                if (t < T) {
                    if (nsl > 1) P[(sl * T + t) * M + o] = sum[e];
                    else if constexpr (YF32) ((float*)Y)[t * ldy + o] = sum[e];
                    else ((uint16_t*)Y)[t * ldy + o] = (uint16_t)f32_to_bf16(sum[e]);
                }
            }
        }
    }
}

// Y[t][o] = sum over slices k = 0.. of P[k][t][o], in slice order.
template <bool YF32>
__global__ __launch_bounds__(256) void k_gs_reduce(const float* __restrict__ P, int64_t nsl, int64_t T, int64_t M,
                                                   void* __restrict__ Y, int64_t ldy) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * M) return;
    const int64_t t = idx / M, o = idx % M;
    float a = P[idx];
    for (int64_t k = 1; k < nsl; ++k) a += P[k * T * M + idx];
    if constexpr (YF32) ((float*)Y)[t * ldy + o] = a;
    else ((uint16_t*)Y)[t * ldy + o] = (uint16_t)f32_to_bf16(a);
}

// bf16 tokens, 4-bit codes, groups of 32 / 64 / 128, K a multiple of 128.
bool qgemv_gs_eligible(int64_t T, int64_t K, int64_t M, int bits, int group, bool xf32, int64_t ldx) {
    return !xf32 && T >= kGsMinT && T <= kGsMaxT && bits == 4 && (group == 32 || group == 64 || group == 128) &&
           K % kGsChunk == 0 && K < ((int64_t)1 << 24) && M * (K / group) * 2 < ((int64_t)1 << 31) &&
           ((T - 1) * ldx + K) * 2 < ((int64_t)1 << 30);
}

size_t qgemv_gs_ws_bytes(int64_t T, int64_t K, int64_t M) { return gs_ws_bytes(T, K, M); }

template <int GROUP, bool YF32, int SZW>
static hipError_t launch_gs3(const GsPlan& pl, const uint16_t* X, int64_t T, int64_t K, int64_t ldx, const float* s,
                             const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, void* Y,
                             int64_t ldy, void* ws, hipStream_t st, StageTimer tm) {
    float* P = (float*)ws;
    const dim3 grid((unsigned)pl.rb, (unsigned)pl.slices), block((unsigned)(pl.gps * kWave));
    if (pl.slices == 1)
        return launch_kernel(k_qgemv_gs<GROUP, YF32, SZW>, grid, block, 0, st, tm.start, tm.stop, X, T, K, ldx, s,
                             codes, scale, zero, M, Y, ldy, P, pl.gps);
    if (hipError_t e = launch_kernel(k_qgemv_gs<GROUP, YF32, SZW>, grid, block, 0, st, tm.start, nullptr, X, T, K, ldx,
                                     s, codes, scale, zero, M, Y, ldy, P, pl.gps))
        return e;
    return launch_kernel(k_gs_reduce<YF32>, dim3((unsigned)((T * M + 255) / 256)), dim3(256), 0, st, nullptr, tm.stop,
                         (const float*)P, pl.slices, T, M, Y, ldy);
}

// Widest step / zero load the row length allows (row o starts o K / GROUP
// halves in; a set reads 4 * 128 / GROUP of them from a multiple of that).
// The row length K / GROUP * 2 bytes is a multiple of 8 (group 32), 4 (64)
// or 2 (128) for K a multiple of 128.
template <int GROUP, bool YF32>
static hipError_t launch_gs2(const GsPlan& pl, const uint16_t* X, int64_t T, int64_t K, int64_t ldx,
                             const float* s, const uint32_t* codes, const uint16_t* scale, const uint16_t* zero,
                             int64_t M, void* Y, int64_t ldy, void* ws, hipStream_t st, StageTimer tm) {
    constexpr int kSetBytes = kGsSet * (kGsChunk / GROUP) * 2;
    constexpr int kMinW = GROUP == 32 ? 8 : GROUP == 64 ? 4 : 2;
    const int64_t rowb = K / GROUP * 2;
    int w = kMinW;
    while (w < 16 && w < kSetBytes && rowb % (2 * w) == 0) w *= 2;
#define TTQ_GS(W) return launch_gs3<GROUP, YF32, W>(pl, X, T, K, ldx, s, codes, scale, zero, M, Y, ldy, ws, st, tm)
    if constexpr (kSetBytes >= 16)
        if (w == 16) TTQ_GS(16);
    if (w == 8) TTQ_GS(8);
    if constexpr (kMinW <= 4)
        if (w == 4) TTQ_GS(4);
    if constexpr (kMinW <= 2) TTQ_GS(2);
#undef TTQ_GS
    return hipErrorInvalidValue;
}

hipError_t launch_qgemv_gs(const void* X, bool xf32, int64_t T, int64_t K, int64_t ldx, const float* s,
                           const uint32_t* codes, const uint16_t* scale, const uint16_t* zero, int64_t M, int bits,
                           int group, void* Y, bool yf32, int64_t ldy, void* ws, hipStream_t st, StageTimer tm) {
    if (!qgemv_gs_eligible(T, K, M, bits, group, xf32, ldx)) return hipErrorInvalidValue;
    const GsPlan pl = gs_plan(T, K, M);
    const uint16_t* Xb = (const uint16_t*)X;
#define TTQ_GS2(G)                                                                                            \
    return yf32 ? launch_gs2<G, true>(pl, Xb, T, K, ldx, s, codes, scale, zero, M, Y, ldy, ws, st, tm) \
                : launch_gs2<G, false>(pl, Xb, T, K, ldx, s, codes, scale, zero, M, Y, ldy, ws, st, tm)
    switch (group) {
        case 32: TTQ_GS2(32);
        case 64: TTQ_GS2(64);
        case 128: TTQ_GS2(128);
    }
#undef TTQ_GS2
    return hipErrorInvalidValue;
}

}  // namespace ttq
