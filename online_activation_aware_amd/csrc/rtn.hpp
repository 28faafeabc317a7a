// Group-wise RTN helpers shared by the quantizer kernels (gfx950).
//
// [TTQ §method b1] group-wise RTN: per group of consecutive input channels of
// one output row, mn = min(0, min v), mx = max(0, max v); step = fp16
// rounded up of fp32(mx - mn) / (2^b - 1) (1 if that is 0); zero =
// clamp(rne(-mn / step), 0, 2^b - 1); code = clamp(rne(v / step) + zero).
#pragma once

#include "common.hpp"

namespace ttq {

constexpr float kMagic = 12582912.0f;      // 1.5 * 2^23: fp32 spacing 1 from 2^23 to 2^24
constexpr uint32_t kMagicBits = 0x4B400000u;

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

// min/max over the GL lanes of a group (aligned runs of GL adjacent lanes).
// NaN is ignored: v_min/v_max return the non-NaN operand.
template <int GL>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
    static_assert(GL == 1 || GL == 2 || GL == 4 || GL == 8 || GL == 16, "lanes per group");
    if constexpr (GL >= 2) {
        mn = fminf(mn, dpp_f<kDppQuadXor1>(mn));
        mx = fmaxf(mx, dpp_f<kDppQuadXor1>(mx));
    }
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

// fp32(x) / QMAXI for finite x >= 0, correctly rounded: q0 = x * r with r the
// rounded reciprocal of the constant, then one fma correction of the
// remainder.  Equal to the IEEE division for every finite non-negative fp32
// x and QMAXI in {3, 7, 15, 31} (checked exhaustively).
template <int QMAXI>
__device__ __forceinline__ float div_qmax(float x) {
    constexpr float q = (float)QMAXI;
    constexpr float r = 1.0f / q;
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, q, x);
    return __builtin_fmaf(e, r, q0);
}

// The group's step (fp16 bits and value), zero point and 1/step from its
// 0-extended range.
struct GroupStep {
    uint16_t dh;
    float df, z, inv;
};
template <int BITS>
__device__ __forceinline__ GroupStep group_step(float mn, float mx) {
    constexpr int QMAXI = (1 << BITS) - 1;
    GroupStep g;
    mn = fminf(0.0f, mn);
    mx = fmaxf(0.0f, mx);
    const float d32 = div_qmax<QMAXI>(mx - mn);
    g.dh = d32 == 0.0f ? (uint16_t)0x3C00 : f32_to_f16_up(d32);
    g.df = f16_to_f32(g.dh);
    g.z = fminf(fmaxf(rintf((-mn) / g.df), 0.0f), (float)QMAXI);
    g.inv = __builtin_amdgcn_rcpf(g.df);
    return g;
}

// kMagic + code for value v: one fma forms v * (1/step) + (kMagic + zero),
// whose rounding to fp32 (spacing 1 there) is the rounded code; the clamp is
// one v_med3 (a NaN value gives the lower bound, code 0).  (code - zero) is
// then exactly qm - (kMagic + zero), and the code is the low bits of qm's bit
// pattern.  v * (1/step) differs from v / step by a few ulps: only values
// within ~1e-6 of a step of a rounding boundary (exact ties among them) can
// be decided differently from v / step.
template <int BITS>
__device__ __forceinline__ float code_magic(float v, const GroupStep& g, float mz) {
    constexpr float QMAX = (float)((1 << BITS) - 1);
    return fminf(fmaxf(__builtin_fmaf(v, g.inv, mz), kMagic), kMagic + QMAX);
}

}  // namespace ttq
