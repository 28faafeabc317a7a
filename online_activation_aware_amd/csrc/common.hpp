// Device helpers shared by the libttq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttq {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t packed) {
    return __builtin_bit_cast(float, packed << 16);
}
__device__ __forceinline__ float bf16hi_to_f32(uint32_t packed) {
    return __builtin_bit_cast(float, packed & 0xFFFF0000u);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)x);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32 (RNE).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp16 bit pattern <-> fp32.
__device__ __forceinline__ float f16_to_f32(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
}
__device__ __forceinline__ uint16_t f32_to_f16_rne(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// fp32 -> fp16 rounded toward +infinity, for x >= 0 (NaN-free).
__device__ __forceinline__ uint16_t f32_to_f16_up(float x) {
    uint16_t h = f32_to_f16_rne(x);
    if (f16_to_f32(h) < x) h = (uint16_t)(h + 1);   // next fp16 up (x >= 0)
    return h;
}

__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T ld_nc(const T* p) {
    return __builtin_nontemporal_load(p);
}

// Store, with the nontemporal (streaming) hint when NT.  A compile-time
// choice: behind a runtime branch the compiler merges the two stores into
// one plain store.
template <bool NT, typename T>
__device__ __forceinline__ void st_nt(T* p, const T& v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Streaming stores for a staged dequantized weight (and its codes) larger
// than this.  Measured on MI355X: with a 117 MB w~ (4096 x 14336 or 14336 x
// 4096 bf16) ordinary stores leave the Infinity Cache (256 MiB, also holding
// the weight being read) full of dirty lines that the projection then
// competes with (4096 -> 14336, T = 512: layer 135.9 -> 126.4-127.2 us with
// streaming stores; 14336 -> 4096, T = 1024: 189.5 -> 183.4-185.2 us); a
// 33.5 MB w~ (4096 x 4096) is read back from that cache by the projection,
// and streaming it cost ~1 us.
constexpr int64_t kStreamStageBytes = (int64_t)64 << 20;
inline bool stream_stage(int64_t M, int64_t K) { return M * K * 2 > kStreamStageBytes; }

}  // namespace ttq
