// Buffer -> LDS staging helpers for the matrix-core kernels (gfx950).
#pragma once

#include "common.hpp"

namespace ttq {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit buffer, gfx9-family descriptor

// Buffer descriptor over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// s_waitcnt vmcnt(n) (expcnt / lgkmcnt left unconstrained), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

// vmcnt(n) for a wave-uniform runtime n (0..11; larger values wait for all).
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

typedef __attribute__((address_space(3))) void lds_void;

// Buffer -> LDS DMA of LS bytes per lane (64 lanes land contiguously at
// `lds`).  Lanes of 16 and 4 bytes land where expected; narrower lanes are
// still spaced 4 bytes apart.  The size operand must be a literal for the
// host compilation pass, hence the explicit dispatch.
template <int LS>
__device__ __forceinline__ void dma_to_lds(rsrc_t r, void* lds, int voff, int soff) {
    static_assert(LS == 4 || LS == 16, "DMA lane size");
    if constexpr (LS == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, soff, 0, 0);
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

// LDS tiles of 64-deep bf16 K slices use 128-byte rows of eight 16-byte
// chunks; chunk j of row r is stored at position j ^ (r & 7), so that 8
// consecutive rows read at the same chunk hit 8 different bank groups
// (conflict-free 16-byte reads and writes).
constexpr int kLdsRowB = 128;
__device__ __forceinline__ int lds_swz(int row, int chunk) {
    return row * kLdsRowB + ((chunk ^ (row & 7)) << 4);
}

// Store 4 consecutive outputs Y[row][o .. o+3] (fp32 accumulators) as fp32 or
// bf16 (RNE); `avail` = M - o outputs exist; one vector store when `vec`.
template <bool YF32>
__device__ __forceinline__ void store_y4(void* Y, int64_t idx, int64_t avail, int vec, const f32x4& v) {
    if constexpr (YF32) {
        float* yp = (float*)Y + idx;
        if (vec && avail >= 4) {
            *(f32x4*)yp = v;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (r < avail) yp[r] = v[r];
        }
    } else {
        uint16_t* yp = (uint16_t*)Y + idx;
        if (vec && avail >= 4) {
            u32x2 p = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *(u32x2*)yp = p;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (r < avail) yp[r] = (uint16_t)f32_to_bf16(v[r]);
        }
    }
}

}  // namespace ttq
