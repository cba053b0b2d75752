// Device-side helpers shared by the sparse-MLA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWave = 64;
constexpr int kPage = 64;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBf16Record = 1152;   // bytes per bf16 token record
constexpr int kFp8Record = 656;     // bytes per FP8 token record

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt[5:4] at bits 15:14, expcnt 6:4,
// lgkmcnt 11:8).  Only the named counter is waited on; the others are left at their maximum.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most n (wave-uniform, 0 <= n <= MAX) vector-memory operations are outstanding.
template <int MAX>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
    if constexpr (MAX > 0) {
        if (n >= MAX) {
            wait_vmcnt<MAX>();
            return;
        }
        wait_vmcnt_upto<MAX - 1>(n);
    } else {
        wait_vmcnt<0>();
    }
}
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// fp32 -> bf16 bit pattern, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Pack two fp32 into a bf16 pair (lo in the low half), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// Order-preserving 32-bit key of an fp32 score: larger key <=> larger score.  -0.0 maps to the
// key of +0.0 (they compare equal) and every NaN maps to 0, below the key of -inf (0x007fffff).
// No number maps to 0: the only patterns whose transform would be 0 are NaNs.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u) return 0u;
    if (mag == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace smla
