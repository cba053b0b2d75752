// KV insert: the records of new tokens written into the paged latent cache, gfx950.
//
// Sources: "Port DeepSeek-V4 optimization PR #174 to v0.26 ..." (MooreThreads/vllm-musa PR 178),
// table "Optimizations carried from PR #174" (the FP8 cache write works on its chunks in parallel
// and keeps the fp32 scale groups contiguous); "[DeepSeek-V4][Preview] Batch-invariant kernels for
// 0-diff RL", section on the fused group-quantization operator (128-element groups with FP32
// scales, 64-bit offsets); "[JJ] Preallocate DeepSeek V4 padded-query output" (local-inference-lab/
// vllm PR 671), "Operation contract" (the KV-insert operator mutates caller-owned storage only);
// "[Bugfix] Make DSV4 sparse MLA work end-to-end ...", section "Purpose" (slot = block id * block
// size + offset).
//
// One wave per token, four tokens per 256-thread workgroup; every token is independent, so the
// result does not depend on how tokens are batched.
//   bf16 record: the 1152 input bytes, copied (lanes 0..63 one 16-byte chunk each, lanes 0..7 one more).
//   FP8 record [512 codes | 4 fp32 scales | 64 bf16 rope]: lane l holds latent values 8l .. 8l+7,
//   which lie in scale group l / 16.  The group's largest magnitude comes from a max over its 16
//   lanes; s = amax / 448 and every code is e4m3(x / s), both IEEE fp32 divisions.  The quotient is
//   clamped to [-448, 448] (saturation) and converted by the hardware OCP E4M3 conversion, which rounds
//   to nearest even.  An all-zero group stores s = 0 and zero codes.  Lane 16g stores s_g; lanes 0..7
//   copy the rope.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kTokPerBlock = 4;   // one wave per token

// Codes of two fp32 values (already inside [-448, 448]) into bytes 0-1 (HI false) or 2-3 of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t pack_e4m3x2(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

__device__ __forceinline__ float sat448(float y) { return fminf(fmaxf(y, -448.f), 448.f); }

template <bool FP8>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(const uint16_t* __restrict__ in, int64_t in_row_stride,
                                                             const int64_t* __restrict__ slots, int32_t T,
                                                             uint8_t* __restrict__ cache, int64_t num_slots) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) return;   // padding or out-of-range slot: nothing written
    const uint16_t* src = in + t * in_row_stride;
    const uint4 lat = *(const uint4*)(src + 8 * lane);
    uint4 rope = make_uint4(0u, 0u, 0u, 0u);
    if (lane < 8) rope = *(const uint4*)(src + 512 + 8 * lane);
    if constexpr (!FP8) {
        uint8_t* dst = cache + slot * kBf16Record;
        *(uint4*)(dst + 16 * lane) = lat;
        if (lane < 8) *(uint4*)(dst + 1024 + 16 * lane) = rope;
        return;
    } else {
        uint8_t* dst = cache + slot * kFp8Record;
        const uint32_t w[4] = {lat.x, lat.y, lat.z, lat.w};
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {   // bf16 -> fp32 is exact
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));   // the group's 16 lanes
        uint32_t lo = 0u, hi = 0u;
        float s = 0.f;
        if (amax > 0.f) {
            s = amax / 448.f;
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = sat448(x[i] / s);
            lo = pack_e4m3x2<false>(y[0], y[1], 0u);
            lo = pack_e4m3x2<true>(y[2], y[3], lo);
            hi = pack_e4m3x2<false>(y[4], y[5], 0u);
            hi = pack_e4m3x2<true>(y[6], y[7], hi);
        }
        *(uint2*)(dst + 8 * lane) = make_uint2(lo, hi);
        if ((lane & 15) == 0) *(float*)(dst + 512 + 4 * (lane >> 4)) = s;
        if (lane < 8) *(uint4*)(dst + 528 + 16 * lane) = rope;
    }
}

}  // namespace

hipError_t launch_kv_cache_write(const void* in, int64_t in_row_stride, const int64_t* slots, int32_t T, void* cache,
                                 int kv_dtype, int64_t num_pages, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((T + kTokPerBlock - 1) / kTokPerBlock);
    const int64_t num_slots = num_pages * kPage;
    if (kv_dtype == 1)
        kv_cache_write_kernel<true><<<grid, 256, 0, stream>>>((const uint16_t*)in, in_row_stride, slots, T,
                                                              (uint8_t*)cache, num_slots);
    else
        kv_cache_write_kernel<false><<<grid, 256, 0, stream>>>((const uint16_t*)in, in_row_stride, slots, T,
                                                               (uint8_t*)cache, num_slots);
    return hipGetLastError();
}

}  // namespace smla
