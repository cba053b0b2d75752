// KV insert: the records of new tokens written into the paged latent cache, gfx950.
//
// Sources: "Port DeepSeek-V4 optimization PR #174 to v0.26 ..." (MooreThreads/vllm-musa PR 178),
// table "Optimizations carried from PR #174" (row "Attention cache write": the inverse-RoPE FP8
// cache write works on its chunks in parallel; row "FP8 quantization": the fp32 scale groups stay
// contiguous); "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL", section on the fused
// group-quantization operator (128-element groups with FP32 scales, 64-bit offsets); "[JJ]
// Preallocate DeepSeek V4 padded-query output" (local-inference-lab/vllm PR 671), "Operation
// contract" (the fused RoPE and KV-insert operator mutates caller-owned storage only); "[Bugfix]
// Make DSV4 sparse MLA work end-to-end ...", section "Purpose" (slot = block id * block size +
// offset).
//
// One wave per two tokens (both tokens' loads are issued before either is converted), eight tokens
// per 256-thread workgroup; every token is independent, so the result does not depend on how
// tokens are batched.
//   bf16 record: the 1152 input bytes, copied (lanes 0..63 one 16-byte chunk each, lanes 0..7 one more).
//   FP8 record [512 codes | 4 fp32 scales | 64 bf16 rope]: lane l holds latent values 8l .. 8l+7,
//   which lie in scale group l / 16.  The group's largest magnitude amax comes from a max over its 16
//   lanes (one DPP row); the stored scale is s = amax / 448 and every code is e4m3(x / s), the
//   inverse of the dequantization (code * s), with IEEE fp32 divisions (round to nearest even).
//   x / s is clamped to [-448, 448] (saturation) and converted by the hardware OCP E4M3 conversion,
//   which rounds to nearest even.  An all-zero group stores s = 0 and zero codes.  Lane 16g stores
//   s_g; lanes 0..7 store the rope.
//   Inverse RoPE (optional): the wave's two tokens have 64 rope pairs, one per lane (lane l: token
//   l / 32, pair l % 32), so every lane rotates one pair and stores its 4 bytes.  Pair i (a, b) of a
//   token at position p becomes (a c + b s, -a s + b c) with c = cos_sin[p][i], s = cos_sin[p][32 + i].
//   Both products are exact in fp64 (8 x 24 significant bits), their sum is rounded once in fp64 and
//   then to bf16 (nearest even) by scaling to the bf16 unit in the last place and rounding to an
//   integer, so the stored value is the exactly rounded rotation unless the fp64 sum itself needed
//   rounding next to a bf16 rounding boundary (at most one bf16 unit apart).
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kTokPerWave = 2;
constexpr int kTokPerBlock = 4 * kTokPerWave;

// Codes of two fp32 values (already inside [-448, 448]) into bytes 0-1 (HI false) or 2-3 of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t pack_e4m3x2(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

__device__ __forceinline__ float sat448(float y) { return __builtin_amdgcn_fmed3f(y, -448.f, 448.f); }

// Max over the 16 lanes of each DPP row (rotations by 8, 4, 2, 1 within the row).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));
    return v;
}

// fp64 -> bf16 bit pattern, rounded to nearest even in one step: the value is scaled by a power of
// two so that one bf16 unit in the last place becomes 1 (exact), rounded to an integer (ties to
// even), and scaled back (exact); the result is a bf16 value, which fp32 holds exactly.  Values below
// 2^-126 share the subnormal unit 2^-133.  A zero result is +0 (the exact sum has no sign).  Finite
// inputs whose rounded value fits bf16 only.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
    if (v == 0.0) return 0u;
    int e = ((int)((__double_as_longlong(v) >> 52) & 0x7ff)) - 1023;   // v is far above fp64 subnormals
    e = e < -126 ? -126 : e;
    const double n = __builtin_rint(__builtin_ldexp(v, 7 - e));        // bf16 keeps 8 significant bits
    const float r = (float)__builtin_ldexp(n, e - 7);                    // exact
    return __float_as_uint(r) >> 16;
}

// One rope pair (two bf16 values) with the rotation of the token's position undone.
__device__ __forceinline__ uint32_t inverse_rope_pair(uint32_t w, float c, float s) {
    const double a = (double)__uint_as_float(w << 16), b = (double)__uint_as_float(w & 0xffff0000u);
    const double ci = (double)c, si = (double)s;
    const double y0 = __builtin_fma(a, ci, b * si);     // b * si is exact in fp64
    const double y1 = __builtin_fma(b, ci, -(a * si));  // a * si is exact in fp64
    return f64_to_bf16_rne(y0) | (f64_to_bf16_rne(y1) << 16);
}

// One token's FP8 record from the lane's 8 latent values `lat`; with COPY_ROPE lanes 0..7 also store
// the rope chunk `rope`.
template <bool COPY_ROPE>
__device__ __forceinline__ void write_fp8_record(uint8_t* dst, int lane, uint4 lat, uint4 rope) {
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
    amax = row16_max(amax);   // lanes 16g .. 16g+15 hold group g
    uint32_t lo = 0u, hi = 0u;
    float s = 0.f;
    if (amax > 0.f) {   // s > 0 for every nonzero bf16 amax (2^-133 / 448 is above the least fp32 subnormal)
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
    if (COPY_ROPE && lane < 8) *(uint4*)(dst + 528 + 16 * lane) = rope;
}

template <bool FP8, bool ROPE>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(const uint16_t* __restrict__ in, int64_t in_row_stride,
                                                             const int64_t* __restrict__ slots,
                                                             const int64_t* __restrict__ positions,
                                                             const float* __restrict__ cos_sin, int64_t max_pos,
                                                             int32_t T, uint8_t* __restrict__ cache,
                                                             int64_t num_slots) {
    static_assert(kTokPerWave * 32 == kWave, "ROPE: one rope pair per lane");
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kTokPerWave;
    const int jr = lane >> 5, pr = lane & 31;   // ROPE: this lane's token (of the wave's two) and rope pair
    uint4 lat[kTokPerWave], rope[kTokPerWave];
    int64_t slot[kTokPerWave], pos[kTokPerWave];
    uint32_t rp = 0u;                           // ROPE: the lane's rope pair
#pragma unroll
    for (int j = 0; j < kTokPerWave; ++j) {   // every load first (wave-uniform guards)
        const int64_t t = t0 + j;
        slot[j] = -1;
        pos[j] = 0;
        lat[j] = rope[j] = make_uint4(0u, 0u, 0u, 0u);
        if (t < T) {
            slot[j] = slots[t];
            if (ROPE) pos[j] = positions[t];
            const uint16_t* src = in + t * in_row_stride;
            lat[j] = *(const uint4*)(src + 8 * lane);
            if (!ROPE && lane < 8) rope[j] = *(const uint4*)(src + 512 + 8 * lane);
        }
    }
    if constexpr (ROPE) {
        if (t0 + jr < T) rp = *(const uint32_t*)(in + (t0 + jr) * in_row_stride + 512 + 2 * pr);
#pragma unroll
        for (int j = 0; j < kTokPerWave; ++j)   // a position outside [0, max_pos) leaves the token unwritten
            if (pos[j] < 0 || pos[j] >= max_pos) slot[j] = -1;
        const int64_t ps = jr ? pos[1] : pos[0];
        if ((jr ? slot[1] : slot[0]) >= 0) {
            const float* row = cos_sin + ps * 64;
            rp = inverse_rope_pair(rp, row[pr], row[32 + pr]);
        }
    }
#pragma unroll
    for (int j = 0; j < kTokPerWave; ++j) {
        if (slot[j] < 0 || slot[j] >= num_slots) continue;   // past T, padding or out of range: nothing written
        if constexpr (!FP8) {
            uint8_t* dst = cache + slot[j] * kBf16Record;
            *(uint4*)(dst + 16 * lane) = lat[j];
            if (!ROPE && lane < 8) *(uint4*)(dst + 1024 + 16 * lane) = rope[j];
        } else {
            write_fp8_record<!ROPE>(cache + slot[j] * kFp8Record, lane, lat[j], rope[j]);
        }
    }
    if constexpr (ROPE) {   // lanes 32 j .. 32 j + 31 store token j's 32 pairs (128 contiguous bytes)
        const int64_t sl = jr ? slot[1] : slot[0];
        if (sl >= 0 && sl < num_slots)
            *(uint32_t*)(cache + sl * (FP8 ? kFp8Record : kBf16Record) + (FP8 ? 528 : 1024) + 4 * pr) = rp;
    }
}

template <bool FP8, bool ROPE>
void launch_one(unsigned grid, hipStream_t stream, const void* in, int64_t in_row_stride, const int64_t* slots,
                const int64_t* positions, const float* cos_sin, int64_t max_pos, int32_t T, void* cache,
                int64_t num_slots) {
    kv_cache_write_kernel<FP8, ROPE><<<grid, 256, 0, stream>>>((const uint16_t*)in, in_row_stride, slots, positions,
                                                                cos_sin, max_pos, T, (uint8_t*)cache, num_slots);
}

}  // namespace

hipError_t launch_kv_cache_write(const void* in, int64_t in_row_stride, const int64_t* slots, const int64_t* positions,
                                 const float* cos_sin, int64_t max_pos, int32_t T, void* cache, int kv_dtype,
                                 int64_t num_pages, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((T + kTokPerBlock - 1) / kTokPerBlock);
    const int64_t num_slots = num_pages * kPage;
    const bool rope = positions != nullptr;
    if (kv_dtype == 1) {
        if (rope) launch_one<true, true>(grid, stream, in, in_row_stride, slots, positions, cos_sin, max_pos, T, cache, num_slots);
        else launch_one<true, false>(grid, stream, in, in_row_stride, slots, nullptr, nullptr, 0, T, cache, num_slots);
    } else {
        if (rope) launch_one<false, true>(grid, stream, in, in_row_stride, slots, positions, cos_sin, max_pos, T, cache, num_slots);
        else launch_one<false, false>(grid, stream, in, in_row_stride, slots, nullptr, nullptr, 0, T, cache, num_slots);
    }
    return hipGetLastError();
}

}  // namespace smla
