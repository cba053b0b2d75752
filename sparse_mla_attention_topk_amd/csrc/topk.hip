// Stable top-k per row with canonical (ascending) output, gfx950.
//
// Method (deterministic sparse top-k of "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff
// RL", section "Deterministic sparse top-k"; length clamping and -1 padding of "[Bugfix] Make DSV4
// sparse MLA work end-to-end ...", "What is fixed"):
//   * every score becomes an order-preserving 32-bit key (score_key); the composite order is
//     (key descending, index ascending), so the n = min(k, L) selected candidates are exactly
//       { j : key_j > T } U { the first `need` indices j with key_j == T }
//     for the key T of the n-th candidate and need = n - #{key > T};
//   * T is found by radix selection over key digits (12, 12, 8 bits), one LDS histogram per digit,
//     stopping early once a whole bucket is taken;
//   * the selection is written by an ordered compaction: the row is scanned in index order, wave
//     ballots and a block-wide prefix sum give each selected candidate its output slot, so the
//     output is ascending by construction (no sort) and the -1 tail is filled afterwards.
// One 1024-thread workgroup owns one row; every decision is made from the clamped length that all
// threads read, so the result is a pure function of the row (batch-invariant, no inter-workgroup
// synchronization of any kind).
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;   // 16
constexpr int kTopkUnroll = 16;                     // elements per thread per chunk
constexpr int64_t kTopkChunk = (int64_t)kTopkThreads * kTopkUnroll;

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum of v over the 1024 threads of the block, in thread order.
// `scratch` holds at least kTopkWaves + 1 words of LDS.  Ends with a barrier.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        uint32_t y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) scratch[wid] = x;
    __syncthreads();
    if (wid == 0) {
        uint32_t w = lane < kTopkWaves ? scratch[lane] : 0u;
        uint32_t z = w;
#pragma unroll
        for (int off = 1; off < kTopkWaves; off <<= 1) {
            uint32_t y = __shfl_up(z, off, kWave);
            if (lane >= off) z += y;
        }
        if (lane < kTopkWaves) scratch[lane] = z - w;
        if (lane == kTopkWaves - 1) scratch[kTopkWaves] = z;
    }
    __syncthreads();
    uint32_t r = scratch[wid] + x - v;
    *total = scratch[kTopkWaves];
    __syncthreads();
    return r;
}

// Histogram of the BITS-bit digit below the DEPTH leading key bits, over the candidates whose
// leading DEPTH bits equal `prefix`.
template <int DEPTH, int BITS>
__device__ void digit_histogram(const float* __restrict__ s, int64_t L, uint32_t prefix, uint32_t* hist) {
    constexpr int kBins = 1 << BITS;
    constexpr int kShift = 32 - DEPTH - BITS;
    for (int i = threadIdx.x; i < kBins; i += kTopkThreads) hist[i] = 0u;
    __syncthreads();
    for (int64_t base = 0; base < L; base += kTopkChunk) {
        uint32_t key[kTopkUnroll];
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
            key[u] = j < L ? score_key(s[j]) : 0u;
        }
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
            bool match = j < L;
            if constexpr (DEPTH > 0) match = match && ((key[u] >> (32 - DEPTH)) == prefix);
            if (match) atomicAdd(&hist[(key[u] >> kShift) & (kBins - 1)], 1u);
        }
    }
    __syncthreads();
}

// Finds the digit d holding the need-th largest candidate: above = #candidates with a larger digit,
// above < need <= above + hist[d].  Results land in res[0..2] = {d, above, hist[d]}.
template <int BITS>
__device__ void find_digit(const uint32_t* hist, uint32_t need, uint32_t* scratch, uint32_t* res) {
    constexpr int kBins = 1 << BITS;
    constexpr int kPer = kBins >= kTopkThreads ? kBins / kTopkThreads : 1;
    uint32_t h[kPer];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int d = kBins - 1 - (threadIdx.x * kPer + i);   // thread 0 owns the top digits
        h[i] = d >= 0 ? hist[d] : 0u;
        local += h[i];
    }
    uint32_t total;
    uint32_t above = block_exclusive_scan(local, scratch, &total);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int d = kBins - 1 - (threadIdx.x * kPer + i);
        if (d >= 0 && above < need && above + h[i] >= need) {
            res[0] = (uint32_t)d;
            res[1] = above;
            res[2] = h[i];
        }
        above += h[i];
    }
    __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(const float* __restrict__ scores,
                                                                 const int64_t* __restrict__ row_offsets,
                                                                 int64_t row_stride,
                                                                 const int32_t* __restrict__ lengths,
                                                                 int32_t k, int32_t* __restrict__ out) {
    __shared__ uint32_t hist[1 << 12];
    __shared__ uint32_t scratch[kTopkWaves + 2];
    __shared__ uint32_t res[3];
    __shared__ uint32_t tbl[kTopkUnroll * kTopkWaves];

    const int row = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int64_t len = lengths ? (int64_t)lengths[row] : row_stride;
    const int64_t L = len < 0 ? 0 : (len > row_stride ? row_stride : len);   // clamp before any decision
    const int64_t off = row_offsets ? row_offsets[row] : (int64_t)row * row_stride;
    const float* __restrict__ s = scores + off;
    int32_t* __restrict__ o = out + (int64_t)row * k;
    const int32_t n = (int32_t)(L < (int64_t)k ? L : (int64_t)k);

    if ((int64_t)n == L) {   // every candidate is selected (also L == 0)
        for (int i = threadIdx.x; i < k; i += kTopkThreads) o[i] = i < n ? i : -1;
        return;
    }

    // ---- threshold by radix selection ----
    uint32_t need = (uint32_t)n;
    digit_histogram<0, 12>(s, L, 0u, hist);
    find_digit<12>(hist, need, scratch, res);
    uint32_t prefix = res[0];
    need -= res[1];
    uint32_t cnt = res[2];
    int depth = 12;
    if (need != cnt) {
        digit_histogram<12, 12>(s, L, prefix, hist);
        find_digit<12>(hist, need, scratch, res);
        prefix = (prefix << 12) | res[0];
        need -= res[1];
        cnt = res[2];
        depth = 24;
        if (need != cnt) {
            digit_histogram<24, 8>(s, L, prefix, hist);
            find_digit<8>(hist, need, scratch, res);
            prefix = (prefix << 8) | res[0];
            need -= res[1];
            depth = 32;
        }
    }
    const int hshift = 32 - depth;   // 20, 8 or 0

    // ---- ordered compaction ----
    uint32_t gt_run = 0, eq_run = 0;
    for (int64_t base = 0; base < L; base += kTopkChunk) {
        uint64_t gtm[kTopkUnroll], eqm[kTopkUnroll];
        uint32_t key[kTopkUnroll];
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
            key[u] = j < L ? score_key(s[j]) : 0u;
        }
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
            const uint32_t hi = key[u] >> hshift;
            gtm[u] = __ballot(j < L && hi > prefix);
            eqm[u] = __ballot(j < L && hi == prefix);
            if (lane == 0)
                tbl[u * kTopkWaves + wid] = ((uint32_t)__popcll(gtm[u]) << 16) | (uint32_t)__popcll(eqm[u]);
        }
        __syncthreads();
        const uint32_t v = threadIdx.x < kTopkUnroll * kTopkWaves ? tbl[threadIdx.x] : 0u;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan(v, scratch, &tot);   // (gt_before << 16) | eq_before
        if (threadIdx.x < kTopkUnroll * kTopkWaves) tbl[threadIdx.x] = ex;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
            const uint32_t pre = tbl[u * kTopkWaves + wid];
            const uint32_t gt_before = gt_run + (pre >> 16) + lanes_below(gtm[u]);
            const uint32_t eq_before = eq_run + (pre & 0xffffu) + lanes_below(eqm[u]);
            uint32_t dst = 0xffffffffu;
            if ((gtm[u] >> lane) & 1ull) dst = gt_before + (eq_before < need ? eq_before : need);
            else if (((eqm[u] >> lane) & 1ull) && eq_before < need) dst = gt_before + eq_before;
            if (dst < (uint32_t)n) o[dst] = (int32_t)j;   // always true; guards the buffer regardless
        }
        gt_run += tot >> 16;
        eq_run += tot & 0xffffu;
        __syncthreads();
    }
    for (int i = n + threadIdx.x; i < k; i += kTopkThreads) o[i] = -1;
}

hipError_t launch_topk(const float* scores, const int64_t* row_offsets, int64_t row_stride,
                       const int32_t* lengths, int32_t rows, int32_t k, int32_t* out, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(kTopkThreads), 0, stream, scores, row_offsets,
                       row_stride, lengths, k, out);
    return hipGetLastError();
}

// ---- A0: causal lengths ----
__global__ __launch_bounds__(256) void causal_lengths_kernel(int64_t first_pos, int32_t T, int32_t* lengths) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < T) {
        int64_t v = first_pos + t + 1;
        v = v < 0 ? 0 : (v > 2147483647LL ? 2147483647LL : v);
        lengths[t] = (int32_t)v;
    }
}

hipError_t launch_causal_lengths(int64_t first_pos, int32_t T, int32_t* lengths, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(causal_lengths_kernel, dim3((T + 255) / 256), dim3(256), 0, stream, first_pos, T, lengths);
    return hipGetLastError();
}

}  // namespace smla
