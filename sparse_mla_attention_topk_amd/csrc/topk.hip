// Stable top-k per row with canonical (ascending) output, gfx950.
//
// Method (deterministic sparse top-k of "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff
// RL", section "Deterministic sparse top-k"; length clamping and -1 padding of "[Bugfix] Make DSV4
// sparse MLA work end-to-end ...", "What is fixed"):
//   * every score becomes an order-preserving 32-bit key (score_key); the composite order is
//     (key descending, index ascending), so the n = min(k, L) selected candidates are exactly
//       { j : key_j > T } U { the first `need` indices j with key_j == T }
//     for the key T of the n-th candidate and need = n - #{key > T};
//   * pass 1 histograms the top 12 key bits in LDS and finds the boundary bucket;
//   * pass 2 marks every candidate above the bucket in an LDS bitmask (wave ballots) and gathers the
//     bucket's candidates into LDS, where T is resolved by radix selection on the remaining 20 bits
//     (or the whole bucket is taken when it holds exactly the missing count);
//   * the selection is emitted by an ordered scan of the bitmasks: block-wide prefix sums of the
//     per-word popcounts give each selected candidate its output slot, so the output is ascending
//     by construction (no sort) and the -1 tail is filled afterwards.
//   Rows longer than the LDS masks, or with a boundary bucket too large for LDS (massive ties),
//   take the general path: further radix passes over the row and an ordered compaction that
//   rereads it with wave ballots and block prefix sums.
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

// Keys of the chunk's candidates base + u*1024 + threadIdx.x (0 past the end).  Every load is
// issued unconditionally (index clamped into the row) and the values are pinned before use, so
// all loads of the chunk are in flight together instead of each waiting behind its own branch.
__device__ __forceinline__ void load_keys(const float* __restrict__ s, int64_t L, int64_t base, uint32_t* key) {
    float v[kTopkUnroll];
#pragma unroll
    for (int u = 0; u < kTopkUnroll; ++u) {
        const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
        v[u] = s[j < L ? j : L - 1];
    }
#pragma unroll
    for (int u = 0; u < kTopkUnroll; ++u) asm volatile("" ::"v"(v[u]));
#pragma unroll
    for (int u = 0; u < kTopkUnroll; ++u) {
        const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
        key[u] = j < L ? score_key(v[u]) : 0u;
    }
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
        load_keys(s, L, base, key);
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

// LDS capacities of the two-pass path.
constexpr int kMaskWords = 4096;     // candidate bitmasks cover rows of up to 131072 candidates
constexpr int kCandCap = 6144;       // boundary-bucket candidates resolved in LDS

// Block-wide exclusive scan of a 64-bit value (two 32-bit scans).
__device__ uint64_t block_exclusive_scan64(uint32_t a, uint32_t b, uint32_t* scratch, uint32_t* ta, uint32_t* tb) {
    const uint32_t ea = block_exclusive_scan(a, scratch, ta);
    const uint32_t eb = block_exclusive_scan(b, scratch, tb);
    return ((uint64_t)ea << 32) | eb;
}

// Ordered emission from two LDS bitmasks over [0, L): every `gt` candidate is selected, and the first
// `need` `eq` candidates in index order.  Output slot = #selected candidates with a smaller index.
__device__ void emit_from_masks(const uint32_t* gtw, const uint32_t* eqw, int64_t L, uint32_t need, int32_t n,
                                int32_t* __restrict__ o, uint32_t* scratch) {
    const int W = (int)((L + 31) >> 5);
    const int per = (W + kTopkThreads - 1) / kTopkThreads;
    const int w0 = threadIdx.x * per;
    const int w1 = min(W, w0 + per);
    uint32_t cg = 0, ce = 0;
    for (int w = w0; w < w1; ++w) {
        cg += __popc(gtw[w]);
        ce += __popc(eqw[w]);
    }
    uint32_t tg, te;
    const uint64_t ex = block_exclusive_scan64(cg, ce, scratch, &tg, &te);
    uint32_t gt_before = (uint32_t)(ex >> 32), eq_before = (uint32_t)ex;
    for (int w = w0; w < w1; ++w) {
        uint32_t mg = gtw[w], me = eqw[w];
        uint32_t both = mg | me;
        while (both) {
            const int b = __ffs(both) - 1;
            both &= both - 1;
            const int32_t j = (w << 5) + b;
            uint32_t dst = 0xffffffffu;
            if ((mg >> b) & 1u) {
                dst = gt_before + (eq_before < need ? eq_before : need);
                ++gt_before;
            } else {
                if (eq_before < need) dst = gt_before + eq_before;
                ++eq_before;
            }
            if (dst < (uint32_t)n) o[dst] = j;
        }
    }
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
    __shared__ uint32_t gtw[kMaskWords], eqw[kMaskWords];
    __shared__ uint32_t cand_key[kCandCap], cand_idx[kCandCap];
    __shared__ uint32_t ncand;

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

    // ---- pass 1: histogram of the top 12 key bits ----
    uint32_t need = (uint32_t)n;
    digit_histogram<0, 12>(s, L, 0u, hist);
    find_digit<12>(hist, need, scratch, res);
    uint32_t prefix = res[0];
    need -= res[1];
    uint32_t cnt = res[2];

    const bool masks_fit = L <= (int64_t)kMaskWords * 32;
    if (masks_fit && (need == cnt || cnt <= (uint32_t)kCandCap)) {
        // ---- pass 2: bitmask of candidates above the boundary bucket; the bucket itself is either
        // taken whole (eq mask) or gathered into LDS for an exact resolution ----
        const bool take_all = need == cnt;
        const int W = (int)((L + 31) >> 5);
        for (int w = threadIdx.x; w < W; w += kTopkThreads) { gtw[w] = 0u; eqw[w] = 0u; }
        if (threadIdx.x == 0) ncand = 0u;
        __syncthreads();
        for (int64_t base = 0; base < L; base += kTopkChunk) {
            uint32_t key[kTopkUnroll];
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) {
                const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
                key[u] = j < L ? score_key(s[j < L ? j : L - 1]) : 0u;   // unconditional load: all in flight
            }
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) {
                const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
                const uint32_t hi = key[u] >> 20;
                const bool ok = j < L;
                const uint64_t gm = __ballot(ok && hi > prefix);
                const bool in_bucket = ok && hi == prefix;
                if (take_all) {
                    const uint64_t em = __ballot(in_bucket);
                    if (lane == 0 && base + (int64_t)u * kTopkThreads + wid * kWave < L) {
                        const int w = (int)((base + (int64_t)u * kTopkThreads + wid * kWave) >> 5);
                        gtw[w] = (uint32_t)gm;
                        eqw[w] = (uint32_t)em;
                        if (w + 1 < W) { gtw[w + 1] = (uint32_t)(gm >> 32); eqw[w + 1] = (uint32_t)(em >> 32); }
                    }
                } else {
                    if (lane == 0 && base + (int64_t)u * kTopkThreads + wid * kWave < L) {
                        const int w = (int)((base + (int64_t)u * kTopkThreads + wid * kWave) >> 5);
                        gtw[w] = (uint32_t)gm;
                        if (w + 1 < W) gtw[w + 1] = (uint32_t)(gm >> 32);
                    }
                    if (in_bucket) {
                        const uint32_t slot = atomicAdd(&ncand, 1u);   // < cnt <= kCandCap (same data as pass 1)
                        if (slot < (uint32_t)kCandCap) {
                            cand_key[slot] = key[u];
                            cand_idx[slot] = (uint32_t)j;
                        }
                    }
                }
            }
        }
        __syncthreads();
        if (!take_all) {
            // ---- resolve the bucket in LDS: radix select on the remaining 20 key bits ----
            const uint32_t nc = ncand < (uint32_t)kCandCap ? ncand : (uint32_t)kCandCap;
            for (int i = threadIdx.x; i < (1 << 12); i += kTopkThreads) hist[i] = 0u;
            __syncthreads();
            for (uint32_t c = threadIdx.x; c < nc; c += kTopkThreads) atomicAdd(&hist[(cand_key[c] >> 8) & 0xfffu], 1u);
            __syncthreads();
            find_digit<12>(hist, need, scratch, res);
            uint32_t p2 = (prefix << 12) | res[0];
            need -= res[1];
            int shift = 8;
            if (need != res[2]) {
                for (int i = threadIdx.x; i < 256; i += kTopkThreads) hist[i] = 0u;
                __syncthreads();
                for (uint32_t c = threadIdx.x; c < nc; c += kTopkThreads)
                    if ((cand_key[c] >> 8) == p2) atomicAdd(&hist[cand_key[c] & 0xffu], 1u);
                __syncthreads();
                find_digit<8>(hist, need, scratch, res);
                p2 = (p2 << 8) | res[0];
                need -= res[1];
                shift = 0;
            }
            for (uint32_t c = threadIdx.x; c < nc; c += kTopkThreads) {
                const uint32_t hi = cand_key[c] >> shift;
                const uint32_t j = cand_idx[c];
                if (hi > p2) atomicOr(&gtw[j >> 5], 1u << (j & 31));
                else if (hi == p2) atomicOr(&eqw[j >> 5], 1u << (j & 31));
            }
            __syncthreads();
        }
        emit_from_masks(gtw, eqw, L, need, n, o, scratch);
        for (int i = n + threadIdx.x; i < k; i += kTopkThreads) o[i] = -1;
        return;
    }

    // ---- general path (rows longer than the LDS masks, or a huge boundary bucket): further radix
    // passes over the row, then an ordered compaction that rereads it ----
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
        load_keys(s, L, base, key);
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
