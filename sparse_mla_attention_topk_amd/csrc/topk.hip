// Stable top-k per row with canonical (ascending) output, gfx950.
//
// Method (deterministic sparse top-k of "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff
// RL", section "Deterministic sparse top-k"; length clamping and -1 padding of "[Bugfix] Make DSV4
// sparse MLA work end-to-end ...", section "Purpose", items "Negative indexer context lengths under
// MTP" and "Top-k kernels hardened against out-of-range lengths"):
//   * every score becomes an order-preserving 32-bit key (score_key); the composite order is
//     (key descending, index ascending), so the n = min(k, L) selected candidates are exactly
//       { j : key_j > T } U { the first `need` indices j with key_j == T }
//     for the key T of the n-th candidate and need = n - #{key > T};
//   * filtered path (select_topk): a threshold from a fixed sample of the row lets roughly 1.25 n
//     candidates through; they are listed in LDS in position order (counts, a block scan, appends),
//     and T is found on that short list by narrowing a key interval with LDS histograms
//     (resolve_list).  Rows of at most kCandCap candidates list all of them;
//   * general path (select_general), for rows the filter cannot serve (a threshold that lets too few
//     or too many through, massive ties): radix passes over the whole row find T, and an ordered
//     compaction rereads it with wave ballots and block prefix sums;
//   * either way a selected candidate's output slot is the number of selected candidates before it in
//     position order, so the output is ascending by construction (no sort), and the -1 tail is filled
//     afterwards;
//   * few long rows may split the filter pass over several workgroups per row (topk_filter_kernel),
//     whose position-ordered lists one workgroup per row then concatenates and resolves
//     (topk_select_kernel).
// One 1024-thread workgroup owns one row (or one chunk of it); every decision is made from the clamped
// length that all threads read, so the result is a pure function of the row (batch-invariant, no
// inter-workgroup synchronization of any kind).
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;   // 16
constexpr int kTopkUnroll = 16;                     // elements per thread per chunk
constexpr int64_t kTopkChunk = (int64_t)kTopkThreads * kTopkUnroll;

// Score source: a selection runs over positions j in [0, L) of a row; at(j) is the score, index(j)
// the index written to the output for it.
struct DirectScores {                 // a contiguous row
    const float* __restrict__ s;
    __device__ __forceinline__ float at(int64_t j) const { return s[j]; }
    __device__ __forceinline__ int32_t index(int64_t j) const { return (int32_t)j; }
};
// Workgroup barrier that orders LDS accesses only.  Threads of a selecting workgroup share data
// through LDS alone, so global loads still in flight (a row streaming into registers) need not be
// waited for here; __syncthreads would wait for them, its fence covering global memory too.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Number of set bits of a wave mask below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16 lanes, then the row
// broadcasts carry the running totals across rows (DPP, no LDS traffic).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return x;
}

// Exclusive prefix sum of v over the 1024 threads of the block, in thread order.
// `scratch` holds at least kTopkWaves words of LDS.  Ends with a barrier.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[wid] = x;
    lds_barrier();
    const uint32_t w = lane < kTopkWaves ? scratch[lane] : 0u;
    const uint32_t z = wave_inclusive_scan(w);       // every wave scans the 16 wave totals itself
    const uint32_t before = __shfl(z - w, wid);       // exclusive prefix of this wave's total
    *total = __shfl(z, kTopkWaves - 1);
    lds_barrier();
    return before + x - v;
}

// Keys of the chunk's candidates base + u*1024 + threadIdx.x (0 past the end).  Every load is
// issued unconditionally (index clamped into the row) and the values are pinned before use, so
// all loads of the chunk are in flight together instead of each waiting behind its own branch.
template <class Src>
__device__ __forceinline__ void load_keys(const Src& src, int64_t L, int64_t base, uint32_t* key) {
    float v[kTopkUnroll];
#pragma unroll
    for (int u = 0; u < kTopkUnroll; ++u) {
        const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
        v[u] = src.at(j < L ? j : L - 1);
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
template <int DEPTH, int BITS, class Src>
__device__ __forceinline__ void digit_histogram(const Src& src, int64_t L, uint32_t prefix, uint32_t* hist) {
    constexpr int kBins = 1 << BITS;
    constexpr int kShift = 32 - DEPTH - BITS;
    for (int i = threadIdx.x; i < kBins; i += kTopkThreads) hist[i] = 0u;
    lds_barrier();
    for (int64_t base = 0; base < L; base += kTopkChunk) {
        uint32_t key[kTopkUnroll];
        load_keys(src, L, base, key);
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
            bool match = j < L;
            if constexpr (DEPTH > 0) match = match && ((key[u] >> (32 - DEPTH)) == prefix);
            if (match) atomicAdd(&hist[(key[u] >> kShift) & (kBins - 1)], 1u);
        }
    }
    lds_barrier();
}

// Finds the digit d holding the need-th largest candidate: above = #candidates with a larger digit,
// above < need <= above + hist[d].  Results land in res[0..2] = {d, above, hist[d]}.
template <int BITS>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t need, uint32_t* scratch, uint32_t* res) {
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
    lds_barrier();
}

// LDS capacity of the filtered path.
constexpr int kCandCap = 12288;      // candidates passing the filter, resolved in LDS
constexpr uint32_t kSegCap = kCandCap / 16;   // one wave's segment of the list (one-pass streaming)
static_assert(kCandCap < (1 << 16), "the emission scan packs two list counts into 16 bits each");
constexpr int kSampleLog2 = 12;      // 4096 sampled candidates, 4 per thread

// The smallest value whose key has top-12 digit d (d >= 8): for every non-NaN v, v >= value <=>
// score_key(v) >= d << 20.  Digits below 8 hold only -inf and NaN keys and have no such value.
__device__ __forceinline__ float digit_floor_value(uint32_t d) {
    const uint32_t key = d << 20;
    return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

// Slot layout of the filtered path.  A row is processed in chunks of U * 1024 positions; in a chunk
// starting at `base`, wave w owns the U * 64 consecutive positions from base + w * U * 64, and lane l
// holds position base + w * U * 64 + u * 64 + l in slot u.  Listing candidates chunk by chunk, wave
// by wave, slot by slot and lane by lane therefore lists them in ascending position order.
// Rows of up to 65536 positions are one chunk of 64 slots held in registers (read once); longer
// rows stream in chunks of 16 slots and are read twice.
constexpr int kResidentU = 64;
constexpr int64_t kResident = (int64_t)kResidentU * kTopkThreads;   // 65536
constexpr int kStreamU = 16;
constexpr int32_t kStreamChunk = kStreamU * kTopkThreads;            // 16384
// one (chunk, wave) count per thread: rows of up to 64 chunks
constexpr int64_t kFilterMax = (int64_t)(kTopkThreads / kTopkWaves) * kStreamChunk;   // 1048576

// Index of the calling wave in its workgroup, as a scalar: branches on it stay uniform.
__device__ __forceinline__ int32_t wave_index() {
    return __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x / kWave));
}

// First position of the calling wave's slot u (uniform in the wave); lane l holds that plus l.
template <int U>
__device__ __forceinline__ int32_t slot_base(int32_t base, int u) {
    return base + wave_index() * (U * kWave) + u * kWave;
}
template <int U>
__device__ __forceinline__ int32_t slot_pos(int32_t base, int u) {
    return slot_base<U>(base, u) + (int32_t)(threadIdx.x & (kWave - 1));
}

// Loads the U slots of the chunk at `base`.  Positions at or beyond L hold NaN, which passes no
// threshold test.  Every load is issued before any wait, and the values become opaque register
// contents, so the compiler cannot re-load them at later uses.
template <int U, class Src>
__device__ __forceinline__ void load_slots(const Src& src, int32_t L, int32_t base, float* v) {
    const float qnan = __builtin_nanf("");
    // Positions from the vector thread index: the loads then issue one by one between per-lane
    // tests, which measured faster on MI355X than the same loads issued back to back (the whole
    // row of 256 KB in registers 1.5 us sooner).
    const int32_t p0 = base + (int32_t)(threadIdx.x / kWave) * (U * kWave) + (int32_t)(threadIdx.x & (kWave - 1));
#pragma unroll
    for (int g = 0; g < U; g += kTopkUnroll) {
        const bool live = p0 + g * kWave - (int32_t)(threadIdx.x & (kWave - 1)) < L;
#pragma unroll
        for (int u = g; u < g + kTopkUnroll; ++u) {
            const int32_t j = p0 + u * kWave;
            v[u] = live ? src.at(j < L ? j : L - 1) : qnan;
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" : "+v"(v[u]));
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (p0 + u * kWave >= L) v[u] = qnan;
}

// The loads of load_slots, issued through a buffer resource over the row's L scores without waiting
// for them: loads at or past the end return 0 and never touch memory, and the slot step sits in each
// load's offset field, so the loads need no address registers (the chunk workgroups of the split
// filter run two to a CU).
template <int U>
__device__ __forceinline__ void issue_slots_buffer(const DirectScores& src, int32_t L, int32_t base, float* v) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)src.s, (short)0, L * (int32_t)sizeof(float), 0x00020000);
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int g = 0; g < U; g += kTopkUnroll) {
        if (slot_base<U>(base, g) < L) {   // uniform
            const int32_t voff = slot_pos<U>(base, g) * (int32_t)sizeof(float);
#pragma unroll
            for (int u = g; u < g + kTopkUnroll; ++u)
                v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                     rs, voff + (u - g) * kWave * (int32_t)sizeof(float), 0, 0));
        } else {
#pragma unroll
            for (int u = g; u < g + kTopkUnroll; ++u) v[u] = qnan;
        }
    }
}

// Waits for the slots of issue_slots_buffer: the values become opaque register contents, and the lanes
// of a slot that straddles L get NaN (which passes no threshold test).
template <int U>
__device__ __forceinline__ void settle_slots_buffer(int32_t L, int32_t base, float* v) {
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" : "+v"(v[u]));
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (slot_base<U>(base, u) + kWave > L)   // uniform: only a slot that straddles L has lanes to fix
            v[u] = slot_pos<U>(base, u) < L ? v[u] : __builtin_nanf("");
}

// Issues every load of the U slots of the chunk at `base` through the row's buffer resource, with no
// branch: slots at or past L read 0 without touching memory (settle_slots_buffer makes them NaN).
// Because no path skips the loads, a later wait for these values can leave loads issued after them
// in flight, which lets a streaming loop keep the next chunk's loads going while it works on this one.
template <int U>
__device__ __forceinline__ void issue_chunk_buffer(const DirectScores& src, int32_t L, int32_t base, float* v) {
    static_assert(U * kWave * (int)sizeof(float) <= 4096, "slot steps must fit the load offset field");
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)src.s, (short)0, L * (int32_t)sizeof(float), 0x00020000);
    const int32_t voff = slot_pos<U>(base, 0) * (int32_t)sizeof(float);
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = __builtin_bit_cast(float,
                                  __builtin_amdgcn_raw_buffer_load_b32(rs, voff + u * kWave * (int32_t)sizeof(float), 0, 0));
}

// One-pass streaming of a long row: wave w takes the positions [w * span, (w + 1) * span) of the row
// (span a multiple of 1024), in steps of kStreamU slots of 64 positions; a step starting at position
// `pb` holds pb + u * 64 + lane in slot u.  Loads go through the row's buffer resource `rs` with no
// branch (positions at or past L read 0 without touching memory).
__device__ __forceinline__ void issue_stretch(__amdgpu_buffer_rsrc_t rs, int32_t pb, float* v) {
    const int32_t voff = (pb + (int32_t)(threadIdx.x & (kWave - 1))) * (int32_t)sizeof(float);
#pragma unroll
    for (int u = 0; u < kStreamU; ++u)
        v[u] = __builtin_bit_cast(float,
                                  __builtin_amdgcn_raw_buffer_load_b32(rs, voff + u * kWave * (int32_t)sizeof(float), 0, 0));
}
// Waits for a step's values; positions at or past L become NaN (only a slot that straddles L has
// lanes to fix, decided per wave).
__device__ __forceinline__ void settle_stretch(int32_t pb, int32_t L, float* v) {
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) asm volatile("" : "+v"(v[u]));
#pragma unroll
    for (int u = 0; u < kStreamU; ++u)
        if (pb + u * kWave + kWave > L)   // uniform
            v[u] = pb + u * kWave + (int32_t)(threadIdx.x & (kWave - 1)) < L ? v[u] : __builtin_nanf("");
}
// Appends a step's candidates with v >= tf to the LDS list from `pos` (uniform), in position order;
// entries at or beyond `limit` are counted but not written.  Returns the offset after the last one.
__device__ __forceinline__ uint32_t append_stretch(const float* v, int32_t pb, float tf, uint32_t pos,
                                                   uint32_t limit, uint32_t* cbits, uint32_t* cidx) {
    const uint32_t pos0 = (uint32_t)(pb + (int32_t)(threadIdx.x & (kWave - 1)));
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
        const bool pred = v[u] >= tf;
        const uint64_t m = __builtin_amdgcn_ballot_w64(pred);
        if (pred) {
            const uint32_t p = pos + lanes_below(m);
            if (p < limit) {
                cbits[p] = __float_as_uint(v[u]);
                cidx[p] = pos0 + (uint32_t)(u * kWave);
            }
        }
        pos += (uint32_t)__popcll(m);
    }
    return pos;
}

// Number of this wave's slots with v >= tf (uniform in the wave).
template <int U>
__device__ __forceinline__ uint32_t wave_count_ge(const float* v, int32_t L, int32_t base, float tf) {
    uint32_t c = 0;
#pragma unroll
    for (int g = 0; g < U; g += kTopkUnroll) {
        if (slot_base<U>(base, g) >= L) break;   // uniform
#pragma unroll
        for (int u = g; u < g + kTopkUnroll; ++u) c += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(v[u] >= tf));
    }
    return c;
}

// Appends this wave's slots with v >= tf (value bits, position) to the LDS list from offset `pos`
// (uniform in the wave), in slot-then-lane order.  With GUARD, slots at or beyond kCandCap are
// never written (the streaming path re-reads the row, so its counts are not taken on faith).
// `cbits` and `cidx` are 48 KB apart at the start of the workgroup's LDS, so both stores of an entry
// use one address register and the stores' offset fields.
template <int U, bool GUARD>
__device__ __forceinline__ void wave_append_ge(const float* v, int32_t L, int32_t base, float tf, uint32_t pos,
                                               uint32_t* cbits, uint32_t* cidx) {
    pos = __builtin_amdgcn_readfirstlane(pos);
    const int32_t wbase = slot_base<U>(base, 0);
    const uint32_t pos0 = (uint32_t)(wbase + (int32_t)(threadIdx.x & (kWave - 1)));   // position in slot 0
#pragma unroll
    for (int g = 0; g < U; g += kTopkUnroll) {
        if (wbase + g * kWave >= L) break;   // uniform
#pragma unroll
        for (int u = g; u < g + kTopkUnroll; ++u) {
            const bool pred = v[u] >= tf;
            const uint64_t m = __builtin_amdgcn_ballot_w64(pred);
            if (pred) {
                const uint32_t p = pos + lanes_below(m);
                if (!GUARD || p < (uint32_t)kCandCap) {
                    cbits[p] = __float_as_uint(v[u]);
                    cidx[p] = pos0 + (uint32_t)(u * kWave);
                }
            }
            pos += (uint32_t)__popcll(m);
        }
    }
}

// LDS of one selecting workgroup.
constexpr uint32_t kSmallBin = 128;  // a boundary bin of at most this many keys is resolved by ranking

struct TopkShared {
    uint32_t cand_key[kCandCap], cand_idx[kCandCap];   // first: both within the LDS offset field's reach
    uint32_t hist[1 << 12];
    uint32_t scratch[kTopkWaves + 2];
    uint32_t res[3];
    uint32_t krange[6];                      // min / max key of the list, then of the interval (2 rounds)
    uint32_t first[2];                       // first digit from the sample: base key, shift
    uint32_t tbl[kTopkUnroll * kTopkWaves];
    uint32_t wcnt[kTopkThreads];             // per-wave candidate counts, then list offsets
    uint32_t mem[kSmallBin];                 // keys of a small boundary bin
    uint32_t mem_n;
};

// Minimum / maximum over the 64 lanes of a wave (every lane gets the result): DPP exchanges within
// each row of 16 lanes (swap neighbours, swap pairs, mirror halves of 8, mirror the row), then the
// cross-row swaps of lanes l <-> l^32 and l <-> l^16; VALU only, no LDS traffic.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
    auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = op(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return op(b[0], b[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_reduce_u32<false>(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_reduce_u32<true>(v); }

// Shift s such that span >> s < 4096: a 12-bit digit (key - base) >> s spreads keys of that span
// over the histogram's bins.
__device__ __forceinline__ int fitted_shift(uint32_t span) {
    const int s = span == 0u ? 0 : 32 - (int)__builtin_clz(span) - 12;
    return s < 0 ? 0 : s;
}

// Filter threshold from the four sampled values per thread: a value tf such that, judging by the
// sample, about 1.25 n + 4 sigma candidates of the row have v >= tf.  Returns false when the sample
// offers none.  Every workgroup that samples the same row at the same positions derives the same tf.
// With `first`, also the first digit for resolve_list: {key of tf, shift fitted to the span from
// that key to the largest sampled key} in first[0..1] (LDS words, readable after the next barrier).
__device__ __forceinline__ bool sample_threshold(const float* sv, int64_t L, int32_t n, uint32_t* hist,
                                                 uint32_t* scratch, uint32_t* res, float* tf,
                                                 uint32_t* first = nullptr) {
    for (int i = threadIdx.x; i < (1 << 12); i += kTopkThreads) hist[i] = 0u;
    if (first && threadIdx.x == 0) first[1] = 0u;
    lds_barrier();
    uint32_t mx = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t key = score_key(sv[i]);
        atomicAdd(&hist[key >> 20], 1u);
        mx = max(mx, key);
    }
    if (first) {
        mx = wave_max_u32(mx);
        if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(&first[1], mx);
    }
    lds_barrier();
    const uint32_t smax = first ? first[1] : 0u;     // read before find_digit's barriers
    const float expect = (float)n * (float)(1 << kSampleLog2) / (float)L;
    const uint32_t want = (uint32_t)(1.25f * expect + 4.f * sqrtf(expect) + 8.f);
    if (want >= (uint32_t)(1 << kSampleLog2)) return false;
    find_digit<12>(hist, want, scratch, res);
    if (res[0] < 8u) return false;
    *tf = digit_floor_value(res[0]);
    if (first && threadIdx.x == 0) {                 // read only after a later barrier
        const uint32_t tkey = res[0] << 20;          // every listed key is at least this
        first[0] = tkey;
        first[1] = (uint32_t)fitted_shift(smax - tkey);   // smax >= tkey: the want-th sample is listed
    }
    return true;
}

// Sampled positions: 128 blocks of 32 consecutive candidates (one cache line each) spread evenly over
// the row; thread t takes 4 of them.  Whole lines keep the sample's memory traffic at 16 KB per row.
template <class Src>
__device__ __forceinline__ void load_sample(const Src& src, int64_t L, float* sv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = (int)threadIdx.x * 4 + i;                      // sample index 0 .. 4095
        const int64_t b = ((int64_t)(q >> 5) * L) >> 7;               // start of block q / 32
        const int64_t j = (b & ~(int64_t)31) + (q & 31);
        sv[i] = src.at(j < L ? j : L - 1);
    }
}

// Rows that go through a candidate filter (decided from L and k alone).
__device__ __forceinline__ bool filter_eligible(int64_t L, int32_t n) {
    return L > kCandCap && L <= kFilterMax && n <= kCandCap;
}

// Clears what resolve_list counts into; a barrier must follow before resolve_list runs.
__device__ __forceinline__ void resolve_prepare(TopkShared& sm) {
    for (int i = threadIdx.x; i < (1 << 12); i += kTopkThreads) sm.hist[i] = 0u;
    if (threadIdx.x == 0) {
        sm.krange[0] = sm.krange[2] = sm.krange[4] = 0xffffffffu;
        sm.krange[1] = sm.krange[3] = sm.krange[5] = 0u;
        sm.mem_n = 0u;
    }
}

// Finishes a selection from the candidate list sm.cand_key (value bits) / sm.cand_idx (positions),
// entries [0, total), which holds every selected candidate, in ascending position order, with
// n <= total <= kCandCap.  resolve_prepare and a barrier must precede it.
//
// The n-th key T is narrowed down as an interval [lo, hi] of keys holding it, with `need` = how many
// of the interval's keys are selected (all keys above hi are).  The first digit is
// min((key - base) >> s, 4095): base and s come from `first` (the sample's threshold key, a lower
// bound of every listed key, and a shift fitted to the sampled span; keys above the sample's
// largest land in the top bin) or, without it, from the list's own key range.  Fitted digits spread
// the keys over the 4096 bins instead of piling them into a few LDS counters.  While the interval
// holds more keys than are needed, it is settled directly when its keys are all equal or number at
// most kSmallBin (ranking), else narrowed by a digit fitted to its keys' own range.  A selected
// candidate's output slot is the number of selected candidates before it in the list.
//
// With `seg`, the list is kTopkWaves segments instead of one run: segment w starts at w * kSegCap and
// holds seg[w] entries, and wave w walks segment w (the segments in order are position order).
template <class Src>
__device__ __forceinline__ void resolve_list(const Src& src, uint32_t total, int32_t n, int32_t k,
                                             int32_t* __restrict__ o, TopkShared& sm,
                                             const uint32_t* first = nullptr, const uint32_t* seg = nullptr) {
    uint32_t* hist = sm.hist;
    uint32_t* scratch = sm.scratch;
    uint32_t* res = sm.res;
    uint32_t* cand_key = sm.cand_key;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t c0, c1;
    if (seg) {
        const uint32_t w = (uint32_t)wave_index(), cw = seg[w];
        const uint32_t per = (cw + kWave - 1) / kWave;                 // <= kSegCap / 64 = 12
        const uint32_t lo = (uint32_t)lane * per < cw ? (uint32_t)lane * per : cw;
        c0 = w * kSegCap + lo;
        c1 = w * kSegCap + (lo + per < cw ? lo + per : cw);
    } else {
        const uint32_t per = (total + kTopkThreads - 1) / kTopkThreads;   // <= 12
        c0 = threadIdx.x * per;
        c1 = c0 + per < total ? c0 + per : total;
    }
    uint32_t base;
    int s;
    if (first) {
        base = first[0];
        s = (int)first[1];
        for (uint32_t c = c0; c < c1; ++c) {
            const uint32_t key = score_key(__uint_as_float(cand_key[c]));
            cand_key[c] = key;
            const uint32_t d = (key - base) >> s;
            atomicAdd(&hist[d < 4095u ? d : 4095u], 1u);
        }
    } else {
        uint32_t lo = 0xffffffffu, hi = 0u;
        for (uint32_t c = c0; c < c1; ++c) {
            const uint32_t key = score_key(__uint_as_float(cand_key[c]));
            cand_key[c] = key;
            lo = min(lo, key);
            hi = max(hi, key);
        }
        lo = wave_min_u32(lo);
        hi = wave_max_u32(hi);
        if (lane == 0) {
            atomicMin(&sm.krange[0], lo);
            atomicMax(&sm.krange[1], hi);
        }
        lds_barrier();
        base = sm.krange[0];
        s = fitted_shift(sm.krange[1] - base);       // digits lie in [0, 4095]
        for (uint32_t c = c0; c < c1; ++c) atomicAdd(&hist[(cand_key[c] - base) >> s], 1u);
    }
    lds_barrier();
    find_digit<12>(hist, (uint32_t)n, scratch, res);
    uint32_t need = (uint32_t)n - res[1];
    uint32_t cnt = res[2];
    uint32_t lo = base + (res[0] << s);
    uint32_t hi = res[0] == 4095u ? 0xffffffffu
                                  : (uint32_t)min((uint64_t)base + ((uint64_t)(res[0] + 1u) << s) - 1u,
                                                  (uint64_t)0xffffffffu);
    for (int round = 0; need != cnt; ++round) {      // uniform; each round shrinks the interval
        // the interval's own key range (and, when few, its keys); krange words of this round
        uint32_t* kr = sm.krange + 2 + 2 * (round & 1);
        uint32_t blo = 0xffffffffu, bhi = 0u;
        for (uint32_t c = c0; c < c1; ++c) {
            const uint32_t key = cand_key[c];
            if (key >= lo && key <= hi) {
                blo = min(blo, key);
                bhi = max(bhi, key);
                if (cnt <= kSmallBin) sm.mem[atomicAdd(&sm.mem_n, 1u)] = key;
            }
        }
        for (int i = threadIdx.x; i < (1 << 12); i += kTopkThreads) hist[i] = 0u;
        if (threadIdx.x == 0) {                       // the other round's words, for the next round
            sm.krange[2 + 2 * ((round + 1) & 1)] = 0xffffffffu;
            sm.krange[3 + 2 * ((round + 1) & 1)] = 0u;
        }
        blo = wave_min_u32(blo);
        bhi = wave_max_u32(bhi);
        if (lane == 0) {
            atomicMin(&kr[0], blo);
            atomicMax(&kr[1], bhi);
        }
        lds_barrier();
        blo = kr[0];
        bhi = kr[1];
        if (blo == bhi) {                            // every key of the interval is equal: T
            lo = hi = blo;
            break;
        }
        if (cnt <= kSmallBin) {                      // rank the interval's keys: the need-th largest is T
            if (threadIdx.x < cnt) {
                const uint32_t my = sm.mem[threadIdx.x];
                uint32_t gt = 0, eq = 0;
                for (uint32_t j = 0; j < cnt; ++j) {
                    const uint32_t v = sm.mem[j];
                    gt += v > my ? 1u : 0u;
                    eq += v == my ? 1u : 0u;
                }
                if (gt < need && need <= gt + eq) {  // every thread holding T writes the same values
                    res[0] = my;
                    res[1] = gt;
                }
            }
            lds_barrier();
            lo = hi = res[0];
            need -= res[1];
            break;
        }
        const int s2 = fitted_shift(bhi - blo);
        for (uint32_t c = c0; c < c1; ++c) {
            const uint32_t key = cand_key[c];
            if (key >= blo && key <= bhi) atomicAdd(&hist[(key - blo) >> s2], 1u);
        }
        lds_barrier();
        find_digit<12>(hist, need, scratch, res);
        need -= res[1];
        cnt = res[2];
        lo = blo + (res[0] << s2);
        hi = (uint32_t)min((uint64_t)blo + ((uint64_t)(res[0] + 1u) << s2) - 1u, (uint64_t)bhi);
    }
    // ---- emission: selected are the keys above hi and the first `need` (in list, i.e. position,
    // order) of those in [lo, hi]; a selected candidate's output slot is the number of selected
    // candidates before it in the list ----
    uint32_t ng = 0, ne = 0;
    for (uint32_t c = c0; c < c1; ++c) {
        const uint32_t key = cand_key[c];
        ng += key > hi ? 1u : 0u;
        ne += key >= lo && key <= hi ? 1u : 0u;
    }
    // one scan of both counts, packed (list totals stay below 2^16: kCandCap = 12288)
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan((ng << 16) | ne, scratch, &tot);
    uint32_t gb = ex >> 16, eb = ex & 0xffffu;
    uint32_t* cand_idx = sm.cand_idx;
    for (uint32_t c = c0; c < c1; ++c) {
        const uint32_t key = cand_key[c];
        uint32_t dst = 0xffffffffu;
        if (key > hi) {
            dst = gb + (eb < need ? eb : need);
            ++gb;
        } else if (key >= lo) {
            if (eb < need) dst = gb + eb;
            ++eb;
        }
        if (dst < (uint32_t)n) o[dst] = src.index((int64_t)cand_idx[c]);
    }
    for (int i = n + threadIdx.x; i < k; i += kTopkThreads) o[i] = -1;
}

// General selection, any row: radix passes over the row, then an ordered compaction that rereads it.
template <class Src>
__device__ __forceinline__ void select_general(const Src& src, int64_t L, int32_t n, int32_t k,
                                               int32_t* __restrict__ o, TopkShared& sm) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    uint32_t* hist = sm.hist;
    uint32_t* scratch = sm.scratch;
    uint32_t* res = sm.res;
    uint32_t* tbl = sm.tbl;
    uint32_t need = (uint32_t)n;
    digit_histogram<0, 12>(src, L, 0u, hist);
    find_digit<12>(hist, need, scratch, res);
    uint32_t prefix = res[0];
    need -= res[1];
    uint32_t cnt = res[2];
    int depth = 12;
    if (need != cnt) {
        digit_histogram<12, 12>(src, L, prefix, hist);
        find_digit<12>(hist, need, scratch, res);
        prefix = (prefix << 12) | res[0];
        need -= res[1];
        cnt = res[2];
        depth = 24;
        if (need != cnt) {
            digit_histogram<24, 8>(src, L, prefix, hist);
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
        load_keys(src, L, base, key);
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
            const uint32_t hi = key[u] >> hshift;
            gtm[u] = __ballot(j < L && hi > prefix);
            eqm[u] = __ballot(j < L && hi == prefix);
            if (lane == 0)
                tbl[u * kTopkWaves + wid] = ((uint32_t)__popcll(gtm[u]) << 16) | (uint32_t)__popcll(eqm[u]);
        }
        lds_barrier();
        const uint32_t v = threadIdx.x < kTopkUnroll * kTopkWaves ? tbl[threadIdx.x] : 0u;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan(v, scratch, &tot);   // (gt_before << 16) | eq_before
        if (threadIdx.x < kTopkUnroll * kTopkWaves) tbl[threadIdx.x] = ex;
        lds_barrier();
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kTopkThreads + threadIdx.x;
            const uint32_t pre = tbl[u * kTopkWaves + wid];
            const uint32_t gt_before = gt_run + (pre >> 16) + lanes_below(gtm[u]);
            const uint32_t eq_before = eq_run + (pre & 0xffffu) + lanes_below(eqm[u]);
            uint32_t dst = 0xffffffffu;
            if ((gtm[u] >> lane) & 1ull) dst = gt_before + (eq_before < need ? eq_before : need);
            else if (((eqm[u] >> lane) & 1ull) && eq_before < need) dst = gt_before + eq_before;
            if (dst < (uint32_t)n) o[dst] = src.index(j);   // always true; guards the buffer regardless
        }
        gt_run += tot >> 16;
        eq_run += tot & 0xffffu;
        lds_barrier();
    }
    for (int i = n + threadIdx.x; i < k; i += kTopkThreads) o[i] = -1;
}

// Selects the min(k, L) best positions of `src` and writes their indices (src.index) to o[0 .. n),
// ascending, then -1 to o[n .. k), in one workgroup.
//
// Filtered path: a threshold value tf is taken from a fixed sample of the row such that roughly
// 1.25 n candidates satisfy v >= tf, and the row is counted against it.  If at least n and at most
// kCandCap candidates pass, every selected candidate is among them (a candidate below tf, or NaN,
// is preceded by all those at or above tf), so the selection is finished on that short list.  The
// sample only decides how fast the row goes; if the count check fails the row takes the general
// path, with the same result.  Rows of at most kCandCap candidates list all of them.
// LONG: rows may be longer than kResident (the streaming forms are compiled in); without it every row
// is at most kResident long and the kernel holds the registers-resident form alone, whose register
// allocation the streaming code would otherwise crowd.
template <bool LONG, class Src>
__device__ __forceinline__ void select_topk(const Src& src, int64_t L, int32_t k, int32_t* __restrict__ o,
                                            TopkShared& sm) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int32_t n = (int32_t)(L < (int64_t)k ? L : (int64_t)k);

    if ((int64_t)n == L) {   // every candidate is selected (also L == 0)
        for (int i = threadIdx.x; i < k; i += kTopkThreads) o[i] = i < n ? src.index(i) : -1;
        return;
    }
    if (L <= kCandCap) {
        const int32_t L32 = (int32_t)L;
        float v[kResidentU];
        load_slots<kResidentU>(src, L32, 0, v);
#pragma unroll
        for (int u = 0; u < kResidentU; ++u) {
            const int32_t j = slot_pos<kResidentU>(0, u);
            if (j < L32) {
                sm.cand_key[j] = __float_as_uint(v[u]);
                sm.cand_idx[j] = (uint32_t)j;
            }
        }
        resolve_prepare(sm);
        lds_barrier();
        resolve_list(src, (uint32_t)L32, n, k, o, sm);
        return;
    }
    if (filter_eligible(L, n)) {   // uniform
        const int32_t L32 = (int32_t)L;
        const bool resident = !LONG || L <= kResident;
        float v[kResidentU];
        float sv[4];
        load_sample(src, L, sv);
        if (resident) load_slots<kResidentU>(src, L32, 0, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(sv[i]));
        float tf = 0.f;
        if (sample_threshold(sv, L, n, sm.hist, sm.scratch, sm.res, &tf, sm.first)) {
            const int nch = resident ? 1 : (L32 + kStreamChunk - 1) / kStreamChunk;
            resolve_prepare(sm);   // ordered before resolve_list by the barriers below
            if (resident) {
                const uint32_t c = wave_count_ge<kResidentU>(v, L32, 0, tf);
                if (lane == 0) sm.wcnt[wid] = c;
            } else {
                // One pass: each wave streams its own stretch of the row (double-buffered: the next
                // step's loads are in flight while this one is appended) into its own list segment;
                // the segments in wave order are position order.  A stretch with more candidates than
                // its segment holds (candidates crowded into few positions) sends the row to the
                // two-pass form below, which lists it as one run.
                const int32_t span = ((L32 + kTopkThreads * kStreamU - 1) / (kTopkThreads * kStreamU)) *
                                     (kWave * kStreamU);
                const int32_t ws = wave_index() * span;
                const int32_t we = min(ws + span, L32);
                const int steps = we > ws ? (we - ws + kWave * kStreamU - 1) / (kWave * kStreamU) : 0;   // uniform
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)src.s, (short)0, L32 * (int32_t)sizeof(float), 0x00020000);
                const uint32_t s0 = (uint32_t)wave_index() * kSegCap;
                uint32_t pos = s0;
                float sa[kStreamU], sb[kStreamU];
                issue_stretch(rs, ws, sa);
                for (int it = 0; it < steps; it += 2) {   // uniform; stops at the stretch's end, no barrier
                    const int32_t p0 = ws + it * kWave * kStreamU, p1 = p0 + kWave * kStreamU;
                    issue_stretch(rs, p1, sb);
                    settle_stretch(p0, L32, sa);
                    pos = append_stretch(sa, p0, tf, pos, s0 + kSegCap, sm.cand_key, sm.cand_idx);
                    issue_stretch(rs, p1 + kWave * kStreamU, sa);
                    settle_stretch(p1, L32, sb);
                    if (it + 1 < steps)   // uniform
                        pos = append_stretch(sb, p1, tf, pos, s0 + kSegCap, sm.cand_key, sm.cand_idx);
                }
                if (lane == 0) sm.wcnt[wid] = pos - s0;
                lds_barrier();
                uint32_t total1 = 0;
                bool fits = true;
#pragma unroll
                for (int w = 0; w < kTopkWaves; ++w) {
                    total1 += sm.wcnt[w];
                    fits = fits && sm.wcnt[w] <= kSegCap;
                }
                if (fits) {   // uniform
                    if (total1 >= (uint32_t)n) {
                        resolve_list(src, total1, n, k, o, sm, sm.first, sm.wcnt);
                        return;
                    }
                    lds_barrier();
                    select_general(src, L, n, k, o, sm);   // too few candidates passed the sample's threshold
                    return;
                }
                lds_barrier();   // every wave has read the counts before the two-pass form rewrites them
                // Chunks in pairs, double-buffered: the next chunk's loads are in flight while this one
                // is counted.  The loop issues up to two chunks past the row, which read nothing.
                float ca[kStreamU], cb[kStreamU];
                issue_chunk_buffer<kStreamU>(src, L32, 0, ca);
                for (int ch = 0; ch < nch; ch += 2) {   // uniform
                    const int32_t b0 = ch * kStreamChunk, b1 = b0 + kStreamChunk;
                    issue_chunk_buffer<kStreamU>(src, L32, b1, cb);
                    settle_slots_buffer<kStreamU>(L32, b0, ca);
                    const uint32_t c0 = wave_count_ge<kStreamU>(ca, L32, b0, tf);
                    if (lane == 0) sm.wcnt[ch * kTopkWaves + wid] = c0;
                    issue_chunk_buffer<kStreamU>(src, L32, b1 + kStreamChunk, ca);
                    settle_slots_buffer<kStreamU>(L32, b1, cb);
                    const uint32_t c1 = wave_count_ge<kStreamU>(cb, L32, b1, tf);
                    if (lane == 0 && ch + 1 < nch) sm.wcnt[(ch + 1) * kTopkWaves + wid] = c1;
                }
            }
            lds_barrier();
            uint32_t total;
            const uint32_t mine = (int)threadIdx.x < nch * kTopkWaves ? sm.wcnt[threadIdx.x] : 0u;
            const uint32_t before = block_exclusive_scan(mine, sm.scratch, &total);
            if ((int)threadIdx.x < nch * kTopkWaves) sm.wcnt[threadIdx.x] = before;
            lds_barrier();
            if (total >= (uint32_t)n && total <= (uint32_t)kCandCap) {   // uniform
                if (resident) {
                    wave_append_ge<kResidentU, false>(v, L32, 0, tf, sm.wcnt[wid], sm.cand_key, sm.cand_idx);
                } else {   // the same double-buffered pairs of chunks as the count
                    float ca[kStreamU], cb[kStreamU];
                    issue_chunk_buffer<kStreamU>(src, L32, 0, ca);
                    for (int ch = 0; ch < nch; ch += 2) {   // uniform
                        const int32_t b0 = ch * kStreamChunk, b1 = b0 + kStreamChunk;
                        issue_chunk_buffer<kStreamU>(src, L32, b1, cb);
                        settle_slots_buffer<kStreamU>(L32, b0, ca);
                        wave_append_ge<kStreamU, true>(ca, L32, b0, tf, sm.wcnt[ch * kTopkWaves + wid], sm.cand_key,
                                                       sm.cand_idx);
                        issue_chunk_buffer<kStreamU>(src, L32, b1 + kStreamChunk, ca);
                        settle_slots_buffer<kStreamU>(L32, b1, cb);
                        if (ch + 1 < nch)   // uniform
                            wave_append_ge<kStreamU, true>(cb, L32, b1, tf, sm.wcnt[(ch + 1) * kTopkWaves + wid],
                                                           sm.cand_key, sm.cand_idx);
                    }
                }
                lds_barrier();
                resolve_list(src, total, n, k, o, sm, sm.first);
                return;
            }
        }
        lds_barrier();
    }
    select_general(src, L, n, k, o, sm);
}

__device__ __forceinline__ int64_t clamped_length(const int32_t* lengths, int row, int64_t row_stride) {
    const int64_t len = lengths ? (int64_t)lengths[row] : row_stride;
    return len < 0 ? 0 : (len > row_stride ? row_stride : len);   // clamp before any decision
}

// One workgroup per row (LONG: see select_topk).
template <bool LONG>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(const float* __restrict__ scores,
                                                                 const int64_t* __restrict__ row_offsets,
                                                                 int64_t row_stride,
                                                                 const int32_t* __restrict__ lengths,
                                                                 int32_t k, int32_t* __restrict__ out) {
    __shared__ TopkShared sm;
    const int row = blockIdx.x;
    const int64_t L = clamped_length(lengths, row, row_stride);
    const int64_t off = row_offsets ? row_offsets[row] : (int64_t)row * row_stride;
    select_topk<LONG>(DirectScores{scores + off}, L, k, out + (int64_t)row * k, sm);
}

// ---- few long rows: the filter pass split over the row's chunks of kFilterChunk positions ----
// Per row, the workspace holds kSplitHeader bytes of chunk counts, then for each chunk a list of up
// to kCandCap (value bits, position) pairs.  Every chunk workgroup derives the same threshold from
// the same sample of the row, and lists its candidates in position order; the select kernel
// concatenates the lists in chunk order, which is position order, and finishes the row exactly as
// the one-workgroup filtered path does.  Rows whose filter fails (a chunk reports kFilterFailed, or
// the total is out of range) are selected by the general path in the select kernel.
constexpr size_t kSplitHeader = 256;
constexpr int kFilterU = 32;                                         // slots per thread of a chunk workgroup
constexpr int32_t kFilterChunk = kFilterU * kTopkThreads;            // 32768 candidates per chunk
constexpr int kMaxSplitChunks = 16;                                  // rows of up to 524288 candidates
constexpr int64_t kMinSplitCandidates = 7 * kStreamChunk + 1;        // rows longer than 114688
constexpr uint32_t kFilterFailed = 0xffffffffu;

__host__ __device__ __forceinline__ size_t split_row_bytes(int nch) {
    return kSplitHeader + (size_t)nch * kCandCap * sizeof(uint2);
}

// Appends this wave's slots with v >= tf to a chunk list in global memory (buffer resource lr), from
// entry `pos` on, in slot-then-lane (position) order.
template <int U>
__device__ __forceinline__ void filter_append(const float* v, int32_t L, int32_t base, float tf, uint32_t pos,
                                              __amdgpu_buffer_rsrc_t lr) {
    pos = __builtin_amdgcn_readfirstlane(pos);
    const int32_t wbase = slot_base<U>(base, 0);
    const uint32_t pos0 = (uint32_t)(wbase + (int32_t)(threadIdx.x & (kWave - 1)));
#pragma unroll
    for (int g = 0; g < U; g += kTopkUnroll) {
        if (wbase + g * kWave >= L) break;   // uniform
#pragma unroll
        for (int u = g; u < g + kTopkUnroll; ++u) {
            const bool pred = v[u] >= tf;
            const uint64_t m = __builtin_amdgcn_ballot_w64(pred);
            if (pred) {
                const uint32_t p = pos + lanes_below(m);   // below the chunk's total, at most kCandCap
                // two 32-bit stores: a 64-bit one would keep every value in the low half of a register pair
                const int32_t off = (int32_t)(p * sizeof(uint2));
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[u]), lr, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(pos0 + (uint32_t)(u * kWave), lr, off + 4, 0, 0);
            }
            pos += (uint32_t)__popcll(m);
        }
    }
}

// At 42 registers per lane two chunk workgroups fit on a CU, so a launch of up to 512 of them runs in
// one round.
__global__ __launch_bounds__(kTopkThreads) void topk_filter_kernel(const float* __restrict__ scores,
                                                                   const int64_t* __restrict__ row_offsets,
                                                                   int64_t row_stride,
                                                                   const int32_t* __restrict__ lengths, int32_t k,
                                                                   int32_t nch, unsigned char* __restrict__ ws) {
    __shared__ uint32_t hist[1 << 12];
    __shared__ uint32_t scratch[kTopkWaves + 2];
    __shared__ uint32_t res[3];
    __shared__ uint32_t wcnt[2 * kTopkWaves];   // per (half, wave) counts, then list offsets
    const int row = blockIdx.x / nch, c = blockIdx.x % nch;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int64_t L = clamped_length(lengths, row, row_stride);
    const int32_t n = (int32_t)(L < (int64_t)k ? L : (int64_t)k);
    if ((int64_t)n == L || !filter_eligible(L, n)) return;   // uniform; the select kernel takes the row whole
    unsigned char* rws = ws + (size_t)row * split_row_bytes(nch);
    uint32_t* counts = (uint32_t*)rws;
    uint2* list = (uint2*)(rws + kSplitHeader) + (size_t)c * kCandCap;
    const int32_t L32 = (int32_t)L;
    const int32_t base = c * kFilterChunk;
    if (base >= L32) {
        if (threadIdx.x == 0) counts[c] = 0u;
        return;
    }
    const DirectScores src{scores + (row_offsets ? row_offsets[row] : (int64_t)row * row_stride)};
    // The chunk is two halves of kStreamChunk positions (the streaming layout, one after the other).
    // The first half's loads go out before the sample is evaluated and land meanwhile; the second
    // half's after it, so the two halves' values and the threshold's working registers are never all
    // live together.
    const int32_t base1 = base + kStreamChunk;
    float sv[4], va[kStreamU], vb[kStreamU];
    load_sample(src, L, sv);
    issue_slots_buffer<kStreamU>(src, L32, base, va);
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(sv[i]));
    float tf = 0.f;
    if (!sample_threshold(sv, L, n, hist, scratch, res, &tf)) {
        if (threadIdx.x == 0) counts[c] = kFilterFailed;
        return;
    }
    issue_slots_buffer<kStreamU>(src, L32, base1, vb);
    settle_slots_buffer<kStreamU>(L32, base, va);
    const uint32_t ca = wave_count_ge<kStreamU>(va, L32, base, tf);
    settle_slots_buffer<kStreamU>(L32, base1, vb);
    const uint32_t cb = wave_count_ge<kStreamU>(vb, L32, base1, tf);
    if (lane == 0) {
        wcnt[wid] = ca;
        wcnt[kTopkWaves + wid] = cb;
    }
    lds_barrier();
    uint32_t total;
    const uint32_t before =
        block_exclusive_scan(threadIdx.x < 2 * kTopkWaves ? wcnt[threadIdx.x] : 0u, scratch, &total);
    if (threadIdx.x < 2 * kTopkWaves) wcnt[threadIdx.x] = before;
    lds_barrier();
    if (threadIdx.x == 0) counts[c] = total;
    if (total > (uint32_t)kCandCap) return;   // uniform; the row's total is then out of range too
    // The chunk's list through a buffer resource: each store's address is one 32-bit offset.
    const __amdgpu_buffer_rsrc_t lr =
        __builtin_amdgcn_make_buffer_rsrc((void*)list, (short)0, (int32_t)(kCandCap * sizeof(uint2)), 0x00020000);
    filter_append<kStreamU>(va, L32, base, tf, wcnt[wid], lr);
    filter_append<kStreamU>(vb, L32, base1, tf, wcnt[kTopkWaves + wid], lr);
}

__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(const float* __restrict__ scores,
                                                                   const int64_t* __restrict__ row_offsets,
                                                                   int64_t row_stride,
                                                                   const int32_t* __restrict__ lengths, int32_t k,
                                                                   int32_t nch, const unsigned char* __restrict__ ws,
                                                                   int32_t* __restrict__ out) {
    __shared__ TopkShared sm;
    const int row = blockIdx.x;
    const int64_t L = clamped_length(lengths, row, row_stride);
    const int32_t n = (int32_t)(L < (int64_t)k ? L : (int64_t)k);
    const DirectScores src{scores + (row_offsets ? row_offsets[row] : (int64_t)row * row_stride)};
    int32_t* o = out + (int64_t)row * k;
    if ((int64_t)n < L && filter_eligible(L, n)) {   // uniform
        const unsigned char* rws = ws + (size_t)row * split_row_bytes(nch);
        const uint32_t* counts = (const uint32_t*)rws;
        const uint2* lists = (const uint2*)(rws + kSplitHeader);
        const int used = (int)((L + kFilterChunk - 1) / kFilterChunk);   // chunks the filter kernel ran
        // Entry i of every chunk's list is loaded by thread i (i < 1024) together with the counts, one
        // round trip for both: every chunk of the row has its list region (entries past a chunk's count
        // are left over from earlier calls and are dropped below).
        uint2 v0[kMaxSplitChunks];
#pragma unroll
        for (int c = 0; c < kMaxSplitChunks; ++c)
            if (c < nch) v0[c] = lists[(size_t)c * kCandCap + threadIdx.x];
        if ((int)threadIdx.x < used) sm.wcnt[threadIdx.x] = counts[threadIdx.x];
        lds_barrier();
        uint32_t total = 0;
        bool ok = true;
        for (int c = 0; c < used; ++c) {
            const uint32_t cc = sm.wcnt[c];
            if (cc == kFilterFailed || cc > (uint32_t)kCandCap) ok = false;
            else total += cc;
        }
        ok = ok && total >= (uint32_t)n && total <= (uint32_t)kCandCap;   // uniform
        if (ok) {
            // Chunk c's entries go to list slots from the sum of the earlier chunks' counts (chunk order
            // is position order): entry i < 1024 from the registers loaded above, entries from 1024 on (a
            // chunk holding more candidates than threads) in a second loop.
            uint32_t cnt[kMaxSplitChunks];   // read before any list store, so the reads do not wait on them
#pragma unroll
            for (int c = 0; c < kMaxSplitChunks; ++c) cnt[c] = c < used ? sm.wcnt[c] : 0u;
            uint32_t before = 0;
#pragma unroll
            for (int c = 0; c < kMaxSplitChunks; ++c) {
                if (threadIdx.x < cnt[c]) {
                    sm.cand_key[before + threadIdx.x] = v0[c].x;
                    sm.cand_idx[before + threadIdx.x] = v0[c].y;
                }
                before += cnt[c];
            }
            before = 0;
            for (int c = 0; c < used; ++c) {   // uniform
                const uint32_t cc = sm.wcnt[c];
                for (uint32_t i = threadIdx.x + kTopkThreads; i < cc; i += kTopkThreads) {
                    const uint2 e = lists[(size_t)c * kCandCap + i];
                    sm.cand_key[before + i] = e.x;
                    sm.cand_idx[before + i] = e.y;
                }
                before += cc;
            }
            resolve_prepare(sm);
            lds_barrier();
            resolve_list(src, total, n, k, o, sm);
            return;
        }
        lds_barrier();
        select_general(src, L, n, k, o, sm);
        return;
    }
    select_topk<true>(src, L, k, o, sm);
}

size_t topk_ws_bytes_per_row(int64_t row_stride, int32_t k) {
    (void)k;
    const int64_t nch = (row_stride + kFilterChunk - 1) / kFilterChunk;
    if (row_stride < kMinSplitCandidates || nch > kMaxSplitChunks) return 0;
    return split_row_bytes((int)nch);
}

hipError_t launch_topk(const float* scores, const int64_t* row_offsets, int64_t row_stride,
                       const int32_t* lengths, int32_t rows, int32_t k, int32_t* out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const size_t per_row = topk_ws_bytes_per_row(row_stride, k);
    // Few very long rows leave most of the GPU idle at one workgroup per row: split the filter pass
    // over the rows' 32768-candidate chunks when the workspace allows (rows of more than 114688
    // candidates, fewer than 256 rows) and the split pays.  Measured on MI355X (lengths uniform in
    // [stride/4, stride], us, split against one workgroup per row, which lists a long row in one pass):
    //   64 rows: 23.1 / 25.0 at stride 131072, 29.6 / 37.5 at 262144, 45.7 / 112 at 524288;
    //   128 rows: 28.9 / 25.9 at 131072, 44.5 / 38.7 at 262144, 57.6 / 53.2 at 393216, 76.1 / 113 at 524288;
    //   200 rows: 43.0 / 26.8 at 131072, 79.8 / 59.4 at 393216, 111 / 172 at 524288.
    // So the split runs for launches of at most a third as many rows as CUs, or rows of more than
    // 393216 candidates.  The result is identical either way.
    int dev = 0, num_cu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    const bool split_pays = 3 * rows <= num_cu || row_stride > 393216;
    const int nch = (int)((row_stride + kFilterChunk - 1) / kFilterChunk);
    if (per_row > 0 && rows < 256 && split_pays && ws && ws_bytes >= per_row) {
        const int per_batch = (int)min((size_t)rows, ws_bytes / per_row);
        for (int r0 = 0; r0 < rows; r0 += per_batch) {
            const int nr = min(per_batch, rows - r0);
            const int64_t* ro = row_offsets ? row_offsets + r0 : nullptr;
            const float* sc = row_offsets ? scores : scores + (int64_t)r0 * row_stride;
            const int32_t* ln = lengths ? lengths + r0 : nullptr;
            hipLaunchKernelGGL(topk_filter_kernel, dim3(nr * nch), dim3(kTopkThreads), 0, stream, sc, ro, row_stride,
                               ln, k, nch, (unsigned char*)ws);
            hipLaunchKernelGGL(topk_select_kernel, dim3(nr), dim3(kTopkThreads), 0, stream, sc, ro, row_stride, ln, k,
                               nch, (const unsigned char*)ws, out + (int64_t)r0 * k);
        }
        return hipGetLastError();
    }
    if (row_stride > kResident)
        hipLaunchKernelGGL(topk_rows_kernel<true>, dim3(rows), dim3(kTopkThreads), 0, stream, scores, row_offsets,
                           row_stride, lengths, k, out);
    else
        hipLaunchKernelGGL(topk_rows_kernel<false>, dim3(rows), dim3(kTopkThreads), 0, stream, scores, row_offsets,
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
