// Indexer scores (paged MQA logits): the per-position scores that the top-k selector consumes, gfx950.
//
// Sources: "[SM120] Sync DS4 with upstream main + validated perf backports", sections "September 12
// follow-up" (the DSA indexer's MQA logits, with a separate kernel for long prefills) and
// "2026-09-12 live validation and promotion update" (the paged form); the pages name the operation
// but give no formula.  The formula used is the published lightning-indexer form of DeepSeek sparse
// attention: one shared index key k_p per token (MQA: 128 bf16), index heads h with query q_h and a
// per-row weight w_h,
//   score[p] = sum_h w_h * relu(<q_h, k_p>),   relu(x) = x if x > 0 else 0,
// for positions p below the row's clamped length whose page is listed; -inf everywhere else in the
// row.  Paging as for the latent cache ("[Bugfix] Make DSV4 sparse MLA work end-to-end ...", section
// "Purpose", item "Graph replay and draft KV"): key p is token p % 64 of physical page
// block_table[req][p / 64]; lengths are clamped to [0, row stride] (same section, items on negative
// and out-of-range lengths).
//
// Work decomposition (persistent).  A page of the key cache is 64 keys x 256 B = 16 KB, contiguous.
// The grid is one workgroup of 4 waves per CU (one wave per SIMD: measured on MI355X, a second wave
// on a SIMD has its loads served after the first's and finishes far later).  Each workgroup first
// computes, in LDS, the prefix sums over the launch's rows of the pages that hold keys to score
// (ceil(L / 64) per row).  Every wave then takes an equal share of that concatenated page list and
// walks it row segment by row segment: per segment it loads the row's Q fragments and head weights
// into registers and up to 64 block-table entries into one vector register (lane i: page i), then
// streams the pages through a double buffer of registers (page n + 1 in flight while page n is
// scored, 16 loads of 16 B per lane per page).  Scores go to LDS and are written out with 16-byte
// stores after the chunk's last key load: on gfx950 stores and loads share one in-order completion
// counter, so a store issued ahead of key loads would delay every wait for them by its own latency.
// Last, each wave writes -inf into an equal share of the remaining page slots (past the rows' lengths).
// Equal shares keep every CU and XCD busy to the end whatever the row lengths.
//
// Contraction (v_mfma_f32_16x16x32_bf16, D[16 x 16] += A[16 x 32] . B[32 x 16]): A = Q (rows = 16
// heads), B = K^T (columns = 16 tokens), 32 dims per step.  Step kk of lane l covers dims 32 kk + 8 g
// .. +8 with g = l / 16, for A (head l % 16 of the head block) and for B (token l % 16 of the token
// block) alike, so each load of K reads 64 contiguous bytes of 16 tokens.  Lane l then holds the
// fp32 dot products of heads 16 hb + 4 g + i (i < 4) with token l % 16.
//
// Epilogue, in a fixed order: each lane sums w_h * relu(s_h) over its heads (head blocks in order,
// then i in order, one fused multiply-add each), the four lanes holding a token add their sums
// pairwise (l + l^32, then + l^16: every one of them gets the same bits), and lane l writes position
// l of the page.  A page's scores depend only on its row's inputs, whichever wave computes them, so
// a row's scores are the same in any batch.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kIdxDim = 128;
constexpr int kIdxRecord = 2 * kIdxDim;         // bytes per index key
constexpr int kIdxWaves = 4;
constexpr int kIdxThreads = kIdxWaves * kWave;

constexpr int kPageBytes = kPage * kIdxRecord;   // 16 KB
constexpr int kMaxRowsPerLaunch = 1024;            // rows whose page prefix sums one launch keeps in LDS
constexpr int kIdxWgPerCu = 1;   // one wave per SIMD: a second wave on a SIMD gets its loads served later than the first

struct IdxParams {
    const uint16_t* q;
    int64_t q_row_stride;
    const float* w;
    int64_t w_row_stride;
    const uint8_t* kidx;
    int64_t num_pages;
    const int32_t* block_table;
    int64_t bt_stride;
    int32_t num_reqs;
    const int32_t* row_req;
    const int32_t* lengths;
    float* out;
    int64_t out_stride;
    int32_t rows;     // rows of this launch, <= kMaxRowsPerLaunch
    int32_t nslots;   // page slots per row: ceil(out_stride / 64)
};

// Sum over lanes l, l^16, l^32, l^48 in an order each of the four reproduces bit for bit.
__device__ __forceinline__ float quad_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <bool LEN>
__device__ __forceinline__ int64_t row_length(const IdxParams& p, int r) {
    const int64_t len = LEN ? (int64_t)p.lengths[r] : p.out_stride;
    return len < 0 ? 0 : (len > p.out_stride ? p.out_stride : len);
}
template <bool REQ>
__device__ __forceinline__ int row_request(const IdxParams& p, int r) {
    const int req = REQ ? p.row_req[r] : 0;
    return req >= 0 && req < p.num_reqs ? req : -1;
}

// NHB: index heads / 16.  LEN / REQ: whether per-row lengths / request ids are given (without them
// every row has length out_stride / reads request 0).
template <int NHB, bool LEN, bool REQ>
__global__ __launch_bounds__(kIdxThreads, 1) void paged_mqa_logits_kernel(const IdxParams p) {
    // dp[r] = sum over rows r' < r of their pages with keys to score: ceil(L / 64) if the row's
    // request is valid, else 0 (such a row is all -inf).
    __shared__ int64_t dp[kMaxRowsPerLaunch + 1];
    __shared__ int64_t wsum[kIdxWaves];
    // per wave: the scores of up to 64 pages, written out after the chunk's last key load (a store ahead of
    // key loads in the in-order memory counter would delay the waits for them by its own latency)
    __shared__ __attribute__((aligned(16))) float stash[kIdxWaves][kWave * kPage];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int g = lane >> 4;
    const float ninf = -__builtin_inff();

    // ---- prefix sums of the data pages per row (each thread: kPer consecutive rows) ----
    {
        constexpr int kPer = kMaxRowsPerLaunch / kIdxThreads;
        // every load first, at clamped rows (rows >= 1), so they are in flight together
        int32_t lenv[kPer], reqv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int r = min((int)threadIdx.x * kPer + i, p.rows - 1);
            lenv[i] = LEN ? p.lengths[r] : 0;
            reqv[i] = REQ ? p.row_req[r] : 0;
        }
        int64_t d[kPer];
        int64_t sum = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int r = (int)threadIdx.x * kPer + i;
            const int64_t len = LEN ? (int64_t)lenv[i] : p.out_stride;
            const int64_t L = len < 0 ? 0 : (len > p.out_stride ? p.out_stride : len);
            const bool ok = r < p.rows && reqv[i] >= 0 && reqv[i] < p.num_reqs;
            d[i] = ok ? (L + kPage - 1) / kPage : 0;
            sum += d[i];
        }
        int64_t incl = sum;   // inclusive scan over the wave
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int64_t v = __shfl_up(incl, off);
            if (lane >= off) incl += v;
        }
        if (lane == kWave - 1) wsum[wid] = incl;
        __syncthreads();
        int64_t before = incl - sum;
        for (int w2 = 0; w2 < wid; ++w2) before += wsum[w2];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            dp[(int)threadIdx.x * kPer + i] = before;
            before += d[i];
        }
        if (threadIdx.x == kIdxThreads - 1) dp[kMaxRowsPerLaunch] = before;
        __syncthreads();
    }
    const int64_t D = dp[p.rows];                                  // pages with keys to score
    const int64_t TS = (int64_t)p.rows * p.nslots - D;            // page slots that only get -inf
    const int64_t NW = (int64_t)gridDim.x * kIdxWaves;
    const int64_t gw = (int64_t)blockIdx.x * kIdxWaves + wid;
    auto row_pages = [&](int r) -> int64_t { return dp[r + 1] - dp[r]; };

    // ---- pages with keys to score ----
    int64_t s = D * gw / NW;
    const int64_t e = D * (gw + 1) / NW;
    int r = 0;
    if (s < e) {
        int lo = 0, hi = p.rows - 1;   // the row holding page s: the largest r with dp[r] <= s
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (dp[mid] <= s) lo = mid; else hi = mid - 1;
        }
        r = lo;
    }
    const int lane_off = (lane & 15) * kIdxRecord + 16 * g;
    constexpr int kBufs = 2;   // page k + 1 in flight while page k is scored
    bf16x8_t kf[kBufs][4][4];   // kf[b][tb][kk]: token 16 tb + l % 16, dims 32 kk + 8 g .. +8
    while (s < e) {
        while (dp[r + 1] <= s) ++r;   // rows without pages are skipped
        const int64_t j0 = s - dp[r];                                        // first page of the segment
        const int64_t cnt = (dp[r + 1] < e ? dp[r + 1] : e) - s;            // pages of the segment
        const int64_t L = row_length<LEN>(p, r);
        const int req = row_request<REQ>(p, r);                              // valid: the row has pages
        float* const orow = p.out + (int64_t)r * p.out_stride;
        // The row's Q fragments (qf[hb][kk]: head 16 hb + l % 16, dims 32 kk + 8 g .. +8) and weights.
        bf16x8_t qf[NHB][4];
        f32x4_t wv[NHB];
        {
            const uint16_t* qrow = p.q + (int64_t)r * p.q_row_stride + (lane & 15) * kIdxDim + 8 * g;
            const float* wrow = p.w + (int64_t)r * p.w_row_stride + 4 * g;
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) qf[hb][kk] = *(const bf16x8_t*)(qrow + hb * 16 * kIdxDim + 32 * kk);
                wv[hb] = *(const f32x4_t*)(wrow + 16 * hb);
            }
        }
        const int32_t* btrow = p.block_table + (int64_t)req * p.bt_stride;
        for (int64_t c0 = 0; c0 < cnt; c0 += kWave) {   // chunks of up to 64 pages
            const int n = (int)(cnt - c0 < kWave ? cnt - c0 : kWave);
            const int64_t jb = j0 + c0;   // first page of the chunk
            // lane i: physical page of page jb + i, or -1 (past the chunk, past the block table, or
            // not a page of the cache)
            int32_t btv = -1;
            {
                const int64_t jl = jb + lane;
                const bool inb = lane < n && jl < p.bt_stride;
                const int32_t v = btrow[inb ? jl : 0];
                if (inb && v >= 0 && (int64_t)v < p.num_pages) btv = v;
            }
            // Page k of the chunk into buffer b.  Past the chunk every lane reads the same 16 bytes
            // (a fixed number of loads keeps the compiler's waits exact; one cache line per load).
            auto issue = [&](int b, int k) {
                const int pg = __builtin_amdgcn_readlane(btv, k < n ? k : 0);
                const bool real = k < n;
                const uint8_t* kp = p.kidx + (real ? (uint64_t)(pg >= 0 ? pg : 0) * kPageBytes + lane_off : 0);
                const int tstride = real ? 16 * kIdxRecord : 0, kstride = real ? 64 : 0;
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        kf[b][tb][kk] = *(const bf16x8_t*)(kp + tb * tstride + kk * kstride);
                asm volatile("" ::: "memory");   // issue here: the compiler would sink the loads to their use
            };
            auto score = [&](int b, int k) {
                float t[4] = {0.f, 0.f, 0.f, 0.f};   // per token block: sum over the lane's heads
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                    for (int hb = 0; hb < NHB; ++hb) {
                        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[hb][kk], kf[b][tb][kk], acc, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float sc = acc[i];
                            t[tb] = __builtin_fmaf(wv[hb][i], sc > 0.f ? sc : 0.f, t[tb]);
                        }
                    }
                }
                float res = ninf;
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const float tot = quad_sum(t[tb]);
                    if (g == tb) res = tot;   // lane l keeps token 16 (l / 16) + l % 16 = l of the page
                }
                const int pg = __builtin_amdgcn_readlane(btv, k);
                const int64_t pos = (jb + k) * kPage + lane;
                stash[wid][k * kWave + lane] = (pg >= 0 && pos < L) ? res : ninf;
            };
#pragma unroll
            for (int b = 0; b < kBufs; ++b) issue(b, b);
#pragma unroll 1
            for (int k = 0; k < n; k += kBufs) {
#pragma unroll
                for (int b = 0; b < kBufs; ++b) {
                    if (b == 0 || k + b < n) score(b, k + b);
                    issue(b, k + b + kBufs);
                }
            }
            // The chunk's n pages of scores (64 n consecutive positions from page jb on) leave as 16-byte
            // stores: store i of lane l writes positions 4 (l + 64 i) .. +3.
#pragma unroll 1
            for (int i = 0; i < kPage / 4; ++i) {
                const int q4 = lane + kWave * i;   // float4 index
                if (q4 >= n * (kPage / 4)) break;
                const f32x4_t v = *(const f32x4_t*)&stash[wid][4 * q4];
                const int64_t pos = jb * kPage + 4 * q4;
                if (pos + 3 < p.out_stride) {
                    __builtin_nontemporal_store(v, (f32x4_t*)&orow[pos]);
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2)
                        if (pos + e2 < p.out_stride) orow[pos + e2] = v[e2];
                }
            }
        }
        s += cnt;
    }

    // ---- -inf page slots, after the scored pages (before them, the stores would sit ahead of the first
    // key loads in the in-order memory counter): tail slot t of the concatenation over rows (row r holds
    // nslots - d_r of them, from its slot d_r on) ----
    {
        int64_t t = TS * gw / NW;
        const int64_t t1 = TS * (gw + 1) / NW;
        if (t < t1) {
            // the row holding tail slot t: the largest r with tp(r) <= t, tp(r) = r nslots - dp[r]
            int lo = 0, hi = p.rows - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((int64_t)mid * p.nslots - dp[mid] <= t) lo = mid; else hi = mid - 1;
            }
            int rt = lo;
            int64_t slot = row_pages(rt) + (t - ((int64_t)rt * p.nslots - dp[rt]));
            for (; t < t1; ++t) {
                while (slot >= p.nslots) { ++rt; slot = row_pages(rt); }
                const int64_t pos = slot * kPage + lane;
                if (pos < p.out_stride) __builtin_nontemporal_store(ninf, &p.out[(int64_t)rt * p.out_stride + pos]);
                ++slot;
            }
        }
    }
}

template <int NHB>
void launch_flags(bool len, bool req, unsigned grid, const IdxParams& p, hipStream_t stream) {
    if (len && req) paged_mqa_logits_kernel<NHB, true, true><<<grid, kIdxThreads, 0, stream>>>(p);
    else if (len) paged_mqa_logits_kernel<NHB, true, false><<<grid, kIdxThreads, 0, stream>>>(p);
    else if (req) paged_mqa_logits_kernel<NHB, false, true><<<grid, kIdxThreads, 0, stream>>>(p);
    else paged_mqa_logits_kernel<NHB, false, false><<<grid, kIdxThreads, 0, stream>>>(p);
}

void launch_nhb(int nhb, bool len, bool req, unsigned grid, const IdxParams& p, hipStream_t stream) {
    switch (nhb) {
        case 1: launch_flags<1>(len, req, grid, p, stream); break;
        case 2: launch_flags<2>(len, req, grid, p, stream); break;
        case 3: launch_flags<3>(len, req, grid, p, stream); break;
        default: launch_flags<4>(len, req, grid, p, stream); break;
    }
}

}  // namespace

hipError_t launch_paged_mqa_logits(const IdxArgs& a, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    IdxParams p;
    p.q = (const uint16_t*)a.q;
    p.q_row_stride = a.q_row_stride;
    p.w = a.weights;
    p.w_row_stride = a.w_row_stride;
    p.kidx = (const uint8_t*)a.kidx;
    p.num_pages = a.num_pages;
    p.block_table = a.block_table;
    p.bt_stride = a.bt_stride;
    p.num_reqs = a.num_reqs;
    p.row_req = a.row_req;
    p.lengths = a.lengths;
    p.out = a.out;
    p.out_stride = a.out_stride;
    p.nslots = (int32_t)((a.out_stride + kPage - 1) / kPage);
    int dev = 0, num_cu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    const unsigned grid = (unsigned)(num_cu * kIdxWgPerCu);
    for (int64_t r0 = 0; r0 < a.rows; r0 += kMaxRowsPerLaunch) {
        IdxParams pr = p;
        pr.rows = (int32_t)(a.rows - r0 < kMaxRowsPerLaunch ? a.rows - r0 : kMaxRowsPerLaunch);
        pr.q = p.q + r0 * p.q_row_stride;
        pr.w = p.w + r0 * p.w_row_stride;
        pr.row_req = p.row_req ? p.row_req + r0 : nullptr;
        pr.lengths = p.lengths ? p.lengths + r0 : nullptr;
        pr.out = p.out + r0 * p.out_stride;
        launch_nhb(a.Hi / 16, pr.lengths != nullptr, pr.row_req != nullptr, grid, pr, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace smla
