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
// Work decomposition.  A page of the key cache is 64 keys x 256 B = 16 KB, contiguous, so one wave
// owns one page: 16 loads of 16 B per lane bring the whole page into registers, and a workgroup of 4
// waves covers 256 consecutive positions of one row.  The workgroup's Q ([heads, 128] bf16, at most
// 16 KB) is staged once in LDS (chunk c of head h at 16-byte position c ^ (h & 15), so the
// fragment reads below touch 16 different bank groups).
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
// 64-page offset l.  Nothing depends on other rows, so a row's scores are the same in any batch.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kIdxDim = 128;
constexpr int kIdxRecord = 2 * kIdxDim;         // bytes per index key
constexpr int kIdxWaves = 4;
constexpr int kIdxThreads = kIdxWaves * kWave;
constexpr int kIdxPositions = kIdxWaves * kPage;   // positions per workgroup

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
    int32_t nchunks;   // workgroups per row
};

// Sum over lanes l, l^16, l^32, l^48 in an order each of the four reproduces bit for bit.
__device__ __forceinline__ float quad_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int NHB>   // index heads / 16
__global__ __launch_bounds__(kIdxThreads) void paged_mqa_logits_kernel(const IdxParams p) {
    __shared__ __attribute__((aligned(16))) bf16x8_t qs[NHB * 16][16];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int g = lane >> 4;

    // Work item: the chunks of one row go to one XCD (workgroups are dispatched round-robin over the
    // 8 XCDs), so the row's Q is fetched from HBM once per XCD.
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3, per = nwg >> 3, rem = nwg & 7;
    const int item = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int64_t row = item / p.nchunks;
    const int64_t chunk0 = (int64_t)(item % p.nchunks) * kIdxPositions;

    const int64_t len = p.lengths ? (int64_t)p.lengths[row] : p.out_stride;
    const int64_t L = len < 0 ? 0 : (len > p.out_stride ? p.out_stride : len);
    float* const orow = p.out + row * p.out_stride;
    const int64_t pos0 = chunk0 + (int64_t)wid * kPage;   // this wave's page of positions
    const int64_t my_pos = pos0 + lane;
    const float ninf = -__builtin_inff();

    if (chunk0 >= L) {   // uniform: nothing to score in this workgroup
        if (my_pos < p.out_stride) orow[my_pos] = ninf;
        return;
    }

    // The wave's physical page (-1: nothing to score on it).
    int64_t page = -1;
    if (pos0 < L) {
        const int req = p.row_req ? p.row_req[row] : 0;
        const int64_t lp = pos0 / kPage;
        if (req >= 0 && req < p.num_reqs && lp < p.bt_stride) {
            const int32_t pg = p.block_table[(int64_t)req * p.bt_stride + lp];
            if (pg >= 0 && (int64_t)pg < p.num_pages) page = pg;
        }
    }
    page = __builtin_amdgcn_readfirstlane((int)page);

    // Q -> LDS (swizzled), issued first so that its wait does not cover the key loads.
    constexpr int kQChunks = NHB * 16 * 16;
    bf16x8_t qstage[kQChunks / kIdxThreads];
    const uint16_t* qrow = p.q + row * p.q_row_stride;
#pragma unroll
    for (int r = 0; r < kQChunks / kIdxThreads; ++r) {
        const int j = (int)threadIdx.x + kIdxThreads * r;
        qstage[r] = *(const bf16x8_t*)(qrow + (j >> 4) * kIdxDim + 8 * (j & 15));
    }
    // The page's keys: kf[tb][kk] = token 16 tb + l % 16, dims 32 kk + 8 g .. +8.  A wave without a
    // page loads page 0 (it exists: num_pages >= 1) and discards it, so that every wave issues the
    // same loads and the waits below count them exactly.
    bf16x8_t kf[4][4];
    {
        const uint64_t pg = page >= 0 ? (uint64_t)page : 0u;
        const uint8_t* kp = p.kidx + pg * (kPage * kIdxRecord) + (lane & 15) * kIdxRecord + 16 * g;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kf[tb][kk] = *(const bf16x8_t*)(kp + tb * 16 * kIdxRecord + 64 * kk);
    }
    // Weights of the lane's heads 16 hb + 4 g + i.
    f32x4_t wv[NHB];
    const float* wrow = p.w + row * p.w_row_stride;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) wv[hb] = *(const f32x4_t*)(wrow + 16 * hb + 4 * g);

#pragma unroll
    for (int r = 0; r < kQChunks / kIdxThreads; ++r) {
        const int j = (int)threadIdx.x + kIdxThreads * r;
        const int h = j >> 4;
        qs[h][(j & 15) ^ (h & 15)] = qstage[r];
    }
    __syncthreads();
    if (page < 0) {
        if (my_pos < p.out_stride) orow[my_pos] = ninf;
        return;
    }

    float res = ninf;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        float t = 0.f;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            const int h = 16 * hb + (lane & 15);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8_t qa = qs[h][(4 * kk + g) ^ (h & 15)];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[tb][kk], acc, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = acc[i];
                t = __builtin_fmaf(wv[hb][i], s > 0.f ? s : 0.f, t);
            }
        }
        const float tot = quad_sum(t);
        if (g == tb) res = tot;   // lane l keeps token 16 (l / 16) + l % 16 = l of the page
    }
    if (my_pos < p.out_stride) orow[my_pos] = my_pos < L ? res : ninf;
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
    const int64_t nchunks = (a.out_stride + kIdxPositions - 1) / kIdxPositions;
    // Rows per launch: the grid stays below 2^31 workgroups and item indices fit in int.
    const int64_t max_rows = ((int64_t)1 << 30) / nchunks;
    p.nchunks = (int32_t)nchunks;
    for (int64_t r0 = 0; r0 < a.rows; r0 += max_rows) {
        const int64_t nr = a.rows - r0 < max_rows ? a.rows - r0 : max_rows;
        IdxParams pr = p;
        pr.q = p.q + r0 * p.q_row_stride;
        pr.w = p.w + r0 * p.w_row_stride;
        pr.row_req = p.row_req ? p.row_req + r0 : nullptr;
        pr.lengths = p.lengths ? p.lengths + r0 : nullptr;
        pr.out = p.out + r0 * p.out_stride;
        const unsigned grid = (unsigned)(nr * nchunks);
        switch (a.Hi / 16) {
            case 1: paged_mqa_logits_kernel<1><<<grid, kIdxThreads, 0, stream>>>(pr); break;
            case 2: paged_mqa_logits_kernel<2><<<grid, kIdxThreads, 0, stream>>>(pr); break;
            case 3: paged_mqa_logits_kernel<3><<<grid, kIdxThreads, 0, stream>>>(pr); break;
            default: paged_mqa_logits_kernel<4><<<grid, kIdxThreads, 0, stream>>>(pr); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace smla
