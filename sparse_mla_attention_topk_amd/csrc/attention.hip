// Sparse MLA attention over canonical top-k indices, gfx950 (CDNA4, wave64, MFMA bf16).
//
// What is computed (MQA over a shared latent; the decode path gathers the selected KV and runs the
// same sparse attention as prefill: "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL",
// section "Sparse MLA and FlashMLA"; slot = block id * block size + offset: "[Bugfix] Make DSV4
// sparse MLA work end-to-end ...", "What is fixed", item "Graph replay and draft KV"):
//   s[h, j] = scale * <q[h, 0:576], K_j[0:576]>,  p = softmax_j(s),  out[h] = sum_j p[h, j] K_j[0:512]
//   lse[h] = log sum_j exp(s[h, j])
// for the tokens j listed in the row's index slots (entries < 0 skipped).
//
// Work decomposition.  One workgroup (4 waves) owns one (row, split, 64-head block).  A split is
// 512 consecutive index slots; the number of splits depends on k only, so the reduction order of a
// row never depends on the batch.  Wave w owns heads [16w, 16w+16) of the block and keeps
//   * Q for its 16 heads in VGPRs (the B operand of the score MFMA, 18 x bf16x8),
//   * the output accumulator O^T [512 dims x 16 heads] in 32 MFMA tiles (AGPRs),
//   * a running max / sum per head (exp2 domain).
// The split's slots are processed in tiles of 32 tokens through a 4-stage LDS ring: each wave
// gathers 8 token records per tile with direct-to-LDS 16-byte loads (global_load_lds_dwordx4), so
// three tiles are in flight while one is consumed.  Records are stored unpadded (1152 B) with the
// 16-byte chunks of token t XOR-swizzled by f(t); the swizzle makes both operand reads below
// bank-conflict free.
//   scores:  S^T[16 tok x 16 heads] = K[16 tok x 576] . Q^T   (A = K rows from LDS via ds_read_b128)
//   values:  O^T[16 dims x 16 heads] += V^T[16 dims x 32 tok] . P^T[32 tok x 16 heads]
//            (A = V^T via ds_read_b64_tr_b16 transposed LDS reads, B = P straight from the score
//             accumulators: the S^T layout already puts a head's 8 token weights in one lane)
// Softmax is an fp32 online softmax in the exp2 domain, tiles in slot order.  A split that is not
// the only one writes its normalized partial (O_s, lse_s) to the workspace and a combine kernel
// merges the splits of a row in split order.  Nothing uses floating-point atomics.
//
// Invalid slots (index < 0, request/page out of range) load a valid dummy record, are zeroed in
// LDS after arrival and get score -inf, so every wave issues exactly the same number of
// direct-to-LDS loads per tile and the vmcnt bookkeeping below stays exact.
#include <math.h>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = 4;
constexpr int kTileTok = 32;
constexpr int kStages = 4;
constexpr int kTilesPerSplit = kSplitSlots / kTileTok;         // 16
constexpr int kStageBytes = kTileTok * kBf16Record;             // 36864
constexpr int kWaveTileBytes = kStageBytes / kAttnWaves;        // 9216: 8 records per wave
constexpr int kLoadsPerWave = kWaveTileBytes / (16 * kWave);    // 9 direct-to-LDS loads per tile
static_assert(kLoadsPerWave * 16 * kWave == kWaveTileBytes, "tile must split into whole wave loads");
constexpr uint32_t kNoToken = 0xffffffffu;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Swizzle key of tile-local token t: bits (t2, t0, t1, t3) -> (b0, b1, b2, b3).  Chunk c of the
// token's record sits at 16-byte position c ^ f (c < 64) or 64 + ((c - 64) ^ (f & 7)) (rope part).
__device__ __forceinline__ int swz_key(int t) {
    return ((t & 1) << 1) | ((t & 2) << 1) | ((t >> 2) & 1) | (t & 8);
}
__device__ __forceinline__ int swz_pos(int c, int f) {
    return c < 64 ? (c ^ f) : (64 + ((c - 64) ^ (f & 7)));
}

struct AttnParams {
    const uint16_t* q;
    int64_t q_row_stride;
    const uint8_t* kv;
    int64_t num_pages;
    const int32_t* block_table;
    int64_t bt_stride;
    int32_t num_reqs;
    const int32_t* row_req;
    const int32_t* idx;
    int32_t k;
    int32_t H;
    int32_t n_splits;
    int32_t n_hblocks;
    float scale_log2;
    int32_t row0;
    uint16_t* out;
    float* lse;
    float* ws_o;
    float* ws_lse;
};

// One direct-to-LDS 16-byte load: lane l's 16 bytes at `g` land at LDS byte lds_base + 16 l.  Issued
// as inline assembly so that the compiler does not pair every later LDS read with a wait for all
// outstanding loads; the kernel waits for these loads itself (wait_vmcnt before each barrier).
__device__ __forceinline__ void dma_b128(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// The running max of a head only moves when a tile's max exceeds it by more than this (log2
// units); in between, weights exp2(s - m) stay below 2^8 and the accumulators need no rescale.
constexpr float kRescaleSlack = 8.f;

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier and the operand prefetch depths.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kQkAhead = 4;   // score steps (2 reads each) in flight ahead of their MFMAs
constexpr int kPvAhead = 6;   // value dim-blocks (2 transposed reads each) in flight

__global__ __launch_bounds__(kAttnThreads, 1) void sparse_mla_bf16_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kStages * kStageBytes];
    __shared__ uint32_t phys[kSplitSlots];
    __shared__ uint32_t tile_valid[kTilesPerSplit];
    __shared__ int s_first, s_last;

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);

    // Work item: consecutive items (the splits / head blocks of one row) go to the same XCD, since
    // workgroups are dispatched round-robin over the 8 XCDs.
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3, per = nwg >> 3, rem = nwg & 7;
    const int item = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int hb = item % p.n_hblocks;
    const int rs = item / p.n_hblocks;
    const int split = rs % p.n_splits;
    const int rloc = rs / p.n_splits;
    const int64_t row = (int64_t)p.row0 + rloc;

    // ---- A4: translate this split's slots to physical token records ----
    const int slot0 = split * kSplitSlots;
    const int nslots = min(kSplitSlots, p.k - slot0);
    const int req = p.row_req ? p.row_req[row] : 0;
    const bool req_ok = req >= 0 && req < p.num_reqs;
    if (tid == 0) { s_first = kSplitSlots; s_last = -1; }
    if (tid < kTilesPerSplit) tile_valid[tid] = 0u;
    __syncthreads();
    for (int j = tid; j < kSplitSlots; j += kAttnThreads) {
        uint32_t ph = kNoToken;
        if (j < nslots && req_ok) {
            const int32_t pos = p.idx[row * p.k + slot0 + j];
            if (pos >= 0) {
                const int64_t lp = pos >> 6;
                if (lp < p.bt_stride) {
                    const int32_t pg = p.block_table[(int64_t)req * p.bt_stride + lp];
                    if (pg >= 0 && (int64_t)pg < p.num_pages) ph = (uint32_t)pg * kPage + (uint32_t)(pos & (kPage - 1));
                }
            }
        }
        phys[j] = ph;
        if (ph != kNoToken) {
            atomicMin(&s_first, j);
            atomicMax(&s_last, j);
            atomicOr(&tile_valid[j / kTileTok], 1u << (j % kTileTok));
        }
    }
    __syncthreads();
    const int ntiles = s_last < 0 ? 0 : s_last / kTileTok + 1;
    const uint32_t dummy = s_last < 0 ? 0u : phys[s_first];

    // ---- Q (B operand of the score MFMA): lane holds head (lane & 15), dims 32kk + 8(lane >> 4) .. +8
    const int h0 = hb * kHeadsPerBlock + wid * 16;
    const bool has_heads = h0 < p.H;
    bf16x8_t qv[18];
    if (has_heads) {
        const uint16_t* qrow = p.q + row * p.q_row_stride + (int64_t)(h0 + (lane & 15)) * kDqk + 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) qv[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
    }
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) asm volatile("" : "+a"(qv[kk]));   // Q lives in AGPRs (MFMA B operand)
    // Drain every compiler-visible global load here: inside the tile loop the only outstanding
    // vector-memory operations are the tile loads, which the loop waits for explicitly.
    wait_vmcnt<0>();

    // ---- A5: gather.  Wave w fills tile-local tokens [8w, 8w+8) of a stage: load i of lane l covers
    // LDS bytes w*9216 + 1024 i + 16 l, i.e. token 8w + (64i + l) / 72, 16-byte position (64i + l) % 72,
    // which holds the record's chunk swz_pos(position, swz_key(token)) (the swizzle is an involution).
    const uint32_t ring_lds = lds_offset(ring);
    const uint32_t wave_lds = ring_lds + (uint32_t)wid * kWaveTileBytes;
    auto issue_tile = [&](int tile, int stage, int ln) {
        const uint32_t m0 = wave_lds + (uint32_t)stage * kStageBytes;
        const uint8_t* src[kLoadsPerWave];
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {   // all slot reads first: the asm below is a compiler barrier
            const int qd = kWave * i + ln;
            const int tt = qd / 72;
            const int t = 8 * wid + tt;
            uint32_t ph = phys[tile * kTileTok + t];
            ph = ph == kNoToken ? dummy : ph;
            src[i] = p.kv + (uint64_t)ph * kBf16Record + 16u * (uint32_t)swz_pos(qd - 72 * tt, swz_key(t));
        }
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) dma_b128(src[i], m0 + 1024u * i);
    };
    // Zero this wave's records of invalid slots (after their dummy data has landed).
    auto zero_invalid = [&](int tile, int stage) {
        const uint32_t wbits = (tile_valid[tile] >> (8 * wid)) & 0xffu;
        if (wbits != 0xffu) {
            uint8_t* wbase = ring + stage * kStageBytes + wid * kWaveTileBytes;
#pragma unroll
            for (int i = 0; i < kLoadsPerWave; ++i) {
                const int qd = kWave * i + lane;
                const int tt = qd / 72;
                if (!((wbits >> tt) & 1u)) *(uint4*)(wbase + 16 * qd) = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    // Per-lane LDS byte offsets inside a stage (computed in the loop):
    //  score operand: token (lane & 15) of a 16-token block, chunk 4kk + g  ->  kb[kk & 3] + 256 (kk >> 2)
    //  for kk < 16, kr[kk - 16] for the two rope steps.
    //  transposed value reads: lane supplies row (token) 4g + ((lane & 15) >> 2) and dims 4(lane & 3)..+3
    //  of a 16-dim block, i.e. chunk 2db + ((lane >> 1) & 1), half (lane & 1)  ->  vb[db & 7] + 256 (db >> 3).
    const int g = lane >> 4;
    float m_run = -INFINITY, l_run = 0.f;   // exp2-domain reference max and weight sum (this lane's tokens)
    f32x4_t oacc[32];
#pragma unroll
    for (int d = 0; d < 32; ++d) oacc[d] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < kStages - 1 && t < ntiles; ++t) issue_tile(t, t, lane);

    for (int it = 0; it < ntiles; ++it) {
        const int stage = it % kStages;
        const int ahead = min(kStages - 2, ntiles - 1 - it);   // tiles issued after `it`
        if (ahead >= 2) wait_vmcnt<2 * kLoadsPerWave>();
        else if (ahead == 1) wait_vmcnt<kLoadsPerWave>();
        else wait_vmcnt<0>();
        zero_invalid(it, stage);
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();   // tile `it` visible; every wave is done with tile it-1
        // Per-lane constants are recomputed every tile from an opaque copy of the lane id: keeping them
        // live across the loop would leave no registers for operand prefetch.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (it + kStages - 1 < ntiles) issue_tile(it + kStages - 1, (it + kStages - 1) % kStages, ln);
        if (!has_heads) continue;
        const int g = ln >> 4;
        const int fa = swz_key(ln & 15);
        const int tv = 4 * g + ((ln & 15) >> 2);
        const int fv = swz_key(tv);
        uint32_t kb[4], kr[2], vb[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) kb[j] = (ln & 15) * kBf16Record + 16 * ((4 * j + g) ^ fa);
#pragma unroll
        for (int j = 0; j < 2; ++j) kr[j] = (ln & 15) * kBf16Record + 16 * (64 + ((4 * j + g) ^ (fa & 7)));
#pragma unroll
        for (int j = 0; j < 8; ++j) vb[j] = tv * kBf16Record + 8 * (ln & 1) + 16 * ((2 * j + ((ln >> 1) & 1)) ^ fv);

        const uint8_t* sb = ring + stage * kStageBytes;
        const uint32_t vmask = tile_valid[it];

        // ---- A7: scores S^T[32 tok x 16 heads] as two 16-token blocks ----
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
            const uint32_t off = kk < 16 ? kb[kk & 3] + 256u * (kk >> 2) : kr[kk - 16];
            const bf16x8_t a0 = *(const bf16x8_t*)(sb + off);
            const bf16x8_t a1 = *(const bf16x8_t*)(sb + off + 16 * kBf16Record);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qv[kk], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qv[kk], s1, 0, 0, 0);
        }
        // Schedule: operand reads run kQkAhead steps ahead of the MFMAs that consume them.
#pragma unroll
        for (int i = 0; i < kQkAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
        for (int i = 0; i < 18 - kQkAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * kQkAhead, 0);

        // ---- A8: online softmax (lane: head lane & 15, tokens 16tb + 4g + i) ----
        float sv[8];
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = ((vmask >> (4 * g + i)) & 1u) ? s0[i] * p.scale_log2 : -INFINITY;
            const float x1 = ((vmask >> (16 + 4 * g + i)) & 1u) ? s1[i] * p.scale_log2 : -INFINITY;
            sv[i] = x0;
            sv[4 + i] = x1;
            mt = fmaxf(mt, fmaxf(x0, x1));
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // The reference max moves only if this tile's max exceeds it by more than the slack; the
        // decision is a function of the row's own scores, so it is identical in every batch.
        if (mt > m_run + kRescaleSlack) {
            const float alpha = exp2f(m_run - mt);   // 0 while nothing has been accumulated
            m_run = mt;
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < 32; ++d) {
                oacc[d][0] *= alpha; oacc[d][1] *= alpha; oacc[d][2] *= alpha; oacc[d][3] *= alpha;
            }
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float pw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pw[j] = exp2f(sv[j] - m_use);
            l_run += pw[j];
        }
        union { bf16x8_t v; uint32_t u[4]; } pb;
        pb.u[0] = pack_bf16x2(pw[0], pw[1]);
        pb.u[1] = pack_bf16x2(pw[2], pw[3]);
        pb.u[2] = pack_bf16x2(pw[4], pw[5]);
        pb.u[3] = pack_bf16x2(pw[6], pw[7]);

        // ---- A9: O^T += V^T P^T over 32 dim blocks ----
#pragma unroll
        for (int db = 0; db < 32; ++db) {
            const uint8_t* vp = sb + vb[db & 7] + 256u * (db >> 3);
            union { bf16x8_t v; i16x4_t h[2]; } va;
            va.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(vp));
            va.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t*)(vp + 16 * kBf16Record));
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, pb.v, oacc[db], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kPvAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
        for (int i = 0; i < 32 - kPvAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPvAhead, 0);
    }

    // ---- A10: epilogue (lane: head h0 + (lane & 15), dims 16db + 4g + i) ----
    if (!has_heads) return;
    // Lanes of one head share m_run (the tile max is reduced over them), so their sums add directly.
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot = l_tot + __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    const int head = h0 + (lane & 15);
    if (p.n_splits == 1) {
        uint16_t* orow = p.out + (row * p.H + head) * (int64_t)kDv + 4 * g;
#pragma unroll
        for (int db = 0; db < 32; ++db) {
            uint2 w;
            w.x = pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv);
            w.y = pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv);
            *(uint2*)(orow + 16 * db) = w;
        }
        if (lane < 16 && p.lse) p.lse[row * p.H + head] = lse_v;
    } else {
        const int64_t part = ((int64_t)rloc * p.n_splits + split) * p.H + head;
        float* wo = p.ws_o + part * kDv + 4 * g;
#pragma unroll
        for (int db = 0; db < 32; ++db) {
            f32x4_t v = {oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv};
            *(f32x4_t*)(wo + 16 * db) = v;
        }
        if (lane < 16) p.ws_lse[part] = lse_v;
    }
}

// A11: merge the splits of each row in split order:  LSE = m + log sum_s e^(lse_s - m),
// out = sum_s (e^(lse_s - m) / sum) * O_s, rounded to bf16.  One thread per (row, head, 4 dims).
__global__ __launch_bounds__(256) void split_combine_kernel(const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_lse, int S, int H,
                                                            int row0, uint16_t* __restrict__ out,
                                                            float* __restrict__ lse) {
    const int pairs = H / 2;
    const int rloc = blockIdx.x / pairs;
    const int head = (blockIdx.x % pairs) * 2 + (threadIdx.x >> 7);
    const int d = 4 * (threadIdx.x & 127);
    const float* ls = ws_lse + (int64_t)rloc * S * H + head;
    float m = -INFINITY;
    for (int s = 0; s < S; ++s) m = fmaxf(m, ls[(int64_t)s * H]);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float LSE = -INFINITY;
    if (m != -INFINITY) {
        float tot = 0.f;
        for (int s = 0; s < S; ++s) tot += expf(ls[(int64_t)s * H] - m);
        LSE = m + logf(tot);
        const float inv = 1.f / tot;
        for (int s = 0; s < S; ++s) {
            const float w = expf(ls[(int64_t)s * H] - m) * inv;
            const f32x4_t o = *(const f32x4_t*)(ws_o + (((int64_t)rloc * S + s) * H + head) * kDv + d);
            acc[0] += w * o[0]; acc[1] += w * o[1]; acc[2] += w * o[2]; acc[3] += w * o[3];
        }
    }
    const int64_t orow = ((int64_t)row0 + rloc) * H + head;
    uint2 w;
    w.x = pack_bf16x2(acc[0], acc[1]);
    w.y = pack_bf16x2(acc[2], acc[3]);
    *(uint2*)(out + orow * kDv + d) = w;
    if (d == 0 && lse) lse[orow] = LSE;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    AttnParams p;
    p.q = (const uint16_t*)a.q;
    p.q_row_stride = a.q_row_stride;
    p.kv = (const uint8_t*)a.kv;
    p.num_pages = a.num_pages;
    p.block_table = a.block_table;
    p.bt_stride = a.bt_stride;
    p.num_reqs = a.num_reqs;
    p.row_req = a.row_req;
    p.idx = a.idx;
    p.k = a.k;
    p.H = a.H;
    p.n_splits = attn_num_splits(a.k);
    p.n_hblocks = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
    p.scale_log2 = a.softmax_scale * kLog2e;
    p.out = (uint16_t*)a.out;
    p.lse = a.lse;
    const size_t per_row = attn_ws_bytes_per_row(a.H, a.k);
    int rows_per_launch = a.rows;
    if (per_row > 0) {
        const size_t fit = a.ws_bytes / per_row;
        rows_per_launch = (int)(fit < (size_t)a.rows ? fit : (size_t)a.rows);
        if (rows_per_launch < 1) return hipErrorInvalidValue;   // host validation prevents this
    }
    for (int row0 = 0; row0 < a.rows; row0 += rows_per_launch) {
        const int n = min(rows_per_launch, a.rows - row0);
        p.row0 = row0;
        p.ws_o = (float*)a.ws;
        p.ws_lse = per_row > 0 ? (float*)a.ws + (size_t)n * p.n_splits * a.H * kDv : nullptr;
        const int grid = n * p.n_splits * p.n_hblocks;
        hipLaunchKernelGGL(sparse_mla_bf16_kernel, dim3(grid), dim3(kAttnThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.n_splits > 1) {
            hipLaunchKernelGGL(split_combine_kernel, dim3(n * (a.H / 2)), dim3(256), 0, stream, p.ws_o, p.ws_lse,
                               p.n_splits, a.H, row0, p.out, p.lse);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace smla
