// Sparse MLA attention over canonical top-k indices, gfx950 (CDNA4, wave64, MFMA bf16).
//
// What is computed (MQA over a shared latent; the decode path gathers the selected KV and runs the
// same sparse attention as prefill: "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL",
// section "Sparse MLA and FlashMLA"; slot = block id * block size + offset: "[Bugfix] Make DSV4
// sparse MLA work end-to-end ...", section "Purpose", item "Graph replay and draft KV"):
//   s[h, j] = scale * <q[h, 0:576], K_j[0:576]>,  p = softmax_j(s),  out[h] = sum_j p[h, j] K_j[0:512]
//   lse[h] = log sum_j exp(s[h, j])
// for the tokens j listed in the row's index slots (entries < 0 skipped).
//
// Work decomposition.  One workgroup (4 waves) owns one (row, split, 64-head block).  A split is
// 512 consecutive index slots; the number of splits depends on k only, so the reduction order of a
// row never depends on the batch.  The split's slots are processed in tiles of 32 tokens through a
// 4-stage LDS ring: each wave gathers 8 token records per tile with direct-to-LDS 16-byte loads
// (global_load_lds_dwordx4), so three tiles are in flight while one is consumed.  Records are
// stored unpadded (1152 B); the 16-byte chunks of tile-local token t are XOR-swizzled with
// f(t) = (t >> 1) & 7, the mapping measured to keep both operand read patterns below free of LDS
// bank conflicts on gfx950.
//
// Waves pair up on 32 heads.  Wave w computes scores for its own 16 heads with Q in AGPRs:
//   S^T[16 tok x 16 heads] = K[16 tok x 576] . Q^T        (A = K rows via ds_read_b128)
// keeps the online-softmax state of those heads, and publishes its bf16 weights P (one 16-byte
// fragment per lane) to its partner through LDS.  Each wave then accumulates the values for BOTH
// head blocks of the pair over one half of the 512 value dims:
//   O^T[16 dims x 16 heads] += V^T[16 dims x 32 tok] . P^T[32 tok x 16 heads]
// (A = V^T via ds_read_b64_tr_b16 transposed LDS reads, shared by the two head blocks), so every
// transposed read feeds two MFMAs.  The S^T accumulator layout already holds a head's token
// weights in the B-operand layout of the value MFMA, so no register transpose is needed.
//
// Softmax is an fp32 online softmax in the exp2 domain, tiles in slot order.  A head's reference
// max only moves when a tile's max exceeds it by more than 2^8 (a decision that depends on the
// row's own scores only), so the accumulators are rescaled rarely.  A split that is not the only
// one writes its normalized partial (O_s, lse_s) to the workspace and a combine kernel merges the
// splits of a row in split order.  Nothing uses floating-point atomics.
//
// Invalid slots (index < 0, request/page out of range) load a valid dummy record, are zeroed in
// LDS after arrival and get score -inf, so every wave issues exactly the same number of
// direct-to-LDS loads per tile and the vmcnt bookkeeping below stays exact.
#include <math.h>

#include <type_traits>

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

// Swizzle of tile-local token t: chunk c of the record sits at 16-byte position c ^ f(t).  f < 8, so
// every chunk stays inside its aligned group of 8 (the 64 latent chunks and the 8 rope chunks alike).
__device__ __forceinline__ int swz_key(int t) { return (t >> 1) & 7; }

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

// max over lanes l, l^16, l^32, l^48 (the four lanes holding one head's tokens)
__device__ __forceinline__ float head_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float w = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(w), __float_as_uint(w), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// sum over the same four lanes, in an order every one of them reproduces bit for bit
__device__ __forceinline__ float head_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float w = __uint_as_float(a[0]) + __uint_as_float(a[1]);    // lanes l < 32: v_l + v_{l+32}
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(w), __float_as_uint(w), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
    typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f2;
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 b2;
    union { b2 v; uint32_t u; } r;
    r.v = __builtin_convertvector((f2){lo, hi}, b2);   // v_cvt_pk_bf16_f32, round to nearest even
    return r.u;
}

// A head's reference max only moves when a tile's max exceeds it by more than this (log2 units);
// in between, weights exp2(s - m) stay below 2^8 and the accumulators need no rescale.
constexpr float kRescaleSlack = 8.f;

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier and the operand prefetch depths.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kQkAhead = 3;   // score steps (2 reads each) in flight ahead of their MFMAs
constexpr int kPvAhead = 4;   // value dim-blocks (2 transposed reads each) in flight

__global__ __launch_bounds__(kAttnThreads, 1) void sparse_mla_bf16_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kStages * kStageBytes];
    __shared__ uint32_t phys[kSplitSlots];
    __shared__ uint32_t tile_valid[kTilesPerSplit];
    __shared__ __attribute__((aligned(16))) uint32_t pfrag[kAttnWaves][kWave * 4];   // P fragments
    __shared__ float xalpha[kAttnWaves][16];    // per-head rescale factor of the current tile
    __shared__ float xsum[kAttnWaves][16];      // per-head weight sums at the end
    __shared__ int s_first, s_last, s_rescale;

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

    // Heads: wave w scores heads hown .. hown+16; its pair (w, w^1) shares heads hpair .. hpair+32;
    // for the values, wave w covers dims dim0 .. dim0+256 of both head blocks of the pair.
    const int hown = hb * kHeadsPerBlock + wid * 16;
    const int hpair = hb * kHeadsPerBlock + (wid >> 1) * 32;
    const int dim0 = (wid & 1) * 256;
    const bool own_ok = hown < p.H;
    const bool blk0_ok = hpair < p.H;          // head block hpair .. +16
    const bool blk1_ok = hpair + 16 < p.H;     // head block hpair+16 .. +32

    // ---- Q (B operand of the score MFMA): lane holds head (lane & 15), dims 32kk + 8(lane >> 4) .. +8
    bf16x8_t qv[18];
    if (own_ok) {
        const uint16_t* qrow = p.q + row * p.q_row_stride + (int64_t)(hown + (lane & 15)) * kDqk + 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) qv[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
    }

    // ---- A4: translate this split's slots to physical token records ----
    const int slot0 = split * kSplitSlots;
    const int nslots = min(kSplitSlots, p.k - slot0);
    const int req = p.row_req ? p.row_req[row] : 0;
    const bool req_ok = req >= 0 && req < p.num_reqs;
    if (tid == 0) { s_first = kSplitSlots; s_last = -1; }
    if (tid < kTilesPerSplit) tile_valid[tid] = 0u;
    __syncthreads();
    int32_t pos[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int j = tid + r * kAttnThreads;
        const int jc = j < nslots ? j : 0;   // unconditional loads (clamped), so both are in flight together
        pos[r] = p.idx[row * p.k + slot0 + jc];
        if (!(j < nslots && req_ok)) pos[r] = -1;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int j = tid + r * kAttnThreads;
        uint32_t ph = kNoToken;
        const int64_t lp = pos[r] >> 6;
        if (pos[r] >= 0 && lp < p.bt_stride) {
            const int32_t pg = p.block_table[(int64_t)req * p.bt_stride + lp];
            if (pg >= 0 && (int64_t)pg < p.num_pages) ph = (uint32_t)pg * kPage + (uint32_t)(pos[r] & (kPage - 1));
        }
        phys[j] = ph;
        const uint64_t vb = __ballot(ph != kNoToken);
        if (lane == 0 && vb) {
            const int jw = j - lane;    // first slot of this wave's 64
            atomicMin(&s_first, jw + (int)__builtin_ctzll(vb));
            atomicMax(&s_last, jw + 63 - (int)__builtin_clzll(vb));
            atomicOr(&tile_valid[jw / kTileTok], (uint32_t)vb);
            atomicOr(&tile_valid[jw / kTileTok + 1], (uint32_t)(vb >> 32));
        }
    }
    // Drain every compiler-visible global load here: inside the tile loop the only outstanding
    // vector-memory operations are the tile loads, which the loop waits for explicitly.
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) asm volatile("" : "+a"(qv[kk]));   // Q lives in AGPRs (MFMA B operand)
    const int ntiles = s_last < 0 ? 0 : s_last / kTileTok + 1;
    const uint32_t dummy = s_last < 0 ? 0u : phys[s_first];

    // ---- A5: gather.  Wave w fills tile-local tokens [8w, 8w+8) of a stage: load i of lane l covers
    // LDS bytes w*9216 + 1024 i + 16 l, i.e. token t = 8w + (64i + l) / 72 at 16-byte position
    // (64i + l) % 72, which holds the record's chunk position ^ f(t).
    uint32_t dtok[kLoadsPerWave], doff[kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int qd = kWave * i + lane;
        const int tt = qd / 72;
        const int t = 8 * wid + tt;
        dtok[i] = 4u * (uint32_t)t;
        doff[i] = 16u * (uint32_t)((qd - 72 * tt) ^ swz_key(t));
    }
    const uint32_t wave_lds = lds_offset(ring) + (uint32_t)wid * kWaveTileBytes;
    auto issue_tile = [&](int tile, int stage) {
        const uint32_t m0 = wave_lds + (uint32_t)stage * kStageBytes;
        const uint8_t* phys_tile = (const uint8_t*)phys + tile * kTileTok * 4;
        const uint8_t* src[kLoadsPerWave];
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {   // all slot reads first: the asm below is a compiler barrier
            uint32_t ph = *(const uint32_t*)(phys_tile + dtok[i]);
            ph = ph == kNoToken ? dummy : ph;
            src[i] = p.kv + (uint64_t)ph * kBf16Record + doff[i];
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

    // Per-lane LDS byte offsets inside a stage.
    //  score operand: token (lane & 15) (+16 for the second block), chunk 4kk + g -> ka[kk & 1] + 128 (kk >> 1)
    //  transposed value reads: lane supplies token 4g + ((lane & 15) >> 2) and dims 4(lane & 3)..+3 of a
    //  16-dim block db, i.e. chunk 2db + ((lane >> 1) & 1), half (lane & 1) -> vb[db & 3] + 128 (db >> 2)
    const int g = lane >> 4;
    uint32_t ka[2], vb[4];
    {
        const int lr = lane & 15;
        const int fa = swz_key(lr);
        const int tv = 4 * g + (lr >> 2);
        const int fv = swz_key(tv);
#pragma unroll
        for (int j = 0; j < 2; ++j) ka[j] = lr * kBf16Record + 16 * ((4 * j + g) ^ fa);
#pragma unroll
        for (int j = 0; j < 4; ++j) vb[j] = tv * kBf16Record + 8 * (lane & 1) + 16 * ((2 * j + ((lane >> 1) & 1)) ^ fv);
    }

    float m_run = -INFINITY, l_run = 0.f;   // own heads: exp2-domain reference max, weight sum (lane's tokens)
    f32x4_t oacc[2][16];                    // [head block of the pair][16-dim block of this wave's half]
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int d = 0; d < 16; ++d) oacc[b][d] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < kStages - 1 && t < ntiles; ++t) issue_tile(t, t);

    for (int it = 0; it < ntiles; ++it) {
        const int stage = it % kStages;
        const int ahead = min(kStages - 2, ntiles - 1 - it);   // tiles issued after `it`
        if (ahead >= 2) wait_vmcnt<2 * kLoadsPerWave>();
        else if (ahead == 1) wait_vmcnt<kLoadsPerWave>();
        else wait_vmcnt<0>();
        zero_invalid(it, stage);
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();   // tile `it` visible; every wave is done with tile it-1
        if (it + kStages - 1 < ntiles) issue_tile(it + kStages - 1, (it + kStages - 1) % kStages);
        // Every wave passes both barriers of every tile, whether or not its heads exist.
        const uint8_t* sb = ring + stage * kStageBytes;
        const uint32_t vmask = tile_valid[it];

        // ---- A7 + A8: scores and online softmax of this wave's own 16 heads ----
        if (own_ok) {
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 18; ++kk) {
                const uint8_t* ap = sb + ka[kk & 1] + 128 * (kk >> 1);
                const bf16x8_t a0 = *(const bf16x8_t*)(ap);
                const bf16x8_t a1 = *(const bf16x8_t*)(ap + 16 * kBf16Record);
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qv[kk], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qv[kk], s1, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < kQkAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
            for (int i = 0; i < 18 - kQkAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * kQkAhead, 0);

            // lane: head (lane & 15), tokens 4g + i (block 0) and 16 + 4g + i (block 1)
            float sv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) { sv[i] = s0[i] * p.scale_log2; sv[4 + i] = s1[i] * p.scale_log2; }
            if (vmask != 0xffffffffu) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (!((vmask >> (4 * g + i)) & 1u)) sv[i] = -INFINITY;
                    if (!((vmask >> (16 + 4 * g + i)) & 1u)) sv[4 + i] = -INFINITY;
                }
            }
            float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                             fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
            mt = head_max(mt);
            float alpha = 1.f;
            if (mt > m_run + kRescaleSlack) {     // same decision in all four lanes of the head
                alpha = __builtin_amdgcn_exp2f(m_run - mt);   // 0 while nothing has been accumulated
                m_run = mt;
                l_run *= alpha;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;
            float pw[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pw[j] = __builtin_amdgcn_exp2f(sv[j] - m_use);
                l_run += pw[j];
            }
            uint4 pf;
            pf.x = pack_bf16x2_hw(pw[0], pw[1]);
            pf.y = pack_bf16x2_hw(pw[2], pw[3]);
            pf.z = pack_bf16x2_hw(pw[4], pw[5]);
            pf.w = pack_bf16x2_hw(pw[6], pw[7]);
            *(uint4*)&pfrag[wid][4 * lane] = pf;
            if (lane < 16) xalpha[wid][lane] = alpha;
        }
        wait_lgkmcnt0();                 // s_barrier does not wait for LDS writes by itself
        __builtin_amdgcn_s_barrier();   // P fragments and rescale factors of both waves published
        if (!blk0_ok) continue;          // no head of this pair exists (uniform across the pair)

        // ---- A9: O^T += V^T P^T for both head blocks of the pair over this wave's 256 dims ----
        const int w0 = wid & ~1;
        float a_blk[2];
        a_blk[0] = blk0_ok ? xalpha[w0][lane & 15] : 1.f;
        a_blk[1] = blk1_ok ? xalpha[w0 + 1][lane & 15] : 1.f;
        bf16x8_t pb[2];
        pb[0] = *(const bf16x8_t*)&pfrag[w0][4 * lane];
        pb[1] = *(const bf16x8_t*)&pfrag[w0 + 1][4 * lane];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (a_blk[b] != 1.f) {   // rare: a reference max moved (exact 1.0 otherwise)
#pragma unroll
                for (int d = 0; d < 16; ++d) {
                    oacc[b][d][0] *= a_blk[b]; oacc[b][d][1] *= a_blk[b];
                    oacc[b][d][2] *= a_blk[b]; oacc[b][d][3] *= a_blk[b];
                }
            }
        }
        const uint8_t* vp0 = sb + 128 * (dim0 / 64);
        // Two copies of the value loop (both head blocks / first block only) keep the branch out of it.
        auto value_pass = [&](auto both_blocks) {
#pragma unroll
            for (int d = 0; d < 16; ++d) {   // dim block within this wave's half
                const uint8_t* vp = vp0 + vb[d & 3] + 128 * (d >> 2);
                union { bf16x8_t v; i16x4_t h[2]; } va;
                va.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(vp));
                va.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4_t*)(vp + 16 * kBf16Record));
                oacc[0][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, pb[0], oacc[0][d], 0, 0, 0);
                if constexpr (decltype(both_blocks)::value)
                    oacc[1][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, pb[1], oacc[1][d], 0, 0, 0);
            }
            constexpr int kM = decltype(both_blocks)::value ? 2 : 1;
#pragma unroll
            for (int i = 0; i < kPvAhead; ++i) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
            for (int i = 0; i < 16 - kPvAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, kM, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kM * kPvAhead, 0);
        };
        if (blk1_ok) value_pass(std::true_type{});
        else value_pass(std::false_type{});
    }

    // ---- A10: epilogue.  Own heads: total weight and LSE; both blocks: normalize and write ----
    const float l_tot = head_sum(l_run);
    if (own_ok && lane < 16) xsum[wid][lane] = l_tot;
    __syncthreads();
    if (!blk0_ok) return;
    if (own_ok && lane < 16) {
        const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        const int64_t hix = row * p.H + hown + lane;
        if (p.n_splits == 1) {
            if (p.lse) p.lse[hix] = lse_v;
        } else {
            p.ws_lse[((int64_t)rloc * p.n_splits + split) * p.H + hown + lane] = lse_v;
        }
    }
    const int w0 = wid & ~1;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (b == 1 && !blk1_ok) break;
        const float lt = xsum[w0 + b][lane & 15];
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int head = hpair + 16 * b + (lane & 15);
        if (p.n_splits == 1) {
            uint16_t* orow = p.out + (row * p.H + head) * (int64_t)kDv + dim0 + 4 * g;
#pragma unroll
            for (int d = 0; d < 16; ++d) {
                uint2 w;
                w.x = pack_bf16x2_hw(oacc[b][d][0] * inv, oacc[b][d][1] * inv);
                w.y = pack_bf16x2_hw(oacc[b][d][2] * inv, oacc[b][d][3] * inv);
                *(uint2*)(orow + 16 * d) = w;
            }
        } else {
            const int64_t part = ((int64_t)rloc * p.n_splits + split) * p.H + head;
            float* wo = p.ws_o + part * kDv + dim0 + 4 * g;
#pragma unroll
            for (int d = 0; d < 16; ++d) {
                f32x4_t v = {oacc[b][d][0] * inv, oacc[b][d][1] * inv, oacc[b][d][2] * inv, oacc[b][d][3] * inv};
                *(f32x4_t*)(wo + 16 * d) = v;
            }
        }
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
    w.x = pack_bf16x2_hw(acc[0], acc[1]);
    w.y = pack_bf16x2_hw(acc[2], acc[3]);
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
