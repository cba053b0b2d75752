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
// Work decomposition.  One workgroup of 16 waves is the only workgroup on its CU and owns one work
// item: a run of consecutive units of one row (a unit is 512 consecutive index slots) for a block of
// 64 heads.  A split is one unit (FP8 caches: two units run one after the other with one softmax
// state); the number of splits depends on k and the cache type only, so the reduction order of a row
// never depends on the batch.  Large launches give a workgroup 2 or 4 consecutive splits of a row, one
// after the other (the index translation and Q serve them all); small launches split the 64 heads over
// 2 or 4 workgroups of 32 or 16 heads.  Either way every split is reduced in the same order with its
// own softmax state, so the bits do not change.  The split's slots are processed
// in tiles of 32 tokens through a 3-stage LDS ring.  The gather of a tile (36 loads of 1 KB, direct
// to LDS with global_load_lds_dwordx4) is spread over all 16 waves: the rate at which random records
// arrive grows with the number of waves per CU issuing loads, measured on MI355X.  Records are stored
// unpadded (1152 B); the 16-byte chunks of tile-local token t are XOR-swizzled with f(t) = (t >> 1) & 7,
// the mapping measured to keep the operand reads below free of LDS bank conflicts on gfx950.  FP8
// caches: a tile is 21 loads of 656-B records, issued by the 8 value waves alone in a phase where
// they would otherwise wait; both roles read the e4m3 codes from the ring and widen them in registers.
//
// Roles (at most 128 registers per wave at 16 waves per CU):
//   score waves 0..7:  wave (hb, half) computes the partial scores of heads hb*16 .. +16 over dims
//                      288*half .. +288 for the tile's 32 tokens with Q in registers:
//                        S^T[16 tok x 16 heads] += K[16 tok x 32 dims] . Q^T    (A = K rows, ds_read_b128)
//                      The second halves publish their partials through LDS; the first halves add them
//                      (first half + second half, always in this order), keep the online-softmax state
//                      of their 16 heads and publish the bf16 weights P and the rescale factors.
//   value waves 8..15: wave 8 + v accumulates dims 64v .. +64 of all 64 heads:
//                        O^T[16 dims x 16 heads] += V^T[16 dims x 32 tok] . P^T[32 tok x 16 heads]
//                      (A = V^T via ds_read_b64_tr_b16 transposed reads, FP8: ds_read_b64_tr_b8 of the
//                      codes, each feeding 4 head blocks).
//   The S^T accumulator layout already holds a head's token weights in the B-operand layout of the
//   value MFMA, so no register transpose is needed.
//
// Softmax is an fp32 online softmax in the exp2 domain, tiles in slot order.  A head's reference
// max only moves when a tile's max exceeds it by more than 2^8 (a decision that depends on the
// row's own scores only), so the accumulators are rescaled rarely.  When a row has several splits,
// each writes its normalized partial (O_s rounded to bf16, lse_s in fp32) to the workspace, and a
// combine kernel merges the splits of a row in split order.  Nothing uses floating-point atomics.
//
// Invalid slots (index < 0, request/page out of range) load record 0 of their cache, are zeroed in
// LDS after arrival and get score -inf, so every loading wave issues the same number of direct-to-LDS
// loads for every tile and the vmcnt bookkeeping below stays exact.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

constexpr int kAttnWaves = 16;
constexpr int kAttnThreads = kAttnWaves * kWave;               // 1024
constexpr int kScoreWaves = 8;
constexpr int kTileTok = 32;
constexpr int kMaxUnitTiles = kMaxUnitSlots / kTileTok;        // 24
constexpr int kStageBytes = kTileTok * kBf16Record;             // 36864
constexpr int kTileLoads = kStageBytes / (16 * kWave);          // 36 direct-to-LDS loads of 1 KB per tile
static_assert(kTileLoads * 16 * kWave == kStageBytes, "tile must split into whole wave loads");
constexpr int kMaxLoadsPerWave = (kTileLoads + kAttnWaves - 1) / kAttnWaves;   // 3 (waves 0..3), else 2
// FP8 records: [512 e4m3 codes | 4 fp32 scales, one per 128 latent dims | 64 bf16 rope] = 656 B,
// 41 chunks of 16 B.  In a stage, tokens 0..15 sit at 656 t and tokens 16..31 at 656 t + 128: at the
// 656-byte pitch tokens t and t + 16 start in the same LDS bank, and the transposed value reads take a
// token from each half in one access.  The stage's 1320 16-byte positions (8 of them the gap) take 21
// loads of 1 KB, the last with 40 active lanes.
constexpr int kFp8Chunks = kFp8Record / 16;                           // 41
constexpr int kFp8Gap = 128;                                          // bytes between tokens 15 and 16
constexpr int kFp8HalfPos = 16 * kFp8Chunks;                          // 656 positions of tokens 0..15
constexpr int kFp8StageBytes = kTileTok * kFp8Record + kFp8Gap;       // 21120
constexpr int kFp8StagePos = kFp8StageBytes / 16;                     // 1320
constexpr int kFp8TileLoads = (kFp8StagePos + kWave - 1) / kWave;     // 21
static_assert(kFp8StageBytes % 16 == 0 && kFp8Gap % 16 == 0, "FP8 stages must stay 16-byte aligned");
constexpr int kFp8Stages = 3;                                         // FP8 ring depth
// byte offset of tile-local token t in an FP8 stage
__device__ __forceinline__ int fp8_tok(int t) { return t * kFp8Record + (t >= 16 ? kFp8Gap : 0); }
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
    int32_t k;              // slots of a row: k_main from idx over kv, then k - k_main from idx_win over kv_win
    int32_t k_main;
    const uint8_t* kv_win;  // sliding-window cache (null: none)
    int64_t num_pages_win;
    const int32_t* block_table_win;
    int64_t bt_win_stride;
    const int32_t* idx_win;
    int32_t H;
    int32_t n_splits;       // splits of a row (one softmax state and one partial each)
    int32_t n_units;        // units of a row (a split is 1 unit, FP8: 2)
    int32_t unit_slots;     // slots of a unit: 512, or a larger multiple of 64 (<= 768) with a window part
    int32_t n_hblocks;
    int32_t heads_per_wg;   // 64, 32 or 16: heads of one workgroup (each head's arithmetic is the same)
    int32_t units_per_wg;   // 1, 2 or 4 consecutive units of a row run by one workgroup, one after the other
    float scale_log2;
    int32_t row0;
    uint16_t* out;
    float* lse;
    void* ws_o;          // [rows][splits][H][512] split partials: bf16 (bf16 cache) or fp16 (FP8 cache, normalized)
    float* ws_lse;       // fp32 [rows][splits][H]
    float* ws_gsc;       // FP8: fp32 [rows][splits][4], the factor 2^(e - 127) of each 128-dim group's partials
    const float* sink;   // fp32 [H] per-head sink logits (natural-log units of the scaled scores), or null
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

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

__device__ __forceinline__ uint32_t pack_f16x2_rne(float lo, float hi) {
    typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f2;
    typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 h2;
    union { h2 v; uint32_t u; } r;
    r.v = __builtin_convertvector((f2){lo, hi}, h2);   // round to nearest even
    return r.u;
}

// Two e4m3 codes (bytes 0-1, or 2-3 when HI, of w) -> two fp16 values.  The scaled conversion with
// scale 1.0 is exact: every e4m3 value is an fp16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
    union { decltype(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(0, 1.f, false)) v; uint32_t u; } r;
    r.v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.f, HI);
    return r.u;
}

// A head's reference max only moves when a tile's max exceeds it by more than this (log2 units);
// in between, weights exp2(s - m) stay below 2^8 and the accumulators need no rescale.
constexpr float kRescaleSlack = 8.f;

// KV_FP8: the ring holds the FP8 records as they are, and both roles read the e4m3 codes from it and
// widen them in registers (exact: every e4m3 value is an fp16 value).  A score wave reads 8 codes of a
// token per MFMA operand; a value wave reads 8 tokens' codes of one dim with one transposed LDS read
// (ds_read_b64_tr_b8).  The latent part of the scores is an fp16 product: each score wave holds its
// latent Q slice in fp16, divided per head by a power of two 2^e that keeps it inside the fp16 range
// (e = 0 unless |q| reaches 2^15).  Entries of at least 2^-14 * 2^e convert from bf16 exactly; smaller
// ones land in fp16's subnormal range, off by at most 2^-25 * 2^e, far below the score's own fp32
// rounding.  The rope part stays bf16.  The scales are applied in fp32: the score waves keep one
// partial per 128-dim scale group and sum 2^e x scale x partial; the softmax publishes the fp32
// weights, and a value wave, whose 64 dims lie in one group, multiplies them by that group's scales,
// rounds to fp16 and runs the value product in fp16 on the codes as they are.
// At the magnitudes these scales produce, rounding the scaled values, or the scaled weights, to bf16
// costs far more accuracy than the fp16 weights.
template <bool KV_FP8>
__global__ __launch_bounds__(kAttnThreads, 1) void sparse_mla_kernel(const AttnParams p) {
    // Ring depth: tiles are loaded kStages - 1 tiles ahead.  An FP8 tile is 21 KB, so FP8 keeps more of
    // them in flight.
    constexpr int kStages = KV_FP8 ? kFp8Stages : 3;
    constexpr int kRingBytes = KV_FP8 ? kStages * kFp8StageBytes : kStages * kStageBytes;
    constexpr int kRecBytes = KV_FP8 ? kFp8Record : kBf16Record;
    constexpr int kRingStage = KV_FP8 ? kFp8StageBytes : kStageBytes;
    __shared__ __attribute__((aligned(16))) uint8_t ring[kRingBytes];
    // Units run by one workgroup (FP8: the 2 units of its split) and their slots' physical records.
    constexpr int kMaxGroup = KV_FP8 ? 2 : 4;
    __shared__ uint32_t phys[kMaxGroup * kMaxUnitSlots];
    __shared__ uint32_t tile_valid[kMaxGroup * kMaxUnitTiles];
    // Weights of each head block: bf16 B-operand fragments (bf16 caches), or the lane's 8 fp32
    // weights (FP8 caches; each value wave scales them by its group's token scales).
    __shared__ __attribute__((aligned(16))) uint32_t pfrag[4][KV_FP8 ? 8 : 4][kWave];
    // Second-half partial scores of each head block.
    __shared__ __attribute__((aligned(16))) f32x4_t xs_own[4][2][kWave];
    __shared__ float xalpha[4][16];    // per-head rescale factor of the current tile
    // Per-head output multiplier at the end of a split, one table per split parity (bf16): after a
    // split's final barrier the score waves may run through a next split without tiles (no barrier)
    // into its end before the value waves have read this split's multipliers.  FP8 workgroups run one
    // split each and keep one table.
    constexpr int kMulTables = KV_FP8 ? 1 : 2;
    __shared__ float xmul[kMulTables][4][16];
    __shared__ int s_first[kMaxGroup], s_last[kMaxGroup];
    auto xs = [&](int b, int j) -> f32x4_t* { return &xs_own[b][j][0]; };
    auto pw32 = [&](int b, int j) -> f32x4_t* { return (f32x4_t*)&pfrag[b][0][0] + j * kWave; };   // FP8 weights

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane >> 4;

    // Work item: consecutive items (the splits / head blocks of one row) go to the same XCD, since
    // workgroups are dispatched round-robin over the 8 XCDs.
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3, per = nwg >> 3, rem = nwg & 7;
    const int item = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int hb_item = item % p.n_hblocks;
    const int rs = item / p.n_hblocks;
    // A workgroup runs units split0 .. split0 + ns - 1 of its row.  bf16: each unit is a split; FP8:
    // units 2s and 2s + 1 form split s, one softmax state over both (the launch gives FP8 workgroups
    // whole splits).
    constexpr int kUnitsPerSplit = KV_FP8 ? kFp8UnitsPerSplit : 1;
    const int n_groups = (p.n_units + p.units_per_wg - 1) / p.units_per_wg;
    const int split0 = (rs % n_groups) * p.units_per_wg;      // first unit of this workgroup
    const int ns = min(p.units_per_wg, p.n_units - split0);  // its units split0 .. split0 + ns - 1
    const int rloc = rs / n_groups;
    const int64_t row = (int64_t)p.row0 + rloc;
    const int head0 = hb_item * p.heads_per_wg;
    const int nhb = min(p.heads_per_wg / 16, (p.H - head0) / 16);   // valid 16-head blocks (H % 16 == 0)

    const bool is_score = wid < kScoreWaves;
    const int shb = wid & 3, half = (wid >> 2) & 1;   // score waves: head block, dim half
    const int vdim0 = 64 * (wid - kScoreWaves);      // value waves: first of their 64 dims
    const bool score_ok = is_score && shb < nhb;

    // ---- Q slice (B operand of the score MFMA): lane holds head (lane & 15), dims 288 half + 32 kk + 8 g .. +8
    bf16x8_t qv[9];
    if (score_ok) {
        const uint16_t* qrow = p.q + row * p.q_row_stride + (int64_t)(head0 + shb * 16 + (lane & 15)) * kDqk +
                               288 * half + 8 * g;
#pragma unroll
        for (int kk = 0; kk < 9; ++kk) qv[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
    } else {
#pragma unroll
        for (int kk = 0; kk < 9; ++kk) qv[kk] = (bf16x8_t){};
    }

    // ---- A4: translate the slots of this workgroup's splits to physical token records: local slot j
    // (split j / 512 of the group) is slot 512 split0 + j of the row.  Each thread owns local slots tid
    // and tid + 1024; both index loads go out before either page-table load. ----
    const int U = p.unit_slots;                  // slots per unit (a multiple of 64)
    const int slot_base = split0 * U;
    const int nslot = min(ns * U, p.k - slot_base);
    const int req = p.row_req ? p.row_req[row] : 0;
    const bool req_ok = req >= 0 && req < p.num_reqs;
    if (tid < kMaxGroup) { s_first[tid] = U; s_last[tid] = -1; }
    if (tid < kMaxGroup * kMaxUnitTiles) tile_valid[tid] = 0u;
    __syncthreads();
    {
        // Row slots [0, k_main) list positions of the main cache (idx, block_table); slots [k_main, k)
        // list positions of the window cache (idx_win, block_table_win).
        constexpr int kRounds = (kMaxGroup * kMaxUnitSlots + kAttnThreads - 1) / kAttnThreads;   // 2 or 3
        const int k_win = p.k - p.k_main;
        int32_t pos[kRounds];
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int j = tid + kAttnThreads * r;
            const int gs = slot_base + (j < nslot ? j : 0);
            const int32_t* ip = gs < p.k_main ? p.idx + row * p.k_main + gs : p.idx_win + row * k_win + (gs - p.k_main);
            pos[r] = *ip;
        }
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            const int j = tid + kAttnThreads * r;
            if (j >= ns * U) break;   // uniform in the wave (64 divides U)
            int32_t ps = pos[r];
            if (!(j < nslot && req_ok)) ps = -1;
            const bool win = slot_base + j >= p.k_main;
            const int32_t* bt = win ? p.block_table_win : p.block_table;
            const int64_t bts = win ? p.bt_win_stride : p.bt_stride;
            const int64_t npg = win ? p.num_pages_win : p.num_pages;
            uint32_t ph = kNoToken;
            const int64_t lp = ps >> 6;
            if (ps >= 0 && lp < bts) {
                const int32_t pg = bt[(int64_t)req * bts + lp];
                if (pg >= 0 && (int64_t)pg < npg) ph = (uint32_t)pg * kPage + (uint32_t)(ps & (kPage - 1));
            }
            phys[j] = ph;
            const uint64_t vbits = __ballot(ph != kNoToken);
            if (lane == 0 && vbits) {
                const int jw = j - lane;                        // first slot of this wave's 64
                const int ls = jw / U, jl = jw % U;
                atomicMin(&s_first[ls], jl + (int)__builtin_ctzll(vbits));
                atomicMax(&s_last[ls], jl + 63 - (int)__builtin_clzll(vbits));
                atomicOr(&tile_valid[ls * kMaxUnitTiles + jl / kTileTok], (uint32_t)vbits);
                atomicOr(&tile_valid[ls * kMaxUnitTiles + jl / kTileTok + 1], (uint32_t)(vbits >> 32));
            }
        }
    }
    // Drain every compiler-visible global load here: inside the tile loop the only outstanding
    // vector-memory operations are the tile loads, which the loop waits for explicitly.
    wait_vmcnt<0>();
    __syncthreads();
    // FP8: the latent steps of the Q slice in fp16, divided by 2^e for the head (lane & 15); the rope
    // steps (the last two of the second half) stay bf16.
    float qscale = 1.f;
    if constexpr (KV_FP8) {
        if (score_ok) {
            const int nlat = half ? 7 : 9;
            float mx = 0.f;
#pragma unroll
            for (int kk = 0; kk < 9; ++kk) {
                if (kk < nlat) {
                    union { bf16x8_t v; uint32_t w[4]; } q;
                    q.v = qv[kk];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(q.w[e] << 16)),
                                             fabsf(__uint_as_float(q.w[e] & 0xffff0000u))));
                }
            }
            mx = head_max(mx);
            const int ex = (int)((__float_as_uint(mx) >> 23) & 0xffu) - 127;
            const int e2 = ex > 14 ? ex - 14 : 0;
            qscale = __uint_as_float((uint32_t)(127 + e2) << 23);
            const float inv = __uint_as_float((uint32_t)(127 - e2) << 23);
#pragma unroll
            for (int kk = 0; kk < 9; ++kk) {
                if (kk < nlat) {
                    union { bf16x8_t v; uint32_t w[4]; } q;
                    q.v = qv[kk];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        q.w[e] = pack_f16x2_rne(__uint_as_float(q.w[e] << 16) * inv,
                                                __uint_as_float(q.w[e] & 0xffff0000u) * inv);
                    qv[kk] = q.v;
                }
            }
        }
    }
#pragma unroll
    for (int kk = 0; kk < 9; ++kk) asm volatile("" : "+v"(qv[kk]));   // opaque: Q is never re-loaded
    // The split being run (ls of the group): its tile count (tiles end at its last valid slot), a valid
    // record for the loads of its invalid slots (record 0 if it has none), and its slot offset.
    // Tile t of the split sits in ring stage (sbase + t) % kStages; sbase runs on from split to split,
    // since a split with at least kStages - 1 tiles requests the next split's first kStages - 1 tiles in
    // the slots where its own tiles ntiles, ntiles + 1, ... would go (pf), so the next split starts with
    // them in flight.
    int cur = 0, ntiles = 0, cur_slot0 = 0, sbase = 0, nx_ntiles = 0;
    bool pf = false, pref_done = false;   // this split requests the next one's first tiles / was requested
    auto split_tiles = [&](int ls) {
        const int last = s_last[ls];
        return __builtin_amdgcn_readfirstlane(last < 0 ? 0 : last / kTileTok + 1);
    };
    auto begin_split = [&](int ls) {
        cur = ls;
        cur_slot0 = ls * U;
        ntiles = split_tiles(ls);
        nx_ntiles = ls + 1 < ns ? split_tiles(ls + 1) : 0;
        pf = ntiles >= kStages - 1 && nx_ntiles >= 1;
    };
    auto end_split = [&]() {
        pref_done = pf;
        sbase = (sbase + ntiles) % kStages;
    };
    auto stg = [&](int t) { return (sbase + t) % kStages; };

    // ---- A5: gather.  Load instruction i of a tile covers stage bytes 1024 i .. +1024.  bf16: all 16
    // waves load, wave w issues i = w, w + 16, w + 32 (below 36).  FP8: the 8 value waves load (after
    // the second barrier, while the score waves run the softmax), value wave v issues i = v, v + 8,
    // v + 16 (below 21).  Lane l of instruction i moves 16-byte chunk Q = 64 i + l of the stage.
    // bf16: token t = Q / 72 at 16-byte position Q % 72, which holds the record's chunk position ^ f(t).
    // FP8: positions below 656 hold token Q / 41, chunk Q % 41; the 8 gap positions are not loaded;
    // position Q >= 664 holds token 16 + (Q - 664) / 41, chunk (Q - 664) % 41; positions past the stage
    // (Q >= 1320, lanes 40..63 of load 20) are not loaded.
    constexpr int kLoads = KV_FP8 ? kFp8TileLoads : kTileLoads;
    constexpr int kLoadWaves = KV_FP8 ? kAttnWaves - kScoreWaves : kAttnWaves;
    static_assert(kLoads <= kMaxLoadsPerWave * kLoadWaves, "loads per wave");
    const int lw = KV_FP8 ? wid - kScoreWaves : wid;   // loading wave index (FP8 score waves: < 0)
    const int nload = (KV_FP8 && lw < 0) ? 0
                             : (lw < kLoads ? 1 : 0) + (lw + kLoadWaves < kLoads ? 1 : 0) +
                                   (lw + 2 * kLoadWaves < kLoads ? 1 : 0);   // loads of this wave per tile (uniform)
    // Per-lane offsets of load r: the token's slot (4 bytes each) and the chunk's byte offset in the
    // record.  Recomputed at every issue from an opaque copy of the lane id, so that they are not held
    // in registers across the tile loop.
    auto load_offsets = [&](uint32_t* dtok, uint32_t* doff) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int r = 0; r < kMaxLoadsPerWave; ++r) {
            const int i = lw + kLoadWaves * r;
            const int qd = kWave * (i < kLoads ? i : 0) + ln;
            if (KV_FP8) {
                const int hi = qd >= kFp8HalfPos;
                int qc = hi ? qd - kFp8HalfPos - kFp8Gap / 16 : qd;   // chunk index within the half
                qc = qc < 0 ? 0 : (qc < kFp8HalfPos ? qc : kFp8HalfPos - 1);   // gap and tail: not loaded
                const int t = qc / kFp8Chunks;
                dtok[r] = 4u * (uint32_t)(t + 16 * hi);
                doff[r] = 16u * (uint32_t)(qc - kFp8Chunks * t);
            } else {
                const int t = qd / 72;
                dtok[r] = 4u * (uint32_t)t;
                doff[r] = 16u * (uint32_t)((qd - 72 * t) ^ swz_key(t));
            }
        }
    };
    const uint32_t ring_lds = lds_offset(ring);
    // FP8: whether stage position qd is loaded (the gap sits in load 10, load 20 ends the stage)
    auto fp8_pos_loaded = [](int qd) {
        return qd < kFp8StagePos && (qd < kFp8HalfPos || qd >= kFp8HalfPos + kFp8Gap / 16);
    };
    // The lane id behind a compiler barrier: per-lane offsets derived from it are recomputed where they
    // are used instead of being held in registers across the tile loop.
    auto opaque_lane = [&]() {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        return ln;
    };
    // Slots at or past k_main of the row (the window part) read the window cache; an invalid slot loads
    // record 0 of its cache (always present: num_pages >= 1), whose bytes are replaced by zeros.
    // (slot0 + tile * 32 is the tile's first slot in the group; the group starts at row slot slot_base.)
    auto issue_tile_of = [&](int slot0, int tile, int stage) {
        if (KV_FP8 && nload == 0) return;
        const uint8_t* phys_tile = (const uint8_t*)(phys + slot0 + tile * kTileTok);
        uint32_t dtok[kMaxLoadsPerWave], doff[kMaxLoadsPerWave];
        load_offsets(dtok, doff);
        const uint8_t* src[kMaxLoadsPerWave];
        const int win_from = p.k_main - (slot_base + slot0 + tile * kTileTok);   // tile tokens >= this: window
#pragma unroll
        for (int r = 0; r < kMaxLoadsPerWave; ++r) {   // all slot reads first: the asm below is a compiler barrier
            uint32_t ph = *(const uint32_t*)(phys_tile + dtok[r]);
            ph = ph == kNoToken ? 0u : ph;
            src[r] = ((int)(dtok[r] >> 2) >= win_from ? p.kv_win : p.kv) + (uint64_t)ph * kRecBytes + doff[r];
        }
        const uint32_t m0 = ring_lds + (uint32_t)stage * kRingStage + 1024u * (uint32_t)lw;
        const int ln = opaque_lane();
        auto fp8_lane_loads = [&](int r) { return fp8_pos_loaded(kWave * (lw + kLoadWaves * r) + ln); };
        if (!KV_FP8) {
            dma_b128(src[0], m0);
            dma_b128(src[1], m0 + 1024u * kAttnWaves);
            if (nload == 3) dma_b128(src[2], m0 + 2048u * kAttnWaves);
        } else {   // value waves 0..4: 3 loads (the third of wave 4 is the 40-lane load), 5..7: 2; a load
                   // is never issued with no active lane, so the wave's vmcnt counts stay exact
            if (fp8_lane_loads(0)) dma_b128(src[0], m0);
            if (fp8_lane_loads(1)) dma_b128(src[1], m0 + 1024u * kLoadWaves);
            if (nload == 3 && fp8_lane_loads(2)) dma_b128(src[2], m0 + 2048u * kLoadWaves);
        }
    };
    auto issue_tile = [&](int tile, int stage) { issue_tile_of(cur_slot0, tile, stage); };
    // The request that would be tile `t` of this split (t >= ntiles) is tile t - ntiles of the next split.
    auto issue_ahead = [&](int t) {
        if (t < ntiles) issue_tile(t, stg(t));
        else if (pf && t - ntiles < nx_ntiles) issue_tile_of(cur_slot0 + U, t - ntiles, stg(t));
    };
    // Zero this wave's chunks of invalid tokens (after their dummy data has landed).
    auto zero_invalid = [&](int tile, int stage) {
        const uint32_t vm = tile_valid[cur * kMaxUnitTiles + tile];
        if (vm != 0xffffffffu) {
            uint8_t* sbase = ring + stage * kRingStage;
            const int ln = opaque_lane();
#pragma unroll
            for (int r = 0; r < kMaxLoadsPerWave; ++r) {
                if (r < nload) {
                    const int qd = kWave * (lw + kLoadWaves * r) + ln;
                    int t;
                    if (KV_FP8) {
                        if (!fp8_pos_loaded(qd)) continue;
                        t = qd < kFp8HalfPos ? qd / kFp8Chunks : 16 + (qd - kFp8HalfPos - kFp8Gap / 16) / kFp8Chunks;
                    } else {
                        t = qd / 72;
                    }
                    if (!((vm >> t) & 1u)) *(uint4*)(sbase + 16 * qd) = make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
    };
    // Per-lane LDS byte offsets inside a stage.
    //  bf16 score operand: token (lane & 15) (+16 for the second block), chunk 4kk + g -> ka[kk & 1] + 128 (kk >> 1)
    //  bf16 transposed value reads: lane supplies token 4g + ((lane & 15) >> 2) and dims 4(lane & 3)..+3 of a
    //  16-dim block db, i.e. chunk 2db + ((lane >> 1) & 1), half (lane & 1) -> vb[db & 3] + 128 (db >> 2)
    //  FP8 score operand: token (lane & 15) at ka[0] (+16: ka[1]); the step's codes at byte dim + 8g
    //  FP8 transposed value reads (ds_read_b64_tr_b8: lane i of a 16-lane group receives byte i & 7 of the
    //  8 bytes supplied by lanes 2e + (i >> 3), e = 0..7): lane supplies token T = 4g + e (e < 4) or
    //  16 + 4g + e - 4 (e >= 4) for e = (lane & 15) >> 1, and codes 8(lane & 1)..+7 of a 16-dim block, so
    //  lane i receives dim i of the 8 tokens in the order of the weights' MFMA operand -> vb[0] + dim0
    uint32_t ka[2], vb[4];
    {
        const int lr = lane & 15;
        if constexpr (!KV_FP8) {
            const int fa = swz_key(lr);
            const int tv = 4 * g + (lr >> 2);
            const int fv = swz_key(tv);
#pragma unroll
            for (int j = 0; j < 2; ++j) ka[j] = lr * kBf16Record + 16 * ((4 * j + g) ^ fa);
#pragma unroll
            for (int j = 0; j < 4; ++j) vb[j] = tv * kBf16Record + 8 * (lane & 1) + 16 * ((2 * j + ((lane >> 1) & 1)) ^ fv);
        } else {
            ka[0] = fp8_tok(lr);
            ka[1] = fp8_tok(16 + lr);
            const int e = lr >> 1;
            const int tv = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
            vb[0] = fp8_tok(tv) + 8 * (lr & 1);
            vb[1] = vb[2] = vb[3] = 0u;
        }
    }

    // Start of split ls of the group (both roles, after the previous split's final barrier): its first
    // tiles are requested.
    auto start_split = [&](int ls) {
        begin_split(ls);
        if (!pref_done)
            for (int t = 0; t < kStages - 1 && t < ntiles; ++t) issue_tile(t, stg(t));
    };

    // Start of tile `it`, common to both roles: wait for this wave's loads of the tile (FP8: only the
    // value waves load), zero its invalid chunks and make the tile visible (first barrier); tile it+1
    // stays in flight.
    auto tile_top = [&](int it) {
        const int stage = stg(it);
        if (it == 0 && pref_done) {   // requested by the previous split: its output stores may follow
            wait_vmcnt<0>();
        } else {   // the requests after tile it (up to tile it + kStages - 2, or the next split's first) stay in flight
            int ahead = 0;
#pragma unroll
            for (int j = 1; j <= kStages - 2; ++j)
                ahead += (it + j < ntiles || (pf && it + j - ntiles < nx_ntiles)) ? 1 : 0;
            wait_vmcnt_upto<3 * (kStages - 2)>(ahead * nload);
        }
        zero_invalid(it, stage);
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        return (const uint8_t*)(ring + stage * kRingStage);
    };
    // After the second barrier of tile it, the stage of tile it-1 receives tile it+2: its value product
    // ends before that barrier.
    // FP8: the value waves issue at the highest wave priority, so their requests go out before the other
    // waves' work in the phase (measured 1% faster per FP8 call; no gain for bf16, where all waves load).
    auto issue_after_second = [&](int it) {
        if (KV_FP8) __builtin_amdgcn_s_setprio(3);
        issue_ahead(it + kStages - 1);
        if (KV_FP8) __builtin_amdgcn_s_setprio(0);
    };
    // The two roles run separate loops with the same barriers per tile, so the registers of
    // one role (Q, the score accumulators) and of the other (the output accumulators) can share storage.
    float m_run = -INFINITY, l_run = 0.f;   // first-half score waves: reference max, weight sum (lane's tokens)
    if (is_score) {
      // The group's units one after the other; each split starts from a fresh softmax state.
      for (int ls = 0; ls < ns; ++ls) {
        start_split(ls);
        const int su = split0 + ls;   // unit of the row
        if (su % kUnitsPerSplit == 0) {
            m_run = -INFINITY;
            l_run = 0.f;
        }
        for (int it = 0; it < ntiles; ++it) {
            const uint8_t* sb = tile_top(it);
            // ---- A7: partial scores over this wave's half of the dims ----
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            if (score_ok) {
                if constexpr (!KV_FP8) {
                    // The K operands are read kKAhead steps ahead of the MFMAs that use them, and the
                    // scheduling barriers keep that order: left to itself, the scheduler put each read
                    // right before its MFMA in the steady-state tile loop, so every MFMA waited for a
                    // whole LDS round trip.
                    constexpr int kKAhead = 2;
                    bf16x8_t ka0[9], ka1[9];
                    auto read_k = [&](int kk) {
                        const int kg = 9 * half + kk;      // kk step over the full 576 dims
                        const uint8_t* ap = sb + ka[kg & 1] + 128 * (kg >> 1);
                        ka0[kk] = *(const bf16x8_t*)(ap);
                        ka1[kk] = *(const bf16x8_t*)(ap + 16 * kBf16Record);
                    };
#pragma unroll
                    for (int kk = 0; kk < kKAhead; ++kk) read_k(kk);
#pragma unroll
                    for (int kk = 0; kk < 9; ++kk) {
                        if (kk + kKAhead < 9) read_k(kk + kKAhead);
                        __builtin_amdgcn_sched_barrier(0);
                        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[kk], qv[kk], s0, 0, 0, 0);
                        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1[kk], qv[kk], s1, 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
                    // One partial per scale group.  Steps kk (32 dims each) of the first half: 0..3 group 0,
                    // 4..7 group 1, 8 group 2; of the second half: 9..11 group 2, 12..15 group 3, 16..17 rope.
                    f32x4_t acc[3][2];
#pragma unroll
                    for (int j = 0; j < 3; ++j) acc[j][0] = acc[j][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                    // As for bf16, the operands are read ahead of their MFMAs: 8 codes of the lane's token
                    // per latent step (widened to fp16 right before the MFMA), 8 bf16 values per rope step.
                    constexpr int kKAhead = 1;
                    const uint8_t* kb0 = sb + ka[0] + 288 * half + 8 * g;   // latent codes, block 0 / 1
                    const uint8_t* kb1 = sb + ka[1] + 288 * half + 8 * g;
                    uint2 kc0[9], kc1[9];
                    bf16x8_t kr0[2], kr1[2];
                    auto read_k = [&](int kk, bool rope) {
                        if (!rope) {
                            kc0[kk] = *(const uint2*)(kb0 + 32 * kk);
                            kc1[kk] = *(const uint2*)(kb1 + 32 * kk);
                        } else {      // rope dims 512 + 32 (kk - 7) + 8g .. +8: bytes 528 + 64 (kk - 7) + 16g
                            kr0[kk - 7] = *(const bf16x8_t*)(sb + ka[0] + 528 + 64 * (kk - 7) + 16 * g);
                            kr1[kk - 7] = *(const bf16x8_t*)(sb + ka[1] + 528 + 64 * (kk - 7) + 16 * g);
                        }
                    };
                    auto widen = [](uint2 c) {
                        union { uint32_t u[4]; f16x8_t h; } r;
                        r.u[0] = fp8x2_to_f16x2<false>(c.x);
                        r.u[1] = fp8x2_to_f16x2<true>(c.x);
                        r.u[2] = fp8x2_to_f16x2<false>(c.y);
                        r.u[3] = fp8x2_to_f16x2<true>(c.y);
                        return r.h;
                    };
                    auto step = [&](int kk, int slot, bool rope, int nlat) {
                        if (kk + kKAhead < 9) read_k(kk + kKAhead, kk + kKAhead >= nlat);
                        __builtin_amdgcn_sched_barrier(0);
                        if (rope) {   // bf16 rope x bf16 Q
                            acc[slot][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr0[kk - 7], qv[kk], acc[slot][0], 0, 0, 0);
                            acc[slot][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr1[kk - 7], qv[kk], acc[slot][1], 0, 0, 0);
                        } else {      // fp16 codes x fp16 Q
                            union { bf16x8_t b; f16x8_t h; } qq;
                            qq.b = qv[kk];
                            acc[slot][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen(kc0[kk]), qq.h, acc[slot][0], 0, 0, 0);
                            acc[slot][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen(kc1[kk]), qq.h, acc[slot][1], 0, 0, 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    };
                    if (!half) {
#pragma unroll
                        for (int kk = 0; kk < kKAhead; ++kk) read_k(kk, false);
#pragma unroll
                        for (int kk = 0; kk < 9; ++kk) step(kk, kk < 4 ? 0 : (kk < 8 ? 1 : 2), false, 9);
                    } else {
#pragma unroll
                        for (int kk = 0; kk < kKAhead; ++kk) read_k(kk, false);
#pragma unroll
                        for (int kk = 0; kk < 9; ++kk) step(kk, kk < 3 ? 0 : (kk < 7 ? 1 : 2), kk >= 7, 7);
                    }
                    // lane: tokens 4g + i (block 0) and 16 + 4g + i (block 1); scale slots per half; the
                    // latent partials carry the Q factor 2^e, the rope partial (second half) does not.
                    // Scale slot j of a token: group j (first half) or 2 + j (second half; its slot 2, the
                    // rope, has none).  A token's 4 group scales follow its codes in the record.
                    const int g0 = half ? 2 : 0;
                    const uint8_t* sp = sb + fp8_tok(4 * g) + 512 + 4 * g0;   // + 656 i: token 4g + i
                    constexpr int kHi = 16 * kFp8Record + kFp8Gap;            // token 16 + 4g + i
                    f32x4_t sa0, sb0, sa1, sb1;
                    f32x4_t sa2 = {1.f, 1.f, 1.f, 1.f}, sb2 = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float2 a = *(const float2*)(sp + kFp8Record * i);
                        const float2 b = *(const float2*)(sp + kHi + kFp8Record * i);
                        sa0[i] = a.x; sa1[i] = a.y;
                        sb0[i] = b.x; sb1[i] = b.y;
                        if (!half) {
                            sa2[i] = *(const float*)(sp + kFp8Record * i + 8);
                            sb2[i] = *(const float*)(sp + kHi + kFp8Record * i + 8);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float a0s = sa0[i] * qscale, a1s = sa1[i] * qscale;
                        const float b0s = sb0[i] * qscale, b1s = sb1[i] * qscale;
                        const float a2s = half ? 1.f : sa2[i] * qscale, b2s = half ? 1.f : sb2[i] * qscale;
                        s0[i] = a0s * acc[0][0][i] + a1s * acc[1][0][i] + a2s * acc[2][0][i];
                        s1[i] = b0s * acc[0][1][i] + b1s * acc[1][1][i] + b2s * acc[2][1][i];
                    }
                }
                if (half) {
                    xs(shb, 0)[lane] = s0;
                    xs(shb, 1)[lane] = s1;
                }
            }
            wait_lgkmcnt0();                 // s_barrier does not wait for LDS writes by itself
            __builtin_amdgcn_s_barrier();   // second-half partials published
            issue_after_second(it);

            // ---- A8: online softmax of the first-half waves' 16 heads ----
            if (score_ok && !half) {
                const f32x4_t t0 = xs(shb, 0)[lane], t1 = xs(shb, 1)[lane];
                const uint32_t vmask = tile_valid[cur * kMaxUnitTiles + it];
                // lane: head (lane & 15), tokens 4g + i (block 0) and 16 + 4g + i (block 1)
                float sv[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sv[i] = (s0[i] + t0[i]) * p.scale_log2;
                    sv[4 + i] = (s1[i] + t1[i]) * p.scale_log2;
                }
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
                if constexpr (!KV_FP8) {
                    uint4 pf;
                    pf.x = pack_bf16x2_hw(pw[0], pw[1]);
                    pf.y = pack_bf16x2_hw(pw[2], pw[3]);
                    pf.z = pack_bf16x2_hw(pw[4], pw[5]);
                    pf.w = pack_bf16x2_hw(pw[6], pw[7]);
                    *(uint4*)&pfrag[shb][0][4 * lane] = pf;
                } else {   // fp32 weights: tokens 4g + i (first vector), 16 + 4g + i (second)
                    pw32(shb, 0)[lane] = (f32x4_t){pw[0], pw[1], pw[2], pw[3]};
                    pw32(shb, 1)[lane] = (f32x4_t){pw[4], pw[5], pw[6], pw[7]};
                }
                if (lane < 16) xalpha[shb][lane] = alpha;
            } else if (!half && shb >= nhb) {   // head block beyond H: zero weights
                if constexpr (!KV_FP8) {
                    *(uint4*)&pfrag[shb][0][4 * lane] = make_uint4(0u, 0u, 0u, 0u);
                } else {
                    pw32(shb, 0)[lane] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                    pw32(shb, 1)[lane] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                }
                if (lane < 16) xalpha[shb][lane] = 1.f;
            }
            wait_lgkmcnt0();
            __builtin_amdgcn_s_barrier();   // P fragments and rescale factors published
        }
        // ---- A10 (score waves), after the split's last unit: output multiplier and LSE of the first
        // halves' heads.  With one split the sink joins here: it adds e^sink to the denominator and
        // nothing to the output.  With several splits the split results exclude it and the combine adds
        // it last. ----
        if (ls == ns - 1 || su % kUnitsPerSplit == kUnitsPerSplit - 1) {
        const float l_tot = head_sum(l_run);
        float mult = 0.f, lse_v = -INFINITY;
        if (score_ok && !half && lane < 16) {
            const int head = head0 + shb * 16 + lane;
            const float snk = (p.sink && p.n_splits == 1) ? p.sink[head] : -INFINITY;
            if (snk == -INFINITY) {
                if (l_tot > 0.f) {
                    mult = 1.f / l_tot;
                    lse_v = (m_run + __log2f(l_tot)) * kLn2;
                }
            } else if (!(l_tot > 0.f)) {
                lse_v = snk;                  // no token: output 0, LSE = the sink
            } else {
                const float s2 = snk * kLog2e;
                const float mn = fmaxf(m_run, s2);
                const float c = __builtin_amdgcn_exp2f(m_run - mn);
                const float lall = l_tot * c + __builtin_amdgcn_exp2f(s2 - mn);
                mult = c / lall;
                lse_v = (mn + __log2f(lall)) * kLn2;
            }
            xmul[KV_FP8 ? 0 : (ls & 1)][shb][lane] = mult;
        }
        __syncthreads();
        if (score_ok && !half && lane < 16) {
            const int head = head0 + shb * 16 + opaque_lane();   // address computed here, not held from the prologue
            if (p.n_splits == 1) {
                if (p.lse) p.lse[row * p.H + head] = lse_v;
            } else {
                p.ws_lse[((int64_t)rloc * p.n_splits + su / kUnitsPerSplit) * p.H + head] = lse_v;
            }
        }
        }
        end_split();
      }
    } else {
        f32x4_t oacc[4][4];                 // [head block][16-dim block of the wave's 64 dims]
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int d = 0; d < 4; ++d) oacc[b][d] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        // FP8: biased exponent of the scale normalization the accumulators carry (0: none yet); the
        // accumulators hold the output times 2^(127 - e_run).
        int e_run = 0;
        // ---- A9: O^T += V^T P^T for the 4 head blocks over this wave's 64 dims (tile it in LDS at sb) ----
        auto value_product = [&](int it, const uint8_t* sb) {
            float a_blk[4];
            uint4 pb[4];   // B operands: bf16 weights, or (FP8) fp16 weights times the wave's group scales
            if constexpr (!KV_FP8) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    a_blk[b] = xalpha[b][lane & 15];
                    pb[b] = *(const uint4*)&pfrag[b][0][4 * lane];
                }
            } else {
                const int gv = vdim0 >> 7;   // the scale group of this wave's dims
                float sc8[8];                // scales of the lane's tokens 4g + i and 16 + 4g + i
                const uint8_t* sp = sb + fp8_tok(4 * g) + 512 + 4 * gv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sc8[i] = *(const float*)(sp + kFp8Record * i);
                    sc8[4 + i] = *(const float*)(sp + 16 * kFp8Record + kFp8Gap + kFp8Record * i);
                }
                // Power-of-two normalization of the scales: every scale of the tile lies below
                // 2^(eb - 126) for the biased exponent eb of the tile's largest scale (lanes l, l^16,
                // l^32, l^48 hold all 32 tokens, so the max is wave-uniform).  The running exponent
                // e_run only grows: when a tile's eb exceeds it the accumulators are scaled by the
                // exact factor 2^(e_run - eb), folded into the rescale factors below.  The scaled
                // weights p * s * 2^(127 - e_run) then stay below 2^9 (p <= 2^8 under the lazy
                // rescale) and far above the fp16 subnormals for the scales that matter, whatever the
                // magnitude of the group scales.
                float mx = fmaxf(fmaxf(fmaxf(sc8[0], sc8[1]), fmaxf(sc8[2], sc8[3])),
                                 fmaxf(fmaxf(sc8[4], sc8[5]), fmaxf(sc8[6], sc8[7])));
                mx = head_max(mx);
                int eb = __builtin_amdgcn_readfirstlane((int)((__float_as_uint(mx) >> 23) & 0xffu));
                if (eb == 0 && mx > 0.f) eb = 1;            // subnormal scales share exponent field 1
                float f = 1.f;
                if (eb > e_run) {
                    if (e_run > 0) f = __builtin_ldexpf(1.f, e_run - eb);
                    e_run = eb;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) sc8[i] = __builtin_ldexpf(sc8[i], 127 - e_run);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    a_blk[b] = xalpha[b][lane & 15] * f;
                    const f32x4_t p0 = pw32(b, 0)[lane], p1 = pw32(b, 1)[lane];
                    pb[b] = make_uint4(pack_f16x2_rne(p0[0] * sc8[0], p0[1] * sc8[1]),
                                       pack_f16x2_rne(p0[2] * sc8[2], p0[3] * sc8[3]),
                                       pack_f16x2_rne(p1[0] * sc8[4], p1[1] * sc8[5]),
                                       pack_f16x2_rne(p1[2] * sc8[6], p1[3] * sc8[7]));
                }
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if (a_blk[b] != 1.f) {   // rare: a reference max moved (exact 1.0 otherwise)
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        oacc[b][d][0] *= a_blk[b]; oacc[b][d][1] *= a_blk[b];
                        oacc[b][d][2] *= a_blk[b]; oacc[b][d][3] *= a_blk[b];
                    }
                }
            }
            if constexpr (!KV_FP8) {
                const uint8_t* vp0 = sb + 128 * (vdim0 / 64);
#pragma unroll
                for (int d = 0; d < 4; ++d) {   // 16-dim block within this wave's 64 dims
                    const uint8_t* vp = vp0 + vb[d];
                    union { bf16x8_t v; i16x4_t h[2]; } va;
                    va.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(vp));
                    va.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(vp + 16 * kBf16Record));
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        union { uint4 u; bf16x8_t v; } pv;
                        pv.u = pb[b];
                        oacc[b][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, pv.v, oacc[b][d], 0, 0, 0);
                    }
                }
            } else {   // 8 tokens' codes of one dim per lane, widened to fp16
                const uint8_t* vp0 = sb + vb[0] + vdim0;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const i32x2_t vc = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2_t*)(vp0 + 16 * d));
                    union { uint32_t u[4]; f16x8_t h; } va;
                    va.u[0] = fp8x2_to_f16x2<false>((uint32_t)vc[0]);
                    va.u[1] = fp8x2_to_f16x2<true>((uint32_t)vc[0]);
                    va.u[2] = fp8x2_to_f16x2<false>((uint32_t)vc[1]);
                    va.u[3] = fp8x2_to_f16x2<true>((uint32_t)vc[1]);
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        union { uint4 u; f16x8_t v; } pv;
                        pv.u = pb[b];
                        oacc[b][d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va.h, pv.v, oacc[b][d], 0, 0, 0);
                    }
                }
            }
        };
        // The value product of tile it runs after the first barrier of tile it+1, beside the scores of
        // tile it+1: its weights and rescale factors are rewritten only after the second barrier of
        // tile it+1, its ring stage only after that too.
      for (int ls = 0; ls < ns; ++ls) {
        start_split(ls);
        const int su = split0 + ls;   // unit of the row
        if (su % kUnitsPerSplit == 0) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int d = 0; d < 4; ++d) oacc[b][d] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            e_run = 0;
        }
        const uint8_t* sb_prev = nullptr;
        for (int it = 0; it < ntiles; ++it) {
            const uint8_t* sb = tile_top(it);
            if (it > 0) value_product(it - 1, sb_prev);
            wait_lgkmcnt0();                 // this wave's reads of tile it-1 are done
            __builtin_amdgcn_s_barrier();   // second-half partials published
            issue_after_second(it);
            __builtin_amdgcn_s_barrier();   // P fragments and rescale factors published
            sb_prev = sb;
        }
        if (ntiles > 0) value_product(ntiles - 1, sb_prev);
        // ---- A10 (value waves), after the split's last unit: wait for the weight sums, normalize and
        // write ----
        if (ls == ns - 1 || su % kUnitsPerSplit == kUnitsPerSplit - 1) {
        __syncthreads();
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b >= nhb) break;
            float inv = xmul[KV_FP8 ? 0 : (ls & 1)][b][lane & 15];
            // undo the scale normalization, except in FP8 split partials, which keep it (and record it)
            if (KV_FP8 && e_run > 0 && p.n_splits == 1) inv = __builtin_ldexpf(inv, e_run - 127);
            // FP8: the lane's addresses are computed per split from an opaque lane id (not held across the loop)
            const int ln = KV_FP8 ? opaque_lane() : lane;
            const int head = head0 + 16 * b + (ln & 15);
            const int64_t pidx = (((int64_t)rloc * p.n_splits + su / kUnitsPerSplit) * p.H + head) * kDv + vdim0 + 4 * (ln >> 4);
            if (KV_FP8 && p.n_splits > 1) {   // fp16 partials in the normalized domain (|value| < 896)
                uint16_t* wo = (uint16_t*)p.ws_o + pidx;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint2 w;
                    w.x = pack_f16x2_rne(oacc[b][d][0] * inv, oacc[b][d][1] * inv);
                    w.y = pack_f16x2_rne(oacc[b][d][2] * inv, oacc[b][d][3] * inv);
                    *(uint2*)(wo + 16 * d) = w;
                }
                if (b == 0 && ln == 0 && (vdim0 & 127) == 0)   // one wave per group records its factor
                    p.ws_gsc[((int64_t)rloc * p.n_splits + su / kUnitsPerSplit) * 4 + (vdim0 >> 7)] =
                        e_run > 0 ? __builtin_ldexpf(1.f, e_run - 127) : 1.f;
            } else {
                uint16_t* orow = p.n_splits == 1 ? p.out + (row * p.H + head) * (int64_t)kDv + vdim0 + 4 * (ln >> 4)
                                                 : (uint16_t*)p.ws_o + pidx;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint2 w;
                    w.x = pack_bf16x2_hw(oacc[b][d][0] * inv, oacc[b][d][1] * inv);
                    w.y = pack_bf16x2_hw(oacc[b][d][2] * inv, oacc[b][d][3] * inv);
                    *(uint2*)(orow + 16 * d) = w;
                }
            }
        }
        }
        end_split();
      }
    }
}

// A11: merge the splits of each row in split order:  LSE = m + log sum_s e^(lse_s - m),
// out = sum_s (e^(lse_s - m) / sum) * O_s, rounded to bf16, computed as an online merge over the
// splits in order (the running max m and sum are updated split by split), and then the head's sink
// logit, if any, as one more term with no output.  64 threads per (row, head), 8 dims each.
// Partials are bf16 (bf16 caches) or fp16 times a per-(split, group) power-of-two factor (FP8 caches).
constexpr int kCombineHeads = 16;   // heads per combine workgroup (64 threads each)

template <bool FP8>
__global__ __launch_bounds__(64 * kCombineHeads) void split_combine_kernel(const void* __restrict__ ws_o,
                                                            const float* __restrict__ ws_lse,
                                                            const float* __restrict__ ws_gsc, int S, int H,
                                                            int row0, const float* __restrict__ sink,
                                                            uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int hq = H / kCombineHeads;
    const int rloc = blockIdx.x / hq;
    const int head = (blockIdx.x % hq) * kCombineHeads + (threadIdx.x >> 6);
    const int d = 8 * (threadIdx.x & 63);
    const float* ls = ws_lse + (int64_t)rloc * S * H + head;
    constexpr int kGroup = 4;   // splits whose loads are in flight together
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, tot = 0.f;
    // Online merge over groups of splits, in split order: the LSEs and partials of a group are loaded
    // together (no load waits for another), and the running sum is rescaled when the max grows.
    for (int s0 = 0; s0 < S; s0 += kGroup) {
        float l4[kGroup], v[kGroup][8];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const int s = s0 + j < S ? s0 + j : S - 1;   // loads stay unconditional (clamped)
            l4[j] = s0 + j < S ? ls[(int64_t)s * H] : -INFINITY;
            const int64_t off = (((int64_t)rloc * S + s) * H + head) * kDv + d;
            const uint4 u = *(const uint4*)((const uint16_t*)ws_o + off);
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
            if (FP8) {   // fp16 pairs times the split's factor for this thread's group (d / 128)
                const float f = ws_gsc[((int64_t)rloc * S + s) * 4 + (d >> 7)];
                typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 h2;
                typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f2 x = __builtin_convertvector(__builtin_bit_cast(h2, wd[e]), f2);
                    v[j][2 * e] = x[0] * f;
                    v[j][2 * e + 1] = x[1] * f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[j][2 * e] = __uint_as_float(wd[e] << 16);
                    v[j][2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            if (l4[j] == -INFINITY) continue;        // empty split (or past S): contributes nothing
            if (l4[j] > m) {                         // rescale what has been merged so far
                const float c = m == -INFINITY ? 0.f : expf(m - l4[j]);
                tot *= c;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] *= c;
                m = l4[j];
            }
            const float w = expf(l4[j] - m);
            tot += w;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += w * v[j][e];
        }
    }
    // The sink, last: one more term e^sink in the denominator with no output (skipped at -inf).
    const float snk = sink ? sink[head] : -INFINITY;
    if (snk != -INFINITY) {
        if (snk > m) {
            const float c = m == -INFINITY ? 0.f : expf(m - snk);
            tot *= c;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= c;
            m = snk;
        }
        tot += expf(snk - m);
    }
    float LSE = -INFINITY;
    if (tot > 0.f) {
        LSE = m + logf(tot);
        const float inv = 1.f / tot;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= inv;
    }
    const int64_t orow = ((int64_t)row0 + rloc) * H + head;
    uint4 o;
    o.x = pack_bf16x2_hw(acc[0], acc[1]);
    o.y = pack_bf16x2_hw(acc[2], acc[3]);
    o.z = pack_bf16x2_hw(acc[4], acc[5]);
    o.w = pack_bf16x2_hw(acc[6], acc[7]);
    *(uint4*)(out + orow * kDv + d) = o;
    if (d == 0 && lse) lse[orow] = LSE;
}

// ---- Workspace-free decode: the split partials live in a static device array ----
// For callers that cannot allocate (code under HIP graph capture, serving loops, harnesses that forbid
// allocation).  Each GPU the library runs on holds its own copy of `scratch` until the process ends;
// every workspace-free call on a GPU shares it, so such calls must be ordered on one stream (calls
// that overlap on one GPU race).  Nothing in it needs clearing: every (row, split, head) partial and
// LSE a launch reads is written by that launch.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

// The device address of the current device's `scratch`, looked up once per device with that
// device current (host code never passes the array's own name, a host-side stand-in).
hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
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
    p.k = a.k + a.k_win;
    p.k_main = a.k;
    // Without a window cache the window fields repeat the main cache's (no slot selects them).
    const bool has_win = a.k_win > 0;
    p.kv_win = (const uint8_t*)(has_win ? a.kv_win : a.kv);
    p.num_pages_win = has_win ? a.num_pages_win : a.num_pages;
    p.block_table_win = has_win ? a.block_table_win : a.block_table;
    p.bt_win_stride = has_win ? a.bt_win_stride : a.bt_stride;
    p.idx_win = has_win ? a.idx_win : a.idx;
    p.H = a.H;
    const bool fp8 = a.kv_dtype == 1;
    p.unit_slots = attn_unit_slots(a.k, a.k_win);
    p.n_units = (p.k + p.unit_slots - 1) / p.unit_slots;
    p.n_splits = fp8 ? (p.n_units + kFp8UnitsPerSplit - 1) / kFp8UnitsPerSplit : p.n_units;
    // Launches with fewer (row, split) items than CUs split the heads over 2 or 4 workgroups (each of
    // which gathers the same records): a head's arithmetic does not depend on the heads it shares a
    // workgroup with, so the results are the same bits either way.
    int dev = 0, num_cu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    p.scale_log2 = a.softmax_scale * kLog2e;
    p.out = (uint16_t*)a.out;
    p.lse = a.lse;
    p.sink = a.sink;
    // Workspace per row: partials of every (split, head), then their LSEs, then (FP8) the group factors
    // of every split (none with one split).  The
    // host validation sizes it for 512-slot units, at least as many splits as any unit size here.
    const size_t o_per_row = p.n_splits > 1 ? (size_t)p.n_splits * a.H * kDv * 2 : 0;
    const size_t lse_per_row = p.n_splits > 1 ? (size_t)p.n_splits * a.H * sizeof(float) : 0;
    const size_t gsc_per_row = p.n_splits > 1 && fp8 ? (size_t)p.n_splits * 4 * sizeof(float) : 0;
    const size_t per_row = o_per_row + lse_per_row + gsc_per_row;
    int rows_per_launch = a.rows;
    if (per_row > 0) {
        const size_t fit = a.ws_bytes / per_row;
        rows_per_launch = (int)(fit < (size_t)a.rows ? fit : (size_t)a.rows);
        if (rows_per_launch < 1) return hipErrorInvalidValue;   // host validation prevents this
    }
    for (int row0 = 0; row0 < a.rows; row0 += rows_per_launch) {
        const int n = min(rows_per_launch, a.rows - row0);
        p.row0 = row0;
        // Workspace regions for a launch of rows_per_launch rows: partials, then LSEs.
        p.ws_o = per_row > 0 ? a.ws : nullptr;
        p.ws_lse = per_row > 0 ? (float*)((uint8_t*)a.ws + (size_t)rows_per_launch * o_per_row) : nullptr;
        p.ws_gsc = gsc_per_row > 0 ? (float*)((uint8_t*)a.ws + (size_t)rows_per_launch * (o_per_row + lse_per_row))
                                   : nullptr;
        // bf16: launches with at least twice as many (row, split) items as CUs run 2 or 4 consecutive
        // splits of a row per workgroup, one after the other: the index translation and Q serve them
        // all.  Each split reduces its own tiles in order with its own softmax state, so the bits are the
        // same.  FP8: a workgroup runs one whole split (its 2 units) in every launch.
        p.heads_per_wg = kHeadsPerBlock;
        const int hb64 = (a.H + kHeadsPerBlock - 1) / kHeadsPerBlock;
        if (fp8) {
            p.units_per_wg = min(kFp8UnitsPerSplit, p.n_units);
        } else {
            p.units_per_wg = 1;
            while (2 * p.units_per_wg <= 4 && 2 * p.units_per_wg <= p.n_units &&
                   (int64_t)n * ((p.n_units + 2 * p.units_per_wg - 1) / (2 * p.units_per_wg)) * hb64 >= num_cu)
                p.units_per_wg *= 2;
        }
        const int groups = (p.n_units + p.units_per_wg - 1) / p.units_per_wg;
        while (p.heads_per_wg > 16 && (int64_t)n * groups * ((a.H + p.heads_per_wg - 1) / p.heads_per_wg) < num_cu)
            p.heads_per_wg /= 2;
        p.n_hblocks = (a.H + p.heads_per_wg - 1) / p.heads_per_wg;
        const int grid = n * groups * p.n_hblocks;
        if (fp8) hipLaunchKernelGGL(sparse_mla_kernel<true>, dim3(grid), dim3(kAttnThreads), 0, stream, p);
        else hipLaunchKernelGGL(sparse_mla_kernel<false>, dim3(grid), dim3(kAttnThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.n_splits > 1) {
            if (fp8)
                hipLaunchKernelGGL(split_combine_kernel<true>, dim3(n * (a.H / kCombineHeads)), dim3(64 * kCombineHeads), 0,
                                   stream, p.ws_o,
                                   p.ws_lse, p.ws_gsc, p.n_splits, a.H, row0, p.sink, p.out, p.lse);
            else
                hipLaunchKernelGGL(split_combine_kernel<false>, dim3(n * (a.H / kCombineHeads)), dim3(64 * kCombineHeads), 0,
                                   stream, p.ws_o,
                                   p.ws_lse, p.ws_gsc, p.n_splits, a.H, row0, p.sink, p.out, p.lse);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace smla
