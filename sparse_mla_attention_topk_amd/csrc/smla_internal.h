// Host-side launcher declarations shared between the C-ABI layer and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smla {

// Geometry of the attention kernels (also used by the host to size workspaces).
constexpr int kSplitSlots = 512;   // index slots of one unit: one pass of the tile loop
constexpr int kHeadsPerBlock = 64; // heads handled by one workgroup (4 waves x 16)
constexpr int kFp8UnitsPerSplit = 2;   // FP8 caches: a split (one softmax state, one partial) is 2 units

inline int attn_num_units(int k) { return (k + kSplitSlots - 1) / kSplitSlots; }
// Calls with a sliding-window part (k_win > 0 slots after the k main ones) stretch the unit so that the
// row keeps the unit count of its main part: units of ceil((k + k_win) / n / 64) * 64 slots for
// n = ceil(k / 512) units (more units if that exceeds kMaxUnitSlots).  A function of k and k_win only.
constexpr int kMaxUnitSlots = 768;
inline int attn_unit_slots(int k, int k_win) {
    if (k_win <= 0) return kSplitSlots;
    const int total = k + k_win;
    for (int n = (k + kSplitSlots - 1) / kSplitSlots;; ++n) {
        const int u = ((total + n - 1) / n + 63) / 64 * 64;
        if (u <= kMaxUnitSlots) return u;
    }
}
// Splits of a row, each reduced by one workgroup before the split combine: units of 512 slots (bf16
// caches) or pairs of them (FP8 caches, whose partials carry per-group power-of-two factors).  A function
// of k and the cache type only, never of the batch.
inline int attn_num_splits(int k, int kv_dtype) {
    const int u = attn_num_units(k);
    return kv_dtype == 1 ? (u + kFp8UnitsPerSplit - 1) / kFp8UnitsPerSplit : u;
}

// Workspace of the attention entry points, per query row (0 when k fits one split): the partial
// outputs of every (split, head) in 16-bit form -- bf16 for bf16 caches; fp16 for FP8 caches, in the
// kernel's normalized domain (the output times 2^(127 - e) for the biased exponent e of the largest
// group scale the split met, which keeps them below 896) -- then their fp32 LSEs, then (FP8) the factor
// 2^(e - 127) of every (split, 128-dim group) in fp32.
inline size_t attn_ws_o_bytes_per_row(int H, int k, int kv_dtype) {
    return (size_t)attn_num_splits(k, kv_dtype) * H * 512 * 2;
}
inline size_t attn_ws_lse_bytes_per_row(int H, int k, int kv_dtype) {
    return (size_t)attn_num_splits(k, kv_dtype) * (H + (kv_dtype == 1 ? 4 : 0)) * 4;
}
inline size_t attn_ws_bytes_per_row(int H, int k, int kv_dtype) {
    if (attn_num_splits(k, kv_dtype) <= 1) return 0;
    return attn_ws_o_bytes_per_row(H, k, kv_dtype) + attn_ws_lse_bytes_per_row(H, k, kv_dtype);
}

struct AttnArgs {
    const void* q;
    int64_t q_row_stride;
    const void* kv;
    int kv_dtype;
    int64_t num_pages;
    const int32_t* block_table;
    int64_t bt_stride;
    int32_t num_reqs;
    const int32_t* row_req;
    const int32_t* idx;
    int32_t rows;
    int32_t H;
    int32_t k;
    float softmax_scale;
    const float* sink;
    void* out;
    float* lse;
    void* ws;
    size_t ws_bytes;
    // Optional sliding-window cache: row slots [k, k + k_win) list positions (idx_win [rows, k_win]) of
    // kv_win through block_table_win; the same request ids (row_req, num_reqs) and record type.
    const void* kv_win = nullptr;
    int64_t num_pages_win = 0;
    const int32_t* block_table_win = nullptr;
    int64_t bt_win_stride = 0;
    const int32_t* idx_win = nullptr;
    int32_t k_win = 0;
};

// Indexer scores (paged MQA logits).
struct IdxArgs {
    const void* q;           // bf16 [rows][Hi][128], row stride q_row_stride elements
    int64_t q_row_stride;
    const float* weights;    // fp32 [rows][Hi], row stride w_row_stride elements
    int64_t w_row_stride;
    const void* kidx;        // bf16 [num_pages][64][128]
    int64_t num_pages;
    const int32_t* block_table;
    int64_t bt_stride;
    int32_t num_reqs;
    const int32_t* row_req;
    const int32_t* lengths;
    int32_t rows;
    int32_t Hi;
    float* out;              // fp32 [rows][out_stride]
    int64_t out_stride;
};

// Top-k workspace bytes per row for the chunked path (0: the row is processed by one workgroup).
size_t topk_ws_bytes_per_row(int64_t row_stride, int32_t k);
hipError_t launch_topk(const float* scores, const int64_t* row_offsets, int64_t row_stride,
                       const int32_t* lengths, int32_t rows, int32_t k, int32_t* out, void* ws, size_t ws_bytes,
                       hipStream_t stream);
hipError_t launch_causal_lengths(int64_t first_pos, int32_t T, int32_t* lengths, hipStream_t stream);
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);
// Workspace-free decode: bytes of the static per-device scratch array, and its device address on the
// current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_paged_mqa_logits(const IdxArgs& a, hipStream_t stream);
// positions == nullptr: the rope values are stored as given; else token t's rope is rotated back by the
// angles of row positions[t] of cos_sin ([max_pos][64] fp32: 32 cosines, then 32 sines).
hipError_t launch_kv_cache_write(const void* in, int64_t in_row_stride, const int64_t* slots, const int64_t* positions,
                                 const float* cos_sin, int64_t max_pos, int32_t T, void* cache, int kv_dtype,
                                 int64_t num_pages, hipStream_t stream);

}  // namespace smla
