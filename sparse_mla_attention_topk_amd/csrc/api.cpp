// C ABI of the sparse-MLA library: argument validation, workspace sizing, dispatch.
//
// Every check runs on the host before anything is enqueued; a failing call enqueues nothing and
// leaves a message naming the parameter (and, for shapes, the supported values) in a thread-local
// buffer.  Unsupported shapes are hard errors, never a fallback to another numeric path
// ("[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL", "Fused activation and FP8
// quantization": missing support is an error; "[Bugfix] Make DSV4 sparse MLA work end-to-end ...",
// section "Purpose", item "SM120 gate": reject at init and name the required shape).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "smla.h"
#include "smla_internal.h"

namespace {

thread_local char g_err[512] = "";

smla_status fail(smla_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

smla_status ok() {
    g_err[0] = '\0';
    return SMLA_OK;
}

constexpr int kMaxK = 16384;
constexpr int64_t kMaxStride = 2147483647LL;
constexpr int64_t kMaxPages = 1LL << 26;   // physical slot index (page * 64 + offset) fits in 32 bits

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

smla_status check_heads(int32_t H) {
    if (H < 16 || H > 128 || H % 16 != 0)
        return fail(SMLA_ERR_UNSUPPORTED, "num_heads=%d is not supported; supported: multiples of 16 in [16, 128]", H);
    return SMLA_OK;
}

smla_status check_k(int32_t k, const char* name) {
    if (k < 1 || k > kMaxK)
        return fail(SMLA_ERR_UNSUPPORTED, "%s=%d is not supported; supported: 1 <= %s <= %d", name, k, name, kMaxK);
    return SMLA_OK;
}

smla_status check_kv_dtype(int32_t d) {
    if (d != SMLA_KV_BF16 && d != SMLA_KV_FP8_E4M3_G128)
        return fail(SMLA_ERR_UNSUPPORTED, "kv_dtype=%d is not supported; supported: %d (SMLA_KV_BF16), %d (SMLA_KV_FP8_E4M3_G128)",
                    d, (int)SMLA_KV_BF16, (int)SMLA_KV_FP8_E4M3_G128);
    return SMLA_OK;
}

smla_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SMLA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
    return ok();
}

// Shared validation of the attention entry points.
smla_status check_attention(const void* q, int64_t q_row_stride, const void* kv, int32_t kv_dtype,
                            int64_t num_pages, const int32_t* block_table, int64_t bt_stride, int32_t num_reqs,
                            const int32_t* idx, int32_t rows, int32_t H, int32_t k, float scale, void* out,
                            const float* lse, void* ws, size_t ws_bytes) {
    smla_status st;
    if ((st = check_heads(H)) != SMLA_OK) return st;
    if ((st = check_k(k, "k")) != SMLA_OK) return st;
    if ((st = check_kv_dtype(kv_dtype)) != SMLA_OK) return st;
    if (rows < 0) return fail(SMLA_ERR_INVALID_ARG, "rows=%d must be >= 0", rows);
    if (num_pages < 1) return fail(SMLA_ERR_INVALID_ARG, "num_pages=%lld must be >= 1", (long long)num_pages);
    if (num_pages > kMaxPages)
        return fail(SMLA_ERR_CAPACITY, "num_pages=%lld exceeds the supported maximum %lld", (long long)num_pages,
                    (long long)kMaxPages);
    if (bt_stride < 1) return fail(SMLA_ERR_INVALID_ARG, "bt_stride=%lld must be >= 1", (long long)bt_stride);
    if (num_reqs < 1) return fail(SMLA_ERR_INVALID_ARG, "num_reqs=%d must be >= 1", num_reqs);
    if (!(scale > 0.f) || scale != scale || scale > 3.0e38f)
        return fail(SMLA_ERR_INVALID_ARG, "softmax_scale=%g must be a finite positive number", (double)scale);
    if (q_row_stride < (int64_t)H * 576)
        return fail(SMLA_ERR_INVALID_ARG, "q_row_stride=%lld must be >= H*576=%lld", (long long)q_row_stride,
                    (long long)H * 576);
    if (rows == 0) return SMLA_OK;
    if (!q) return fail(SMLA_ERR_INVALID_ARG, "q is NULL");
    if (!kv) return fail(SMLA_ERR_INVALID_ARG, "kv is NULL");
    if (!block_table) return fail(SMLA_ERR_INVALID_ARG, "block_table is NULL");
    if (!idx) return fail(SMLA_ERR_INVALID_ARG, "idx is NULL");
    if (!out) return fail(SMLA_ERR_INVALID_ARG, "out is NULL");
    if (!aligned(q, 16)) return fail(SMLA_ERR_ALIGNMENT, "q must be 16-byte aligned");
    if (q_row_stride % 8 != 0)
        return fail(SMLA_ERR_ALIGNMENT, "q_row_stride=%lld must be a multiple of 8 elements", (long long)q_row_stride);
    if (!aligned(kv, 16)) return fail(SMLA_ERR_ALIGNMENT, "kv must be 16-byte aligned");
    if (!aligned(out, 16)) return fail(SMLA_ERR_ALIGNMENT, "out must be 16-byte aligned");
    if (!aligned(block_table, 4)) return fail(SMLA_ERR_ALIGNMENT, "block_table must be 4-byte aligned");
    if (!aligned(idx, 4)) return fail(SMLA_ERR_ALIGNMENT, "idx must be 4-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(SMLA_ERR_ALIGNMENT, "lse must be 4-byte aligned");
    const size_t per_row = smla::attn_ws_bytes_per_row(H, k, kv_dtype);
    if (per_row > 0) {
        if (!ws) return fail(SMLA_ERR_WORKSPACE, "ws is NULL but k=%d needs %zu workspace bytes per row", k, per_row);
        if (!aligned(ws, 256)) return fail(SMLA_ERR_ALIGNMENT, "ws must be 256-byte aligned");
        if (ws_bytes < per_row)
            return fail(SMLA_ERR_WORKSPACE, "ws_bytes=%zu is smaller than the %zu bytes one row needs (H=%d, k=%d)",
                        ws_bytes, per_row, H, k);
    }
    return SMLA_OK;
}

// Shared validation of the cache-write entry points.
smla_status check_cache_write(const void* kv_in, int64_t in_row_stride, const int64_t* slot_mapping, int32_t T,
                              void* cache, int32_t kv_dtype, int64_t num_pages) {
    smla_status st;
    if ((st = check_kv_dtype(kv_dtype)) != SMLA_OK) return st;
    if (T < 0) return fail(SMLA_ERR_INVALID_ARG, "T=%d must be >= 0", T);
    if (num_pages < 1) return fail(SMLA_ERR_INVALID_ARG, "num_pages=%lld must be >= 1", (long long)num_pages);
    if (num_pages > kMaxPages)
        return fail(SMLA_ERR_CAPACITY, "num_pages=%lld exceeds the supported maximum %lld", (long long)num_pages,
                    (long long)kMaxPages);
    if (in_row_stride < 576)
        return fail(SMLA_ERR_INVALID_ARG, "in_row_stride=%lld must be >= 576", (long long)in_row_stride);
    if (in_row_stride % 8 != 0)
        return fail(SMLA_ERR_ALIGNMENT, "in_row_stride=%lld must be a multiple of 8 elements", (long long)in_row_stride);
    if (T == 0) return ok();
    if (!kv_in) return fail(SMLA_ERR_INVALID_ARG, "kv_in is NULL");
    if (!slot_mapping) return fail(SMLA_ERR_INVALID_ARG, "slot_mapping is NULL");
    if (!cache) return fail(SMLA_ERR_INVALID_ARG, "cache is NULL");
    if (!aligned(kv_in, 16)) return fail(SMLA_ERR_ALIGNMENT, "kv_in must be 16-byte aligned");
    if (!aligned(slot_mapping, 8)) return fail(SMLA_ERR_ALIGNMENT, "slot_mapping must be 8-byte aligned");
    if (!aligned(cache, 16)) return fail(SMLA_ERR_ALIGNMENT, "cache must be 16-byte aligned");
    return SMLA_OK;
}

}  // namespace

extern "C" {

const char* smla_last_error(void) { return g_err; }

const char* smla_version(void) { return "smla 0.1.0 (gfx950)"; }

smla_status smla_is_supported(const smla_capacity* cap) {
    if (!cap) return fail(SMLA_ERR_INVALID_ARG, "cap is NULL");
    smla_status st;
    if ((st = check_heads(cap->num_heads)) != SMLA_OK) return st;
    if ((st = check_k(cap->max_k, "max_k")) != SMLA_OK) return st;
    if (cap->d_qk != 576)
        return fail(SMLA_ERR_UNSUPPORTED, "d_qk=%d is not supported; supported: 576 (512 latent + 64 rope)", cap->d_qk);
    if (cap->d_v != 512) return fail(SMLA_ERR_UNSUPPORTED, "d_v=%d is not supported; supported: 512", cap->d_v);
    if (cap->page_block_size != 64)
        return fail(SMLA_ERR_UNSUPPORTED, "page_block_size=%d is not supported; supported: 64", cap->page_block_size);
    if ((st = check_kv_dtype(cap->kv_dtype)) != SMLA_OK) return st;
    if (cap->max_rows < 1) return fail(SMLA_ERR_CAPACITY, "max_rows=%d must be >= 1", cap->max_rows);
    if (cap->max_candidates < 1 || cap->max_candidates > kMaxStride)
        return fail(SMLA_ERR_CAPACITY, "max_candidates=%lld is outside [1, %lld]", (long long)cap->max_candidates,
                    (long long)kMaxStride);
    if (cap->reserved != 0) return fail(SMLA_ERR_INVALID_ARG, "reserved must be 0");
    return ok();
}

smla_status smla_workspace_size(const smla_capacity* cap, size_t* topk_ws_bytes, size_t* attn_ws_bytes) {
    smla_status st = smla_is_supported(cap);
    if (st != SMLA_OK) return st;
    if (topk_ws_bytes) {
        const size_t per_row = smla::topk_ws_bytes_per_row(cap->max_candidates, cap->max_k);
        const size_t rows = cap->max_rows < 255 ? (size_t)cap->max_rows : 255;   // the chunked path serves < 256 rows
        *topk_ws_bytes = per_row * rows;
    }
    if (attn_ws_bytes) {
        const size_t per_row = smla::attn_ws_bytes_per_row(cap->num_heads, cap->max_k, cap->kv_dtype);
        *attn_ws_bytes = per_row * (size_t)cap->max_rows;
    }
    return ok();
}

smla_status smla_fill_causal_lengths(int64_t first_pos, int32_t T, int32_t* lengths, void* stream) {
    if (T < 0) return fail(SMLA_ERR_INVALID_ARG, "T=%d must be >= 0", T);
    if (T == 0) return ok();
    if (!lengths) return fail(SMLA_ERR_INVALID_ARG, "lengths is NULL");
    if (!aligned(lengths, 4)) return fail(SMLA_ERR_ALIGNMENT, "lengths must be 4-byte aligned");
    return hip_status(smla::launch_causal_lengths(first_pos, T, lengths, (hipStream_t)stream), "fill_causal_lengths");
}

smla_status smla_topk_per_row(const float* scores, const int64_t* row_offsets, int64_t row_stride,
                              const int32_t* lengths, int32_t rows, int32_t k, int32_t* out_idx, void* ws,
                              size_t ws_bytes, void* stream) {
    smla_status st;
    if ((st = check_k(k, "k")) != SMLA_OK) return st;
    if (rows < 0) return fail(SMLA_ERR_INVALID_ARG, "rows=%d must be >= 0", rows);
    if (row_stride < 1 || row_stride > kMaxStride)
        return fail(SMLA_ERR_CAPACITY, "row_stride=%lld is outside [1, %lld]", (long long)row_stride,
                    (long long)kMaxStride);
    if (rows == 0) return ok();
    if (!scores) return fail(SMLA_ERR_INVALID_ARG, "scores is NULL");
    if (!out_idx) return fail(SMLA_ERR_INVALID_ARG, "out_idx is NULL");
    if (!aligned(scores, 4)) return fail(SMLA_ERR_ALIGNMENT, "scores must be 4-byte aligned");
    if (!aligned(out_idx, 4)) return fail(SMLA_ERR_ALIGNMENT, "out_idx must be 4-byte aligned");
    if (row_offsets && !aligned(row_offsets, 8)) return fail(SMLA_ERR_ALIGNMENT, "row_offsets must be 8-byte aligned");
    if (lengths && !aligned(lengths, 4)) return fail(SMLA_ERR_ALIGNMENT, "lengths must be 4-byte aligned");
    if (ws && !aligned(ws, 256)) return fail(SMLA_ERR_ALIGNMENT, "ws must be 256-byte aligned");
    return hip_status(smla::launch_topk(scores, row_offsets, row_stride, lengths, rows, k, out_idx, ws,
                                        ws ? ws_bytes : 0, (hipStream_t)stream),
                      "topk_per_row");
}

smla_status smla_sparse_mla_decode(const void* q, int64_t q_row_stride, const void* kv, int32_t kv_dtype,
                                   int64_t num_pages, const int32_t* block_table, int64_t bt_stride,
                                   int32_t num_reqs, const int32_t* row_req, const int32_t* idx, int32_t rows,
                                   int32_t H, int32_t k, float softmax_scale, const float* sink, void* out, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
    smla_status st = check_attention(q, q_row_stride, kv, kv_dtype, num_pages, block_table, bt_stride, num_reqs, idx,
                                     rows, H, k, softmax_scale, out, lse, ws, ws_bytes);
    if (st != SMLA_OK) return st;
    if (rows == 0) return ok();
    if (row_req && !aligned(row_req, 4)) return fail(SMLA_ERR_ALIGNMENT, "row_req must be 4-byte aligned");
    if (sink && !aligned(sink, 4)) return fail(SMLA_ERR_ALIGNMENT, "sink must be 4-byte aligned");
    smla::AttnArgs a{q,   q_row_stride, kv,  kv_dtype,      num_pages, block_table, bt_stride, num_reqs, row_req,
                     idx, rows,         H,   k,             softmax_scale, sink,    out,       lse,      ws,
                     ws_bytes};
    return hip_status(smla::launch_attention(a, (hipStream_t)stream), "sparse_mla_decode");
}

smla_status smla_sparse_mla_decode_with_window(const void* q, int64_t q_row_stride, const void* kv, int32_t kv_dtype,
                                              int64_t num_pages, const int32_t* block_table, int64_t bt_stride,
                                              const int32_t* idx, int32_t k, const void* kv_win,
                                              int64_t num_pages_win, const int32_t* block_table_win,
                                              int64_t bt_win_stride, const int32_t* idx_win, int32_t k_win,
                                              int32_t num_reqs, const int32_t* row_req, int32_t rows, int32_t H,
                                              float softmax_scale, const float* sink, void* out, float* lse,
                                              void* ws, size_t ws_bytes, void* stream) {
    if (k_win < 64 || k_win % 64 != 0)
        return fail(SMLA_ERR_UNSUPPORTED, "k_win=%d is not supported; supported: a positive multiple of 64 (the "
                    "64-entry tile: 192 for 128 window + 5 draft entries)", k_win);
    if (k < 1 || (int64_t)k + k_win > kMaxK)
        return fail(SMLA_ERR_UNSUPPORTED, "k=%d with k_win=%d is not supported; supported: k >= 1 and k + k_win <= %d",
                    k, k_win, kMaxK);
    // the whole row (k + k_win slots) is validated as one index list of the main cache ...
    smla_status st = check_attention(q, q_row_stride, kv, kv_dtype, num_pages, block_table, bt_stride, num_reqs, idx,
                                     rows, H, k + k_win, softmax_scale, out, lse, ws, ws_bytes);
    if (st != SMLA_OK) return st;
    // ... and the window cache on its own
    if (num_pages_win < 1) return fail(SMLA_ERR_INVALID_ARG, "num_pages_win=%lld must be >= 1", (long long)num_pages_win);
    if (num_pages_win > kMaxPages)
        return fail(SMLA_ERR_CAPACITY, "num_pages_win=%lld exceeds the supported maximum %lld", (long long)num_pages_win,
                    (long long)kMaxPages);
    if (bt_win_stride < 1) return fail(SMLA_ERR_INVALID_ARG, "bt_win_stride=%lld must be >= 1", (long long)bt_win_stride);
    if (rows == 0) return ok();
    if (!kv_win) return fail(SMLA_ERR_INVALID_ARG, "kv_win is NULL");
    if (!block_table_win) return fail(SMLA_ERR_INVALID_ARG, "block_table_win is NULL");
    if (!idx_win) return fail(SMLA_ERR_INVALID_ARG, "idx_win is NULL");
    if (!aligned(kv_win, 16)) return fail(SMLA_ERR_ALIGNMENT, "kv_win must be 16-byte aligned");
    if (!aligned(block_table_win, 4)) return fail(SMLA_ERR_ALIGNMENT, "block_table_win must be 4-byte aligned");
    if (!aligned(idx_win, 4)) return fail(SMLA_ERR_ALIGNMENT, "idx_win must be 4-byte aligned");
    if (row_req && !aligned(row_req, 4)) return fail(SMLA_ERR_ALIGNMENT, "row_req must be 4-byte aligned");
    if (sink && !aligned(sink, 4)) return fail(SMLA_ERR_ALIGNMENT, "sink must be 4-byte aligned");
    smla::AttnArgs a{q,   q_row_stride, kv,  kv_dtype,      num_pages, block_table, bt_stride, num_reqs, row_req,
                     idx, rows,         H,   k,             softmax_scale, sink,    out,       lse,      ws,
                     ws_bytes};
    a.kv_win = kv_win;
    a.num_pages_win = num_pages_win;
    a.block_table_win = block_table_win;
    a.bt_win_stride = bt_win_stride;
    a.idx_win = idx_win;
    a.k_win = k_win;
    return hip_status(smla::launch_attention(a, (hipStream_t)stream), "sparse_mla_decode_with_window");
}

smla_status smla_sparse_mla_decode_noalloc(const void* q, int64_t q_row_stride, const void* kv, int32_t kv_dtype,
                                           int64_t num_pages, const int32_t* block_table, int64_t bt_stride,
                                           int32_t num_reqs, const int32_t* row_req, const int32_t* idx,
                                           int32_t rows, int32_t H, int32_t k, float softmax_scale,
                                           const float* sink, void* out, float* lse, void* stream) {
    const size_t per_row = smla::attn_ws_bytes_per_row(H, k, kv_dtype);
    if (per_row > smla::kNoAllocScratchBytes)
        return fail(SMLA_ERR_CAPACITY,
                    "one row needs %zu bytes of split partials (H=%d, k=%d) but the static scratch holds %zu", per_row,
                    H, k, smla::kNoAllocScratchBytes);
    // validated as the workspace form with a stand-in workspace of the scratch size; the real address
    // is looked up below (no allocation either way)
    static const size_t kStandIn = 256;
    smla_status st = check_attention(q, q_row_stride, kv, kv_dtype, num_pages, block_table, bt_stride, num_reqs, idx,
                                     rows, H, k, softmax_scale, out, lse, (void*)kStandIn,
                                     smla::kNoAllocScratchBytes);
    if (st != SMLA_OK) return st;
    if (rows == 0) return ok();
    if (row_req && !aligned(row_req, 4)) return fail(SMLA_ERR_ALIGNMENT, "row_req must be 4-byte aligned");
    if (sink && !aligned(sink, 4)) return fail(SMLA_ERR_ALIGNMENT, "sink must be 4-byte aligned");
    void* ws = nullptr;
    if (per_row > 0) {
        hipError_t e = smla::noalloc_scratch(&ws);
        if (e != hipSuccess) return hip_status(e, "sparse_mla_decode_noalloc: scratch lookup");
    }
    smla::AttnArgs a{q,   q_row_stride, kv,  kv_dtype,      num_pages, block_table, bt_stride, num_reqs, row_req,
                     idx, rows,         H,   k,             softmax_scale, sink,    out,       lse,      ws,
                     per_row > 0 ? smla::kNoAllocScratchBytes : 0};
    return hip_status(smla::launch_attention(a, (hipStream_t)stream), "sparse_mla_decode_noalloc");
}

smla_status smla_sparse_mla_prefill_chunk(const void* q, int64_t q_row_stride, const void* kv, int32_t kv_dtype,
                                          int64_t num_pages, const int32_t* block_table_row, int64_t bt_len,
                                          const int32_t* idx, int32_t T, int32_t H, int32_t k, float softmax_scale,
                                          const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                                          void* stream) {
    smla_status st = check_attention(q, q_row_stride, kv, kv_dtype, num_pages, block_table_row, bt_len, 1, idx, T, H,
                                     k, softmax_scale, out, lse, ws, ws_bytes);
    if (st != SMLA_OK) return st;
    if (T == 0) return ok();
    if (sink && !aligned(sink, 4)) return fail(SMLA_ERR_ALIGNMENT, "sink must be 4-byte aligned");
    smla::AttnArgs a{q,   q_row_stride, kv, kv_dtype, num_pages,     block_table_row, bt_len, 1,   nullptr,
                     idx, T,            H,  k,        softmax_scale, sink,            out,    lse, ws,
                     ws_bytes};
    return hip_status(smla::launch_attention(a, (hipStream_t)stream), "sparse_mla_prefill_chunk");
}

smla_status smla_kv_cache_write(const void* kv_in, int64_t in_row_stride, const int64_t* slot_mapping, int32_t T,
                                void* cache, int32_t kv_dtype, int64_t num_pages, void* stream) {
    smla_status st = check_cache_write(kv_in, in_row_stride, slot_mapping, T, cache, kv_dtype, num_pages);
    if (st != SMLA_OK || T == 0) return st;
    return hip_status(smla::launch_kv_cache_write(kv_in, in_row_stride, slot_mapping, nullptr, nullptr, 0, T, cache,
                                                  kv_dtype, num_pages, (hipStream_t)stream),
                      "kv_cache_write");
}

smla_status smla_kv_cache_write_rope(const void* kv_in, int64_t in_row_stride, const int64_t* slot_mapping,
                                     const int64_t* positions, const float* cos_sin, int64_t max_pos, int32_t T,
                                     void* cache, int32_t kv_dtype, int64_t num_pages, void* stream) {
    smla_status st = check_cache_write(kv_in, in_row_stride, slot_mapping, T, cache, kv_dtype, num_pages);
    if (st != SMLA_OK) return st;
    if (max_pos < 1) return fail(SMLA_ERR_INVALID_ARG, "max_pos=%lld must be >= 1", (long long)max_pos);
    if (T == 0) return ok();
    if (!positions) return fail(SMLA_ERR_INVALID_ARG, "positions is NULL");
    if (!cos_sin) return fail(SMLA_ERR_INVALID_ARG, "cos_sin is NULL");
    if (!aligned(positions, 8)) return fail(SMLA_ERR_ALIGNMENT, "positions must be 8-byte aligned");
    if (!aligned(cos_sin, 4)) return fail(SMLA_ERR_ALIGNMENT, "cos_sin must be 4-byte aligned");
    return hip_status(smla::launch_kv_cache_write(kv_in, in_row_stride, slot_mapping, positions, cos_sin, max_pos, T,
                                                  cache, kv_dtype, num_pages, (hipStream_t)stream),
                      "kv_cache_write_rope");
}

smla_status smla_paged_mqa_logits(const void* q, int64_t q_row_stride, const float* weights, int64_t w_row_stride,
                                  const void* kidx, int64_t num_pages, const int32_t* block_table, int64_t bt_stride,
                                  int32_t num_reqs, const int32_t* row_req, const int32_t* lengths, int32_t rows,
                                  int32_t Hi, float* out, int64_t out_stride, void* stream) {
    if (Hi < 16 || Hi > 64 || Hi % 16 != 0)
        return fail(SMLA_ERR_UNSUPPORTED, "index heads Hi=%d is not supported; supported: 16, 32, 48, 64", Hi);
    if (rows < 0) return fail(SMLA_ERR_INVALID_ARG, "rows=%d must be >= 0", rows);
    if (out_stride < 1 || out_stride > kMaxStride)
        return fail(SMLA_ERR_CAPACITY, "out_stride=%lld is outside [1, %lld]", (long long)out_stride,
                    (long long)kMaxStride);
    if (num_pages < 1) return fail(SMLA_ERR_INVALID_ARG, "num_pages=%lld must be >= 1", (long long)num_pages);
    if (num_pages > kMaxPages)
        return fail(SMLA_ERR_CAPACITY, "num_pages=%lld exceeds the supported maximum %lld", (long long)num_pages,
                    (long long)kMaxPages);
    if (bt_stride < 1) return fail(SMLA_ERR_INVALID_ARG, "bt_stride=%lld must be >= 1", (long long)bt_stride);
    if (num_reqs < 1) return fail(SMLA_ERR_INVALID_ARG, "num_reqs=%d must be >= 1", num_reqs);
    if (q_row_stride < (int64_t)Hi * 128)
        return fail(SMLA_ERR_INVALID_ARG, "q_row_stride=%lld must be >= Hi*128=%lld", (long long)q_row_stride,
                    (long long)Hi * 128);
    if (w_row_stride < Hi)
        return fail(SMLA_ERR_INVALID_ARG, "w_row_stride=%lld must be >= Hi=%d", (long long)w_row_stride, Hi);
    if (rows == 0) return ok();
    if (!q) return fail(SMLA_ERR_INVALID_ARG, "q is NULL");
    if (!weights) return fail(SMLA_ERR_INVALID_ARG, "weights is NULL");
    if (!kidx) return fail(SMLA_ERR_INVALID_ARG, "kidx is NULL");
    if (!block_table) return fail(SMLA_ERR_INVALID_ARG, "block_table is NULL");
    if (!out) return fail(SMLA_ERR_INVALID_ARG, "out is NULL");
    if (!aligned(q, 16)) return fail(SMLA_ERR_ALIGNMENT, "q must be 16-byte aligned");
    if (q_row_stride % 8 != 0)
        return fail(SMLA_ERR_ALIGNMENT, "q_row_stride=%lld must be a multiple of 8 elements", (long long)q_row_stride);
    if (!aligned(weights, 16)) return fail(SMLA_ERR_ALIGNMENT, "weights must be 16-byte aligned");
    if (w_row_stride % 4 != 0)
        return fail(SMLA_ERR_ALIGNMENT, "w_row_stride=%lld must be a multiple of 4 elements", (long long)w_row_stride);
    if (!aligned(kidx, 16)) return fail(SMLA_ERR_ALIGNMENT, "kidx must be 16-byte aligned");
    if (!aligned(block_table, 4)) return fail(SMLA_ERR_ALIGNMENT, "block_table must be 4-byte aligned");
    if (row_req && !aligned(row_req, 4)) return fail(SMLA_ERR_ALIGNMENT, "row_req must be 4-byte aligned");
    if (lengths && !aligned(lengths, 4)) return fail(SMLA_ERR_ALIGNMENT, "lengths must be 4-byte aligned");
    if (!aligned(out, 4)) return fail(SMLA_ERR_ALIGNMENT, "out must be 4-byte aligned");
    smla::IdxArgs a{q,         q_row_stride, weights, w_row_stride, kidx, num_pages, block_table, bt_stride,
                    num_reqs, row_req,      lengths, rows,         Hi,   out,       out_stride};
    return hip_status(smla::launch_paged_mqa_logits(a, (hipStream_t)stream), "paged_mqa_logits");
}

}  // extern "C"
