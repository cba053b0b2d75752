/*
 * smla.h — C ABI of the deterministic, batch-invariant sparse-MLA library for AMD MI355X (gfx950).
 *
 * Per query row the library
 *   1. selects the top k of the row's indexer scores under a composite (score, index) order with a
 *      stable tie-break                          [smla_topk_per_row]
 *   2. emits the selected token positions in ascending order, padded with -1
 *   3. gathers those latent-KV records from a paged cache
 *   4. runs MQA attention in which every head reads the same 576-wide latent record
 *      (512 latent + 64 rope; values are the first 512 entries), with one fixed reduction order
 *                                                [smla_sparse_mla_decode, smla_sparse_mla_prefill_chunk]
 * and writes new tokens' records into the paged cache, quantizing them for FP8 caches and
 * optionally undoing the rotary embedding of the rope part
 *                                                [smla_kv_cache_write, smla_kv_cache_write_rope]
 * and produces the indexer scores the selector ranks  [smla_paged_mqa_logits]
 * The result for a row never depends on the other rows of the call.
 *
 * Sources (pages by title, section):
 *   - "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL" (vllm-project/vllm PR 54955),
 *     sections "Deterministic sparse top-k" (composite score/index key, stable tie-break, canonical
 *     index order before attention, persistent row-start buffers) and "Sparse MLA and FlashMLA"
 *     (decode gathers the selected KV and runs the prefill attention path; prefill chunks each
 *     request on its own; top-k width, gather capacity and workspaces come from model capacity;
 *     length buffers are filled without a host sync).
 *   - "[Bugfix] Make DSV4 sparse MLA work end-to-end for plain decode, MTP, and DSpark"
 *     (vllm-project/vllm PR 51538), section "Purpose": lengths clamped to [0, stride] before any
 *     decision, -1 padding of short rows, slot = block id * block size + offset, unsupported
 *     shapes rejected at init with the missing parameter named.
 *   - "[JJ] Preallocate DeepSeek V4 padded-query output" (local-inference-lab/vllm PR 671),
 *     "Operation contract" / "Resulting behavior": caller-owned outputs, no hidden allocation,
 *     shapes/dtypes/layouts validated before launch.
 *
 * Conventions for every entry point:
 *   - Every buffer pointer is a DEVICE pointer owned by the caller; the library never allocates,
 *     never frees and never synchronizes the host.  Work is enqueued on `stream` (a hipStream_t;
 *     NULL means the null stream) and completes asynchronously.  Addresses may stay fixed across
 *     HIP graph capture and replay; no call records a memset.
 *   - Arguments are validated on the host before anything is enqueued.  On failure nothing is
 *     enqueued, the status says which class of problem it is, and smla_last_error() names the
 *     parameter and the supported values.
 *   - Device-side values are guarded instead of trusted: lengths are clamped to [0, row_stride];
 *     index entries < 0, request ids outside [0, num_reqs), positions past the block table and
 *     page ids outside [0, num_pages) are treated as "no token" (they contribute nothing); nothing
 *     is read outside the buffers described below.
 *   - All offsets are 64-bit.
 *   - Calls that share a workspace must be ordered on one stream.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SMLA_OK = 0,
    SMLA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent strides            */
    SMLA_ERR_UNSUPPORTED = 2,   /* a shape parameter outside the compiled set (message names it) */
    SMLA_ERR_WORKSPACE = 3,     /* workspace pointer missing or smaller than required            */
    SMLA_ERR_ALIGNMENT = 4,     /* a pointer or stride violates the stated alignment             */
    SMLA_ERR_CAPACITY = 5,      /* a size exceeds the capacity limits of this library            */
    SMLA_ERR_HIP = 6            /* the HIP runtime reported an error while enqueueing            */
} smla_status;

typedef enum {
    SMLA_KV_BF16 = 0,           /* record = 576 bf16 (1152 B): 512 latent then 64 rope           */
    SMLA_KV_FP8_E4M3_G128 = 1   /* record = 656 B: 512 OCP e4m3fn codes | 4 fp32 scales (one per
                                   128 latent entries, little endian) | 64 bf16 rope              */
} smla_kv_dtype;

/* Model capacity.  Workspace sizes derive from these numbers only, never from batch contents. */
typedef struct {
    int32_t max_rows;           /* most query rows one attention call carries (>= 1)              */
    int32_t max_k;              /* largest top-k width                                            */
    int32_t num_heads;          /* query heads H                                                  */
    int32_t d_qk;               /* must be 576                                                    */
    int32_t d_v;                /* must be 512                                                    */
    int32_t page_block_size;    /* must be 64                                                     */
    int64_t max_candidates;     /* longest score row (row_stride) top-k will see                  */
    int32_t kv_dtype;           /* smla_kv_dtype                                                  */
    int32_t reserved;           /* must be 0                                                      */
} smla_capacity;

/* Message for the last failing call on this host thread ("" if none).  Never NULL. */
const char* smla_last_error(void);

/* Library version string. */
const char* smla_version(void);

/* Init-time gate: SMLA_OK if the capacity is within what the compiled kernels support, else
 * SMLA_ERR_UNSUPPORTED / SMLA_ERR_CAPACITY with the offending parameter and the supported set
 * in smla_last_error().  Supported: num_heads a multiple of 16 in [16, 128]; d_qk 576; d_v 512;
 * page_block_size 64; 1 <= max_k <= 16384; 1 <= max_candidates <= 2^31 - 1; max_rows >= 1. */
smla_status smla_is_supported(const smla_capacity* cap);

/* Workspace bytes the top-k and attention entry points need for this capacity (either output
 * pointer may be NULL).  Workspaces must be 256-byte aligned.  A larger attention workspace lets
 * one call carry more rows per launch; results do not depend on it. */
smla_status smla_workspace_size(const smla_capacity* cap, size_t* topk_ws_bytes, size_t* attn_ws_bytes);

/* A0, causal candidate counts of a prefill chunk:
 *   lengths[t] = max(0, first_pos + t + 1), clamped to INT32_MAX, for t in [0, T).
 * Query token t sits at position first_pos + t and may attend to positions 0..first_pos+t
 * ("Negative indexer context lengths under MTP": never below 0).
 * lengths: int32 [T] device buffer, 4-byte aligned.  T = 0 enqueues nothing. */
smla_status smla_fill_causal_lengths(int64_t first_pos, int32_t T, int32_t* lengths, void* stream);

/* A1-A3, stable top-k with canonical order, one row per query row.
 *   Row r's candidates are scores[off_r + j] for j in [0, L_r), where
 *   off_r = row_offsets ? row_offsets[r] : r * row_stride   (element offsets, int64) and
 *   L_r = clamp(lengths ? lengths[r] : row_stride, 0, row_stride).
 *   Order: higher score first; equal scores (IEEE ==, so -0.0 == +0.0) by lower index; NaN after
 *   every number, NaNs by lower index.  The first n_r = min(k, L_r) candidates in that order are
 *   written to out_idx[r*k + 0 .. n_r) in ASCENDING index order, and out_idx[r*k + n_r .. k) = -1.
 *   The result is a pure function of the row: bit-identical in any batch.
 * scores: fp32, 4-byte aligned; row_offsets: int64 [rows] or NULL; lengths: int32 [rows] or NULL;
 * out_idx: int32 [rows, k].  Requires 1 <= k <= 16384, 1 <= row_stride <= 2^31 - 1, rows >= 0.
 * ws/ws_bytes: optional top-k workspace, 256-byte aligned (NULL/0 allowed).  With fewer than 256
 *   rows and 114688 < row_stride <= 524288, a workspace of at least 256 + ceil(row_stride/32768) *
 *   98304 bytes per row lets the filtering pass over each row run on several workgroups (one per
 *   32768-candidate chunk); smla_workspace_size reports the size for 255 rows.  The output is
 *   identical with or without it.  Calls sharing a workspace must be stream-ordered. */
smla_status smla_topk_per_row(const float* scores, const int64_t* row_offsets, int64_t row_stride,
                              const int32_t* lengths, int32_t rows, int32_t k, int32_t* out_idx,
                              void* ws, size_t ws_bytes, void* stream);

/* A4-A11, sparse MLA attention over canonical indices (decode rows, or any mix of rows).
 * (smla_sparse_mla_decode_with_window below adds a sliding-window cache to the same call.)
 *   q:      bf16 [rows, H, 576], row r at q + r*q_row_stride elements (q_row_stride >= H*576,
 *           multiple of 8); 16-byte aligned.
 *   kv:     paged cache, [num_pages, 64, record] bytes per kv_dtype; 16-byte aligned.
 *   block_table: int32 [num_reqs, bt_stride]; logical page p of request q is physical page
 *           block_table[q*bt_stride + p].
 *   row_req: int32 [rows] request id of each row, or NULL for "request 0".
 *   idx:    int32 [rows, k] logical token positions (from smla_topk_per_row); entries < 0 skipped.
 *   For row r and head h: s_j = softmax_scale * <q[r,h,:], K_j> over the 576 entries of each
 *   listed token's record K_j; D = sum_j e^{s_j} + e^{sink[h]}; out[r,h,:] = sum_j (e^{s_j} / D)
 *   K_j[0:512] rounded to bf16 (RNE); lse[r,h] = ln D (fp32).  Without a sink (sink NULL, or
 *   sink[h] = -inf) the e^{sink} term is absent and p is the plain softmax.  A row with no valid
 *   token gets out = 0 and lse = sink[h] (-inf without a sink).  Slots are reduced in a fixed order
 *   that depends only on k and kv_dtype: the k slots are cut into splits of 512 slots (FP8 caches:
 *   1024), each split accumulates its tiles in slot order with an fp32 online softmax, the splits
 *   are combined in split order, and the sink term comes last.
 *   sink:   fp32 [H] per-head attention-sink logits, in the units of the scaled scores, or NULL
 *           ("[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL", section "MHC, CUDA
 *           graphs, and weight reload": sink weights keep -inf padding, i.e. -inf = no sink);
 *           entries must be finite or -inf; 4-byte aligned.
 *   out: bf16 [rows, H, 512], 16-byte aligned; lse: fp32 [rows, H] or NULL.
 *   ws: attention workspace (256-byte aligned) of at least the size smla_workspace_size reports for
 *   a capacity with max_rows >= 1; rows beyond what it holds are processed in further launches.
 *   It holds the split partials (bf16; FP8 caches: fp16 with one fp32 power-of-two factor per split
 *   and 128-dim group) and their fp32 LSEs (only with more than one split); calls that share a
 *   workspace must be ordered on one stream.
 * Requires H a multiple of 16 in [16, 128], 1 <= k <= 16384, rows >= 0, num_pages >= 1. */
smla_status smla_sparse_mla_decode(const void* q, int64_t q_row_stride, const void* kv, int32_t kv_dtype,
                                   int64_t num_pages, const int32_t* block_table, int64_t bt_stride,
                                   int32_t num_reqs, const int32_t* row_req, const int32_t* idx,
                                   int32_t rows, int32_t H, int32_t k, float softmax_scale, const float* sink,
                                   void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Decode over compressed and sliding-window KV in one softmax.
 * Sources: "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL", section "Sparse MLA and
 * FlashMLA" (decode gathers compressed and sliding-window KV); "[Bugfix] Make DSV4 sparse MLA work
 * end-to-end ...", section "Purpose", item "SWA widths" (the window + draft width pads to a multiple of
 * the 64-entry tile: 192 for 128 window + 5 draft entries).
 *   Row r attends to the k positions idx[r*k ...] of the main paged cache kv (through block_table) and
 *   to the k_win positions idx_win[r*k_win ...] of the window cache kv_win (through block_table_win,
 *   [num_reqs, bt_win_stride], num_pages_win pages, the same record type and request ids row_req):
 *   one set of keys, one softmax, entries < 0 skipped; everything else (arithmetic, sink, lse, invalid
 *   entries, batch invariance) as smla_sparse_mla_decode over a row of k + k_win slots, the window slots
 *   last.  The reduction order depends on k, k_win and kv_dtype only.
 *   Requires k >= 1, k_win a positive multiple of 64, k + k_win <= 16384; the workspace is that of
 *   smla_sparse_mla_decode at width k + k_win (smla_workspace_size with max_k >= k + k_win). */
smla_status smla_sparse_mla_decode_with_window(const void* q, int64_t q_row_stride, const void* kv, int32_t kv_dtype,
                                              int64_t num_pages, const int32_t* block_table, int64_t bt_stride,
                                              const int32_t* idx, int32_t k, const void* kv_win,
                                              int64_t num_pages_win, const int32_t* block_table_win,
                                              int64_t bt_win_stride, const int32_t* idx_win, int32_t k_win,
                                              int32_t num_reqs, const int32_t* row_req, int32_t rows, int32_t H,
                                              float softmax_scale, const float* sink, void* out, float* lse,
                                              void* ws, size_t ws_bytes, void* stream);

/* smla_sparse_mla_decode without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Arguments,
 * arithmetic, results (bit for bit) and errors are those of smla_sparse_mla_decode; the split partials
 * go to a static 32 MiB device array of the library instead (one per GPU, held until the process ends;
 * its address is looked up once per device).  The call allocates nothing.  Every workspace-free call on
 * a GPU shares that array: such calls must be ordered on one stream (calls that overlap on one GPU
 * race).  Rows beyond what the array holds per launch are processed in further launches; a shape whose
 * single row needs more than 32 MiB of partials is rejected with SMLA_ERR_CAPACITY (no supported shape
 * does: at most 4.2 MB per row). */
smla_status smla_sparse_mla_decode_noalloc(const void* q, int64_t q_row_stride, const void* kv, int32_t kv_dtype,
                                           int64_t num_pages, const int32_t* block_table, int64_t bt_stride,
                                           int32_t num_reqs, const int32_t* row_req, const int32_t* idx,
                                           int32_t rows, int32_t H, int32_t k, float softmax_scale,
                                           const float* sink, void* out, float* lse, void* stream);

/* Prefill chunk of one request: T query rows that all read the request whose block table row is
 * block_table_row (bt_len entries).  Same arithmetic and the same kernels as smla_sparse_mla_decode
 * (row t of a chunk and the same row inside a mixed decode batch give bit-identical results). */
smla_status smla_sparse_mla_prefill_chunk(const void* q, int64_t q_row_stride, const void* kv,
                                          int32_t kv_dtype, int64_t num_pages,
                                          const int32_t* block_table_row, int64_t bt_len,
                                          const int32_t* idx, int32_t T, int32_t H, int32_t k,
                                          float softmax_scale, const float* sink, void* out, float* lse,
                                          void* ws, size_t ws_bytes, void* stream);

/* KV insert: writes the records of T new tokens into the paged cache (the step that produces the
 * records smla_sparse_mla_decode gathers).
 * Sources: "Port DeepSeek-V4 optimization PR #174 to v0.26 ..." (MooreThreads/vllm-musa PR 178), table
 * "Optimizations carried from PR #174" (FP8 cache write, contiguous fp32 scale groups);
 * "[DeepSeek-V4][Preview] Batch-invariant kernels for 0-diff RL", fused group-quantization section
 * (128-element groups, FP32 scales); "[JJ] Preallocate DeepSeek V4 padded-query output", "Operation
 * contract" (the KV-insert operator mutates caller-owned storage only).
 *   kv_in:  bf16 [T, 576] (512 latent then 64 rope), token t at kv_in + t*in_row_stride elements
 *           (in_row_stride >= 576, multiple of 8); 16-byte aligned.
 *   slot_mapping: int64 [T]; token t is written to physical slot slot_mapping[t] = block id * 64 +
 *           offset in the block.  Slots < 0 or >= num_pages*64 are skipped (nothing written).
 *   cache:  [num_pages, 64, record] bytes per kv_dtype, 16-byte aligned; only the records of the
 *           listed slots change.
 *   SMLA_KV_BF16: the record is the 1152 input bytes.
 *   SMLA_KV_FP8_E4M3_G128: for each 128-entry group g of the latent, amax = largest |x|; the
 *           stored scale is s_g = amax / 448 and code = e4m3(x / s_g), the inverse of the
 *           dequantization code * s_g (IEEE fp32 divisions, round-to-nearest-even), the quotient
 *           saturated to [-448, 448] and rounded to the nearest e4m3 value (ties to even mantissa);
 *           a group of zeros stores s_g = 0 and zero codes; the rope is stored unchanged.  Latent
 *           values must be finite (the codes of a group holding inf or NaN are unspecified).
 * Tokens mapped to the same slot race: which record remains is unspecified.  T = 0 enqueues nothing. */
smla_status smla_kv_cache_write(const void* kv_in, int64_t in_row_stride, const int64_t* slot_mapping, int32_t T,
                                void* cache, int32_t kv_dtype, int64_t num_pages, void* stream);

/* KV insert with the rotary embedding of the rope part undone ("inverse-RoPE" cache write).
 * Source: "Port DeepSeek-V4 optimization PR #174 to v0.26 ..." (MooreThreads/vllm-musa PR 178), table
 * "Optimizations carried from PR #174", row "Attention cache write" (inverse-RoPE FP8 cache write,
 * chunks in parallel); "[JJ] Preallocate DeepSeek V4 padded-query output", "Operation contract" (the
 * fused RoPE and KV-insert operator).  The pages do not define the rotation; the convention here:
 *   positions: int64 [T], the position of each token; 8-byte aligned.
 *   cos_sin:   fp32 [max_pos, 64]: row p holds cos(theta_p,i) for i < 32, then sin(theta_p,i);
 *              4-byte aligned.  Rope pair i is (rope[2i], rope[2i+1]).
 *   The stored rope pair is (a c + b s, -a s + b c) for the input pair (a, b), c = cos_sin[p][i],
 *   s = cos_sin[p][32 + i]: the rotation by -theta, which undoes a rotation by +theta.  It is
 *   evaluated with exact products and one fp64 sum, then rounded to bf16 (nearest even); the result
 *   is within one bf16 unit of the exactly rounded rotation (equal to it unless the fp64 sum itself
 *   was inexact next to a bf16 rounding boundary).  A zero result is stored as +0.  Rope inputs must
 *   be finite and the rotated values must fit bf16.
 *   A token whose position lies outside [0, max_pos) is not written (like an invalid slot).
 * Everything else is exactly smla_kv_cache_write; the latent part is not rotated. */
smla_status smla_kv_cache_write_rope(const void* kv_in, int64_t in_row_stride, const int64_t* slot_mapping,
                                     const int64_t* positions, const float* cos_sin, int64_t max_pos, int32_t T,
                                     void* cache, int32_t kv_dtype, int64_t num_pages, void* stream);

/* Indexer scores (paged MQA logits): the per-position scores smla_topk_per_row consumes.
 * Sources: "[SM120] Sync DS4 with upstream main + validated perf backports", sections "September 12
 * follow-up" and "2026-09-12 live validation and promotion update" name the DSA indexer's paged MQA
 * logits without a formula; the formula is the published lightning-indexer form of DeepSeek sparse
 * attention (a reading).  Paging and length clamping as for the latent cache ("[Bugfix] Make DSV4
 * sparse MLA work end-to-end ...", section "Purpose").
 *   q:       bf16 [rows, Hi, 128] index queries, row r at q + r*q_row_stride elements
 *            (q_row_stride >= Hi*128, multiple of 8); 16-byte aligned.
 *   weights: fp32 [rows, Hi] per-row head weights, row r at weights + r*w_row_stride
 *            (w_row_stride >= Hi, multiple of 4); 16-byte aligned.
 *   kidx:    bf16 [num_pages, 64, 128] paged index-key cache (one 128-wide key per token, shared by
 *            every index head); 16-byte aligned.
 *   block_table / bt_stride / num_reqs / row_req: as for smla_sparse_mla_decode.
 *   lengths: int32 [rows] or NULL (NULL: out_stride); L_r = clamp(lengths[r], 0, out_stride).
 *   out:     fp32 [rows, out_stride], 4-byte aligned.  For p < L_r whose page
 *            block_table[req*bt_stride + p/64] lies in [0, num_pages) (with p/64 < bt_stride and req
 *            in [0, num_reqs)):
 *              out[r*out_stride + p] = sum_h weights[r, h] * relu(<q[r, h, :], key_p>),
 *            relu(x) = x if x > 0 else 0, key_p = token p % 64 of that page; every other p in
 *            [0, out_stride) gets -inf.  Every entry of the row is written.
 *   Arithmetic: bf16 products accumulated in fp32 (MFMA, 32 dims per step), then one fp32 fused
 *   multiply-add per head in a fixed order and a fixed pairwise sum over four partial sums; the
 *   result for a row does not depend on the other rows of the call.
 * Requires Hi in {16, 32, 48, 64}, 1 <= out_stride <= 2^31 - 1, rows >= 0, num_pages >= 1.  rows = 0
 * enqueues nothing. */
smla_status smla_paged_mqa_logits(const void* q, int64_t q_row_stride, const float* weights, int64_t w_row_stride,
                                  const void* kidx, int64_t num_pages, const int32_t* block_table, int64_t bt_stride,
                                  int32_t num_reqs, const int32_t* row_req, const int32_t* lengths, int32_t rows,
                                  int32_t Hi, float* out, int64_t out_stride, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
